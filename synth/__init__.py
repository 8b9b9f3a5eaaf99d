"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This package holds no attention arithmetic: it draws N(0, 1) tensors on the
CPU from fixed seeds, rounds them to the stored formats with torch's own casts,
and names the workloads. Both the oracle and the HIP path consume what it
returns; neither is imported here.
"""

from .inputs import (  # noqa: F401
    WORKLOADS,
    Workload,
    normal,
    to_bf16_bits,
    quant_e4m3fn_per_tensor,
    make_inputs,
    random_codes,
    plant_needles,
)
