"""CPU oracle for the fused attention forward with per-row log-sum-exp.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call,
link or execute anything in this package: only the tests, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it. The
oracle shares no code, header, table or constant with the HIP path under
``head_attention_amd/``, and never imports it.

Contents
--------
``formats``    exact decoders of the stored element formats (bf16 bit patterns,
               OCP FP8 e4m3fn codes) into float64, written from the formats'
               definitions.
``attention``  the plain fp64 forward: dequantise, GQA head map, scores,
               causal mask with a key offset, softmax normalisation, output and
               natural-log LSE; plus the merge of partial (O, LSE) results.
``backward``   the plain fp64 backward (dQ, dK, dV) by the chain rule on the
               same forward definition, with P recomputed from Q and K.
``brute``      a pure-Python nested-loop version for tiny shapes, computed by a
               different route (no max subtraction, ``math.fsum``), used only to
               pin the numpy version.

Every function is pinned by ``tests/test_oracle_pins.py`` against values the
mathematics or the pages fix (closed forms, invariants, brute force, library
routines, the pages' printed figures). No function here is "parity unpinned".
"""

from .formats import decode_bf16, decode_e4m3fn, dequantise  # noqa: F401
from .attention import attention_forward, merge_lse  # noqa: F401
from .backward import attention_backward  # noqa: F401
