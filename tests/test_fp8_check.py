"""The fp8 parity check against kernels emulated on the CPU (no GPU).

An fp8 attention forward feeds each softmax weight to the P V product as an
e4m3fn value: its relative rounding error is at most 2^-4. ``check_fp8`` holds
a kernel to that: range-normalised NRMS <= 1e-2 (the pass bar), plus the
Frobenius-relative error <= 1.5 x its expected size 2^-4 / sqrt(8 ln 2) and the
elementwise first-order bound
|dO| <= 2^-4 sum_j P_ij |v_jd| + 2^-8 |O| + 2^-10. Here a numpy emulation of
such a kernel (exact P, rounded to e4m3fn after a 2^4 pre-scale, normalised by
the unrounded row sum, O rounded to bf16) must pass, and the same emulation
with one plausible slip of a tiled kernel (a tile's P meeting the wrong V rows,
keys permuted inside a tile, a tile missing from O, a stale P) must fail, some
of them only through the guards.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import check_fp8, nrms
from synth import normal, quant_e4m3fn_per_tensor

TILE = 64


def e4m3(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).to(torch.float64).numpy()


def emulate(q, k, v, scale, mistake=None):
    """One head: q [Sq, D], k/v [Skv, D] dequantised fp64. Returns (O, LSE)."""
    s = scale * q @ k.T
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    w = e4m3(p * 16.0) / 16.0
    vv = v.copy()
    t = 3 * TILE                       # the tile a slip hits
    if mistake == "v_of_previous_tile":     # P of tile 3 meets V of tile 2
        vv[t:t + TILE] = v[t - TILE:t]
    elif mistake == "keys_permuted_in_tile":  # P's key order inside a tile differs from V's
        vv[t:t + TILE] = np.concatenate([v[t + 32:t + TILE], v[t:t + 32]])
    elif mistake == "tile_missing_from_o":     # a tile counted in l but not in O
        w[:, t:t + TILE] = 0.0
    elif mistake == "stale_p":                 # P of tile 2 used again for tile 3
        w[:, t:t + TILE] = w[:, t - TILE:t]
    O = bf16((w @ vv) / l)
    return O, (m + np.log(l))[:, 0]


def case(Sq=256, Skv=2048, D=128, seed=31):
    q32, k32, v32 = normal((Sq, D), seed), normal((Skv, D), seed + 1), normal((Skv, D), seed + 2)
    (qc, qd), (kc, kd), (vc, vd) = (quant_e4m3fn_per_tensor(x) for x in (q32, k32, v32))
    q, k, v = (oracle.dequantise(c, "e4m3fn", d) for c, d in ((qc, qd), (kc, kd), (vc, vd)))
    scale = 1 / np.sqrt(D)
    Oref, Lref = oracle.attention_forward(q[None, None], k[None, None], v[None, None], scale)
    Aref, _ = oracle.attention_forward(q[None, None], k[None, None], np.abs(v)[None, None], scale)
    return q, k, v, scale, Oref[0, 0], Lref[0, 0], Aref[0, 0]


def test_correct_emulation_passes():
    q, k, v, scale, Oref, Lref, Aref = case()
    O, L = emulate(q, k, v, scale)
    check_fp8(O, L, Oref, Lref, Aref, what="e4m3 P emulation")


@pytest.mark.parametrize("mistake", ["v_of_previous_tile", "keys_permuted_in_tile", "tile_missing_from_o",
                                     "stale_p"])
def test_slips_fail(mistake):
    q, k, v, scale, Oref, Lref, Aref = case()
    O, L = emulate(q, k, v, scale, mistake)
    with pytest.raises(AssertionError):
        check_fp8(O, L, Oref, Lref, Aref, what=mistake)


def test_guards_catch_what_nrms_alone_misses():
    """Over 512 key tiles a one-tile slip stays inside the NRMS bar; the guards still
    reject it, while the correct emulation passes them."""
    q, k, v, scale, Oref, Lref, Aref = case(Sq=128, Skv=32768)
    O, L = emulate(q, k, v, scale)
    check_fp8(O, L, Oref, Lref, Aref, what="e4m3 P emulation, 32768 keys")
    for mistake in ("v_of_previous_tile", "keys_permuted_in_tile", "tile_missing_from_o", "stale_p"):
        O, L = emulate(q, k, v, scale, mistake)
        assert nrms(O, Oref) <= 1e-2, mistake
        with pytest.raises(AssertionError):
            check_fp8(O, L, Oref, Lref, Aref, what=mistake)
