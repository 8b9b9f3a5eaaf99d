"""The largest single-head slices the boundary accepts, against the fp64 oracle.

The limits are the ones attn.h documents for ATTN_ERR_OVERFLOW (one head's slice
plus one tile stays below 2^31 bytes); ``test_abi.py`` checks that one more row
or key is refused. Inputs are stored-format codes drawn as bits
(``synth.random_codes``), because 10^9 N(0, 1) draws would take minutes.

Longest key range: each query row r gets a "needle", key ``pos[r]`` = 2^e q_r,
at positions spread over the whole range from key 0 to the very last key, with
the smallest e in 1..4 that lifts the needle's score to ln(Skv) + 1.5, so that
the needle dominates the row's output (a misread or skipped key tile anywhere
in the range, most of all in the last tiles where the byte offsets are largest,
changes the row); in the rows whose needle lands just above that score the
other keys still move the LSE by more than its tolerance. The oracle runs over
key chunks of 2^20 and merges them by LSE (its ``merge_lse``), so its memory
stays bounded.

Longest query range: the keys are few, the rows sampled include the first and
the last tiles of the range.

The backward (bf16) has its own limits, (Skv + 256) * D * 4 < 2^31 (fp32 key
partials) and (Sq + 256) * D * 2 < 2^31. Its longest key range, with the same
needles, is compared with the full fp64 backward oracle (about 20 GB of host
memory). There the rows are nearly one key each, so dP - D is a small
difference of larger numbers and the bf16 rounding of O in D = dO . O decides
it: both sides are given the same O and LSE, the oracle's own forward (over
key chunks) rounded to bf16 / fp32, and the oracle forms D from that O. The
longest query range runs the whole pipeline (the kernel's forward feeds its
backward) against the exact oracle over blocks of 2^20 query rows (without a
mask each row's softmax is its own, so the blocks' dK and dV add up to the
whole).
"""

import math

import numpy as np
import pytest
import torch

import head_attention_amd as ha
import oracle
from synth import random_codes, plant_needles, to_bf16_bits
from gpu_helpers import say, check_bf16, check_fp8, check_grad, to_dev

pytestmark = pytest.mark.gpu

MAX_SKV = {"bf16": 8388543, "e4m3fn": 16777151}   # D = 128: (Skv + 64) * 128 * elt < 2^31
MAX_SQ = {128: 8388351, 64: 16776959}             # (Sq + 256) * D * 2 < 2^31
BWD_MAX_SKV = 4194047                             # D = 128: (Skv + 256) * 128 * 4 < 2^31


def oracle_chunked(qc, kc, vc, fmt, scale, chunk=1 << 20):
    """Oracle over [0, Skv) in key chunks, merged by LSE; qc [R, D], kc/vc [Skv, D] codes."""
    q = oracle.dequantise(qc, fmt, 1.0)[None, None]
    parts = []
    for a in range(0, kc.shape[0], chunk):
        k = oracle.dequantise(kc[a:a + chunk], fmt, 1.0)[None, None]
        v = oracle.dequantise(vc[a:a + chunk], fmt, 1.0)[None, None]
        parts.append(oracle.attention_forward(q, k, v, scale))
    O, L = oracle.merge_lse(parts)
    return O[0, 0], L[0, 0]


@pytest.mark.parametrize("fmt", ["bf16", "e4m3fn"])
def test_longest_key_range_needles(fmt):
    Skv, Sq, D = MAX_SKV[fmt], 40, 128
    say(f"case max Skv {fmt}: Sq={Sq} Skv={Skv}")
    q = random_codes((Sq, D), fmt, 71)
    k = random_codes((Skv, D), fmt, 72)
    v = random_codes((Skv, D), fmt, 73)
    pos = [round(r * (Skv - 1) / (Sq - 1)) for r in range(Sq)]
    assert pos[0] == 0 and pos[-1] == Skv - 1
    scale = 1 / math.sqrt(D)
    qn = scale * (oracle.dequantise(q, fmt, 1.0) ** 2).sum(axis=1)      # a needle of 2^e q scores 2^e qn
    steps = [next((e for e in (1, 2, 3, 4) if (1 << e) * x >= math.log(Skv) + 1.5), 4) for x in qn]
    plant_needles(q, k, pos, fmt, steps)
    Q, K, V = (to_dev(x.reshape(1, 1, *x.shape), fmt) for x in (q, k, v))
    one = torch.ones(1, dtype=torch.float32, device="cuda") if fmt == "e4m3fn" else None
    Oref, Lref = oracle_chunked(q, k, v, fmt, scale)
    for split in (False, True):
        if split:
            n = ha.attn_splitkv_auto_splits(1, 1, Sq, Skv, D)
            assert n > 16, n            # a single query tile against 2^17+ key tiles
            O, L = ha.forward_splitkv(Q, K, V, n_splits=0, scale=scale, q_descale=one, k_descale=one,
                                      v_descale=one)
        else:
            O, L = ha.forward(Q, K, V, scale=scale, q_descale=one, k_descale=one, v_descale=one)
        torch.cuda.synchronize()
        On, Ln = O.float().cpu().numpy()[0, 0], L.cpu().numpy()[0, 0]
        what = f"max Skv {fmt} {'split' if split else 'unsplit'}"
        # the needle decides each row: its value row must dominate the output
        w = np.einsum("rd,rd->r", On, oracle.dequantise(v[pos], fmt, 1.0)) / \
            np.einsum("rd,rd->r", oracle.dequantise(v[pos], fmt, 1.0), oracle.dequantise(v[pos], fmt, 1.0))
        say(f"  {what}: needle weight min {w.min():.3f}")
        assert (w > 0.5).all(), what
        if fmt == "bf16":
            check_bf16(On, Ln, Oref, Lref, what=what)
        else:
            check_fp8(On, Ln, Oref, Lref, what=what)
        del O, L
    del Q, K, V
    torch.cuda.empty_cache()


@pytest.mark.parametrize("D", [128, 64])
def test_longest_query_range_sampled_rows(D):
    Sq, Skv, fmt = MAX_SQ[D], 100, "bf16"
    say(f"case max Sq D{D}: Sq={Sq} Skv={Skv}")
    q = random_codes((Sq, D), fmt, 81)
    k = random_codes((Skv, D), fmt, 82)
    v = random_codes((Skv, D), fmt, 83)
    scale = 1 / math.sqrt(D)
    Q, K, V = (to_dev(x.reshape(1, 1, *x.shape), fmt) for x in (q, k, v))
    O, L = ha.forward(Q, K, V, scale=scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(84)
    rows = np.unique(np.concatenate([np.arange(0, 300), np.arange(Sq - 600, Sq),
                                     rng.integers(0, Sq, 200)]))
    idx = torch.from_numpy(rows).cuda()
    On = O[0, 0].index_select(0, idx).float().cpu().numpy()
    Ln = L[0, 0].index_select(0, idx).cpu().numpy()
    assert bool(torch.isfinite(L).all()), "every row has keys: LSE must be finite"
    Oref, Lref = oracle.attention_forward(oracle.dequantise(q[rows], fmt, 1.0)[None, None],
                                          oracle.dequantise(k, fmt, 1.0)[None, None],
                                          oracle.dequantise(v, fmt, 1.0)[None, None], scale)
    check_bf16(On, Ln, Oref[0, 0], Lref[0, 0], what=f"max Sq D{D} ({len(rows)} sampled rows)")
    del O, L, Q, K, V
    torch.cuda.empty_cache()


def needle_steps(q, fmt, scale, Skv):
    """Per-row needle exponent: the smallest e in 1..4 with 2^e * scale * |q_r|^2 >= ln Skv + 1.5."""
    qn = scale * (oracle.dequantise(q, fmt, 1.0) ** 2).sum(axis=1)
    return [next((e for e in (1, 2, 3, 4) if (1 << e) * x >= math.log(Skv) + 1.5), 4) for x in qn]


def test_backward_longest_key_range_needles():
    Skv, Sq, D, fmt = BWD_MAX_SKV, 40, 128, "bf16"
    say(f"case backward max Skv: Sq={Sq} Skv={Skv}")
    scale = 1 / math.sqrt(D)
    q = random_codes((Sq, D), fmt, 91)
    k = random_codes((Skv, D), fmt, 92)
    v = random_codes((Skv, D), fmt, 93)
    do = random_codes((Sq, D), fmt, 94)
    pos = [round(r * (Skv - 1) / (Sq - 1)) for r in range(Sq)]
    plant_needles(q, k, pos, fmt, needle_steps(q, fmt, scale, Skv))
    Oref, Lref = oracle_chunked(q, k, v, fmt, scale)
    o_in = to_bf16_bits(torch.from_numpy(Oref.astype(np.float32)))
    Q, K, V, dO, O = (to_dev(x.reshape(1, 1, *x.shape), fmt) for x in (q, k, v, do, o_in))
    L = torch.from_numpy(Lref.astype(np.float32).reshape(1, 1, Sq)).cuda()
    dQ, dK, dV = ha.backward(Q, K, V, O, dO, L, scale=scale)
    torch.cuda.synchronize()
    gq, gk, gv = (t.float().cpu().numpy()[0, 0].astype(np.float64) for t in (dQ, dK, dV))
    del Q, K, V, dO, O, L, dQ, dK, dV
    torch.cuda.empty_cache()
    rq, rk, rv = oracle.attention_backward(*(oracle.dequantise(x, fmt, 1.0)[None, None] for x in (q, k, v, do)), scale,
                                           out=oracle.dequantise(o_in, fmt, 1.0)[None, None])
    rq, rk, rv = rq[0, 0], rk[0, 0], rv[0, 0]
    check_grad(gq, rq, "max Skv dQ")
    check_grad(gk, rk, "max Skv dK")
    check_grad(gv, rv, "max Skv dV")
    # the keys other than the needles carry little weight each: checked on their own
    bulk = np.ones(Skv, dtype=bool)
    bulk[pos] = False
    check_grad(gk[bulk], rk[bulk], "max Skv dK, non-needle keys")
    check_grad(gv[bulk], rv[bulk], "max Skv dV, non-needle keys")


def test_backward_longest_query_range():
    Sq, Skv, D, fmt = MAX_SQ[128], 100, 128, "bf16"
    say(f"case backward max Sq: Sq={Sq} Skv={Skv}")
    scale = 1 / math.sqrt(D)
    q = random_codes((Sq, D), fmt, 101)
    k = random_codes((Skv, D), fmt, 102)
    v = random_codes((Skv, D), fmt, 103)
    do = random_codes((Sq, D), fmt, 104)
    Q, K, V, dO = (to_dev(x.reshape(1, 1, *x.shape), fmt) for x in (q, k, v, do))
    O, L = ha.forward(Q, K, V, scale=scale)
    dQ, dK, dV = ha.backward(Q, K, V, O, dO, L, scale=scale)
    torch.cuda.synchronize()
    gk, gv = (t.float().cpu().numpy()[0, 0].astype(np.float64) for t in (dK, dV))
    kd, vd = oracle.dequantise(k, fmt, 1.0)[None, None], oracle.dequantise(v, fmt, 1.0)[None, None]
    rk, rv = np.zeros((Skv, D)), np.zeros((Skv, D))
    n2d = n2r = mx = mref = 0.0
    blk = 1 << 20
    for a in range(0, Sq, blk):
        rq, pk, pv = oracle.attention_backward(oracle.dequantise(q[a:a + blk], fmt, 1.0)[None, None], kd, vd,
                                               oracle.dequantise(do[a:a + blk], fmt, 1.0)[None, None], scale)
        rk += pk[0, 0]
        rv += pv[0, 0]
        g = dQ[0, 0, a:a + blk].float().cpu().numpy().astype(np.float64)
        d = g - rq[0, 0]
        n2d += float((d * d).sum())
        n2r += float((rq * rq).sum())
        mx = max(mx, float(np.abs(d).max()))
        mref = max(mref, float(np.abs(rq).max()))
    del Q, K, V, dO, O, L, dQ, dK, dV
    torch.cuda.empty_cache()
    fro = math.sqrt(n2d / n2r)
    say(f"  max Sq dQ: frob_rel={fro:.3e} max|d|={mx:.3e} (max|ref|={mref:.3e})")
    assert fro <= 1e-2 and mx <= 2e-2 * mref, "max Sq dQ"
    check_grad(gk, rk, "max Sq dK")
    check_grad(gv, rv, "max Sq dV")
