"""Attention backward (attn_bwd) against the fp64 backward oracle.

The forward (O, LSE) comes from the HIP path itself (attn_fwd), as a caller's
would; dO is a seeded N(0, 1) draw rounded to bf16. The oracle differentiates
the attention of the same bf16-rounded q, k, v (and dO) in float64.

Bar (each of dQ, dK, dV): ||G - G_ref||_F <= 1e-2 * ||G_ref||_F and
max |G - G_ref| <= 2e-2 * max |G_ref|. Derivation: the kernel rounds three
things to bf16 (unit roundoff u = 2^-8): P and dS as MFMA operands and the
output itself; each rounding is a relative perturbation of RMS u / sqrt(12)
~ 1.1e-3, independent across elements, and O enters D_i = dO_i . O_i as the
forward's bf16 output (another ~1.1e-3). Errors of independent terms add in
quadrature, so the expected relative Frobenius error is a few 1e-3; 1e-2 leaves
a factor of about three. The max-error bar is relative to the tensor's largest
entry because entries near zero carry the absolute error of their larger
neighbours' sums.

Also checked: identical inputs give identical bits; a batch entry's
gradients do not depend on the other entries of the batch (the property the
page "feat(attention): add strict bitwise ROCm path" tests as batch
composition).
"""

import math

import numpy as np
import pytest
import torch

import head_attention_amd as ha
import oracle
from gpu_helpers import say, to_dev, DEV, check_grad
from synth import normal, to_bf16_bits, WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


def bf16_inputs(B, Hq, Hkv, Sq, Skv, D, seed):
    q = to_bf16_bits(normal((B, Hq, Sq, D), seed))
    k = to_bf16_bits(normal((B, Hkv, Skv, D), seed + 1))
    v = to_bf16_bits(normal((B, Hkv, Skv, D), seed + 2))
    do = to_bf16_bits(normal((B, Hq, Sq, D), seed + 3))
    return q, k, v, do


def run_bwd(q, k, v, do, scale, causal):
    Q, K, V, dO = (to_dev(x, "bf16") for x in (q, k, v, do))
    O, L = ha.forward(Q, K, V, scale=scale, causal=causal)
    dQ, dK, dV = ha.backward(Q, K, V, O, dO, L, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return dQ, dK, dV


def f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def dec(x):
    return oracle.dequantise(x, "bf16", 1.0)


CASES = [
    # B, Hq, Hkv, Sq, Skv, D, causal
    (1, 2, 2, 256, 256, 128, False),
    (1, 2, 2, 300, 300, 128, True),      # ragged query and key tiles
    (2, 4, 2, 200, 333, 128, False),     # GQA (per-head partials summed over the group)
    (1, 4, 1, 257, 513, 64, True),       # D64, GQA 4:1, causal with Sq < Skv
    (1, 2, 2, 513, 129, 64, False),      # Sq > Skv
    (1, 2, 2, 129, 700, 128, True),      # keys past the last query get zero gradients
    (1, 1, 1, 1, 1, 128, False),         # one query, one key: dQ = dK = 0, dV = dO
    (1, 8, 2, 1024, 1024, 128, True),
    (64, 4, 2, 64, 1024, 128, False),    # enough KV-head blocks to sum the group in registers
    (64, 4, 2, 100, 1024, 64, True),
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}H{c[1]}/{c[2]}S{c[3]}x{c[4]}D{c[5]}c{int(c[6])}" for c in CASES])
def test_backward_matches_oracle(case):
    B, Hq, Hkv, Sq, Skv, D, causal = case
    say(f"case backward {case}")
    q, k, v, do = bf16_inputs(B, Hq, Hkv, Sq, Skv, D, seed=100 + Sq + 3 * Skv)
    scale = 1 / math.sqrt(D)
    dQ, dK, dV = run_bwd(q, k, v, do, scale, causal)
    rq, rk, rv = oracle.attention_backward(dec(q), dec(k), dec(v), dec(do), scale, causal)
    for got, ref, name in ((dQ, rq, "dQ"), (dK, rk, "dK"), (dV, rv, "dV")):
        check_grad(f64(got), ref, f"{name} {case}")
    if causal and Skv > Sq:
        assert (f64(dK)[:, :, Sq:] == 0).all() and (f64(dV)[:, :, Sq:] == 0).all()


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("Sq,Skv,bounds", [(700, 700, (0, 300, 700)), (700, 700, (0, 64, 333, 700)),
                                           (500, 900, (0, 256, 257, 900))])
def test_backward_key_chunks_sum_to_full(causal, Sq, Skv, bounds):
    """attn_bwd_chunk over key chunks, each with the full softmax's O and LSE: the
    chunks' dQ add up to the full dQ and their dK / dV are the full ones' slices
    (the backward of a context-parallel split of the keys)."""
    say(f"case backward chunks causal={causal} Sq={Sq} Skv={Skv} bounds={bounds}")
    B, Hq, Hkv, D = 1, 4, 2, 128
    q, k, v, do = bf16_inputs(B, Hq, Hkv, Sq, Skv, D, seed=55 + len(bounds))
    scale = 1 / math.sqrt(D)
    Q, K, V, dO = (to_dev(x, "bf16") for x in (q, k, v, do))
    O, L = ha.forward(Q, K, V, scale=scale, causal=causal)
    dq = np.zeros((B, Hq, Sq, D))
    dks, dvs = [], []
    for a, b in zip(bounds[:-1], bounds[1:]):
        Kc, Vc = K[:, :, a:b].contiguous(), V[:, :, a:b].contiguous()
        gq, gk, gv = ha.backward(Q, Kc, Vc, O, dO, L, scale=scale, causal=causal, kv_start=a)
        torch.cuda.synchronize()
        dq += f64(gq)
        dks.append(f64(gk))
        dvs.append(f64(gv))
    rq, rk, rv = oracle.attention_backward(dec(q), dec(k), dec(v), dec(do), scale, causal)
    check_grad(dq, rq, "dQ (sum over chunks)")
    check_grad(np.concatenate(dks, axis=2), rk, "dK (chunks)")
    check_grad(np.concatenate(dvs, axis=2), rv, "dV (chunks)")


def test_backward_is_deterministic_and_batch_invariant():
    say("case backward determinism / batch composition")
    B, Hq, Hkv, S, D = 3, 4, 2, 333, 128
    q, k, v, do = bf16_inputs(B, Hq, Hkv, S, S, D, seed=7)
    scale = 1 / math.sqrt(D)
    a = run_bwd(q, k, v, do, scale, True)
    b = run_bwd(q, k, v, do, scale, True)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    for i in range(B):
        s = run_bwd(*(np.ascontiguousarray(t[i:i + 1]) for t in (q, k, v, do)), scale, True)
        for x, y in zip(a, s):
            assert torch.equal(x[i:i + 1], y), f"batch entry {i} differs when run alone"


def test_backward_grouped_heads_in_registers_equal_partials():
    """The two ways of summing a KV head's group (in registers, or fp32 partials
    summed by a second kernel) agree to fp32 rounding: 64 batch entries select the
    first, one entry the second."""
    say("case backward group-sum paths")
    q, k, v, do = bf16_inputs(64, 4, 2, 64, 1024, 128, seed=21)
    scale = 1 / math.sqrt(128)
    assert ha.attn_bwd_workspace_bytes(64, 4, 2, 64, 1024, 128) == 64 * 4 * 64 * 8
    assert ha.attn_bwd_workspace_bytes(1, 4, 2, 64, 1024, 128) > 4 * 64 * 8
    full = run_bwd(q, k, v, do, scale, False)
    one = run_bwd(*(np.ascontiguousarray(t[5:6]) for t in (q, k, v, do)), scale, False)
    for x, y in zip(full, one):
        d = float((x[5:6].float() - y.float()).abs().max())
        assert d <= 2e-2 * float(y.float().abs().max())


def test_backward_empty_sides():
    say("case backward Skv = 0 and Sq = 0")
    q, k, v, do = bf16_inputs(1, 2, 2, 40, 0, 128, seed=3)
    Q, K, V, dO = (to_dev(x, "bf16") for x in (q, k, v, do))
    O = torch.zeros_like(Q)
    L = torch.full((1, 2, 40), float("-inf"), device=DEV)
    dQ, dK, dV = ha.backward(Q, K, V, O, dO, L)
    torch.cuda.synchronize()
    assert (dQ == 0).all() and dK.numel() == 0
    q, k, v, do = bf16_inputs(1, 2, 2, 0, 50, 128, seed=4)
    Q, K, V, dO = (to_dev(x, "bf16") for x in (q, k, v, do))
    dQ, dK, dV = ha.backward(Q, K, V, torch.zeros_like(Q), dO, torch.zeros((1, 2, 0), device=DEV))
    torch.cuda.synchronize()
    assert (dK == 0).all() and (dV == 0).all()


def test_backward_llm_full_size_properties():
    """The timed backward shape (B1 Hq32 Hkv8 S4096 D128 causal) at full size:
    sampled dQ rows against the oracle (row i of dQ needs only query i and keys
    0..i), and the softmax identities for dK and dV over every key and head."""
    w = WORKLOADS["bwd_llm"]
    say(f"case backward full size {w.name}")
    q, k, v, do = bf16_inputs(w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.D, seed=1000 * w.wid)
    dQ, dK, dV = run_bwd(q, k, v, do, w.scale, True)
    dq, dk, dv = f64(dQ), f64(dK), f64(dV)
    qd, kd, vd, dod = dec(q), dec(k), dec(v), dec(do)
    for i in (0, 1, 63, 64, 1000, 2047, 4095):
        rq, _, _ = oracle.attention_backward(qd[:, :, i:i + 1], kd[:, :, :i + 1], vd[:, :, :i + 1],
                                             dod[:, :, i:i + 1], w.scale, False)
        check_grad(dq[:, :, i:i + 1], rq, f"dQ row {i}")
    # sum over keys of dK is zero (up to the bf16 rounding of each entry)
    tot = np.abs(dk).sum(axis=2)
    assert (np.abs(dk.sum(axis=2)) <= 2e-2 * tot + 1e-6).all()
    # sum over keys of dV equals the sum of dO over the group's rows
    want = dod.reshape(w.B, w.Hkv, w.Hq // w.Hkv, w.Sq, w.D).sum(axis=(2, 3))
    got = dv.sum(axis=2)
    assert np.abs(got - want).max() <= 1e-2 * np.abs(dv).sum(axis=2).max()


def test_backward_graph_capture_replays():
    """attn_bwd (dQ, dK/dV and group-sum kernels, no memsets) captured in a HIP graph on a
    side stream: every replay, with eager work in between, gives the eager bits."""
    say("case backward hip graph capture")
    B, Hq, Hkv, S, D = 1, 4, 2, 500, 128
    q, k, v, do = bf16_inputs(B, Hq, Hkv, S, S, D, seed=31)
    scale = 1 / math.sqrt(D)
    Q, K, V, dO = (to_dev(x, "bf16") for x in (q, k, v, do))
    O, L = ha.forward(Q, K, V, scale=scale, causal=True)
    ref = ha.backward(Q, K, V, O, dO, L, scale=scale, causal=True)
    need = ha.attn_bwd_workspace_bytes(B, Hq, Hkv, S, S, D)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        st = ha.attn_bwd(Q, K, V, O, dO, L, dQ, dK, dV, B, Hq, Hkv, S, S, D, scale, True, ha.ATTN_BF16,
                         ws, need, side.cuda_stream)
    assert st == 0
    for rep in range(3):
        dQ.fill_(float("nan"))
        dK.fill_(float("nan"))
        dV.fill_(float("nan"))
        ws.fill_(255)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((dQ, dK, dV), ref):
            assert torch.equal(got, want), f"replay {rep} differs from the eager result"

