"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Every case names itself before it touches the GPU. Sizes are chosen so the
oracle finishes in seconds yet the kernel sees several query tiles (256 rows),
several key tiles (64 keys) and ragged tails. At the full video-DiT and GQA
sizes the oracle is evaluated on sampled query rows (each output row depends
only on its own query), always including the first and last rows.

Bars: bf16 max|dO| <= 1e-2 and max|dLSE| <= 1e-3 against the oracle on the
bf16-rounded inputs; fp8 range-normalised NRMS(O) <= 1e-2 against the oracle
on the dequantised e4m3fn inputs, and max|dLSE| <= 1e-3.
"""

import math

import numpy as np
import pytest
import torch

import head_attention_amd as ha
from gpu_helpers import (say, run_gpu, oracle_ref, synth_inputs, check_bf16, check_fp8, make_inputs,
                         WORKLOADS, nrms, frob_rel, to_dev, descale_dev)

pytestmark = pytest.mark.gpu


def sample_rows(S, n, seed):
    r = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, 1, S - 1, S - 2], r.choice(S, size=min(n, S), replace=False)]))
    return rows[(rows >= 0) & (rows < S)]


def check(inp, O, L, Oref, Lref, what):
    if inp["fmt"] == "bf16":
        return check_bf16(O, L, Oref, Lref, what=what)
    return check_fp8(O, L, Oref, Lref, what=what)


# ---------------------------------------------------------------- the five workloads

def test_tiny_fp32_workload():
    w = WORKLOADS["tiny"]
    say(f"case tiny {w}")
    inp = make_inputs(w)
    O, L, _ = run_gpu(inp, w.scale, False)
    Oref, Lref = oracle_ref(inp, w.scale, False)
    check_bf16(O, L, Oref, Lref, what="tiny vs oracle(bf16 inputs)")
    # context only: the same GPU output against the oracle on the unrounded fp32 draws
    import oracle
    O32, L32 = oracle.attention_forward(inp["q32"].double().numpy(), inp["k32"].double().numpy(),
                                        inp["v32"].double().numpy(), w.scale)
    say(f"  tiny vs oracle(fp32 inputs): max|dO|={np.abs(O - O32).max():.3e} max|dLSE|={np.abs(L - L32).max():.3e}")


@pytest.mark.parametrize("causal", [False, True])
def test_llm_workload_full(causal):
    w = WORKLOADS["llm"]
    say(f"case llm causal={causal}")
    inp = make_inputs(w)
    O, L, _ = run_gpu(inp, w.scale, causal)
    Oref, Lref = oracle_ref(inp, w.scale, causal)
    check_bf16(O, L, Oref, Lref, what=f"llm causal={causal}")


@pytest.mark.parametrize("name", ["video_dit", "video_dit_fp8"])
def test_video_dit_full_size_sampled_rows(name):
    w = WORKLOADS[name]
    say(f"case {name} full size, sampled rows")
    inp = make_inputs(w)
    O, L, _ = run_gpu(inp, w.scale, False)
    rows = sample_rows(w.Sq, 60, 3)
    Oref, Lref = oracle_ref(inp, w.scale, False, rows=rows)
    check(inp, O[:, :, rows], L[:, :, rows], Oref, Lref, what=f"{name} rows={len(rows)}")


def test_video_dit_fp8_reduced_full_tensor():
    """fp8 at 1/16 of the sequence, full-tensor NRMS (all rows)."""
    w = WORKLOADS["video_dit_fp8"]
    say("case video_dit_fp8 S=4725 full tensor")
    inp = make_inputs(w, sq=4725, skv=4725)
    O, L, _ = run_gpu(inp, w.scale, False)
    Oref, Lref = oracle_ref(inp, w.scale, False)
    check_fp8(O, L, Oref, Lref, what="fp8 S=4725")
    # context: against the oracle on the unquantised draws
    import oracle
    O32, _ = oracle.attention_forward(inp["q32"].double().numpy(), inp["k32"].double().numpy(),
                                      inp["v32"].double().numpy(), w.scale)
    say(f"  vs unquantised inputs: nrms={nrms(O, O32):.3e} frob_rel={frob_rel(O, O32):.3e} max|dO|={np.abs(O - O32).max():.3e}")


def test_gqa_causal_full_and_chunked_merge():
    w = WORKLOADS["gqa_causal"]
    say("case gqa_causal full + two chunks merged on host")
    inp = make_inputs(w)
    O, L, Og = run_gpu(inp, w.scale, True)
    rows = sample_rows(w.Sq, 48, 5)
    Oref, Lref = oracle_ref(inp, w.scale, True, rows=rows)
    check_bf16(O[:, :, rows], L[:, :, rows], Oref, Lref, what="gqa causal unsplit")
    # two chunks of 4096 keys, each (O, LSE), merged by LSE on the host
    c0 = w.chunks[0]
    O1, L1, O1g = run_gpu(inp, w.scale, True, kv_start=0, k_slice=slice(0, c0))
    O2, L2, O2g = run_gpu(inp, w.scale, True, kv_start=c0, k_slice=slice(c0, None))
    assert np.isneginf(L2[:, :, :c0]).all() and (O2[:, :, :c0, :] == 0).all()
    bits = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
    Om, Lm = ha.merge_lse2_host(bits(O1g), L1, bits(O2g), L2)
    Om = torch.from_numpy(Om.view(np.int16)).view(torch.bfloat16).float().numpy()
    check_bf16(Om, Lm, O, L, what="merged vs unsplit GPU")
    check_bf16(Om[:, :, rows], Lm[:, :, rows], Oref, Lref, what="merged vs oracle")


@pytest.mark.parametrize("name", ["window30", "wan_cross", "wan_cross_fp8"])
def test_sq_ne_skv_full_size_sampled_rows(name):
    """Sq != Skv at full size: query 4680 x key 51480 (12 heads) and 90000 x 512 (40 heads)."""
    w = WORKLOADS[name]
    say(f"case {name} full size, sampled rows")
    inp = make_inputs(w)
    O, L, _ = run_gpu(inp, w.scale, False)
    rows = sample_rows(w.Sq, 40, 11)
    Oref, Lref = oracle_ref(inp, w.scale, False, rows=rows)
    check(inp, O[:, :, rows], L[:, :, rows], Oref, Lref, what=f"{name} rows={len(rows)}")


# ---------------------------------------------------------------- ragged, degenerate, mixed shapes

EDGE = [
    # B, Hq, Hkv, Sq, Skv, D, causal, kv_start
    (1, 1, 1, 1, 1, 128, False, 0),
    (1, 1, 1, 1, 1, 64, True, 0),
    (1, 3, 1, 300, 77, 128, False, 0),
    (2, 2, 2, 77, 1000, 64, False, 0),
    (1, 2, 1, 513, 513, 128, True, 0),
    (1, 4, 2, 700, 300, 128, True, 0),      # causal, Sq > Skv
    (1, 2, 2, 300, 700, 64, True, 0),       # causal, Sq < Skv: top-left, later keys masked
    (1, 2, 1, 600, 250, 128, True, 350),    # causal chunk with a key offset: rows < 350 empty
    (1, 6, 2, 257, 129, 128, False, 0),
    (1, 5, 5, 1000, 2000, 128, False, 0),   # odd head count
    (1, 4, 4, 1000, 512, 128, False, 0),    # even head count, short keys (cross-attention-like)
    (1, 40, 40, 1500, 512, 128, False, 0),  # the cross-attention head count, even
    (1, 9, 9, 1500, 512, 128, False, 0),    # and an odd one
]


@pytest.mark.parametrize("fmt", ["bf16", "e4m3fn"])
@pytest.mark.parametrize("shape", EDGE, ids=[f"B{s[0]}H{s[1]}/{s[2]}S{s[3]}x{s[4]}D{s[5]}c{int(s[6])}o{s[7]}" for s in EDGE])
def test_edge_shapes(shape, fmt):
    B, Hq, Hkv, Sq, Skv, D, causal, ks = shape
    say(f"case edge {shape} {fmt}")
    inp = synth_inputs(B, Hq, Hkv, Sq, Skv, D, fmt, seed=17 + Sq + Skv)
    scale = 1 / math.sqrt(D)
    O, L, _ = run_gpu(inp, scale, causal, kv_start=ks)
    Oref, Lref = oracle_ref(inp, scale, causal, kv_start=ks)
    if fmt == "bf16":
        check_bf16(O, L, Oref, Lref, what=str(shape))
    else:
        live = ~np.isneginf(Lref)
        assert np.array_equal(np.isneginf(L), ~live) and (O[~live] == 0).all()
        check_fp8(O[live], L[live], Oref[live], Lref[live], what=str(shape))


def test_empty_keys_give_zero_and_neg_inf():
    say("case Skv=0")
    Q = torch.randn(1, 2, 100, 128, device="cuda").to(torch.bfloat16)
    K = torch.empty(1, 2, 0, 128, device="cuda", dtype=torch.bfloat16)
    O, L = ha.forward(Q, K, K.clone(), causal=False)
    torch.cuda.synchronize()
    assert (O.float() == 0).all() and torch.isneginf(L).all()


def test_empty_queries_is_a_no_op():
    say("case Sq=0")
    Q = torch.empty(1, 2, 0, 64, device="cuda", dtype=torch.bfloat16)
    K = torch.randn(1, 2, 10, 64, device="cuda").to(torch.bfloat16)
    O, L = ha.forward(Q, K, K.clone())
    torch.cuda.synchronize()
    assert O.numel() == 0 and L.numel() == 0


def test_large_scores_stay_finite():
    """Scores of magnitude ~100 (keys scaled by 30): the running max keeps exp2 in range.

    Outside the N(0,1) regime one key can carry almost all the weight. The
    kernel keeps its running max while every p = 2^(c s - m) of a tile stays
    at most 2^8, so the dominant p is a bf16-rounded value in [1, 256] rather
    than exactly 1:
    its relative rounding error (2^-8 at most) passes straight into O, hence
    the bound 1e-2 + 2^-8 * max|V| here instead of 1e-2.
    """
    say("case large scores")
    inp = synth_inputs(1, 2, 2, 300, 500, 128, "bf16", seed=99, scale_k=30.0)
    O, L, _ = run_gpu(inp, 1 / math.sqrt(128), False)
    Oref, Lref = oracle_ref(inp, 1 / math.sqrt(128), False)
    import oracle
    vmax = float(np.abs(oracle.dequantise(inp["v"], "bf16")).max())
    check_bf16(O, L, Oref, Lref, o_tol=1e-2 + 2 ** -8 * vmax, lse_tol=2e-3, what="large scores")
