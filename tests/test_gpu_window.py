"""Local attention (attn_fwd_window: window_size_left / window_size_right and sink
keys) against the fp64 oracle.

The bars are those of the dense path (bf16: max|dO| <= 1e-2, max|dLSE| <= 1e-3;
fp8: range-normalised NRMS <= 1e-2, max|dLSE| <= 1e-3). Rows whose window holds no
key must come back as O = 0, LSE = -inf. The shapes put the band edges inside
key tiles, across tile boundaries and past the ragged tail, so the kernel's three
tile kinds (skipped, whole, masked) all occur.
"""

import math

import numpy as np
import pytest
import torch

import head_attention_amd as ha
import oracle
from gpu_helpers import say, synth_inputs, check_bf16, check_fp8, to_dev, descale_dev, make_inputs, WORKLOADS

pytestmark = pytest.mark.gpu


def run_window(inp, scale, causal, wl, wr, sink, kv_start=0):
    fmt = inp["fmt"]
    qd, kd, vd = (descale_dev(inp[n]) for n in ("q_descale", "k_descale", "v_descale")) if fmt == "e4m3fn" else (None,) * 3
    Q, K, V = to_dev(inp["q"], fmt), to_dev(inp["k"], fmt), to_dev(inp["v"], fmt)
    O, L = ha.forward(Q, K, V, scale=scale, causal=causal, q_descale=qd, k_descale=kd, v_descale=vd,
                      kv_start=kv_start, window_left=wl, window_right=wr, sink=sink)
    torch.cuda.synchronize()
    return O.float().cpu().numpy(), L.cpu().numpy()


def oracle_window(inp, scale, causal, wl, wr, sink, kv_start=0, rows=None, abs_v=False):
    fmt = inp["fmt"]
    q = oracle.dequantise(inp["q"], fmt, inp["q_descale"])
    k = oracle.dequantise(inp["k"], fmt, inp["k_descale"])
    v = oracle.dequantise(inp["v"], fmt, inp["v_descale"])
    return oracle.attention_forward(q, k, np.abs(v) if abs_v else v, scale, causal, kv_start, rows=rows,
                                    window_left=wl, window_right=wr, sink=sink)


def check(inp, O, L, Oref, Lref, what, Aref=None):
    if inp["fmt"] == "bf16":
        check_bf16(O, L, Oref, Lref, what=what)
    else:
        live = ~np.isneginf(Lref)
        assert np.array_equal(np.isneginf(L), ~live), f"{what}: -inf LSE rows differ"
        assert (O[~live] == 0).all()
        check_fp8(O[live], L[live], Oref[live], Lref[live], Aref[live] if Aref is not None else None, what=what)


CASES = [
    # B, Hq, Hkv, Sq, Skv, D, causal, window_left, window_right, sink, kv_start, fmt
    (1, 2, 2, 700, 700, 128, False, 100, 100, 0, 0, "bf16"),     # symmetric band across tiles
    (1, 4, 2, 1000, 1000, 128, True, 256, -1, 4, 0, "bf16"),     # causal sliding window + sinks, GQA
    (1, 2, 2, 600, 900, 64, False, -1, 50, 0, 0, "bf16"),        # right side only, D64
    (2, 2, 1, 513, 777, 128, False, 0, 0, 0, 0, "bf16"),         # width zero: O_i = v_i
    (1, 2, 2, 500, 500, 128, True, 63, -1, 64, 0, "bf16"),       # sink = one whole key tile
    (1, 2, 2, 400, 300, 128, False, 50, 50, 3, 200, "bf16"),     # chunk call: keys start at 200
    (1, 2, 2, 300, 1000, 128, False, 40, 700, 0, 0, "bf16"),     # band reaching past the last key
    (1, 2, 2, 300, 300, 128, False, 5000, 5000, 0, 0, "bf16"),   # window wider than everything
    (1, 2, 2, 700, 700, 128, False, 128, 128, 0, 0, "e4m3fn"),
    (1, 4, 2, 600, 600, 128, True, 200, -1, 8, 0, "e4m3fn"),
    (1, 2, 2, 500, 800, 64, False, 30, 60, 2, 0, "e4m3fn"),
]


@pytest.mark.parametrize("case", CASES, ids=[
    f"B{c[0]}H{c[1]}/{c[2]}S{c[3]}x{c[4]}D{c[5]}c{int(c[6])}w{c[7]},{c[8]}s{c[9]}o{c[10]}{c[11]}" for c in CASES])
def test_window_matches_oracle(case):
    B, Hq, Hkv, Sq, Skv, D, causal, wl, wr, sink, ks, fmt = case
    say(f"case window {case}")
    inp = synth_inputs(B, Hq, Hkv, Sq, Skv, D, fmt, seed=11 + Sq + Skv + max(wl, 0))
    scale = 1 / math.sqrt(D)
    O, L = run_window(inp, scale, causal, wl, wr, sink, ks)
    Oref, Lref = oracle_window(inp, scale, causal, wl, wr, sink, ks)
    Aref = oracle_window(inp, scale, causal, wl, wr, sink, ks, abs_v=True)[0] if inp["fmt"] != "bf16" else None
    check(inp, O, L, Oref, Lref, what=f"window {case}", Aref=Aref)


def test_zero_width_window_returns_own_value_row():
    say("case window width zero, exact")
    inp = synth_inputs(1, 2, 2, 300, 300, 128, "bf16", seed=77)
    O, _ = run_window(inp, 1 / math.sqrt(128), False, 0, 0, 0)
    v = oracle.dequantise(inp["v"], "bf16", 1.0)
    # one key of weight exactly 1: the bf16 output is the bf16 value row itself
    np.testing.assert_array_equal(O, v.astype(np.float32))


@pytest.mark.parametrize("causal", [False, True])
def test_unbounded_window_equals_dense_kernel(causal):
    """Both sides unbounded with no sinks routes to the dense kernel; a window wider
    than the sequence must give the dense kernel's bits. The grid (40 heads of 777
    rows) is large enough for 8-wave workgroups on both paths: a small bf16 grid runs
    its dense rows as key-split workgroups, whose row sums are ordered differently."""
    say(f"case window unbounded == dense, causal={causal}")
    inp = synth_inputs(1, 40, 8, 777, 777, 128, "bf16", seed=91)
    fmt = "bf16"
    Q, K, V = to_dev(inp["q"], fmt), to_dev(inp["k"], fmt), to_dev(inp["v"], fmt)
    Od, Ld = ha.forward(Q, K, V, causal=causal)
    Ow, Lw = ha.forward(Q, K, V, causal=causal, window_left=10 ** 6, window_right=10 ** 6)
    torch.cuda.synchronize()
    assert torch.equal(Od, Ow) and torch.equal(Ld, Lw)


def test_rows_with_no_key_in_window():
    """Keys start at 1000 (a chunk call) but the window of rows < 900 ends before 1000."""
    say("case window empty rows")
    inp = synth_inputs(1, 2, 2, 1000, 200, 128, "bf16", seed=5)
    O, L = run_window(inp, 1 / math.sqrt(128), False, 10, 100, 0, kv_start=1000)
    Oref, Lref = oracle_window(inp, 1 / math.sqrt(128), False, 10, 100, 0, kv_start=1000)
    assert np.isneginf(Lref[..., :900]).all() and np.isfinite(Lref[..., 900:]).all()
    check(inp, O, L, Oref, Lref, what="window empty rows")


@pytest.mark.parametrize("name", ["swa_llm", "video_band"])
def test_local_workloads_full_size_sampled_rows(name):
    """The measured local-attention workloads at full size, sampled rows against the oracle."""
    w = WORKLOADS[name]
    say(f"case window workload {name} full size")
    inp = make_inputs(w)
    causal = bool(w.causal[-1])
    O, L = run_window(inp, w.scale, causal, w.window_left, w.window_right, w.sink)
    rs = np.random.default_rng(9).choice(w.Sq, 12, replace=False)
    rows = np.unique(np.concatenate([[0, 1, w.sink, w.Sq // 2, w.Sq - 1], rs]))
    Oref, Lref = oracle_window(inp, w.scale, causal, w.window_left, w.window_right, w.sink, rows=rows)
    check(inp, O[:, :, rows], L[:, :, rows], Oref, Lref, what=f"{name} sampled rows")
