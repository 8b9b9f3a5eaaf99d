"""Split-KV forward (attn_fwd_splitkv) against the fp64 oracle and the unsplit kernel.

Each split computes the (O, LSE) of its key range into an fp32 workspace and a
second kernel merges them by LSE; the bars are the ones of the unsplit path
(bf16: max|dO| <= 1e-2, max|dLSE| <= 1e-3; fp8: range-normalised NRMS <= 1e-2,
max|dLSE| <= 1e-3), and the split result must also agree with the unsplit
kernel far more tightly than that.
"""

import math

import numpy as np
import pytest
import torch

import head_attention_amd as ha
from gpu_helpers import say, oracle_ref, refs, check_any, synth_inputs, check_bf16, check_fp8, to_dev, descale_dev, make_inputs, WORKLOADS

pytestmark = pytest.mark.gpu


def run_split(inp, scale, causal, n_splits, workspace=None):
    fmt = inp["fmt"]
    qd, kd, vd = (descale_dev(inp[n]) for n in ("q_descale", "k_descale", "v_descale")) if fmt == "e4m3fn" else (None,) * 3
    Q, K, V = to_dev(inp["q"], fmt), to_dev(inp["k"], fmt), to_dev(inp["v"], fmt)
    O, L = ha.forward_splitkv(Q, K, V, n_splits=n_splits, scale=scale, causal=causal,
                              q_descale=qd, k_descale=kd, v_descale=vd, workspace=workspace)
    Ou, Lu = ha.forward(Q, K, V, scale=scale, causal=causal, q_descale=qd, k_descale=kd, v_descale=vd)
    torch.cuda.synchronize()
    return O.float().cpu().numpy(), L.cpu().numpy(), Ou.float().cpu().numpy(), Lu.cpu().numpy()


CASES = [
    # B, Hq, Hkv, Sq, Skv, D, causal, n_splits, fmt
    (1, 2, 2, 300, 2000, 128, False, 2, "bf16"),
    (1, 2, 2, 300, 2000, 128, False, 7, "bf16"),
    (1, 4, 2, 257, 1999, 128, False, 3, "bf16"),     # GQA, ragged key tail
    (1, 2, 2, 700, 700, 128, True, 3, "bf16"),       # causal: some splits lie wholly above some rows
    (2, 2, 1, 300, 1000, 64, False, 4, "bf16"),
    (1, 2, 2, 300, 100, 128, False, 8, "bf16"),      # more splits than key tiles
    (1, 3, 3, 500, 3000, 128, False, 0, "bf16"),     # the library's choice
    (1, 2, 2, 300, 2000, 128, False, 5, "e4m3fn"),
    (1, 4, 2, 600, 600, 128, True, 2, "e4m3fn"),
    (1, 2, 2, 300, 1000, 64, False, 3, "e4m3fn"),
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}H{c[1]}/{c[2]}S{c[3]}x{c[4]}D{c[5]}c{int(c[6])}n{c[7]}{c[8]}" for c in CASES])
def test_splitkv_matches_oracle_and_unsplit(case):
    B, Hq, Hkv, Sq, Skv, D, causal, ns, fmt = case
    say(f"case splitkv {case}")
    inp = synth_inputs(B, Hq, Hkv, Sq, Skv, D, fmt, seed=3 + Sq + Skv + ns)
    scale = 1 / math.sqrt(D)
    O, L, Ou, Lu = run_split(inp, scale, causal, ns)
    R = refs(inp, scale, causal)
    if fmt == "bf16":
        check_any(inp, O, L, R, what=f"split {case}")
    else:
        live = ~np.isneginf(R[1])
        assert np.array_equal(np.isneginf(L), ~live) and (O[~live] == 0).all()
        check_any(inp, O, L, R, what=f"split {case}", live=live)
    # against the unsplit kernel: only fp32 rounding of the partials separates them
    fin = np.isfinite(Lu)
    assert np.array_equal(np.isfinite(L), fin)
    dO = float(np.abs(O - Ou).max())
    dL = float(np.abs(L[fin] - Lu[fin]).max()) if fin.any() else 0.0
    say(f"  vs unsplit kernel: max|dO|={dO:.3e} max|dLSE|={dL:.3e}")
    assert dO <= (8e-3 if fmt == "bf16" else 4e-2) and dL <= 1e-4


AUTO_CASES = [
    # B, Hq, Hkv, Sq, Skv, D, causal, fmt: what the library's choice (n_splits = 0) does there
    (1, 1, 1, 200, 40000, 128, False, "bf16"),     # one query tile: the least-time count (37 splits)
    (1, 2, 1, 100, 30000, 128, False, "e4m3fn"),   # two tiles, GQA, fp8 (28 splits)
    (1, 2, 2, 256, 20000, 64, True, "bf16"),       # causal, D64: nearly every split above the diagonal
    (1, 4, 2, 2000, 8000, 128, False, "bf16"),     # 32 tiles: 7 splits of 18 key tiles
    (1, 64, 64, 1100, 4000, 64, False, "bf16"),    # 320 tiles: 3 whole-grid splits (94 % of 4 rounds)
    (1, 40, 40, 1700, 2100, 128, True, "bf16"),    # 280 tiles, causal: the tail count sizes the workspace,
                                                   # the call itself runs unsplit
]


@pytest.mark.parametrize("case", AUTO_CASES,
                         ids=[f"B{c[0]}H{c[1]}/{c[2]}S{c[3]}x{c[4]}D{c[5]}c{int(c[6])}{c[7]}" for c in AUTO_CASES])
def test_splitkv_library_choice(case):
    """n_splits = 0 with exactly the workspace attn_splitkv_auto_splits sizes, against the
    oracle and the unsplit kernel."""
    B, Hq, Hkv, Sq, Skv, D, causal, fmt = case
    n = ha.attn_splitkv_auto_splits(B, Hq, Sq, Skv, D)
    say(f"case splitkv library choice {case}: {n} splits")
    need = ha.attn_splitkv_workspace_bytes(B, Hq, Sq, D, n)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    inp = synth_inputs(B, Hq, Hkv, Sq, Skv, D, fmt, seed=11 + Sq + Skv)
    scale = 1 / math.sqrt(D)
    O, L, Ou, Lu = run_split(inp, scale, causal, 0, workspace=ws)
    check_any(inp, O, L, refs(inp, scale, causal), what=f"library choice {case}")
    fin = np.isfinite(Lu)
    assert np.array_equal(np.isfinite(L), fin)
    if causal and B * Hq * ((Sq + 255) // 256) >= 256:
        # a causal call never takes a tail split: it is the unsplit kernel, bit for bit
        assert np.array_equal(O, Ou) and np.array_equal(L, Lu)
    else:
        assert n > 1
        assert float(np.abs(O - Ou).max()) <= (8e-3 if fmt == "bf16" else 4e-2)
        assert float(np.abs(L[fin] - Lu[fin]).max()) <= 1e-4


def test_splitkv_ignores_workspace_contents():
    """A workspace full of NaN from an earlier use gives the same result."""
    say("case splitkv dirty workspace")
    inp = synth_inputs(1, 2, 2, 300, 1500, 128, "bf16", seed=41)
    need = ha.attn_splitkv_workspace_bytes(1, 2, 300, 128, 4)
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda").view(torch.uint8)
    O1, L1, _, _ = run_split(inp, 1 / math.sqrt(128), False, 4, workspace=ws)
    O2, L2, _, _ = run_split(inp, 1 / math.sqrt(128), False, 4, workspace=ws)
    assert np.isfinite(O1).all() and np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_splitkv_video_dit_shard_full_size_auto():
    """An eighth of the video-DiT queries against all 75600 keys (185 query tiles on
    256 CUs) with the library's split choice."""
    w = WORKLOADS["video_dit_shard"]
    ns = ha.attn_splitkv_auto_splits(w.B, w.Hq, w.Sq, w.Skv, w.D)
    say(f"case splitkv video_dit_shard full size, auto splits = {ns}")
    assert ns > 1
    inp = make_inputs(w)
    O, L, Ou, Lu = run_split(inp, w.scale, False, 0)
    rows = np.unique(np.concatenate([[0, 1, w.Sq - 1], np.random.default_rng(5).choice(w.Sq, 30, replace=False)]))
    Oref, Lref = oracle_ref(inp, w.scale, False, rows=rows)
    check_bf16(O[:, :, rows], L[:, :, rows], Oref, Lref, what="video_dit_shard split")
    assert float(np.abs(O - Ou).max()) <= 8e-3


@pytest.mark.parametrize("fmt", ["bf16", "e4m3fn"])
def test_splitkv_tail_only_split(fmt):
    """With the library's choice at 280 query tiles on 256 CUs, only the last 24 tiles
    (one partial round) are split over their keys; the rest are computed whole. Every
    row against the oracle, and against attn_fwd."""
    B, Hq, Hkv, Sq, Skv, D = 1, 40, 40, 1700, 2100, 128
    assert ha.attn_splitkv_auto_splits(B, Hq, Sq, Skv, D) == 2
    say(f"case splitkv tail-only split {fmt}")
    inp = synth_inputs(B, Hq, Hkv, Sq, Skv, D, fmt, seed=77)
    scale = 1 / math.sqrt(D)
    O, L, Ou, Lu = run_split(inp, scale, False, 0)
    check_any(inp, O, L, refs(inp, scale, False), what="tail split")
    # rows of whole tiles are the unsplit kernel's bits; tail rows agree to fp32 rounding
    whole_rows = (256 // 7) * Sq + (256 % 7) * 256          # first row of the first tail tile
    flatO, flatOu = O.reshape(-1, D), Ou.reshape(-1, D)
    assert np.array_equal(flatO[:whole_rows], flatOu[:whole_rows])
    assert float(np.abs(flatO[whole_rows:] - flatOu[whole_rows:]).max()) <= (8e-3 if fmt == "bf16" else 4e-2)


def test_splitkv_tail_only_split_long_rows():
    """460 tiles (one full round of 256, then 204 tail tiles split 5 ways over 460 key
    tiles): whole-tile rows equal the unsplit kernel's bits; sampled rows on both sides
    of the first tail tile and in the last head against the oracle."""
    B, Hq, Hkv, Sq, Skv, D = 1, 4, 4, 29440, 29440, 128
    assert ha.attn_splitkv_auto_splits(B, Hq, Sq, Skv, D) == 5
    say("case splitkv tail-only split, long rows")
    inp = synth_inputs(B, Hq, Hkv, Sq, Skv, D, "bf16", seed=78)
    scale = 1 / math.sqrt(D)
    O, L, Ou, Lu = run_split(inp, scale, False, 0)
    first_tail = 256 - 2 * 115                               # tile 256 is head 2, query tile 26
    rows = np.array([0, 100, first_tail * 256 - 1, first_tail * 256, first_tail * 256 + 200, Sq - 1])
    Oref, Lref = oracle_ref(inp, scale, False, rows=rows)
    check_bf16(O[:, :, rows], L[:, :, rows], Oref, Lref, what="tail split long rows")
    assert np.array_equal(O[:, :2], Ou[:, :2])               # heads 0 and 1: whole tiles only
    assert np.array_equal(O[:, 2, :first_tail * 256], Ou[:, 2, :first_tail * 256])
    assert float(np.abs(O - Ou).max()) <= 8e-3
