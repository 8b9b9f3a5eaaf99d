"""Pins of the CPU oracle against what the mathematics and the pages fix.

None of these tests needs a GPU. Each pin is chosen so that a plausible slip in
the oracle (a dropped scale, a wrong GQA index, an off-by-one causal offset, a
transposed operand, a log in the wrong base, a wrong merge weight, a wrong fp8
exponent bias) fails at least one of them; ``test_pins_catch_planted_mistakes``
plants such slips in a copy of the oracle and checks that they are caught.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention_forward, merge_lse, decode_bf16, decode_e4m3fn, dequantise
from oracle.brute import attention_brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(1234)


def rand(*shape, scale=1.0):
    return rng.standard_normal(shape) * scale


# ---------------------------------------------------------------- formats

def test_e4m3fn_closed_form_codes():
    cases = {
        0x00: 0.0, 0x80: -0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
        0x38: 1.0, 0x3C: 1.5, 0x40: 2.0, 0x7E: 448.0, 0xFE: -448.0, 0x77: 240.0,
        0x30: 0.5, 0xB8: -1.0, 0x39: 1.125,
    }
    got = decode_e4m3fn(np.array(list(cases), dtype=np.uint8))
    np.testing.assert_array_equal(got, np.array(list(cases.values())))
    assert np.isnan(decode_e4m3fn(np.array([0x7F, 0xFF], dtype=np.uint8))).all()
    finite = decode_e4m3fn(np.arange(256))
    assert np.nanmax(np.abs(finite)) == 448.0
    assert np.isnan(finite).sum() == 2


def test_e4m3fn_matches_torch_cast_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = decode_e4m3fn(codes.numpy())
    both_nan = np.isnan(ref) & np.isnan(got)
    np.testing.assert_array_equal(np.where(both_nan, 0, got), np.where(both_nan, 0, ref))


def test_bf16_matches_torch_cast():
    bits = torch.randint(0, 65536, (20000,), dtype=torch.int32)
    bits = bits[(bits & 0x7F80) != 0x7F80]  # finite patterns
    ref = bits.to(torch.int16).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(decode_bf16(bits.numpy()), ref)
    np.testing.assert_array_equal(decode_bf16(np.array([0x3F80, 0xC000, 0x0001, 0x7F7F])),
                                  [1.0, -2.0, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127])


def test_dequantise_applies_descale_only_to_fp8():
    codes = np.array([0x38, 0x40], dtype=np.uint8)
    np.testing.assert_array_equal(dequantise(codes, "e4m3fn", 0.25), [0.25, 0.5])
    np.testing.assert_array_equal(dequantise(np.array([0x3F80]), "bf16", 0.25), [1.0])


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("Sq,Skv,D", [(1, 1, 1), (2, 3, 2), (5, 3, 4), (3, 5, 2), (17, 5, 4), (5, 17, 1)])
@pytest.mark.parametrize("causal,kv_start", [(False, 0), (True, 0), (True, 2)])
def test_oracle_matches_brute_force(Sq, Skv, D, causal, kv_start):
    Hq, Hkv = 4, 2                       # GQA with distinct KV heads
    q, k, v = rand(1, Hq, Sq, D), rand(1, Hkv, Skv, D), rand(1, Hkv, Skv, D)
    scale = 0.7
    O, L = attention_forward(q, k, v, scale, causal, kv_start)
    Ob, Lb = attention_brute(q.tolist(), k.tolist(), v.tolist(), scale, causal, kv_start)
    np.testing.assert_allclose(O, np.array(Ob), rtol=1e-12, atol=1e-13)
    Lb = np.array(Lb)
    assert np.array_equal(np.isinf(L), np.isinf(Lb))
    np.testing.assert_allclose(L[np.isfinite(L)], Lb[np.isfinite(Lb)], rtol=1e-12, atol=1e-13)


def test_tiny_config_matches_brute_force_sampled_rows():
    # The tiny fp32 workload shape (B1 H2 S256 D64), every 37th row checked by brute force.
    q, k, v = rand(1, 2, 256, 64), rand(1, 2, 256, 64), rand(1, 2, 256, 64)
    scale = 1 / 8
    rows = np.arange(0, 256, 37)
    O, L = attention_forward(q, k, v, scale, rows=rows)
    Ob, Lb = attention_brute(q[:, :, rows].tolist(), k.tolist(), v.tolist(), scale)
    np.testing.assert_allclose(O, np.array(Ob), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(L, np.array(Lb), rtol=1e-12)


# ---------------------------------------------------------------- library routines

@pytest.mark.parametrize("causal", [False, True])
def test_oracle_matches_torch_sdpa_fp64(causal):
    B, Hq, Hkv, S, D = 2, 6, 3, 70, 16
    q, k, v = rand(B, Hq, S, D), rand(B, Hkv, S, D), rand(B, Hkv, S, D)
    scale = 0.3
    O, L = attention_forward(q, k, v, scale, causal)
    g = Hq // Hkv
    qt = torch.from_numpy(q)
    kt = torch.from_numpy(k).repeat_interleave(g, dim=1)
    vt = torch.from_numpy(v).repeat_interleave(g, dim=1)
    Ot = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, scale=scale)
    np.testing.assert_allclose(O, Ot.numpy(), rtol=1e-12, atol=1e-13)
    s = scale * (qt @ kt.transpose(-1, -2))
    if causal:
        s = s.masked_fill(torch.ones(S, S, dtype=torch.bool).triu(1), -math.inf)
    np.testing.assert_allclose(L, torch.logsumexp(s, dim=-1).numpy(), rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- closed forms and invariants

def test_identical_keys_give_mean_of_v_and_lse_score_plus_ln_skv():
    Skv, D = 37, 8
    q = rand(1, 1, 5, D)
    k = np.broadcast_to(rand(1, 1, 1, D), (1, 1, Skv, D)).copy()
    v = rand(1, 1, Skv, D)
    scale = 0.4
    O, L = attention_forward(q, k, v, scale)
    np.testing.assert_allclose(O[0, 0], np.broadcast_to(v[0, 0].mean(0), (5, D)), rtol=1e-12, atol=1e-14)
    score = scale * (q[0, 0] @ k[0, 0, 0])
    np.testing.assert_allclose(L[0, 0], score + np.log(Skv), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_rows_sum_to_one(causal):
    q, k = rand(1, 2, 33, 8, scale=3.0), rand(1, 2, 33, 8, scale=3.0)
    O, _ = attention_forward(q, k, np.ones((1, 2, 33, 8)), 1.0, causal)
    np.testing.assert_allclose(O, 1.0, rtol=0, atol=1e-13)


def test_zero_queries_closed_forms():
    S, D = 19, 4
    v = rand(1, 1, S, D)
    k = rand(1, 1, S, D)
    O, L = attention_forward(np.zeros((1, 1, S, D)), k, v, 0.9, causal=False)
    np.testing.assert_allclose(O[0, 0], np.broadcast_to(v[0, 0].mean(0), (S, D)), atol=1e-14)
    np.testing.assert_allclose(L, np.log(S), rtol=1e-14)
    O, L = attention_forward(np.zeros((1, 1, S, D)), k, v, 0.9, causal=True)
    cum = np.cumsum(v[0, 0], axis=0) / np.arange(1, S + 1)[:, None]
    np.testing.assert_allclose(O[0, 0], cum, atol=1e-14)
    np.testing.assert_allclose(L[0, 0], np.log(np.arange(1, S + 1)), rtol=1e-14)


def test_single_key_and_causal_row_zero():
    q, k, v = rand(1, 1, 4, 6), rand(1, 1, 1, 6), rand(1, 1, 1, 6)
    O, L = attention_forward(q, k, v, 0.5)
    np.testing.assert_allclose(O[0, 0], np.broadcast_to(v[0, 0, 0], (4, 6)), atol=1e-15)
    np.testing.assert_allclose(L[0, 0], 0.5 * (q[0, 0] @ k[0, 0, 0]), rtol=1e-14)
    q, k, v = rand(1, 1, 4, 6), rand(1, 1, 4, 6), rand(1, 1, 4, 6)
    O, L = attention_forward(q, k, v, 0.5, causal=True)
    np.testing.assert_array_equal(O[0, 0, 0], v[0, 0, 0])
    np.testing.assert_allclose(L[0, 0, 0], 0.5 * q[0, 0, 0] @ k[0, 0, 0], rtol=1e-14)


def test_key_permutation_invariance():
    q, k, v = rand(1, 2, 24, 8), rand(1, 2, 24, 8), rand(1, 2, 24, 8)
    O, L = attention_forward(q, k, v, 0.5, False)
    perm = rng.permutation(24)
    Op, Lp = attention_forward(q, k[:, :, perm], v[:, :, perm], 0.5, False)
    np.testing.assert_allclose(Op, O, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(Lp, L, rtol=1e-13)


def test_causal_equals_explicit_tril_mask():
    S, D = 21, 5
    q, k, v = rand(1, 1, S, D), rand(1, 1, S, D), rand(1, 1, S, D)
    O, L = attention_forward(q, k, v, 0.8, causal=True)
    for i in range(S):
        Oi, Li = attention_forward(q[:, :, i:i + 1], k[:, :, :i + 1], v[:, :, :i + 1], 0.8)
        np.testing.assert_allclose(O[0, 0, i], Oi[0, 0, 0], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(L[0, 0, i], Li[0, 0, 0], rtol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("split", [1, 7, 16, 29])
def test_chunked_keys_merged_by_lse_equal_unsplit(causal, split):
    Hq, Hkv, S, D = 4, 2, 30, 8
    q, k, v = rand(1, Hq, S, D), rand(1, Hkv, S, D), rand(1, Hkv, S, D)
    O, L = attention_forward(q, k, v, 0.6, causal)
    p1 = attention_forward(q, k[:, :, :split], v[:, :, :split], 0.6, causal, kv_start=0)
    p2 = attention_forward(q, k[:, :, split:], v[:, :, split:], 0.6, causal, kv_start=split)
    if causal:   # rows before the second chunk start attend to none of its keys
        assert np.isneginf(p2[1][..., :split]).all() and (p2[0][..., :split, :] == 0).all()
    Om, Lm = merge_lse([p1, p2])
    np.testing.assert_allclose(Om, O, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(Lm, L, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("bounds", [(0, 5, 11, 30), (0, 1, 2, 3, 30), (0, 29, 30), (0, 10, 10, 20, 30)])
def test_n_way_key_split_merged_by_lse_equals_unsplit(causal, bounds):
    """N key ranges (including an empty one), each with its absolute start, merged by LSE."""
    Hq, Hkv, S, D = 4, 2, 30, 8
    q, k, v = rand(1, Hq, S, D), rand(1, Hkv, S, D), rand(1, Hkv, S, D)
    O, L = attention_forward(q, k, v, 0.6, causal)
    parts = [attention_forward(q, k[:, :, a:b], v[:, :, a:b], 0.6, causal, kv_start=a)
             for a, b in zip(bounds[:-1], bounds[1:])]
    Om, Lm = merge_lse(parts)
    np.testing.assert_allclose(Om, O, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(Lm, L, rtol=1e-13, atol=1e-14)


def test_merge_of_empty_chunks():
    O1, L1 = np.zeros((3, 2)), np.full(3, -np.inf)
    O2, L2 = rand(3, 2), np.array([-np.inf, 0.5, 2.0])
    Om, Lm = merge_lse([(O1, L1), (O2, L2)])
    assert np.isneginf(Lm[0]) and (Om[0] == 0).all()
    np.testing.assert_array_equal(Om[1:], O2[1:])
    np.testing.assert_array_equal(Lm[1:], L2[1:])
    # merge weights: two equal-LSE chunks average and add ln 2
    Om, Lm = merge_lse([(np.ones((1, 2)), np.array([1.0])), (3 * np.ones((1, 2)), np.array([1.0]))])
    np.testing.assert_allclose(Om, 2.0)
    np.testing.assert_allclose(Lm, 1.0 + np.log(2.0))


def test_row_subset_equals_full():
    q, k, v = rand(1, 2, 40, 8), rand(1, 2, 40, 8), rand(1, 2, 40, 8)
    O, L = attention_forward(q, k, v, 0.5, causal=True, row_block=7)
    rows = np.array([0, 3, 39, 17])
    Os, Ls = attention_forward(q, k, v, 0.5, causal=True, rows=rows)
    np.testing.assert_array_equal(Os, O[:, :, rows])
    np.testing.assert_array_equal(Ls, L[:, :, rows])


# ---------------------------------------------------------------- local attention (window, sink)

WINDOWS = [(-1, -1, 0), (0, 0, 0), (2, -1, 0), (-1, 1, 0), (1, 2, 0), (3, 0, 1), (0, 0, 2), (-1, -1, 3), (6, 6, 0)]


@pytest.mark.parametrize("wl,wr,sink", WINDOWS)
@pytest.mark.parametrize("causal,kv_start", [(False, 0), (True, 0), (False, 3), (True, 2)])
def test_local_attention_matches_brute_force(wl, wr, sink, causal, kv_start):
    Hq, Hkv, Sq, Skv, D = 4, 2, 9, 7, 3
    q, k, v = rand(1, Hq, Sq, D), rand(1, Hkv, Skv, D), rand(1, Hkv, Skv, D)
    O, L = attention_forward(q, k, v, 0.7, causal, kv_start, window_left=wl, window_right=wr, sink=sink)
    Ob, Lb = attention_brute(q.tolist(), k.tolist(), v.tolist(), 0.7, causal, kv_start, wl, wr, sink)
    np.testing.assert_allclose(O, np.array(Ob), rtol=1e-12, atol=1e-13)
    Lb = np.array(Lb)
    assert np.array_equal(np.isinf(L), np.isinf(Lb))
    np.testing.assert_allclose(L[np.isfinite(L)], Lb[np.isfinite(Lb)], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("wl,wr,sink,causal", [(4, 2, 0, False), (5, -1, 2, True), (0, 3, 1, False)])
def test_local_attention_matches_torch_sdpa_with_band_mask(wl, wr, sink, causal):
    """torch's SDPA with an explicit boolean band mask built from index arithmetic."""
    S, D = 40, 8
    q, k, v = rand(1, 2, S, D), rand(1, 2, S, D), rand(1, 2, S, D)
    O, L = attention_forward(q, k, v, 0.5, causal, window_left=wl, window_right=wr, sink=sink)
    i = torch.arange(S)[:, None]
    j = torch.arange(S)[None, :]
    band = torch.ones(S, S, dtype=torch.bool)
    if wl >= 0:
        band &= j >= i - wl
    if wr >= 0:
        band &= j <= i + wr
    mask = band | (j < sink)
    if causal:
        mask &= j <= i
    Ot = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k),
                                                          torch.from_numpy(v), attn_mask=mask, scale=0.5)
    np.testing.assert_allclose(O, Ot.numpy(), rtol=1e-12, atol=1e-13)
    s = (0.5 * (torch.from_numpy(q) @ torch.from_numpy(k).transpose(-1, -2))).masked_fill(~mask, -math.inf)
    np.testing.assert_allclose(L, torch.logsumexp(s, dim=-1).numpy(), rtol=1e-13, atol=1e-13)


def test_zero_width_window_picks_own_key():
    """A window of width zero keeps exactly key i for query i: O_i = v_i, LSE_i = scale q_i.k_i;
    with one sink key as well, row i > 0 is the two-key softmax of keys 0 and i."""
    S, D = 12, 5
    q, k, v = rand(1, 1, S, D), rand(1, 1, S + 3, D), rand(1, 1, S + 3, D)
    O, L = attention_forward(q, k, v, 0.9, window_left=0, window_right=0)
    np.testing.assert_array_equal(O[0, 0], v[0, 0, :S])
    np.testing.assert_allclose(L[0, 0], 0.9 * np.einsum("id,id->i", q[0, 0], k[0, 0, :S]), rtol=1e-14)
    O, L = attention_forward(q, k, v, 0.9, window_left=0, window_right=0, sink=1)
    for i in range(1, S):
        s0, si = 0.9 * q[0, 0, i] @ k[0, 0, 0], 0.9 * q[0, 0, i] @ k[0, 0, i]
        w0 = 1.0 / (1.0 + math.exp(si - s0))
        np.testing.assert_allclose(O[0, 0, i], w0 * v[0, 0, 0] + (1 - w0) * v[0, 0, i], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(L[0, 0, i], np.logaddexp(s0, si), rtol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_window_covering_every_key_is_full_attention(causal):
    Sq, Skv, D = 11, 17, 4
    q, k, v = rand(1, 2, Sq, D), rand(1, 2, Skv, D), rand(1, 2, Skv, D)
    O, L = attention_forward(q, k, v, 0.6, causal)
    for wl, wr, sink in [(Sq, Skv, 0), (10 ** 6, 10 ** 6, 0), (-1, -1, Skv), (0, 0, Skv)]:
        Ow, Lw = attention_forward(q, k, v, 0.6, causal, window_left=wl, window_right=wr, sink=sink)
        np.testing.assert_array_equal(Ow, O)
        np.testing.assert_array_equal(Lw, L)
    # under causal, a right side >= 0 changes nothing
    if causal:
        Ow, Lw = attention_forward(q, k, v, 0.6, True, window_left=3, window_right=0)
        Ox, Lx = attention_forward(q, k, v, 0.6, True, window_left=3, window_right=-1)
        np.testing.assert_array_equal(Ow, Ox)
        np.testing.assert_array_equal(Lw, Lx)


@pytest.mark.parametrize("wl,wr,sink,causal", [(4, 4, 0, False), (6, -1, 2, True), (-1, 2, 3, False)])
def test_local_attention_key_chunks_merged_by_lse_equal_unsplit(wl, wr, sink, causal):
    """Window and sink are functions of absolute key position, so chunks with kv_start merge exactly."""
    Hq, Hkv, S, D = 2, 1, 30, 6
    q, k, v = rand(1, Hq, S, D), rand(1, Hkv, S, D), rand(1, Hkv, S, D)
    kw = dict(window_left=wl, window_right=wr, sink=sink)
    O, L = attention_forward(q, k, v, 0.6, causal, **kw)
    parts = [attention_forward(q, k[:, :, a:b], v[:, :, a:b], 0.6, causal, kv_start=a, **kw)
             for a, b in [(0, 2), (2, 13), (13, 30)]]
    Om, Lm = merge_lse(parts)
    np.testing.assert_allclose(Om, O, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(Lm, L, rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------- the pages' printed figures

def test_metric_arithmetic_reproduces_printed_summary():
    import bench
    g = json.load(open(os.path.join(GOLDEN, "aiter_fp8_fmha_summary.json")))
    s = g["shape"]
    for us, tfl, gbs, elt in [(g["fwd_us"], g["fwd_tflops"], g["fwd_gb_per_sec"], 2),
                              (g["quant_fwd_us"], g["quant_fwd_tflops"], g["quant_fwd_gb_per_sec"], 1)]:
        assert bench.attn_tflops(s["B"], s["H"], s["Sq"], s["Skv"], s["D"], us * 1e-6, False) == pytest.approx(tfl, rel=1e-8)
        assert bench.pages_gbps(s["B"], s["H"], s["H"], s["Sq"], s["Skv"], s["D"], elt, us * 1e-6) == pytest.approx(gbs, rel=1e-6)


@pytest.mark.parametrize("Sq,Skv,causal,wl,wr,sink", [
    (9, 7, False, 2, 1, 0), (9, 7, True, 2, -1, 3), (20, 30, False, -1, -1, 0), (20, 30, True, -1, -1, 0),
    (12, 12, False, 0, 0, 5), (15, 9, False, 3, 50, 2), (15, 9, True, 1, 0, 20), (40, 40, False, 5, 5, 9)])
def test_local_flop_count_matches_enumeration(Sq, Skv, causal, wl, wr, sink):
    """The kept-pair count behind the local-attention TFLOPS equals the oracle's own mask."""
    import bench
    q, k, v = np.zeros((1, 1, Sq, 1)), np.zeros((1, 1, Skv, 1)), np.ones((1, 1, Skv, 1))
    _, L = attention_forward(q, k, v, 1.0, causal, window_left=wl, window_right=wr, sink=sink)
    kept = np.where(np.isfinite(L), np.rint(np.exp(L)), 0).sum()   # all scores 0: LSE = ln(#kept)
    assert bench.allowed_pairs(Sq, Skv, causal, wl, wr, sink) == int(kept)


def test_nrms_definition_is_bf16_scale():
    # The printed fp8 accuracy figures are exact bf16 numbers (8 significant bits): the
    # comparison ran on bf16 outputs, which the range-normalised reading uses.
    g = json.load(open(os.path.join(GOLDEN, "aiter_fp8_fmha_summary.json")))
    for x in (g["fp8_output_nrms"], g["fp8_output_max_diff"]):
        assert float(torch.tensor(x).to(torch.bfloat16).float()) == x


# ---------------------------------------------------------------- the pins catch planted slips

def _load_mutant(module_file, old, new):
    import importlib.util
    import types
    src = open(module_file).read()
    assert old in src, old
    mod = types.ModuleType("mutant")
    mod.__dict__["np"] = np
    exec(compile(src.replace(old, new, 1), module_file, "exec"), mod.__dict__)
    return mod


def _attention_pins_pass(fwd, merge):
    """A compact run of the pins above against candidate functions."""
    r = np.random.default_rng(7)
    try:
        q, k, v = r.standard_normal((1, 4, 6, 3)), r.standard_normal((1, 2, 5, 3)), r.standard_normal((1, 2, 5, 3))
        for causal, ks in [(False, 0), (True, 0), (True, 2)]:
            O, L = fwd(q, k, v, 0.7, causal, ks)
            Ob, Lb = attention_brute(q.tolist(), k.tolist(), v.tolist(), 0.7, causal, ks)
            Lb = np.array(Lb)
            if not np.allclose(O, np.array(Ob), atol=1e-10):
                return False
            if not np.array_equal(np.isinf(L), np.isinf(Lb)) or not np.allclose(L[np.isfinite(L)], Lb[np.isfinite(Lb)]):
                return False
        for causal, ks, wl, wr, sk in [(False, 0, 1, 2, 0), (True, 1, 2, 0, 1), (False, 0, 0, 0, 2)]:
            O, L = fwd(q, k, v, 0.7, causal, ks, window_left=wl, window_right=wr, sink=sk)
            Ob, Lb = attention_brute(q.tolist(), k.tolist(), v.tolist(), 0.7, causal, ks, wl, wr, sk)
            Lb = np.array(Lb)
            if not np.allclose(O, np.array(Ob), atol=1e-10):
                return False
            if not np.array_equal(np.isinf(L), np.isinf(Lb)) or not np.allclose(L[np.isfinite(L)], Lb[np.isfinite(Lb)]):
                return False
        O, L = fwd(q, k, v, 0.6, True, 0)
        p1 = fwd(q, k[:, :, :2], v[:, :, :2], 0.6, True, 0)
        p2 = fwd(q, k[:, :, 2:], v[:, :, 2:], 0.6, True, 2)
        Om, Lm = merge(p1, p2)
        return bool(np.allclose(Om, O, atol=1e-10) and np.allclose(Lm, L))
    except Exception:
        return False


ATT_FILE = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "attention.py")
FMT_FILE = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "formats.py")


@pytest.mark.parametrize("old,new", [
    ("float(scale) * (", "("),                                            # dropped scale
    ("kv_h = h // group", "kv_h = h % Hkv"),                              # wrong GQA map
    ("key_pos[None, :] <= ridx[:, None]", "key_pos[None, :] < ridx[:, None]"),  # off-by-one causal
    ("+ int(kv_start)", "- int(kv_start)"),                               # wrong offset sign
    ("(p @ V)", "(p @ K)"),                                               # wrong operand
    ("m[live] + np.log(l)", "m[live] + np.log2(l)"),                      # wrong log base
    ("m[live] + np.log(l)", "np.log(l)"),                                 # dropped max term
    ("w / np.where(finite, tot, 1.0)[None]", "w"),                        # unnormalised merge
    ("p = np.exp(s[live] - m[live, None])", "p = np.exp(s[live] + m[live, None])"),  # sign slip
    ("key_pos[None, :] >= ridx[:, None] - int(window_left)",
     "key_pos[None, :] > ridx[:, None] - int(window_left)"),             # off-by-one left edge
    ("key_pos[None, :] <= ridx[:, None] + int(window_right)",
     "key_pos[None, :] <= ridx[:, None] - int(window_right)"),           # mirrored right edge
    ("(key_pos[None, :] < int(sink))", "(key_pos[None, :] <= int(sink))"),  # one sink key too many
    ("in_win | (key_pos", "in_win & (key_pos"),                          # sink intersected, not joined
])
def test_pins_catch_planted_mistakes(old, new):
    good = _load_mutant(ATT_FILE, "def merge_lse", "def merge_lse")
    assert _attention_pins_pass(good.attention_forward, lambda a, b: good.merge_lse([a, b]))
    bad = _load_mutant(ATT_FILE, old, new)
    assert not _attention_pins_pass(bad.attention_forward, lambda a, b: bad.merge_lse([a, b]))


@pytest.mark.parametrize("old,new", [
    ("(exp - 7)", "(exp - 8)"),
    ("frac / 8.0", "frac / 16.0"),
    ("np.ldexp(frac / 8.0, -6)", "np.ldexp(frac / 8.0, -7)"),
    ("(exp - 127)", "(exp - 128)"),
    ("frac / 128.0", "frac / 64.0"),
])
def test_format_pins_catch_planted_mistakes(old, new):
    bad = _load_mutant(FMT_FILE, old, new)
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref8 = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    bits = torch.arange(0, 65536, 97, dtype=torch.int32)
    bits = bits[(bits & 0x7F80) != 0x7F80]
    ref16 = bits.to(torch.int16).view(torch.bfloat16).to(torch.float64).numpy()
    ok8 = np.array_equal(np.nan_to_num(bad.decode_e4m3fn(codes.numpy())), np.nan_to_num(ref8))
    ok16 = np.array_equal(bad.decode_bf16(bits.numpy()), ref16)
    assert not (ok8 and ok16)
