"""Seeded random shapes over the whole entry-point surface, against the fp64 oracle.

Each case draws batch, KV heads, group size, ragged query and key lengths, head
dim, causal, dtype, a key offset (chunk call) and sometimes a window / sink
setting, runs the matching entry point (attn_fwd_chunk, attn_fwd_window,
attn_fwd_splitkv, attn_bwd_chunk) and compares with the oracle at the bars of
the dedicated tests (bf16: max|dO| <= 1e-2, max|dLSE| <= 1e-3; fp8: NRMS <=
1e-2; backward: relative Frobenius <= 1e-2 and max <= 2e-2 max|ref|). The
draws are fixed by the seed, so a failure names a reproducible case.
"""

import math

import numpy as np
import pytest
import torch

import head_attention_amd as ha
import oracle
from gpu_helpers import say, synth_inputs, check_bf16, check_fp8, to_dev, descale_dev

pytestmark = pytest.mark.gpu


def draw_forward(i):
    r = np.random.default_rng(9000 + i)
    hkv = int(r.integers(1, 4))
    case = dict(
        B=int(r.integers(1, 3)), Hkv=hkv, Hq=hkv * int(r.choice([1, 2, 4])),
        Sq=int(r.integers(1, 700)), Skv=int(r.integers(1, 900)), D=int(r.choice([64, 128])),
        causal=bool(r.random() < 0.5), fmt=str(r.choice(["bf16", "e4m3fn"])),
        kv_start=int(r.choice([0, 0, int(r.integers(0, 600))])),
        wl=-1, wr=-1, sink=0, splits=1)
    u = r.random()
    if u < 0.3:
        case.update(wl=int(r.choice([-1, int(r.integers(0, 300))])), wr=int(r.choice([-1, int(r.integers(0, 300))])),
                    sink=int(r.choice([0, 0, int(r.integers(1, 100))])))
        if case["wl"] < 0 and case["wr"] < 0 and case["sink"] == 0:
            case["wl"] = 16
    elif u < 0.5:
        case["splits"] = int(r.integers(2, 6))
    return case


FWD = [draw_forward(i) for i in range(32)]


def fmt_case(c):
    return (f"B{c['B']}H{c['Hq']}/{c['Hkv']}S{c['Sq']}x{c['Skv']}D{c['D']}c{int(c['causal'])}{c['fmt']}"
            f"o{c['kv_start']}w{c['wl']},{c['wr']}s{c['sink']}n{c['splits']}")


@pytest.mark.parametrize("c", FWD, ids=[fmt_case(c) for c in FWD])
def test_random_forward(c):
    say(f"case random forward {fmt_case(c)}")
    inp = synth_inputs(c["B"], c["Hq"], c["Hkv"], c["Sq"], c["Skv"], c["D"], c["fmt"], seed=c["Sq"] * 7 + c["Skv"])
    fmt, scale = c["fmt"], 1 / math.sqrt(c["D"])
    qd, kd, vd = (descale_dev(inp[n]) for n in ("q_descale", "k_descale", "v_descale")) if fmt == "e4m3fn" else (None,) * 3
    Q, K, V = to_dev(inp["q"], fmt), to_dev(inp["k"], fmt), to_dev(inp["v"], fmt)
    if c["splits"] > 1:
        assert c["kv_start"] >= 0
        # split-KV has no key offset: run it at kv_start = 0
        c = dict(c, kv_start=0)
        O, L = ha.forward_splitkv(Q, K, V, n_splits=c["splits"], scale=scale, causal=c["causal"],
                                  q_descale=qd, k_descale=kd, v_descale=vd)
    else:
        O, L = ha.forward(Q, K, V, scale=scale, causal=c["causal"], q_descale=qd, k_descale=kd, v_descale=vd,
                          kv_start=c["kv_start"], window_left=c["wl"], window_right=c["wr"], sink=c["sink"])
    torch.cuda.synchronize()
    O, L = O.float().cpu().numpy(), L.cpu().numpy()
    q = oracle.dequantise(inp["q"], fmt, inp["q_descale"])
    k = oracle.dequantise(inp["k"], fmt, inp["k_descale"])
    v = oracle.dequantise(inp["v"], fmt, inp["v_descale"])
    Oref, Lref = oracle.attention_forward(q, k, v, scale, c["causal"], c["kv_start"],
                                          window_left=c["wl"], window_right=c["wr"], sink=c["sink"])
    if fmt == "bf16":
        check_bf16(O, L, Oref, Lref, what=fmt_case(c))
    else:
        Aref, _ = oracle.attention_forward(q, k, np.abs(v), scale, c["causal"], c["kv_start"],
                                           window_left=c["wl"], window_right=c["wr"], sink=c["sink"])
        live = ~np.isneginf(Lref)
        assert np.array_equal(np.isneginf(L), ~live) and (O[~live] == 0).all()
        if live.any():
            check_fp8(O[live], L[live], Oref[live], Lref[live], Aref[live], what=fmt_case(c))


def draw_backward(i):
    r = np.random.default_rng(7000 + i)
    hkv = int(r.integers(1, 4))
    sq = int(r.integers(1, 600))
    skv_full = int(r.integers(1, 700))
    causal = bool(r.random() < 0.6)
    a = int(r.integers(0, skv_full)) if r.random() < 0.4 else 0      # key chunk [a, b)
    b = int(r.integers(a + 1, skv_full + 1)) if a else skv_full
    return dict(B=int(r.integers(1, 3)), Hkv=hkv, Hq=hkv * int(r.choice([1, 2, 4])), Sq=sq, Skv=skv_full,
                D=int(r.choice([64, 128])), causal=causal, a=a, b=b)


BWD = [draw_backward(i) for i in range(16)]


@pytest.mark.parametrize("c", BWD, ids=[f"B{c['B']}H{c['Hq']}/{c['Hkv']}S{c['Sq']}x{c['Skv']}D{c['D']}c{int(c['causal'])}"
                                        f"k{c['a']}-{c['b']}" for c in BWD])
def test_random_backward(c):
    """Backward of one key chunk [a, b) (the whole key range when a = 0, b = Skv), with the
    full softmax's O and LSE; compared with the oracle's full gradients (dK, dV sliced;
    dQ only when the chunk is the whole range)."""
    say(f"case random backward {c}")
    from synth import normal, to_bf16_bits
    B, Hq, Hkv, Sq, Skv, D = c["B"], c["Hq"], c["Hkv"], c["Sq"], c["Skv"], c["D"]
    seed = 31 * Sq + Skv
    q = to_bf16_bits(normal((B, Hq, Sq, D), seed))
    k = to_bf16_bits(normal((B, Hkv, Skv, D), seed + 1))
    v = to_bf16_bits(normal((B, Hkv, Skv, D), seed + 2))
    do = to_bf16_bits(normal((B, Hq, Sq, D), seed + 3))
    scale = 1 / math.sqrt(D)
    Q, K, V, dO = (to_dev(x, "bf16") for x in (q, k, v, do))
    O, L = ha.forward(Q, K, V, scale=scale, causal=c["causal"])
    a, b = c["a"], c["b"]
    gq, gk, gv = ha.backward(Q, K[:, :, a:b].contiguous(), V[:, :, a:b].contiguous(), O, dO, L, scale=scale,
                             causal=c["causal"], kv_start=a)
    torch.cuda.synchronize()
    dec = lambda x: oracle.dequantise(x, "bf16", 1.0)
    rq, rk, rv = oracle.attention_backward(dec(q), dec(k), dec(v), dec(do), scale, c["causal"])
    f64 = lambda t: t.float().cpu().numpy().astype(np.float64)
    pairs = [(f64(gk), rk[:, :, a:b], "dK"), (f64(gv), rv[:, :, a:b], "dV")]
    if a == 0 and b == Skv:
        pairs.append((f64(gq), rq, "dQ"))
    for got, ref, name in pairs:
        assert np.isfinite(got).all()
        nref = float(np.linalg.norm(ref))
        mx = float(np.abs(got - ref).max()) if ref.size else 0.0
        if nref == 0.0:
            assert mx <= 1e-5, f"{name}: expected ~0, got {mx}"
            continue
        fro = float(np.linalg.norm(got - ref)) / nref
        say(f"  {name}: frob_rel={fro:.3e} max|d|={mx:.3e}")
        assert fro <= 1e-2 and mx <= 2e-2 * float(np.abs(ref).max()), name
