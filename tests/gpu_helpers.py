"""Shared plumbing of the GPU tests: move stored inputs to the device, run the
C-ABI path, and compute the oracle on the very same stored values."""

import math
import sys

import numpy as np
import torch

import head_attention_amd as ha
import oracle
from synth import make_inputs, WORKLOADS, normal, to_bf16_bits, quant_e4m3fn_per_tensor

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(stored: np.ndarray, fmt: str) -> torch.Tensor:
    if fmt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(stored).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(stored)).view(torch.float8_e4m3fn).to(DEV)


def descale_dev(x: float) -> torch.Tensor:
    return torch.tensor([x], dtype=torch.float32, device=DEV)


def synth_inputs(B, Hq, Hkv, Sq, Skv, D, fmt, seed, scale_k=1.0):
    """Seeded N(0,1) inputs of an arbitrary shape (edge-case tests)."""
    q32 = normal((B, Hq, Sq, D), seed)
    k32 = normal((B, Hkv, Skv, D), seed + 1) * scale_k
    v32 = normal((B, Hkv, Skv, D), seed + 2)
    out = dict(fmt=fmt, q32=q32, k32=k32, v32=v32)
    if fmt == "bf16":
        out.update(q=to_bf16_bits(q32), k=to_bf16_bits(k32), v=to_bf16_bits(v32),
                   q_descale=1.0, k_descale=1.0, v_descale=1.0)
    else:
        (qc, qd), (kc, kd), (vc, vd) = (quant_e4m3fn_per_tensor(t) for t in (q32, k32, v32))
        out.update(q=qc, k=kc, v=vc, q_descale=float(qd), k_descale=float(kd), v_descale=float(vd))
    return out


def run_gpu(inp, scale, causal, kv_start=0, k_slice=None, stream=None):
    """Run the HIP path on stored inputs; returns (O float32 numpy, LSE numpy)."""
    fmt = inp["fmt"]
    q, k, v = inp["q"], inp["k"], inp["v"]
    if k_slice is not None:
        k, v = k[:, :, k_slice], v[:, :, k_slice]
    qd, kd, vd = (descale_dev(inp[n]) for n in ("q_descale", "k_descale", "v_descale")) if fmt == "e4m3fn" else (None,) * 3
    Q, K, V = to_dev(q, fmt), to_dev(k, fmt), to_dev(v, fmt)
    O, L = ha.forward(Q, K, V, scale=scale, causal=causal, q_descale=qd, k_descale=kd, v_descale=vd,
                      kv_start=kv_start, stream=stream)
    torch.cuda.synchronize()
    return O.float().cpu().numpy(), L.cpu().numpy(), O


def oracle_ref(inp, scale, causal, kv_start=0, rows=None, k_slice=None, with_abs=False):
    """(O_ref, LSE_ref) from the oracle on the stored inputs; with with_abs, also
    A_ref = the oracle's output with |V| in place of V (sum_j P_ij |v_jd|, the
    scale of the first-order effect of rounding each P weight)."""
    fmt = inp["fmt"]
    if rows is not None and not causal:
        # Without a mask each output row depends only on its own query: decode
        # just the sampled rows (the full float64 Q of a large case is GBs).
        q = oracle.dequantise(np.ascontiguousarray(inp["q"][:, :, rows]), fmt, inp["q_descale"])
        rows_arg, causal_arg = None, False
    else:
        q = oracle.dequantise(inp["q"], fmt, inp["q_descale"])
        rows_arg, causal_arg = rows, causal
    k = oracle.dequantise(inp["k"], fmt, inp["k_descale"])
    v = oracle.dequantise(inp["v"], fmt, inp["v_descale"])
    if k_slice is not None:
        k, v = k[:, :, k_slice], v[:, :, k_slice]
    O, L = oracle.attention_forward(q, k, v, scale, causal_arg, kv_start, rows=rows_arg)
    if not with_abs:
        return O, L
    A, _ = oracle.attention_forward(q, k, np.abs(v), scale, causal_arg, kv_start, rows=rows_arg)
    return O, L, A


def oracle_full(inp, scale, causal, kv_start=0, workers=16, block=256):
    """The oracle's (O, LSE) over every query row of the stored inputs, evaluated as
    independent blocks of query rows on a thread pool. Each block is the unchanged
    oracle restricted to its rows (each output row depends only on its own query);
    BLAS runs one thread per block so that the blocks run side by side."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    fmt = inp["fmt"]
    B, Hq, Sq, D = inp["q"].shape
    g = Hq // inp["k"].shape[1]
    q = oracle.dequantise(inp["q"], fmt, inp["q_descale"])
    k = oracle.dequantise(inp["k"], fmt, inp["k_descale"])
    v = oracle.dequantise(inp["v"], fmt, inp["v_descale"])
    O = np.empty((B, Hq, Sq, D), np.float64)
    L = np.empty((B, Hq, Sq), np.float64)
    tasks = [(b, h, r0) for b in range(B) for h in range(Hq) for r0 in range(0, Sq, block)]

    def run(t):
        b, h, r0 = t
        rows = np.arange(r0, min(r0 + block, Sq))
        o, l = oracle.attention_forward(q[b:b + 1, h:h + 1], k[b:b + 1, h // g:h // g + 1],
                                        v[b:b + 1, h // g:h // g + 1], scale, causal, kv_start, rows=rows)
        O[b, h, rows] = o[0, 0]
        L[b, h, rows] = l[0, 0]

    with threadpool_limits(limits=1), ThreadPoolExecutor(max_workers=workers) as ex:
        for i, _ in enumerate(ex.map(run, tasks)):
            if (i + 1) % max(1, len(tasks) // 8) == 0:
                say(f"  oracle {i + 1}/{len(tasks)} row blocks")
    return O, L


def refs(inp, scale, causal, **kw):
    """(O_ref, LSE_ref, A_ref) for the stored inputs; A_ref (the oracle on |V|) only
    for fp8 inputs, else None."""
    if inp["fmt"] == "e4m3fn":
        return oracle_ref(inp, scale, causal, with_abs=True, **kw)
    O, L = oracle_ref(inp, scale, causal, **kw)
    return O, L, None


def check_any(inp, O, L, R, what="", live=None):
    """The bf16 or fp8 bar for the stored inputs' format; R = refs(...); live: optional
    mask of the rows to compare (rows without keys are checked separately)."""
    Oref, Lref, Aref = R
    if live is not None:
        O, L, Oref, Lref = O[live], L[live], Oref[live], Lref[live]
        Aref = Aref[live] if Aref is not None else None
    if inp["fmt"] == "bf16":
        return check_bf16(O, L, Oref, Lref, what=what)
    return check_fp8(O, L, Oref, Lref, Aref, what=what)


def nrms(got, ref):
    """Range-normalised RMS error: RMS(got - ref) / (max(ref) - min(ref))."""
    d = np.asarray(got, np.float64) - np.asarray(ref, np.float64)
    rng = float(np.max(ref) - np.min(ref))
    return float(np.sqrt(np.mean(d * d)) / rng) if rng > 0 else float(np.sqrt(np.mean(d * d)))


def frob_rel(got, ref):
    d = np.asarray(got, np.float64) - np.asarray(ref, np.float64)
    return float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300))


def check_bf16(O, L, Oref, Lref, o_tol=1e-2, lse_tol=1e-3, what=""):
    """bf16 bar: max |O - O_ref| <= 1e-2 and max |LSE - LSE_ref| <= 1e-3 (-inf rows must match)."""
    assert O.shape == Oref.shape and L.shape == Lref.shape, (O.shape, Oref.shape)
    assert np.isfinite(O).all(), f"{what}: non-finite O"
    inf_ref = np.isneginf(Lref)
    assert np.array_equal(np.isneginf(L), inf_ref), f"{what}: -inf LSE rows differ"
    assert (O[inf_ref] == 0).all(), f"{what}: empty rows must be 0"
    eo = float(np.max(np.abs(O - Oref))) if O.size else 0.0
    el = float(np.max(np.abs(L[~inf_ref] - Lref[~inf_ref]))) if (~inf_ref).any() else 0.0
    say(f"  {what}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= o_tol, f"{what}: max|dO| {eo} > {o_tol}"
    assert el <= lse_tol, f"{what}: max|dLSE| {el} > {lse_tol}"
    return eo, el


# e4m3fn keeps 3 mantissa bits: round-to-nearest changes a normal value by at most
# E4M3_U = 2^-4 of itself. Over values spread evenly (in log) across a binade the
# rounding error is uniform on +-2^-4 * 2^e while the value runs over [2^e, 2^(e+1)),
# so its RMS relative size is E4M3_RHO = 2^-4 / sqrt(8 ln 2) ~ 0.0265. With weights
# rounded independently and V drawn N(0,1) independent of them, the output error
# dO_i = sum_j P_ij e_j v_j and O_i = sum_j P_ij v_j have the same structure, so
# ||dO||_F / ||O||_F ~ E4M3_RHO; the bar allows 1.5 times that.
# bf16 output rounding: at most 2^-8 relative.
E4M3_U = 2.0 ** -4
E4M3_RHO = E4M3_U / math.sqrt(8.0 * math.log(2.0))
FP8_FROB_BAR = 1.5 * E4M3_RHO
BF16_U = 2.0 ** -8
FP8_ABS_SLACK = 2.0 ** -10


def check_fp8(O, L, Oref, Lref, Aref=None, what=""):
    """fp8 bars against the oracle on the dequantised e4m3fn inputs.

    Gate: range-normalised NRMS(O) <= 1e-2; LSE within 1e-3. Guards derived from the
    e4m3fn rounding of P (each weight enters the P V product with relative error at
    most E4M3_U, independently from key to key): the Frobenius-relative error of O is
    at most FP8_FROB_BAR (1.5 times its expected size E4M3_RHO for N(0,1) values),
    and, where A_ref (the oracle's output on |V|) is given, every element obeys
    |dO| <= E4M3_U * A_ref + BF16_U * |O_ref| + FP8_ABS_SLACK (the first-order
    bound, plus slack for e4m3fn subnormal weights and fp32 sums)."""
    assert np.isfinite(O).all(), f"{what}: non-finite O"
    e = nrms(O, Oref)
    fr = frob_rel(O, Oref)
    d = np.abs(np.asarray(O, np.float64) - Oref)
    el = float(np.max(np.abs(L - Lref))) if L.size else 0.0
    msg = f"  {what}: nrms={e:.3e} frob_rel={fr:.3e} max|dO|={d.max() if d.size else 0.0:.3e} max|dLSE|={el:.3e}"
    if Aref is not None and d.size:
        bound = E4M3_U * Aref + BF16_U * np.abs(Oref) + FP8_ABS_SLACK
        worst = float(np.max(d / bound))
        msg += f" max|dO|/bound={worst:.3f}"
    say(msg)
    assert e <= 1e-2, f"{what}: nrms {e} > 1e-2"
    assert fr <= FP8_FROB_BAR, f"{what}: frob_rel {fr} > {FP8_FROB_BAR}"
    if Aref is not None and d.size:
        assert worst <= 1.0, f"{what}: |dO| exceeds the e4m3 rounding bound by {worst:.3f}x"
    assert el <= 1e-3, f"{what}: max|dLSE| {el} > 1e-3"
    return e, el


def check_grad(got, ref, what):
    """Backward bar for one gradient tensor: ||G - G_ref||_F <= 1e-2 ||G_ref||_F and
    max |G - G_ref| <= 2e-2 max |G_ref| (an all-zero reference: max |G| <= 1e-5)."""
    assert np.isfinite(got).all(), f"{what}: non-finite"
    nref = float(np.linalg.norm(ref))
    fro = float(np.linalg.norm(got - ref)) / max(nref, 1e-300)
    mref = float(np.abs(ref).max()) if ref.size else 0.0
    mx = float(np.abs(got - ref).max()) if ref.size else 0.0
    say(f"  {what}: frob_rel={fro:.3e} max|d|={mx:.3e} (max|ref|={mref:.3e})")
    if nref == 0.0:
        # e.g. a causal row with one key: P = 1 and dS = dP - D is zero in exact
        # arithmetic, but the kernel sums dP (MFMA) and D (VALU) in different fp32
        # orders; their difference is fp32 rounding of a dot product of size
        # ~|dO||v| ~ 10, i.e. ~1e-6, times scale * |k|.
        assert mx <= 1e-5, f"{what}: expected ~0, got {mx}"
        return
    assert fro <= 1e-2, f"{what}: frob_rel {fro} > 1e-2"
    assert mx <= 2e-2 * mref, f"{what}: max|d| {mx} > 2e-2 * {mref}"
