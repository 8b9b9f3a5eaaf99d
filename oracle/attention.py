"""Plain float64 attention forward with per-row LSE, and the LSE merge.

Test infrastructure only (see the package docstring).

What is computed, and where the pages say so
--------------------------------------------
* Fused scaled-dot-product attention forward that also returns the row
  log-sum-exp: page "[Proposal] ROCm (AMD Instinct) support for the core
  attention and distributed init" (sections "Where it breaks on ROCm" and the
  follow-up on the efficient kernel with compute_log_sumexp), and page
  "F8 fmha ASM gfx950", Test Result section (fmha_v3_fwd with softmax_scale,
  is_causal, return_softmax_lse and q/k/v_descale).
* The LSE is the attention-domain LSE of the scaled scores, and partial
  (out, lse) results combine in a fixed order: page "feat(attention): add
  strict bitwise ROCm path", Summary table (Vime boundary returns
  (out, lse); CP communication reduce-scatters Out/LSE).
* Grouped KV heads, 32 query heads over 8 KV heads: same page, ROCm
  Validation table (Qwen3-8B dense heads).
* Causal prefill: same page, Benchmark results.

Readings where the pages are silent (each listed in the design notes):
* LSE is in natural log and includes the softmax scale: LSE_i = ln sum_j
  exp(scale * q_i . k_j) over allowed keys.
* Causal keeps key j for query i iff j + kv_start <= i (top-left alignment,
  with an explicit key offset for chunked calls).
* A row with no allowed key has O = 0 and LSE = -inf.
* Query head h reads KV head h // (Hq / Hkv).
* Local attention: window sides and sink count are in key positions (the
  same absolute positions as the causal test); a key is kept if it is inside
  the window or is a sink key, and causal applies on top of both.

Query rows are processed in independent blocks purely to bound memory (one
fp64 score row at 75600 keys is 605 KB); no sum is split or reordered by it.
"""

import numpy as np


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, S, D]")
    B, Hq, Sq, D = q.shape
    Bk, Hkv, Skv, Dk = k.shape
    if v.shape != k.shape or Bk != B or Dk != D:
        raise ValueError("k and v must be [B, Hkv, Skv, D] matching q")
    if Hkv == 0 or Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, Hq, Hkv, Sq, Skv, D


def attention_forward(q, k, v, scale, causal=False, kv_start=0, rows=None, row_block=512,
                      window_left=-1, window_right=-1, sink=0):
    """Attention forward in float64.

    q: [B, Hq, Sq, D], k and v: [B, Hkv, Skv, D], real values (already
    dequantised). ``rows`` optionally selects a subset of query rows (an index
    array into Sq); each output row depends only on its own query, so a subset is
    the same computation restricted to those rows.

    Local attention (window_size_left / window_size_right of the fmha_v3_fwd
    call on the page "F8 fmha ASM gfx950", Test Result section; window and sink
    settings of the page "[Proposal] ROCm (AMD Instinct) support for the core
    attention and distributed init"): with key position j = key index +
    kv_start, key j is allowed for query i iff it lies in the window
    [i - window_left, i + window_right] (a side of -1 is unbounded) or j < sink;
    causal additionally requires j <= i.

    Returns (O [B, Hq, R, D], LSE [B, Hq, R]) with R = Sq or len(rows).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Hkv, Sq, Skv, D = _check_shapes(q, k, v)
    if kv_start < 0:
        raise ValueError("kv_start must be >= 0")
    if window_left < -1 or window_right < -1 or sink < 0:
        raise ValueError("window sides must be >= -1 and sink >= 0")
    local = window_left >= 0 or window_right >= 0 or sink > 0
    group = Hq // Hkv
    row_idx = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    R = row_idx.shape[0]
    out = np.zeros((B, Hq, R, D), dtype=np.float64)
    lse = np.full((B, Hq, R), -np.inf, dtype=np.float64)
    key_pos = np.arange(Skv, dtype=np.int64) + int(kv_start)
    for b in range(B):
        for h in range(Hq):
            kv_h = h // group                      # GQA head map
            K = k[b, kv_h]
            V = v[b, kv_h]
            for r0 in range(0, R, row_block):
                ridx = row_idx[r0:r0 + row_block]
                s = float(scale) * (q[b, h, ridx] @ K.T)          # [r, Skv] scores
                if causal:
                    allowed = key_pos[None, :] <= ridx[:, None]
                    s = np.where(allowed, s, -np.inf)
                if local:
                    in_win = np.ones((len(ridx), Skv), dtype=bool)
                    if window_left >= 0:
                        in_win &= key_pos[None, :] >= ridx[:, None] - int(window_left)
                    if window_right >= 0:
                        in_win &= key_pos[None, :] <= ridx[:, None] + int(window_right)
                    s = np.where(in_win | (key_pos[None, :] < int(sink)), s, -np.inf)
                m = s.max(axis=1) if Skv > 0 else np.full(len(ridx), -np.inf)
                live = np.isfinite(m)
                p = np.exp(s[live] - m[live, None])               # exp(-inf) = 0 for masked
                l = p.sum(axis=1)
                out[b, h, r0 + np.nonzero(live)[0]] = (p @ V) / l[:, None]
                lse[b, h, r0 + np.nonzero(live)[0]] = m[live] + np.log(l)
    return out, lse


def merge_lse(parts):
    """Merge partial results over disjoint key sets.

    parts: sequence of (O_c [..., D], L_c [...]) in float64, each the attention of
    the same queries over one key chunk. Returns (O, L) with
    L = ln sum_c exp(L_c) (-inf when every L_c is -inf) and
    O = sum_c exp(L_c - L) * O_c (0 where L = -inf).
    """
    Ls = np.stack([np.asarray(L, dtype=np.float64) for _, L in parts])
    Os = np.stack([np.asarray(O, dtype=np.float64) for O, _ in parts])
    Lmax = Ls.max(axis=0)
    finite = np.isfinite(Lmax)
    shift = np.where(finite, Lmax, 0.0)
    w = np.exp(Ls - shift[None])                    # exp(-inf) = 0 for empty chunks
    tot = w.sum(axis=0)
    L = np.where(finite, shift + np.log(np.where(finite, tot, 1.0)), -np.inf)
    wn = np.where(finite[None], w / np.where(finite, tot, 1.0)[None], 0.0)
    O = (wn[..., None] * Os).sum(axis=0)
    return O, L
