"""Plain float64 attention backward: dQ, dK, dV from Q, K, V and dO.

Test infrastructure only (see the package docstring).

What is computed, and where the pages say so
--------------------------------------------
The gradients of the attention forward with respect to its three inputs,
the dQ / dK / dV tensors that the page "feat(attention): add strict bitwise
ROCm path" checks next to out and lse (Latest status) and times as the
deterministic and non-deterministic backward (section "What the strict
contract costs"). The forward is the one of ``oracle.attention``: with
s_ij = scale * q_i . k_j over the allowed keys, P = softmax_j(s), O = P V.

The gradients follow from the chain rule on that definition, written out
step by step:

    dV_j = sum_i P_ij dO_i                       (O = P V)
    dP_ij = dO_i . v_j
    D_i  = sum_j P_ij dP_ij = dO_i . O_i         (softmax Jacobian)
    dS_ij = P_ij (dP_ij - D_i)                   (gradient w.r.t. s_ij)
    dQ_i = scale * sum_j dS_ij k_j
    dK_j = scale * sum_i dS_ij q_i

Masked pairs have P_ij = 0 and so contribute nothing; a row with no allowed
key has zero gradients. With grouped KV heads each KV head's dK and dV are
the sums over the query heads that read it. Reading: the loss is only seen
through dO (no gradient flows into the LSE output).

P is recomputed here from Q and K with its own row maximum; nothing is taken
from a forward pass of the HIP path.

A backward receives the forward's output next to dO (the dense MHA core of
that page pairs an mha_fwd with an mha_bwd, and the strict path checks dQ / dK
/ dV computed from its own out and lse); D_i is the one quantity taken from
it. ``out`` lets the caller state that O, for example the forward's output
rounded to bf16: D_i = dO_i . out_i is then formed from it instead of from the
float64 O = P V (with the exact O both agree). In rows where P is nearly one
key, dP_ij - D_i is a small difference of two larger numbers, and the rounding
of O decides it.
"""

import numpy as np


def attention_backward(q, k, v, dout, scale, causal=False, kv_start=0, row_block=512, out=None):
    """(dQ [B,Hq,Sq,D], dK [B,Hkv,Skv,D], dV [B,Hkv,Skv,D]) in float64.

    q: [B, Hq, Sq, D], k and v: [B, Hkv, Skv, D], dout: [B, Hq, Sq, D], real
    values (already dequantised). Causal keeps key j for query i iff
    j + kv_start <= i, as in the forward. ``out`` (optional, [B, Hq, Sq, D]):
    the forward output the backward is given; D_i = dO_i . out_i then comes
    from it rather than from the float64 O.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    if q.ndim != 4 or k.ndim != 4 or v.shape != k.shape or dout.shape != q.shape:
        raise ValueError("q, dout must be [B, Hq, Sq, D] and k, v [B, Hkv, Skv, D]")
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != D or Hkv == 0 or Hq % Hkv != 0:
        raise ValueError("inconsistent shapes")
    if kv_start < 0:
        raise ValueError("kv_start must be >= 0")
    out64 = None if out is None else np.asarray(out, dtype=np.float64)
    if out64 is not None and out64.shape != q.shape:
        raise ValueError("out must be [B, Hq, Sq, D]")
    group = Hq // Hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    key_pos = np.arange(Skv, dtype=np.int64) + int(kv_start)
    for b in range(B):
        for h in range(Hq):
            kv_h = h // group
            K, V = k[b, kv_h], v[b, kv_h]
            for r0 in range(0, Sq, row_block):
                rows = np.arange(r0, min(Sq, r0 + row_block))
                s = float(scale) * (q[b, h, rows] @ K.T)
                if causal:
                    s = np.where(key_pos[None, :] <= rows[:, None], s, -np.inf)
                m = s.max(axis=1) if Skv > 0 else np.full(len(rows), -np.inf)
                live = np.isfinite(m)
                P = np.zeros_like(s)
                e = np.exp(s[live] - m[live, None])
                P[live] = e / e.sum(axis=1, keepdims=True)
                dO = dout[b, h, rows]
                O = P @ V if out64 is None else out64[b, h, rows]
                dP = dO @ V.T
                Drow = (dO * O).sum(axis=1)
                dS = P * (dP - Drow[:, None])
                dq[b, h, rows] = float(scale) * (dS @ K)
                dk[b, kv_h] += float(scale) * (dS.T @ q[b, h, rows])
                dv[b, kv_h] += P.T @ dO
    return dq, dk, dv
