"""Pure-Python attention for tiny shapes, used only to pin ``oracle.attention``.

Test infrastructure only (see the package docstring).

It follows the plain definition by a different route from the numpy oracle:
no running or row maximum is subtracted (inputs are tiny, so exp cannot
overflow), the softmax weights are formed as exp(s_j) / sum exp(s), every sum
is ``math.fsum``, and the allowed key set is enumerated explicitly per query.
Inputs are nested lists (or anything indexable) of real numbers.
"""

import math


def attention_brute(q, k, v, scale, causal=False, kv_start=0, window_left=-1, window_right=-1, sink=0):
    B, Hq, Sq, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv, Skv = len(k[0]), len(k[0][0])
    group = Hq // Hkv
    out = [[[[0.0] * D for _ in range(Sq)] for _ in range(Hq)] for _ in range(B)]
    lse = [[[-math.inf] * Sq for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            hk = h // group
            for i in range(Sq):
                keys = []
                for j in range(Skv):
                    pos = j + kv_start
                    if causal and pos > i:
                        continue
                    lo_ok = window_left < 0 or pos >= i - window_left
                    hi_ok = window_right < 0 or pos <= i + window_right
                    if (lo_ok and hi_ok) or pos < sink:
                        keys.append(j)
                if not keys:
                    continue
                e = [math.exp(scale * math.fsum(q[b][h][i][d] * k[b][hk][j][d] for d in range(D)))
                     for j in keys]
                z = math.fsum(e)
                lse[b][h][i] = math.log(z)
                for d in range(D):
                    out[b][h][i][d] = math.fsum(e[t] * v[b][hk][j][d] for t, j in enumerate(keys)) / z
    return out, lse
