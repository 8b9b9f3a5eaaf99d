"""Pins of the fp64 backward oracle against what the mathematics fixes.

None of these tests needs a GPU. The backward is checked against (a) central
finite differences of the pinned forward oracle, (b) torch's autograd through
the forward written with plain CPU float64 ops, and (c) identities of the
softmax: shifting every key of a row by the same vector changes nothing, so
the dK of a head sum to zero; P's rows sum to one, so the dV of a head sum to
the dO rows; identical keys give dQ = 0; value rows all equal give zero dQ and
dK. Planted slips in a copy of the oracle are shown to fail them.
"""

import os

import numpy as np
import pytest
import torch

from oracle import attention_forward, attention_backward

rng = np.random.default_rng(4321)
BWD_FILE = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "backward.py")


def rand(*shape, scale=1.0):
    return rng.standard_normal(shape) * scale


def autograd_ref(q, k, v, dout, scale, causal, kv_start=0):
    """Gradients of sum(O * dout) by torch autograd through the plain forward."""
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    g = q.shape[1] // k.shape[1]
    K = kt.repeat_interleave(g, dim=1)
    V = vt.repeat_interleave(g, dim=1)
    s = scale * (qt @ K.transpose(-1, -2))
    if causal:
        i = torch.arange(q.shape[2])[:, None]
        j = torch.arange(k.shape[2])[None, :] + kv_start
        s = s.masked_fill(j > i, -float("inf"))
    p = torch.softmax(s, dim=-1)
    p = torch.nan_to_num(p, nan=0.0)                      # rows with no key
    O = p @ V
    (O * torch.tensor(dout)).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("Hq,Hkv,Sq,Skv,D", [(1, 1, 5, 7, 3), (4, 2, 9, 6, 4), (6, 2, 17, 17, 8), (2, 1, 3, 40, 5)])
@pytest.mark.parametrize("causal,kv_start", [(False, 0), (True, 0), (True, 3)])
def test_backward_matches_autograd(Hq, Hkv, Sq, Skv, D, causal, kv_start):
    q, k, v, do = rand(2, Hq, Sq, D), rand(2, Hkv, Skv, D), rand(2, Hkv, Skv, D), rand(2, Hq, Sq, D)
    dq, dk, dv = attention_backward(q, k, v, do, 0.6, causal, kv_start, row_block=4)
    rq, rk, rv = autograd_ref(q, k, v, do, 0.6, causal, kv_start)
    for got, ref in ((dq, rq), (dk, rk), (dv, rv)):
        np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_finite_differences_of_forward_oracle(causal):
    """Every input element, central differences of sum(O * W) through attention_forward."""
    Hq, Hkv, Sq, Skv, D = 2, 1, 3, 4, 2
    q, k, v, W = rand(1, Hq, Sq, D), rand(1, Hkv, Skv, D), rand(1, Hkv, Skv, D), rand(1, Hq, Sq, D)
    scale = 0.8

    def loss(q_, k_, v_):
        return float((attention_forward(q_, k_, v_, scale, causal)[0] * W).sum())

    dq, dk, dv = attention_backward(q, k, v, W, scale, causal)
    h = 1e-6
    for x, grad, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-8)


def test_dk_sums_to_zero_and_dv_sums_to_dout():
    Hq, Hkv, S, D = 4, 2, 20, 6
    q, k, v, do = rand(1, Hq, S, D), rand(1, Hkv, S, D), rand(1, Hkv, S, D), rand(1, Hq, S, D)
    for causal in (False, True):
        _, dk, dv = attention_backward(q, k, v, do, 0.5, causal)
        np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
        want = do.reshape(1, Hkv, Hq // Hkv, S, D).sum(axis=(2, 3))
        np.testing.assert_allclose(dv.sum(axis=2), want, rtol=1e-12, atol=1e-12)


def test_identical_keys_give_zero_dq():
    S, D = 15, 5
    q, v, do = rand(1, 2, S, D), rand(1, 2, S, D), rand(1, 2, S, D)
    k = np.broadcast_to(rand(1, 2, 1, D), (1, 2, S, D)).copy()
    dq, _, _ = attention_backward(q, k, v, do, 0.7, False)
    np.testing.assert_allclose(dq, 0.0, atol=1e-12)


def test_equal_value_rows_give_zero_dq_dk():
    S, D = 13, 4
    q, k, do = rand(1, 1, S, D), rand(1, 1, S, D), rand(1, 1, S, D)
    v = np.broadcast_to(rand(1, 1, 1, D), (1, 1, S, D)).copy()
    for causal in (False, True):
        dq, dk, dv = attention_backward(q, k, v, do, 0.9, causal)
        np.testing.assert_allclose(dq, 0.0, atol=1e-12)
        np.testing.assert_allclose(dk, 0.0, atol=1e-12)
        assert np.abs(dv).max() > 0.1


def test_rows_without_keys_have_zero_gradient():
    """kv_start = 3 under causal: rows 0-2 see no key; rows 3-5 see what rows 0-2 of an
    unshifted causal call see."""
    q, k, v, do = rand(1, 1, 6, 3), rand(1, 1, 4, 3), rand(1, 1, 4, 3), rand(1, 1, 6, 3)
    dq, dk, dv = attention_backward(q, k, v, do, 0.5, True, kv_start=3)
    assert (dq[0, 0, :3] == 0).all() and np.abs(dq[0, 0, 3:]).max() > 0
    dq2, dk2, dv2 = attention_backward(q[:, :, 3:], k, v, do[:, :, 3:], 0.5, True, kv_start=0)
    np.testing.assert_array_equal(dq[:, :, 3:], dq2)
    np.testing.assert_allclose(dk, dk2, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(dv, dv2, rtol=1e-13, atol=1e-15)


def test_given_exact_out_equals_default():
    """Passing the forward's own float64 O as ``out`` changes nothing."""
    q, k, v, do = rand(2, 4, 9, 5), rand(2, 2, 11, 5), rand(2, 2, 11, 5), rand(2, 4, 9, 5)
    for causal in (False, True):
        O, _ = attention_forward(q, k, v, 0.6, causal, kv_start=2)
        got = attention_backward(q, k, v, do, 0.6, causal, kv_start=2, out=O)
        ref = attention_backward(q, k, v, do, 0.6, causal, kv_start=2)
        for a, b in zip(got, ref):
            np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


def _one_key_closed_form(q, k, v, do, scale, out):
    """One key: P = 1 for every row, so dV = sum of dO, and dS_i = dO_i . (v - out_i)
    (dP_i = dO_i . v, D_i = dO_i . out_i), dQ_i = scale dS_i k, dK = scale sum_i dS_i q_i."""
    B, Hkv, Sq, D = q.shape[0], k.shape[1], q.shape[2], q.shape[3]
    g = q.shape[1] // Hkv
    vv = v[:, :, 0, :][:, :, None, None, :]                                    # [B, Hkv, 1, 1, D]
    ds = ((vv - out.reshape(B, Hkv, g, Sq, D)) * do.reshape(B, Hkv, g, Sq, D)).sum(axis=-1)   # [B, Hkv, g, Sq]
    kk = k[:, :, 0, :]
    dq = scale * ds[..., None] * kk[:, :, None, None, :]
    dk = scale * (ds[..., None] * q.reshape(q.shape[0], k.shape[1], g, q.shape[2], -1)).sum(axis=(2, 3))
    dv = do.reshape(q.shape[0], k.shape[1], g, q.shape[2], -1).sum(axis=(2, 3))
    return dq.reshape(q.shape), dk[:, :, None, :], dv[:, :, None, :]


def test_given_out_one_key_closed_form():
    """With a given out that is not the exact O (here v plus noise), one key: the closed
    form above. A slip that ignores ``out`` or takes it for the wrong head fails it."""
    q, k, v, do = rand(1, 4, 3, 5), rand(1, 2, 1, 5), rand(1, 2, 1, 5), rand(1, 4, 3, 5)
    out = np.repeat(v, 2, axis=1).repeat(3, axis=2) + 0.1 * rand(1, 4, 3, 5)
    got = attention_backward(q, k, v, do, 0.7, False, out=out)
    ref = _one_key_closed_form(q, k, v, do, 0.7, out)
    for a, b in zip(got, ref):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)
    mut = _load_mutant("O = P @ V if out64 is None else out64[b, h, rows]", "O = P @ V").attention_backward
    assert not np.allclose(mut(q, k, v, do, 0.7, False, out=out)[0], ref[0])


def _load_mutant(old, new):
    import types
    src = open(BWD_FILE).read()
    assert old in src, old
    mod = types.ModuleType("mutant_bwd")
    mod.__dict__["np"] = np
    exec(compile(src.replace(old, new, 1), BWD_FILE, "exec"), mod.__dict__)
    return mod


def _pins_pass(fn):
    r = np.random.default_rng(11)
    try:
        q, k, v, do = r.standard_normal((1, 4, 5, 3)), r.standard_normal((1, 2, 6, 3)), \
            r.standard_normal((1, 2, 6, 3)), r.standard_normal((1, 4, 5, 3))
        for causal, ks in ((False, 0), (True, 1)):
            got = fn(q, k, v, do, 0.7, causal, ks)
            ref = autograd_ref(q, k, v, do, 0.7, causal, ks)
            if not all(np.allclose(a, b, atol=1e-9) for a, b in zip(got, ref)):
                return False
        return True
    except Exception:
        return False


@pytest.mark.parametrize("old,new", [
    ("dS = P * (dP - Drow[:, None])", "dS = P * dP"),                                  # dropped softmax term
    ("dk[b, kv_h] += float(scale) * (dS.T @ q[b, h, rows])",
     "dk[b, kv_h] += (dS.T @ q[b, h, rows])"),                                         # dropped scale in dK
    ("dv[b, kv_h] += P.T @ dO", "dv[b, kv_h] = P.T @ dO"),                             # GQA heads not summed
    ("dq[b, h, rows] = float(scale) * (dS @ K)", "dq[b, h, rows] = float(scale) * (dS @ V)"),  # wrong operand
    ("Drow = (dO * O).sum(axis=1)", "Drow = (dO * O).sum(axis=1) / 2"),                # wrong row term
    ("key_pos[None, :] <= rows[:, None]", "key_pos[None, :] < rows[:, None]"),          # off-by-one mask
])
def test_backward_pins_catch_planted_mistakes(old, new):
    assert _pins_pass(_load_mutant("def attention_backward", "def attention_backward").attention_backward)
    assert not _pins_pass(_load_mutant(old, new).attention_backward)
