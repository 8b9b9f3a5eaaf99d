"""attn_fwd_splitkv_static: the split-KV forward with its partials in the library's
static device array, for callers that cannot allocate. Its outputs must equal those of
attn_fwd_splitkv with a caller workspace (same kernels, same split count: the same
bits) and meet the oracle bars, on two calls in a row per format, the second smaller;
a request whose partials exceed the array is refused before anything is launched."""

import math

import numpy as np
import pytest
import torch

import head_attention_amd as ha
from gpu_helpers import say, synth_inputs, to_dev, descale_dev, refs, check_any

pytestmark = pytest.mark.gpu

# B, Hq, Hkv, Sq, Skv, D, causal, fmt: per format a larger call, then a smaller one
CALLS = [
    (1, 8, 2, 256, 40000, 128, False, "bf16"),
    (1, 2, 1, 100, 3000, 64, True, "bf16"),
    (1, 4, 4, 256, 30000, 128, False, "e4m3fn"),
    (2, 1, 1, 50, 2000, 128, True, "e4m3fn"),
]


def test_static_scratch_equals_workspace_entry_point():
    stream = torch.cuda.current_stream()
    for i, (B, Hq, Hkv, Sq, Skv, D, causal, fmt) in enumerate(CALLS):
        say(f"case static scratch call {i}: B{B} Hq{Hq} Hkv{Hkv} Sq{Sq} Skv{Skv} D{D} causal={causal} {fmt}")
        n = ha.attn_splitkv_auto_splits(B, Hq, Sq, Skv, D)
        need = ha.attn_splitkv_workspace_bytes(B, Hq, Sq, D, n)
        assert n > 1 and 0 < need <= ha.SPLITKV_STATIC_SCRATCH_BYTES, (n, need)
        inp = synth_inputs(B, Hq, Hkv, Sq, Skv, D, fmt, seed=900 + i)
        scale = 1 / math.sqrt(D)
        Q, K, V = (to_dev(inp[x], fmt) for x in "qkv")
        ds = [descale_dev(inp[x]) for x in ("q_descale", "k_descale", "v_descale")] if fmt == "e4m3fn" else [None] * 3
        Ow, Lw = ha.forward_splitkv(Q, K, V, n_splits=0, scale=scale, causal=causal,
                                    q_descale=ds[0], k_descale=ds[1], v_descale=ds[2])
        Os = torch.full((B, Hq, Sq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        Ls = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device="cuda")
        dt = ha.ATTN_BF16 if fmt == "bf16" else ha.ATTN_FP8_E4M3FN
        st = ha.attn_fwd_splitkv_static(Q, K, V, Os, Ls, B, Hq, Hkv, Sq, Skv, D, scale, causal, dt,
                                        ds[0], ds[1], ds[2], 0, stream.cuda_stream)
        assert st == 0, ha.attn_status_string(st)
        torch.cuda.synchronize()
        assert torch.equal(Os.view(torch.int16), Ow.view(torch.int16)), "O differs from the workspace entry point"
        assert torch.equal(Ls.view(torch.int32), Lw.view(torch.int32)), "LSE differs from the workspace entry point"
        O, L = Os.float().cpu().numpy(), Ls.cpu().numpy()
        R = refs(inp, scale, causal)
        live = ~np.isneginf(R[1])
        assert np.array_equal(np.isneginf(L), ~live) and (O[~live] == 0).all()
        check_any(inp, O, L, R, what=f"static scratch call {i}", live=live)


def test_static_scratch_refuses_more_than_it_holds():
    """256 splits of 4 heads x 8192 rows need 4.3 GB of partials: ATTN_ERR_WORKSPACE,
    with nothing launched (the outputs keep their sentinel)."""
    B, Hq, Hkv, Sq, Skv, D = 1, 4, 4, 8192, 65536, 128
    need = ha.attn_splitkv_workspace_bytes(B, Hq, Sq, D, 256)
    assert need > ha.SPLITKV_STATIC_SCRATCH_BYTES
    say("case static scratch too small")
    Q = torch.zeros((B, Hq, Sq, D), dtype=torch.bfloat16, device="cuda")
    K = torch.zeros((B, Hkv, Skv, D), dtype=torch.bfloat16, device="cuda")
    V = torch.zeros_like(K)
    O = torch.full((B, Hq, Sq, D), 7.0, dtype=torch.bfloat16, device="cuda")
    L = torch.full((B, Hq, Sq), 7.0, dtype=torch.float32, device="cuda")
    st = ha.attn_fwd_splitkv_static(Q, K, V, O, L, B, Hq, Hkv, Sq, Skv, D, 1 / math.sqrt(D), False, ha.ATTN_BF16,
                                    None, None, None, 256, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert ha.STATUS[st] == "ATTN_ERR_WORKSPACE", ha.attn_status_string(st)
    assert (O.float() == 7.0).all() and (L == 7.0).all()
