"""Properties of the HIP path that hold at any size (GPU).

* run-to-run bitwise determinism;
* batch-composition invariance: a B=2 call equals the two B=1 calls bit for bit
  (the property the page "feat(attention): add strict bitwise ROCm path"
  measures in its Batch composition table); every workgroup owns one
  (batch, head, query tile), so this holds by construction;
* head-count invariance: a call over a subset of heads reproduces those heads
  bit for bit (that page's TP-degree invariance, single-GPU part);
* guard bands: nothing is written outside out / lse; NaN-prefilled outputs are
  fully overwritten;
* identical keys give O = mean(V) and LSE = score + ln(Skv); V = 1 gives O = 1;
  permuting K and V rows together leaves O and LSE unchanged (to tolerance);
* the launch is capturable in a HIP graph and replays give the eager bits;
  so are split-KV launches (the attention kernel, its workspace and the merge
  kernel; whole-grid and tail-only splits) and local-attention launches.
"""

import math

import numpy as np
import pytest
import torch

import head_attention_amd as ha
from gpu_helpers import say, synth_inputs, to_dev, descale_dev, run_gpu, oracle_ref, check_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def dev_inputs(B, Hq, Hkv, Sq, Skv, D, fmt, seed):
    inp = synth_inputs(B, Hq, Hkv, Sq, Skv, D, fmt, seed)
    Q, K, V = (to_dev(inp[n], fmt) for n in "qkv")
    ds = (descale_dev(inp["q_descale"]), descale_dev(inp["k_descale"]), descale_dev(inp["v_descale"])) \
        if fmt == "e4m3fn" else (None, None, None)
    return Q, K, V, ds


def fwd(Q, K, V, ds, causal, **kw):
    return ha.forward(Q, K, V, causal=causal, q_descale=ds[0], k_descale=ds[1], v_descale=ds[2], **kw)


def bits(t):
    return t.contiguous().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu()


@pytest.mark.parametrize("fmt,causal", [("bf16", False), ("bf16", True), ("e4m3fn", False)])
def test_determinism(fmt, causal):
    say(f"case determinism {fmt} causal={causal}")
    Q, K, V, ds = dev_inputs(1, 4, 2, 1000, 1000, 128, fmt, 5)
    O1, L1 = fwd(Q, K, V, ds, causal)
    O2, L2 = fwd(Q, K, V, ds, causal)
    torch.cuda.synchronize()
    assert torch.equal(bits(O1), bits(O2)) and torch.equal(L1.view(torch.int32).cpu(), L2.view(torch.int32).cpu())


@pytest.mark.parametrize("fmt,causal", [("bf16", True), ("e4m3fn", False)])
def test_batch_composition_invariance(fmt, causal):
    say(f"case batch composition {fmt} causal={causal}")
    Q, K, V, ds = dev_inputs(2, 4, 2, 512, 512, 128, fmt, 6)
    O, L = fwd(Q, K, V, ds, causal)
    for b in range(2):
        Ob, Lb = fwd(Q[b:b + 1].contiguous(), K[b:b + 1].contiguous(), V[b:b + 1].contiguous(), ds, causal)
        torch.cuda.synchronize()
        assert torch.equal(bits(Ob), bits(O[b:b + 1])) and torch.equal(Lb.cpu(), L[b:b + 1].cpu())


def test_head_subset_invariance():
    say("case head subset")
    Q, K, V, ds = dev_inputs(1, 8, 4, 700, 700, 128, "bf16", 7)
    O, L = fwd(Q, K, V, ds, True)
    # query heads 2..5 read KV heads 1..2
    Os, Ls = fwd(Q[:, 2:6].contiguous(), K[:, 1:3].contiguous(), V[:, 1:3].contiguous(), ds, True)
    torch.cuda.synchronize()
    assert torch.equal(bits(Os), bits(O[:, 2:6])) and torch.equal(Ls.cpu(), L[:, 2:6].cpu())


@pytest.mark.parametrize("fmt", ["bf16", "e4m3fn"])
def test_guard_bands_and_full_coverage(fmt):
    say(f"case guard bands {fmt}")
    B, H, Sq, Skv, D = 1, 3, 333, 200, 128
    Q, K, V, ds = dev_inputs(B, H, H, Sq, Skv, D, fmt, 8)
    pad = 4096
    obuf = torch.full((pad + B * H * Sq * D + pad,), float("nan"), dtype=torch.bfloat16, device=DEV)
    lbuf = torch.full((pad + B * H * Sq + pad,), float("nan"), dtype=torch.float32, device=DEV)
    canary_o = obuf.clone()
    O = obuf[pad:pad + B * H * Sq * D].view(B, H, Sq, D)
    L = lbuf[pad:pad + B * H * Sq].view(B, H, Sq)
    fwd(Q, K, V, ds, False, out=O, lse=L)
    torch.cuda.synchronize()
    assert torch.isnan(obuf[:pad].float()).all() and torch.isnan(obuf[-pad:].float()).all()
    assert torch.isnan(lbuf[:pad]).all() and torch.isnan(lbuf[-pad:]).all()
    assert torch.isfinite(O.float()).all() and torch.isfinite(L).all()
    del canary_o


def test_identical_keys_and_ones():
    say("case identical keys / V = 1")
    Skv, D = 1000, 128
    q = torch.randn(1, 2, 300, D).to(torch.bfloat16)
    k = torch.randn(1, 2, 1, D).to(torch.bfloat16).expand(1, 2, Skv, D).contiguous()
    v = torch.randn(1, 2, Skv, D).to(torch.bfloat16)
    scale = 1 / math.sqrt(D)
    O, L = ha.forward(q.to(DEV), k.to(DEV), v.to(DEV), scale=scale)
    torch.cuda.synchronize()
    mean_v = v.double().mean(2, keepdim=True).expand(1, 2, 300, D)
    assert (O.cpu().double() - mean_v).abs().max() <= 1e-2
    score = scale * (q.double() @ k[:, :, :1].double().transpose(-1, -2))[..., 0]
    assert (L.cpu().double() - (score + math.log(Skv))).abs().max() <= 1e-3
    O1, _ = ha.forward(q.to(DEV), torch.randn(1, 2, Skv, D, device=DEV).to(torch.bfloat16),
                       torch.ones(1, 2, Skv, D, device=DEV, dtype=torch.bfloat16), causal=True)
    torch.cuda.synchronize()
    assert (O1.float() == 1.0).all()


def test_key_permutation():
    say("case key permutation")
    Q, K, V, ds = dev_inputs(1, 2, 2, 400, 777, 128, "bf16", 9)
    O, L = fwd(Q, K, V, ds, False)
    perm = torch.randperm(777, generator=torch.Generator().manual_seed(3)).to(DEV)
    Op, Lp = fwd(Q, K[:, :, perm].contiguous(), V[:, :, perm].contiguous(), ds, False)
    torch.cuda.synchronize()
    assert (O.float() - Op.float()).abs().max() <= 1e-2
    assert (L - Lp).abs().max() <= 1e-4


def test_graph_capture_replays():
    say("case hip graph capture")
    Q, K, V, ds = dev_inputs(1, 4, 4, 600, 600, 128, "bf16", 10)
    O, L = fwd(Q, K, V, ds, True)
    torch.cuda.synchronize()
    Og = torch.empty_like(O)
    Lg = torch.empty_like(L)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fwd(Q, K, V, ds, True, out=Og, lse=Lg, stream=s)
    for _ in range(3):
        Og.zero_()
        Lg.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(Og), bits(O)) and torch.equal(Lg.cpu(), L.cpu())


def test_graph_capture_splitkv_and_window_replays():
    """One graph holding a whole-grid split-KV launch, a tail-only split-KV launch (the
    library's choice at 280 query tiles) and a local-attention launch, on a side stream:
    every replay, with the outputs NaN-filled and the workspaces overwritten in between,
    gives the eager bits."""
    say("case hip graph capture: split-KV and window")
    scale = 1 / math.sqrt(128)
    Qa, Ka, Va, dsa = dev_inputs(1, 2, 2, 300, 4000, 128, "bf16", 41)          # whole-grid split (auto)
    Qb, Kb, Vb, dsb = dev_inputs(1, 40, 40, 1700, 2100, 128, "e4m3fn", 42)      # tail-only split (auto)
    Qc, Kc, Vc, dsc = dev_inputs(1, 4, 2, 900, 900, 128, "bf16", 43)            # window + sink, causal
    na = ha.attn_splitkv_auto_splits(1, 2, 300, 4000, 128)
    nb = ha.attn_splitkv_auto_splits(1, 40, 1700, 2100, 128)
    assert na > 1 and nb == 2
    wa = torch.empty(ha.attn_splitkv_workspace_bytes(1, 2, 300, 128, na), dtype=torch.uint8, device=DEV)
    wb = torch.empty(ha.attn_splitkv_workspace_bytes(1, 40, 1700, 128, nb), dtype=torch.uint8, device=DEV)
    outs = [(torch.empty(1, 2, 300, 128, dtype=torch.bfloat16, device=DEV), torch.empty(1, 2, 300, device=DEV)),
            (torch.empty(1, 40, 1700, 128, dtype=torch.bfloat16, device=DEV), torch.empty(1, 40, 1700, device=DEV)),
            (torch.empty(1, 4, 900, 128, dtype=torch.bfloat16, device=DEV), torch.empty(1, 4, 900, device=DEV))]

    def launch(stream):
        sa = ha.attn_fwd_splitkv(Qa, Ka, Va, outs[0][0], outs[0][1], 1, 2, 2, 300, 4000, 128, scale, 0,
                                 ha.ATTN_BF16, None, None, None, 0, wa, wa.numel(), stream)
        sb = ha.attn_fwd_splitkv(Qb, Kb, Vb, outs[1][0], outs[1][1], 1, 40, 40, 1700, 2100, 128, scale, 0,
                                 ha.ATTN_FP8_E4M3FN, dsb[0], dsb[1], dsb[2], 0, wb, wb.numel(), stream)
        sc = ha.attn_fwd_window(Qc, Kc, Vc, outs[2][0], outs[2][1], 1, 4, 2, 900, 900, 128, scale, 1,
                                ha.ATTN_BF16, None, None, None, 0, 200, 0, 70, stream)
        assert (sa, sb, sc) == (0, 0, 0)

    launch(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ref = [(bits(o), bits(l)) for o, l in outs]
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        launch(side.cuda_stream)
    for rep in range(3):
        for o, l in outs:
            o.fill_(float("nan"))
            l.fill_(float("nan"))
        wa.fill_(255)
        wb.fill_(255)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (o, l), (ro, rl) in zip(outs, ref):
            assert torch.equal(bits(o), ro) and torch.equal(bits(l), rl), f"replay {rep} differs from eager"
