"""The C-ABI library on the CPU: it loads, exports every declared symbol,
refuses bad arguments before touching a device, and its host-side merge
matches the oracle's merge. No kernel is launched here."""

import os
import re

import numpy as np
import pytest
import torch

import head_attention_amd as ha
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ha.library_path):
        from head_attention_amd.build import build
        build()
    return ha.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) == set(ha.EXPORTED), names
    for n in names:
        assert hasattr(L, n), f"missing export {n}"


def test_mfma_probe_library_loads_and_refuses_bad_arguments():
    """The benchmark's MFMA probes (a measurement aid beside the attention library)
    export their four entry points and reject bad arguments without launching."""
    import ctypes
    path = os.path.join(ROOT, "head_attention_amd", "libmfma_probe.so")
    if not os.path.exists(path):
        from head_attention_amd.build import build
        build()
    P = ctypes.CDLL(path)
    P.mfma_probe_launch.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p]
    P.mfma_probe_launch.restype = ctypes.c_int
    assert hasattr(P, "mfma_probe_device")
    assert P.mfma_probe_launch(0, 0, 10, 1 << 20, 1 << 20, None) == 1      # no workgroups
    assert P.mfma_probe_launch(0, 4, 0, 1 << 20, 1 << 20, None) == 1       # no iterations
    assert P.mfma_probe_launch(1, 4, 10, None, 1 << 20, None) == 1         # no operand buffer
    P.mfma_softmax_probe_launch.argtypes = P.mfma_probe_launch.argtypes
    P.mfma_softmax_probe_launch.restype = ctypes.c_int
    assert P.mfma_softmax_probe_launch(1, 0, 10, 1 << 20, 1 << 20, None) == 1
    assert P.mfma_softmax_probe_launch(0, 4, 0, 1 << 20, 1 << 20, None) == 1
    assert P.mfma_softmax_probe_launch(1, 4, 10, 1 << 20, None, None) == 1   # no output buffer
    P.valu_rate_probe_launch.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    P.valu_rate_probe_launch.restype = ctypes.c_int
    assert P.valu_rate_probe_launch(3, 4, 10, 1 << 20, None) == 1             # no such kind
    assert P.valu_rate_probe_launch(-1, 4, 10, 1 << 20, None) == 1
    assert P.valu_rate_probe_launch(0, 0, 10, 1 << 20, None) == 1             # no workgroups
    assert P.valu_rate_probe_launch(1, 4, 0, 1 << 20, None) == 1              # no iterations
    assert P.valu_rate_probe_launch(2, 4, 10, None, None) == 1                # no output buffer


def test_status_strings(L):
    for code, name in ha.STATUS.items():
        assert ha.attn_status_string(code).startswith(name)
    assert ha.attn_status_string(99) == "ATTN_ERR_UNKNOWN"


# A fake, 16-byte aligned, never-dereferenced address: validation returns before any use.
P = 1 << 20


@pytest.mark.parametrize("args,status", [
    (dict(D=96), 3),
    (dict(D=0), 3),
    (dict(dtype=2), 4),
    (dict(Hq=3, Hkv=2), 2),
    (dict(Hkv=0), 2),
    (dict(Sq=-1), 2),
    (dict(B=-2), 2),
    (dict(kv_start=-1), 2),
    (dict(scale=float("nan")), 7),
    (dict(scale=float("inf")), 7),
    (dict(scale=0.0), 7),
    (dict(scale=-1.0), 7),
    (dict(q=None), 1),
    (dict(out=None), 1),
    (dict(lse=None), 1),
    (dict(k=None), 1),
    (dict(q=P + 8), 5),
    (dict(v=P + 4), 5),
    (dict(lse=P + 2), 5),
    (dict(Sq=1 << 30), 6),
    (dict(Skv=1 << 30), 6),
    (dict(Sq=8388352), 6),                   # one past the largest D128 query slice
    (dict(Skv=8388544), 6),                  # one past the largest D128 bf16 key slice
    (dict(Skv=16777152, dtype=1), 6),        # one past the largest D128 fp8 key slice
    (dict(Sq=16776960, D=64), 6),            # one past the largest D64 query slice
    (dict(kv_start=(1 << 30) - 100), 6),     # key positions must stay below 2^30
    (dict(kv_start=(1 << 30) - 65, Skv=1), 6),    # kv_start + Skv + one key tile = 2^30
    # zero sizes: nothing to compute is OK and enqueues nothing, even with null pointers
    (dict(B=0), 0),
    (dict(Sq=0), 0),
    (dict(Hq=0, Hkv=0), 0),
    (dict(Sq=0, q=None, out=None, lse=None, k=None, v=None), 0),
    # lse needs 4-byte alignment only: a 4-aligned lse passes the alignment check and is
    # stopped by the next one (index overflow), a 2-aligned one is not
    (dict(lse=P + 4, Sq=1 << 30), 6),
    (dict(lse=P + 2, Sq=1 << 30), 5),
])
def test_fail_closed_validation(L, args, status):
    a = dict(q=P, k=P, v=P, out=P, lse=P, B=1, Hq=4, Hkv=2, Sq=100, Skv=100, D=128, scale=0.1,
             causal=0, dtype=0, kv_start=0)
    a.update(args)
    st = ha.attn_fwd_chunk(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["Sq"],
                           a["Skv"], a["D"], a["scale"], a["causal"], a["dtype"], None, None, None,
                           a["kv_start"], 0)
    assert st == status, (args, ha.STATUS.get(st, st))


@pytest.mark.parametrize("args,status", [
    (dict(n_splits=-1), 2),
    (dict(n_splits=257), 2),
    (dict(n_splits=2, workspace=None), 9),
    (dict(n_splits=2, workspace=P + 8), 9),
    (dict(n_splits=2, wbytes=100), 9),
    (dict(n_splits=2, D=96), 3),
    (dict(n_splits=2, q=None), 1),
])
def test_splitkv_fail_closed_validation(L, args, status):
    a = dict(q=P, k=P, v=P, out=P, lse=P, B=1, Hq=4, Hkv=2, Sq=100, Skv=1000, D=128, n_splits=2,
             workspace=P, wbytes=1 << 40)
    a.update(args)
    st = ha.attn_fwd_splitkv(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["Sq"],
                             a["Skv"], a["D"], 0.1, 0, 0, None, None, None, a["n_splits"], a["workspace"],
                             a["wbytes"], 0)
    assert st == status, (args, ha.STATUS.get(st, st))


@pytest.mark.parametrize("args,status", [
    (dict(wl=-2), 2),
    (dict(wr=-5), 2),
    (dict(sink=-1), 2),
    (dict(wl=3, D=96), 3),
    (dict(wl=3, q=None), 1),
    (dict(wl=3, kv_start=-1), 2),
    (dict(wl=3, kv_start=1 << 30), 6),
])
def test_window_fail_closed_validation(L, args, status):
    a = dict(q=P, k=P, v=P, out=P, lse=P, D=128, kv_start=0, wl=-1, wr=-1, sink=0)
    a.update(args)
    st = ha.attn_fwd_window(a["q"], a["k"], a["v"], a["out"], a["lse"], 1, 4, 2, 100, 100, a["D"], 0.1, 0, 0,
                            None, None, None, a["kv_start"], a["wl"], a["wr"], a["sink"], 0)
    assert st == status, (args, ha.STATUS.get(st, st))


@pytest.mark.parametrize("args,status", [
    (dict(dtype=1), 4),
    (dict(D=96), 3),
    (dict(Hq=3), 2),
    (dict(Sq=-1), 2),
    (dict(scale=0.0), 7),
    (dict(dq=None), 1),
    (dict(dk=None), 1),
    (dict(lse=None), 1),
    (dict(dout=P + 8), 5),
    (dict(dv=P + 4), 5),
    (dict(workspace=None), 9),
    (dict(workspace=P + 16), 9),
    (dict(wbytes=10), 9),
    (dict(Skv=1 << 30), 6),
])
def test_backward_fail_closed_validation(L, args, status):
    a = dict(q=P, k=P, v=P, out=P, dout=P, lse=P, dq=P, dk=P, dv=P, Hq=4, Sq=100, D=128, scale=0.1,
             dtype=0, workspace=P, wbytes=1 << 40, Skv=100)
    a.update(args)
    st = ha.attn_bwd(a["q"], a["k"], a["v"], a["out"], a["dout"], a["lse"], a["dq"], a["dk"], a["dv"],
                     1, a["Hq"], 2, a["Sq"], a["Skv"], a["D"], a["scale"], 1, a["dtype"], a["workspace"],
                     a["wbytes"], 0)
    assert st == status, (args, ha.STATUS.get(st, st))


@pytest.mark.parametrize("args,status", [
    (dict(kv_start=-1), 2),
    (dict(kv_start=(1 << 30) - 100), 6),
    (dict(kv_start=5, D=96), 3),
    (dict(kv_start=5, dq=None), 1),
])
def test_backward_chunk_fail_closed_validation(L, args, status):
    a = dict(q=P, dq=P, D=128, kv_start=0)
    a.update(args)
    st = ha.attn_bwd_chunk(a["q"], P, P, P, P, P, a["dq"], P, P, 1, 4, 2, 100, 100, a["D"], 0.1, 1, 0,
                           a["kv_start"], P, 1 << 40, 0)
    assert st == status, (args, ha.STATUS.get(st, st))


def test_backward_workspace_size():
    # 8 bytes of row statistics per query row, padded to 256 bytes ...
    assert ha.attn_bwd_workspace_bytes(1, 2, 2, 100, 100, 128) == 1792
    assert ha.attn_bwd_workspace_bytes(2, 3, 3, 64, 999, 64) == 2 * 3 * 64 * 8
    # ... plus fp32 partial dK and dV per query head when a KV head's group is
    # split over workgroups (few KV-head key blocks) ...
    assert ha.attn_bwd_workspace_bytes(1, 32, 8, 4096, 4096, 128) == 32 * 4096 * 8 + 2 * 32 * 4096 * 128 * 4
    # ... but not when the group is summed in registers (enough blocks to fill the chip)
    assert ha.attn_bwd_workspace_bytes(64, 4, 2, 64, 1024, 128) == 64 * 4 * 64 * 8
    assert ha.attn_bwd_workspace_bytes(1, 4, 3, 10, 10, 128) == -1
    assert ha.attn_bwd_workspace_bytes(1, 4, 2, 10, 10, 96) == -1


def test_splitkv_workspace_size():
    assert ha.attn_splitkv_workspace_bytes(2, 3, 100, 128, 1) == 0
    assert ha.attn_splitkv_workspace_bytes(2, 3, 100, 128, 4) == 4 * 2 * 3 * 100 * 129 * 4
    assert ha.attn_splitkv_workspace_bytes(1, 1, 10, 64, 2) == 2 * 10 * 65 * 4
    assert ha.attn_splitkv_workspace_bytes(1, 1, 10, 96, 2) == -1
    assert ha.attn_splitkv_workspace_bytes(1, 1, 10, 128, 300) == -1


def test_splitkv_auto_split_choice():
    # 1480 video-DiT query tiles fill 5 rounds of 256 CUs and 200 tiles of a sixth: only those
    # 200 are split, 5 ways (1000 short workgroups need 0.8 of a round; 2-4 ways would need 1).
    assert ha.attn_splitkv_auto_splits(1, 5, 75600, 75600, 128) == 5
    # 228 tiles (window-30 shape) nearly fill one round: no split.
    assert ha.attn_splitkv_auto_splits(1, 12, 4680, 51480, 128) == 1
    # 258 tiles fill only half of their second round: the whole grid is split (9 x 258 =
    # 2322 workgroups, 91 % of 10 rounds).
    assert ha.attn_splitkv_auto_splits(1, 2, 33000, 33000, 128) == 9
    # 460 tiles: one full round and 204 tiles; those are split 5 ways (0.8 of a round).
    assert ha.attn_splitkv_auto_splits(1, 4, 29440, 29440, 128) == 5
    # 280 tiles, 33 key tiles: 2 ways (each split keeps at least 16 key tiles).
    assert ha.attn_splitkv_auto_splits(1, 40, 1700, 2100, 128) == 2
    # 185 (an eighth of the video-DiT queries) fill 72 %: four splits make 740 = 96 % of 3 rounds.
    assert ha.attn_splitkv_auto_splits(1, 5, 9450, 75600, 128) == 4
    assert ha.attn_splitkv_auto_splits(2, 8, 2048, 2048, 128) == 2
    assert ha.attn_splitkv_auto_splits(1, 1, 256, 512, 128) == 1      # too few key tiles to split
    # Grids that 16 splits cannot bring to 90 %: the count with the least estimated time.
    # One 256-row tile against 16384 key tiles: 249 splits of 66 tiles (the fewest within 3 %
    # of 256 splits of 64), one round.
    assert ha.attn_splitkv_auto_splits(1, 1, 256, 1 << 20, 128) == 249
    assert ha.attn_splitkv_auto_splits(1, 8, 1, 8192, 128) == 8       # 128 key tiles: 8 of 16
    assert ha.attn_splitkv_auto_splits(1, 1, 300, 3000, 128) == 2     # 47 key tiles: 2 of 23
    assert ha.attn_splitkv_auto_splits(1, 1, 256, 96, 100) == -1


def test_zero_queries_return_ok_without_launch(L):
    assert ha.attn_fwd(None, None, None, None, None, 1, 4, 2, 0, 100, 128, 0.1, 0, 0) == 0
    assert ha.attn_fwd(None, None, None, None, None, 0, 4, 2, 10, 100, 128, 0.1, 0, 0) == 0


def _bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _unbits(b):
    return torch.from_numpy(np.asarray(b).view(np.int16)).view(torch.bfloat16).double().numpy()


def test_host_merge_matches_oracle_merge(L):
    r = np.random.default_rng(0)
    B, H, S, D = 2, 3, 50, 64
    o1, o2 = r.standard_normal((B, H, S, D)), r.standard_normal((B, H, S, D))
    l1, l2 = r.standard_normal((B, H, S)) * 3, r.standard_normal((B, H, S)) * 3
    l1[0, 0, :5] = -np.inf
    l2[0, 0, 3:8] = -np.inf
    b1, b2 = _bits(o1), _bits(o2)
    f1, f2 = np.float32(l1), np.float32(l2)
    om, lm = ha.merge_lse2_host(b1, f1, b2, f2)
    Oref, Lref = oracle.merge_lse([(_unbits(b1), f1.astype(np.float64)), (_unbits(b2), f2.astype(np.float64))])
    got = _unbits(om)
    assert np.array_equal(np.isneginf(lm), np.isneginf(Lref))
    assert (got[np.isneginf(Lref)] == 0).all()
    # one bf16 rounding (half an ulp: 2^-8 relative) plus fp32 arithmetic
    assert (np.abs(got - Oref) <= 2 ** -8 * np.abs(Oref) * 1.01 + 1e-6).all()
    fin = np.isfinite(Lref)
    assert np.abs(lm[fin] - Lref[fin]).max() <= 1e-5


def test_host_merge_rejects_bad_arguments(L):
    assert ha.attn_merge_lse2_host(None, None, None, None, None, None, 1, 1, 1, 4) == 1
    assert ha.attn_merge_lse2_host(None, None, None, None, None, None, -1, 1, 1, 4) == 2
    assert ha.attn_merge_lse2_host(None, None, None, None, None, None, 0, 1, 1, 4) == 0
