"""Python binding of the gfx950 fused attention forward and backward (``libattn.so``).

Argument marshalling only: every step of the attention runs in the HIP
kernels behind the C ABI declared in ``include/attn.h``. The functions
``attn_fwd``, ``attn_fwd_chunk``, ``attn_fwd_window``, ``attn_fwd_splitkv``,
``attn_splitkv_workspace_bytes``, ``attn_splitkv_auto_splits``,
``attn_bwd``, ``attn_bwd_chunk``, ``attn_bwd_workspace_bytes``, ``attn_fwd_splitkv_static``,
``attn_merge_lse2_host`` and ``attn_status_string`` carry the C names and
arguments one for one (pointer arguments accept a torch tensor, a plain integer
address or None) and return what the C function returns. ``forward`` and
``forward_splitkv`` are convenience wrappers that read the sizes off torch
tensors, allocate the outputs (and the split workspace) with torch and raise
``AttnError`` on a non-OK status; ``backward`` does the same for ``attn_bwd``.

There is no fallback: if the library is missing, loading raises.
"""

import ctypes
import math
import os

__all__ = [
    "ATTN_BF16", "ATTN_FP8_E4M3FN", "STATUS", "AttnError", "lib", "library_path",
    "attn_fwd", "attn_fwd_chunk", "attn_fwd_window", "attn_fwd_splitkv", "attn_splitkv_workspace_bytes",
    "attn_splitkv_auto_splits", "attn_merge_lse2_host", "attn_status_string", "forward",
    "forward_splitkv", "merge_lse2_host", "attn_bwd", "attn_bwd_chunk", "attn_bwd_workspace_bytes", "backward",
    "attn_fwd_splitkv_static", "SPLITKV_STATIC_SCRATCH_BYTES",
]

ATTN_BF16 = 0
ATTN_FP8_E4M3FN = 1
STATUS = {
    0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_SHAPE", 3: "ATTN_ERR_HEAD_DIM", 4: "ATTN_ERR_DTYPE",
    5: "ATTN_ERR_ALIGN", 6: "ATTN_ERR_OVERFLOW", 7: "ATTN_ERR_SCALE", 8: "ATTN_ERR_HIP",
    9: "ATTN_ERR_WORKSPACE",
}
EXPORTED = ("attn_fwd", "attn_fwd_chunk", "attn_fwd_window", "attn_fwd_splitkv", "attn_splitkv_workspace_bytes",
            "attn_splitkv_auto_splits", "attn_merge_lse2_host", "attn_status_string", "attn_bwd",
            "attn_bwd_chunk", "attn_bwd_workspace_bytes", "attn_fwd_splitkv_static")
SPLITKV_STATIC_SCRATCH_BYTES = 64 << 20   # ATTN_SPLITKV_STATIC_SCRATCH_BYTES of attn.h

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libattn.so")
_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str = ""):
        self.status = int(status)
        super().__init__(f"{where}: {attn_status_string(status)}" if where else attn_status_string(status))


def lib():
    """Load libattn.so (once). Raises OSError if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise OSError(f"{library_path} not built; run `python -m head_attention_amd.build`")
        L = ctypes.CDLL(library_path)
        vp, i64, f32, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
        fwd_args = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, f32, i32, i32, vp, vp, vp]
        L.attn_fwd.argtypes = fwd_args + [vp]
        L.attn_fwd.restype = i32
        L.attn_fwd_chunk.argtypes = fwd_args + [i64, vp]
        L.attn_fwd_chunk.restype = i32
        L.attn_fwd_window.argtypes = fwd_args + [i64, i64, i64, i64, vp]
        L.attn_fwd_window.restype = i32
        L.attn_fwd_splitkv.argtypes = fwd_args + [i64, vp, i64, vp]
        L.attn_fwd_splitkv.restype = i32
        L.attn_fwd_splitkv_static.argtypes = fwd_args + [i64, vp]
        L.attn_fwd_splitkv_static.restype = i32
        L.attn_splitkv_workspace_bytes.argtypes = [i64, i64, i64, i64, i64]
        L.attn_splitkv_workspace_bytes.restype = i64
        L.attn_splitkv_auto_splits.argtypes = [i64, i64, i64, i64, i64]
        L.attn_splitkv_auto_splits.restype = i64
        L.attn_merge_lse2_host.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64]
        L.attn_merge_lse2_host.restype = i32
        L.attn_bwd.argtypes = [vp] * 9 + [i64] * 6 + [f32, i32, i32, vp, i64, vp]
        L.attn_bwd.restype = i32
        L.attn_bwd_chunk.argtypes = [vp] * 9 + [i64] * 6 + [f32, i32, i32, i64, vp, i64, vp]
        L.attn_bwd_chunk.restype = i32
        L.attn_bwd_workspace_bytes.argtypes = [i64] * 6
        L.attn_bwd_workspace_bytes.restype = i64
        L.attn_status_string.argtypes = [i32]
        L.attn_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _addr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr() or None
    if hasattr(x, "ctypes"):  # numpy array (host pointers of the merge)
        return x.ctypes.data or None
    raise TypeError(f"cannot take the address of {type(x)!r}")


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def attn_fwd(q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, scale, causal, dtype,
             q_descale=None, k_descale=None, v_descale=None, stream=0):
    return lib().attn_fwd(_addr(q), _addr(k), _addr(v), _addr(out), _addr(lse), B, Hq, Hkv, Sq, Skv, D,
                          float(scale), int(bool(causal)), int(dtype),
                          _addr(q_descale), _addr(k_descale), _addr(v_descale), _stream(stream))


def attn_fwd_chunk(q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, scale, causal, dtype,
                   q_descale=None, k_descale=None, v_descale=None, kv_start=0, stream=0):
    return lib().attn_fwd_chunk(_addr(q), _addr(k), _addr(v), _addr(out), _addr(lse), B, Hq, Hkv, Sq, Skv,
                                D, float(scale), int(bool(causal)), int(dtype),
                                _addr(q_descale), _addr(k_descale), _addr(v_descale), int(kv_start),
                                _stream(stream))


def attn_fwd_window(q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, scale, causal, dtype,
                    q_descale=None, k_descale=None, v_descale=None, kv_start=0, window_left=-1,
                    window_right=-1, sink=0, stream=0):
    return lib().attn_fwd_window(_addr(q), _addr(k), _addr(v), _addr(out), _addr(lse), B, Hq, Hkv, Sq, Skv,
                                 D, float(scale), int(bool(causal)), int(dtype),
                                 _addr(q_descale), _addr(k_descale), _addr(v_descale), int(kv_start),
                                 int(window_left), int(window_right), int(sink), _stream(stream))


def attn_fwd_splitkv(q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, scale, causal, dtype,
                     q_descale=None, k_descale=None, v_descale=None, n_splits=0, workspace=None,
                     workspace_bytes=0, stream=0):
    return lib().attn_fwd_splitkv(_addr(q), _addr(k), _addr(v), _addr(out), _addr(lse), B, Hq, Hkv, Sq, Skv,
                                  D, float(scale), int(bool(causal)), int(dtype),
                                  _addr(q_descale), _addr(k_descale), _addr(v_descale), int(n_splits),
                                  _addr(workspace), int(workspace_bytes), _stream(stream))


def attn_fwd_splitkv_static(q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, scale, causal, dtype,
                            q_descale=None, k_descale=None, v_descale=None, n_splits=0, stream=0):
    return lib().attn_fwd_splitkv_static(_addr(q), _addr(k), _addr(v), _addr(out), _addr(lse), B, Hq, Hkv, Sq,
                                         Skv, D, float(scale), int(bool(causal)), int(dtype),
                                         _addr(q_descale), _addr(k_descale), _addr(v_descale), int(n_splits),
                                         _stream(stream))



def attn_splitkv_workspace_bytes(B, Hq, Sq, D, n_splits):
    return lib().attn_splitkv_workspace_bytes(B, Hq, Sq, D, n_splits)


def attn_splitkv_auto_splits(B, Hq, Sq, Skv, D):
    return lib().attn_splitkv_auto_splits(B, Hq, Sq, Skv, D)


def attn_merge_lse2_host(o1, lse1, o2, lse2, o_out, lse_out, B, H, S, D):
    return lib().attn_merge_lse2_host(_addr(o1), _addr(lse1), _addr(o2), _addr(lse2), _addr(o_out),
                                      _addr(lse_out), B, H, S, D)


def attn_status_string(status):
    return lib().attn_status_string(int(status)).decode()


def forward(q, k, v, scale=None, causal=False, q_descale=None, k_descale=None, v_descale=None,
            kv_start=0, out=None, lse=None, stream=None, window_left=-1, window_right=-1, sink=0):
    """(out, lse) for torch tensors q [B,Hq,Sq,D], k/v [B,Hkv,Skv,D] on the GPU.

    q/k/v are torch.bfloat16 or torch.float8_e4m3fn; descales are one-element
    float32 device tensors or None. A window side >= 0 or sink > 0 runs
    ``attn_fwd_window``, else ``attn_fwd_chunk``.
    """
    import torch
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    if q.dtype == torch.bfloat16:
        dt = ATTN_BF16
    elif q.dtype == torch.float8_e4m3fn:
        dt = ATTN_FP8_E4M3FN
    else:
        raise TypeError(f"unsupported dtype {q.dtype}")
    for t in (q, k, v):
        if t.dtype != q.dtype or not t.is_contiguous() or t.device.type != "cuda":
            raise ValueError("q, k, v must be contiguous GPU tensors of one dtype")
    if out is None:
        out = torch.empty((B, Hq, Sq, D), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if window_left >= 0 or window_right >= 0 or sink > 0:
        st = attn_fwd_window(q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, scale, causal, dt,
                             q_descale, k_descale, v_descale, kv_start, window_left, window_right, sink, stream)
        if st != 0:
            raise AttnError(st, "attn_fwd_window")
        return out, lse
    st = attn_fwd_chunk(q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, scale, causal, dt,
                        q_descale, k_descale, v_descale, kv_start, stream)
    if st != 0:
        raise AttnError(st, "attn_fwd_chunk")
    return out, lse


def forward_splitkv(q, k, v, n_splits=0, scale=None, causal=False, q_descale=None, k_descale=None,
                    v_descale=None, out=None, lse=None, workspace=None, stream=None):
    """(out, lse) like ``forward``, computed by ``attn_fwd_splitkv`` with n_splits key
    splits (0: the library's choice). The fp32 split workspace is allocated with
    torch unless one (a uint8 GPU tensor) is passed."""
    import torch
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    if q.dtype == torch.bfloat16:
        dt = ATTN_BF16
    elif q.dtype == torch.float8_e4m3fn:
        dt = ATTN_FP8_E4M3FN
    else:
        raise TypeError(f"unsupported dtype {q.dtype}")
    for t in (q, k, v):
        if t.dtype != q.dtype or not t.is_contiguous() or t.device.type != "cuda":
            raise ValueError("q, k, v must be contiguous GPU tensors of one dtype")
    # n_splits = 0 is passed on as the library's choice (which may split only the
    # query tiles of a last, partly filled round); the workspace is sized for the
    # split count that choice uses.
    sized = attn_splitkv_auto_splits(B, Hq, Sq, Skv, D) if n_splits == 0 else n_splits
    if out is None:
        out = torch.empty((B, Hq, Sq, D), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    need = attn_splitkv_workspace_bytes(B, Hq, Sq, D, sized)
    if need < 0:
        raise AttnError(2, "attn_splitkv_workspace_bytes")
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = attn_fwd_splitkv(q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, scale, causal, dt,
                          q_descale, k_descale, v_descale, n_splits, workspace, wbytes, stream)
    if st != 0:
        raise AttnError(st, "attn_fwd_splitkv")
    return out, lse


def attn_bwd(q, k, v, out, dout, lse, dq, dk, dv, B, Hq, Hkv, Sq, Skv, D, scale, causal, dtype,
             workspace, workspace_bytes, stream=0):
    return lib().attn_bwd(_addr(q), _addr(k), _addr(v), _addr(out), _addr(dout), _addr(lse), _addr(dq),
                          _addr(dk), _addr(dv), B, Hq, Hkv, Sq, Skv, D, float(scale), int(bool(causal)),
                          int(dtype), _addr(workspace), int(workspace_bytes), _stream(stream))


def attn_bwd_chunk(q, k, v, out, dout, lse, dq, dk, dv, B, Hq, Hkv, Sq, Skv, D, scale, causal, dtype, kv_start,
                   workspace, workspace_bytes, stream=0):
    return lib().attn_bwd_chunk(_addr(q), _addr(k), _addr(v), _addr(out), _addr(dout), _addr(lse), _addr(dq),
                                _addr(dk), _addr(dv), B, Hq, Hkv, Sq, Skv, D, float(scale), int(bool(causal)),
                                int(dtype), int(kv_start), _addr(workspace), int(workspace_bytes), _stream(stream))


def attn_bwd_workspace_bytes(B, Hq, Hkv, Sq, Skv, D):
    return lib().attn_bwd_workspace_bytes(B, Hq, Hkv, Sq, Skv, D)


def backward(q, k, v, out, dout, lse, scale=None, causal=False, workspace=None, stream=None, kv_start=0):
    """(dq, dk, dv) for bf16 GPU tensors q/out/dout [B,Hq,Sq,D], k/v [B,Hkv,Skv,D] and
    lse [B,Hq,Sq] fp32 from ``forward``. The workspace (a uint8 GPU tensor) is
    allocated with torch unless one is passed. kv_start > 0 runs ``attn_bwd_chunk``
    (out and lse then belong to the attention over all keys)."""
    import torch
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    for t in (q, k, v, out, dout):
        if t.dtype != torch.bfloat16 or not t.is_contiguous() or t.device.type != "cuda":
            raise ValueError("q, k, v, out, dout must be contiguous bf16 GPU tensors")
    if lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    need = attn_bwd_workspace_bytes(B, Hq, Hkv, Sq, Skv, D)
    if need < 0:
        raise AttnError(2, "attn_bwd_workspace_bytes")
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = attn_bwd_chunk(q, k, v, out, dout, lse, dq, dk, dv, B, Hq, Hkv, Sq, Skv, D, scale, causal, ATTN_BF16,
                        kv_start, workspace, wbytes, stream)
    if st != 0:
        raise AttnError(st, "attn_bwd_chunk")
    return dq, dk, dv


def merge_lse2_host(o1, lse1, o2, lse2):
    """Merge two host (numpy) partial results: o* uint16 bf16 bits [B,H,S,D], lse* float32 [B,H,S]."""
    import numpy as np
    o1 = np.ascontiguousarray(o1, dtype=np.uint16)
    o2 = np.ascontiguousarray(o2, dtype=np.uint16)
    l1 = np.ascontiguousarray(lse1, dtype=np.float32)
    l2 = np.ascontiguousarray(lse2, dtype=np.float32)
    B, H, S, D = o1.shape
    if o2.shape != o1.shape or l1.shape != (B, H, S) or l2.shape != (B, H, S):
        raise ValueError("shape mismatch")
    oo = np.empty_like(o1)
    lo = np.empty_like(l1)
    st = attn_merge_lse2_host(o1, l1, o2, l2, oo, lo, B, H, S, D)
    if st != 0:
        raise AttnError(st, "attn_merge_lse2_host")
    return oo, lo
