"""Workload table and seeded input generators.

Values are drawn N(0, 1) in float32 on the CPU with ``torch.Generator`` seeded
as ``1000 * workload_id + {0: q, 1: k, 2: v}``, so the oracle and the GPU see
identical numbers. Storage formats:

* "bf16": round-to-nearest-even through ``tensor.to(torch.bfloat16)``;
  returned as uint16 bit patterns.
* "e4m3fn": per-tensor amax scaling, descale = amax / 448 (1 when amax = 0),
  codes = e4m3fn(x / descale) through ``torch.float8_e4m3fn`` (round to nearest
  even, clamped to +/-448 first); returned as uint8 codes plus the float32
  descale. The +/-448 range is the e4m3fn range given on the page "[ops] feat:
  run the DeepSeek-V4 TileLang kernels and FP8 QAT on AMD gfx942/gfx950"; the
  amax rule is the plainest reading of "per-tensor amax scales".

The shapes are the five workloads of the attention forward: a tiny fp32 case,
an LLM-style case, the video-DiT self-attention (bf16 and fp8) and a GQA causal
case that is also run as two key chunks. The video-DiT shape is the one the
page "F8 fmha ASM gfx950" benchmarks (b 1, n 5, q 75600, d 128). Three more
have Sq != Skv: the window-30 shape of the page "[Proposal] ROCm (AMD
Instinct) support for the core attention and distributed init" (query 4680 x
key 51480, 12 heads), and the cross-attention of the page "F8 fmha ASM gfx950"
(90000 queries against 512 keys, 40 heads; an even head count), bf16 and fp8.

Two local-attention workloads carry a window and sink keys (the pages give
window / sink configurations, in video frames, but no token counts, so these
sizes are chosen here): "swa_llm", causal GQA with the 32/8 heads of the
pages' Qwen3-8B validation, 16384 tokens, a 4096-token sliding window
(window_left 4095) and 4 sink tokens; and "video_band", the video-DiT shape
(75600 tokens = 21 frames of 3600) with a band of three frames on either side
(window 10800 / 10800) and the first frame as sinks (3600).

The backward is timed on "bwd_llm": B1, 32/8 heads, S4096, D128, causal, the
largest sequence length of the deterministic-backward table on the page
"feat(attention): add strict bitwise ROCm path" (section "What the strict
contract costs"), with that page's Qwen3-8B head layout; dO is a fourth
N(0, 1) draw (seed base + 3).
"""

from dataclasses import dataclass, field
import math

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Skv: int
    D: int
    fmt: str                     # "f32" (tiny case, rounded to bf16 for the GPU), "bf16", "e4m3fn"
    causal: tuple = (False,)
    chunks: tuple = ()           # key chunk lengths for the chunked-merge run
    note: str = ""
    window_left: int = -1        # local attention: -1 = unbounded side
    window_right: int = -1
    sink: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def flops(self, causal: bool) -> float:
        """4*B*Hq*Sq*Skv*D, halved for causal (the metric's own convention)."""
        f = 4.0 * self.B * self.Hq * self.Sq * self.Skv * self.D
        return f / 2 if causal else f


WORKLOADS = {
    w.name: w
    for w in [
        Workload(1, "tiny", 1, 2, 2, 256, 256, 64, "f32", (False,),
                 note="fp32 N(0,1), scale 1/sqrt(64), non-causal"),
        Workload(2, "llm", 2, 8, 8, 2048, 2048, 128, "bf16", (False, True)),
        Workload(3, "video_dit", 1, 5, 5, 75600, 75600, 128, "bf16", (False,)),
        Workload(4, "video_dit_fp8", 1, 5, 5, 75600, 75600, 128, "e4m3fn", (False,)),
        Workload(5, "gqa_causal", 1, 32, 8, 8192, 8192, 128, "bf16", (True,), chunks=(4096, 4096)),
        # Sq != Skv shapes beyond the five above
        Workload(6, "window30", 1, 12, 12, 4680, 51480, 128, "bf16", (False,),
                 note="raw SDPA at the window-30 shape, query 4680 x key 51480"),
        Workload(7, "wan_cross", 1, 40, 40, 90000, 512, 128, "bf16", (False,),
                 note="cross-attention, 90000 queries against 512 keys, 40 heads"),
        Workload(8, "wan_cross_fp8", 1, 40, 40, 90000, 512, 128, "e4m3fn", (False,),
                 note="the same cross-attention in fp8 e4m3fn with per-tensor descales"),
        Workload(9, "video_dit_shard", 1, 5, 5, 9450, 75600, 128, "bf16", (False,),
                 note="one eighth of the video-DiT queries against all its keys (one GPU's share "
                      "when the queries are split over eight GPUs)"),
        Workload(10, "swa_llm", 1, 32, 8, 16384, 16384, 128, "bf16", (True,),
                 note="causal sliding window of 4096 tokens with 4 sink tokens, GQA 32/8",
                 window_left=4095, sink=4),
        Workload(11, "video_band", 1, 5, 5, 75600, 75600, 128, "bf16", (False,),
                 note="video-DiT shape with a +/-3-frame band and the first frame as sinks",
                 window_left=10800, window_right=10800, sink=3600),
        # the backward's timed shape
        Workload(12, "bwd_llm", 1, 32, 8, 4096, 4096, 128, "bf16", (True,),
                 note="attention backward, B1, 32 query / 8 KV heads, S4096, D128, causal"),
    ]
}


def normal(shape, seed: int) -> torch.Tensor:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return torch.randn(*shape, generator=g, dtype=torch.float32)


def to_bf16_bits(x: torch.Tensor) -> np.ndarray:
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def quant_e4m3fn_per_tensor(x: torch.Tensor):
    """-> (uint8 codes, float32 descale) with x ~= decode(codes) * descale."""
    amax = float(x.abs().max()) if x.numel() else 0.0
    descale = np.float32(amax / 448.0) if amax > 0 else np.float32(1.0)
    y = (x / torch.tensor(float(descale), dtype=torch.float32)).clamp(-448.0, 448.0)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, descale


def random_codes(shape, fmt: str, seed: int) -> np.ndarray:
    """Stored-format codes drawn directly as bits, for tensors too large for
    ``normal`` (10^9 elements): a random sign and mantissa and one of the
    exponents of [2^-7, 2) for bf16 (uint16), of [2^-3, 2) for e4m3fn (uint8);
    never zero, never a NaN or infinity."""
    rng = np.random.default_rng(int(seed))
    if fmt == "bf16":
        r = rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
        return (r & np.uint16(0x807F)) | ((np.uint16(120) + ((r >> np.uint16(7)) & np.uint16(7))) << np.uint16(7))
    if fmt == "e4m3fn":
        r = rng.integers(0, 1 << 8, size=shape, dtype=np.uint8)
        return (r & np.uint8(0x87)) | ((np.uint8(4) + ((r >> np.uint8(3)) & np.uint8(3))) << np.uint8(3))
    raise ValueError(fmt)


def plant_needles(q: np.ndarray, k: np.ndarray, positions, fmt: str, steps=None) -> None:
    """In place on codes from ``random_codes`` ([S, D] views): key row
    ``positions[r]`` becomes query row r times 2^steps[r] (default 4: the
    exponent field raised by steps[r], exact; steps in 1..4), so that query r's
    largest score is with that key."""
    shift = 7 if fmt == "bf16" else 3
    for r, pos in enumerate(positions):
        st = 2 if steps is None else int(steps[r])
        assert 1 <= st <= 4
        k[pos] = q[r] + k.dtype.type(st << shift)


def make_inputs(w: Workload, fmt: str = None, sq: int = None, skv: int = None):
    """Draw q, k, v for workload ``w`` (optionally with shorter Sq / Skv).

    Returns a dict with ``fmt`` ("bf16" or "e4m3fn"), the stored arrays ``q``,
    ``k``, ``v`` (uint16 bf16 bits or uint8 e4m3fn codes), the descales (1.0 for
    bf16) and ``q32``/``k32``/``v32``, the float32 draws before rounding.
    """
    fmt = fmt or ("bf16" if w.fmt in ("f32", "bf16") else w.fmt)
    Sq = sq if sq is not None else w.Sq
    Skv = skv if skv is not None else w.Skv
    base = 1000 * w.wid
    q32 = normal((w.B, w.Hq, Sq, w.D), base + 0)
    k32 = normal((w.B, w.Hkv, Skv, w.D), base + 1)
    v32 = normal((w.B, w.Hkv, Skv, w.D), base + 2)
    out = dict(fmt=fmt, q32=q32, k32=k32, v32=v32)
    if fmt == "bf16":
        out.update(q=to_bf16_bits(q32), k=to_bf16_bits(k32), v=to_bf16_bits(v32),
                   q_descale=1.0, k_descale=1.0, v_descale=1.0)
    elif fmt == "e4m3fn":
        (qc, qd), (kc, kd), (vc, vd) = (quant_e4m3fn_per_tensor(t) for t in (q32, k32, v32))
        out.update(q=qc, k=kc, v=vc, q_descale=float(qd), k_descale=float(kd), v_descale=float(vd))
    else:
        raise ValueError(fmt)
    return out
