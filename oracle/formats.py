"""Exact float64 decoders for the element formats the attention kernel reads.

Test infrastructure only (see the package docstring).

Both decoders are written from the format definitions, field by field, not by
reinterpreting memory:

* bf16 is the upper half of an IEEE-754 binary32: 1 sign bit, 8 exponent bits
  with bias 127, 7 fraction bits.
* OCP FP8 e4m3fn ("fn": finite, no infinities) has 1 sign bit, 4 exponent bits
  with bias 7 and 3 fraction bits. Exponent field 0 is subnormal
  (value = 2^-6 * m/8); the code with exponent 15 and fraction 7 is NaN; the
  largest finite magnitude is 2^8 * 1.75 = 448. The page "[ops] feat: run the
  DeepSeek-V4 TileLang kernels and FP8 QAT on AMD gfx942/gfx950" (its FP8
  section) states that e4m3fn saturates at +/-448 and that gfx950 uses e4m3fn
  natively, while gfx94x's e4m3fnuz holds half the value of the same bits; the
  kernel here targets gfx950, so the fn decoding applies.

Every function here is pinned in tests/test_oracle_pins.py (closed-form codes,
torch's own casts for all 256 fp8 codes and for random bf16 bit patterns).
"""

import numpy as np


def decode_bf16(bits):
    """bf16 bit patterns (any integer array, values 0..65535) -> float64 array."""
    b = np.asarray(bits).astype(np.int64) & 0xFFFF
    sign = np.where(b >> 15, -1.0, 1.0)
    exp = (b >> 7) & 0xFF
    frac = (b & 0x7F).astype(np.float64)
    normal = sign * np.ldexp(1.0 + frac / 128.0, (exp - 127).astype(np.int64))
    subnormal = sign * np.ldexp(frac / 128.0, -126)
    out = np.where(exp == 0, subnormal, normal)
    special = exp == 0xFF
    if np.any(special):
        out = np.where(special & (frac == 0), sign * np.inf, out)
        out = np.where(special & (frac != 0), np.nan, out)
    return out


def decode_e4m3fn(codes):
    """OCP e4m3fn byte codes (values 0..255) -> float64 array (NaN for 0x7F, 0xFF)."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(c >> 7, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    frac = (c & 0x7).astype(np.float64)
    normal = sign * np.ldexp(1.0 + frac / 8.0, (exp - 7).astype(np.int64))
    subnormal = sign * np.ldexp(frac / 8.0, -6)
    out = np.where(exp == 0, subnormal, normal)
    return np.where((exp == 15) & (frac == 7), np.nan, out)


def dequantise(stored, fmt, descale=1.0):
    """Real values the kernel is asked to attend over, in float64.

    ``fmt`` is "bf16" (``stored`` holds bit patterns), "e4m3fn" (``stored`` holds
    byte codes; the per-tensor ``descale`` multiplies the decoded value, as the
    q/k/v_descale arguments of the fp8 forward on the page "F8 fmha ASM gfx950",
    Test Result section, do) or "f64" (plain numbers, used for tiny fp32 inputs).
    """
    if fmt == "bf16":
        return decode_bf16(stored)
    if fmt == "e4m3fn":
        return decode_e4m3fn(stored) * float(descale)
    if fmt == "f64":
        return np.asarray(stored, dtype=np.float64)
    raise ValueError(f"unknown format {fmt!r}")
