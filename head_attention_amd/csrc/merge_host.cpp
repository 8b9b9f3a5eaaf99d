// Host-side helpers of the C ABI: the two-chunk (out, lse) merge and status names.
//
// The merge combines the attention of the same queries over two disjoint key
// chunks into the attention over their union, the out/LSE combination the page
// "feat(attention): add strict bitwise ROCm path" performs across
// context-parallel ranks (Summary table: attention-domain LSE, fixed merge
// order; CP communication: Out/LSE reduce-scatter). With L_c the natural-log
// LSE of chunk c: L = ln(e^L1 + e^L2) and O = e^(L1 - L) O1 + e^(L2 - L) O2.

#include <math.h>
#include <stdint.h>
#include <string.h>

#include "attn.h"

namespace {

inline float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

}  // namespace

extern "C" attn_status_t attn_merge_lse2_host(const uint16_t* o1, const float* lse1, const uint16_t* o2,
                                              const float* lse2, uint16_t* o_out, float* lse_out, int64_t B,
                                              int64_t H, int64_t S, int64_t D) {
  if (B < 0 || H < 0 || S < 0 || D < 0) return ATTN_ERR_SHAPE;
  const int64_t rows = B * H * S;
  if (rows == 0) return ATTN_OK;
  if (!lse1 || !lse2 || !lse_out) return ATTN_ERR_NULL;
  if (D > 0 && (!o1 || !o2 || !o_out)) return ATTN_ERR_NULL;
  for (int64_t r = 0; r < rows; ++r) {
    const float L1 = lse1[r], L2 = lse2[r];
    const float Lm = fmaxf(L1, L2);
    const int64_t base = r * D;
    if (Lm == -INFINITY) {
      for (int64_t d = 0; d < D; ++d) o_out[base + d] = 0;
      lse_out[r] = -INFINITY;
      continue;
    }
    const float w1 = expf(L1 - Lm), w2 = expf(L2 - Lm);
    const float tot = w1 + w2;
    const float a1 = w1 / tot, a2 = w2 / tot;
    for (int64_t d = 0; d < D; ++d) {
      const float x = a1 * bf16_to_f32(o1[base + d]) + a2 * bf16_to_f32(o2[base + d]);
      o_out[base + d] = f32_to_bf16_rne(x);
    }
    lse_out[r] = Lm + logf(tot);
  }
  return ATTN_OK;
}

extern "C" const char* attn_status_string(attn_status_t s) {
  switch (s) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_NULL: return "ATTN_ERR_NULL: a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "ATTN_ERR_SHAPE: negative size, Hq not a multiple of Hkv, kv_start < 0, or a bad split count";
    case ATTN_ERR_HEAD_DIM: return "ATTN_ERR_HEAD_DIM: head dimension must be 64 or 128";
    case ATTN_ERR_DTYPE: return "ATTN_ERR_DTYPE: unknown input dtype";
    case ATTN_ERR_ALIGN: return "ATTN_ERR_ALIGN: q/k/v/out must be 16-byte aligned, lse 4-byte aligned";
    case ATTN_ERR_OVERFLOW: return "ATTN_ERR_OVERFLOW: a head slice or the grid exceeds 32-bit addressing";
    case ATTN_ERR_SCALE: return "ATTN_ERR_SCALE: scale must be finite and > 0";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP: kernel launch failed";
    case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE: workspace missing, misaligned or too small";
  }
  return "ATTN_ERR_UNKNOWN";
}
