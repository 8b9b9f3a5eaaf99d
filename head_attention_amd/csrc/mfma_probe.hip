// MFMA throughput probes for gfx950 (MI355X), a measurement aid for the
// benchmark, not part of the attention boundary. The first shows what the
// matrix cores sustain on this device under the attention kernels' own MFMA
// forms (bf16 32x32x16 and the unscaled fp8 32x32x64) when nothing else runs;
// the second (mfma_softmax_kernel, below) adds the attention tile's own
// softmax VALU instructions between the MFMAs; the third (valu_rate_kernel)
// times the softmax's two main VALU forms, exp2 and fma, alone and mixed.
// Every wave issues only MFMAs on register operands loaded once from a buffer
// of random values, rotating over eight A and eight B fragments so that the
// operand data changes from one MFMA to the next as it does in attention (the
// chip's clock, and so its MFMA rate, depends on that activity); four
// independent accumulators keep the MFMA pipe supplied. Workgroups are 4
// waves; two workgroups per compute unit give each SIMD two waves, like the
// attention kernels.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace probe {

using hat::f32x16;
using hat::bf16x8;
using hat::i32x4;
using hat::i32x8;

constexpr int kFrags = 8;   // operand fragments per matrix, rotated

// The unscaled fp8 MFMA: the scaled builtin with zero scale operands, which the
// compiler emits as v_mfma_f32_32x32x64_f8f6f4 (the attention kernels' form).
__device__ __forceinline__ f32x16 mfma_e4m3(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

template <bool FP8>
__global__ void __launch_bounds__(256) mfma_ceiling_kernel(const int* __restrict__ src, float* __restrict__ out,
                                                           int iters) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
  if constexpr (!FP8) {
    // a fragment is 4 ints (8 bf16) per lane; src holds 2 * kFrags * 64 of them
    bf16x8 a[kFrags], b[kFrags];
#pragma unroll
    for (int j = 0; j < kFrags; ++j) {
      a[j] = __builtin_bit_cast(bf16x8, *(const i32x4*)(src + (j * 64 + lane) * 4));
      b[j] = __builtin_bit_cast(bf16x8, *(const i32x4*)(src + ((kFrags + j) * 64 + lane) * 4));
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < kFrags; ++j)
        acc[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[(3 * j + 1) & (kFrags - 1)], acc[j & 3], 0, 0, 0);
    }
  } else {
    // a fragment is 8 ints (32 e4m3fn codes) per lane
    i32x8 a[kFrags], b[kFrags];
#pragma unroll
    for (int j = 0; j < kFrags; ++j) {
      a[j] = *(const i32x8*)(src + (j * 64 + lane) * 8);
      b[j] = *(const i32x8*)(src + ((kFrags + j) * 64 + lane) * 8);
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < kFrags; ++j)
        acc[j & 3] = mfma_e4m3(a[j], b[(3 * j + 1) & (kFrags - 1)], acc[j & 3]);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int k = 0; k < 16; ++k) s += acc[i][k];
  out[gw * 64 + lane] = s;   // keeps the MFMAs live
}

// MFMA plus the attention tile's own softmax VALU work, interleaved in each
// wave as the pipelined attention loop interleaves them: after every MFMA its
// share of the per-score instructions (fma for the scale and offset, exp2, the
// row-sum add, and the pack to the P operand format). Per 32-key block of one
// tile a lane owns 16 scores: fp8 issues 8 MFMAs (4 for S, 4 for O) per 32
// scores, so 14 VALU per MFMA (4 fma, 4 exp2, 4 add, 2 packs to e4m3fn);
// bf16 issues 32 MFMAs per 32 scores, so 4 per MFMA (1 fma, 1 exp2, 1 add,
// and every other MFMA one pack to bf16 and one dot2 summing the rounded
// pair). The VALU operands never depend on MFMA results, so this is the rate
// of that instruction mix with perfect independence: an upper bound for an
// attention loop, which also moves K and V and reads them from LDS.
template <bool FP8>
__global__ void __launch_bounds__(256) mfma_softmax_kernel(const int* __restrict__ src, float* __restrict__ out,
                                                           int iters) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
  const float c = 0.173f, d = -1.5f;   // p = exp2(c x + d) stays in (0, 1)
  float r = 0.f;
  if constexpr (FP8) {
    i32x8 a[kFrags], b[kFrags];
#pragma unroll
    for (int j = 0; j < kFrags; ++j) {
      a[j] = *(const i32x8*)(src + (j * 64 + lane) * 8);
      b[j] = *(const i32x8*)(src + ((kFrags + j) * 64 + lane) * 8);
    }
    float x[kFrags][4];
    int pk[kFrags];
#pragma unroll
    for (int j = 0; j < kFrags; ++j) {
      pk[j] = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[j][e] = (float)(lane + 4 * j + e) * 1e-3f;
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < kFrags; ++j) {
        acc[j & 3] = mfma_e4m3(a[j], b[(3 * j + 1) & (kFrags - 1)], acc[j & 3]);
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[j][e], c, d));
        r += (p[0] + p[1]) + (p[2] + p[3]);
        const int w = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], pk[j], false);
        pk[j] = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], w, true);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[j][e] = p[e];
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 14, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < kFrags; ++j) r += (float)(pk[j] & 1);
  } else {
    bf16x8 a[kFrags], b[kFrags];
#pragma unroll
    for (int j = 0; j < kFrags; ++j) {
      a[j] = __builtin_bit_cast(bf16x8, *(const i32x4*)(src + (j * 64 + lane) * 4));
      b[j] = __builtin_bit_cast(bf16x8, *(const i32x4*)(src + ((kFrags + j) * 64 + lane) * 4));
    }
    float x[kFrags], rb = 0.f;
#pragma unroll
    for (int j = 0; j < kFrags; ++j) x[j] = (float)(lane + j) * 1e-3f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < kFrags; ++j) {
        acc[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[(3 * j + 1) & (kFrags - 1)], acc[j & 3], 0, 0, 0);
        x[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[j], c, d));
        r += x[j];
        if (j & 1) {
          rb = hat::sum_bf16x2(hat::pack_bf16(x[j - 1], x[j]), rb);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
        } else {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
        }
      }
    }
    r += rb;
  }
  float s = r;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int k = 0; k < 16; ++k) s += acc[i][k];
  out[gw * 64 + lane] = s;   // keeps the MFMAs and the VALU work live
}

// VALU issue rates of the softmax's main forms: KIND 0 issues only v_exp_f32
// (eight independent chains x <- exp2(-x), which stay in (0, 1)), KIND 1 only
// v_fma_f32 (eight chains x <- 0.999 x + 0.001), KIND 2 both, one fma after
// each exp2. Workgroups of 4 waves; eight workgroups per compute unit give
// each SIMD eight waves, so that latency never limits the issue rate.
template <int KIND>
__global__ void __launch_bounds__(256) valu_rate_kernel(float* __restrict__ out, int iters) {
  float e[8], f[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    e[i] = 0.5f + 0.01f * i + 1e-6f * threadIdx.x;
    f[i] = 0.5f + 0.02f * i + 1e-6f * threadIdx.x;
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (KIND != 1) e[i] = __builtin_amdgcn_exp2f(-e[i]);
      if (KIND != 0) f[i] = __builtin_fmaf(f[i], 0.999f, 0.001f);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += e[i] + f[i];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace probe

// Launches nblocks workgroups of 4 waves on `stream`, each wave issuing
// iters * 8 MFMAs (fp8 = 0: bf16 32x32x16, 32768 flops each; fp8 = 1: fp8
// 32x32x64, 131072 flops each). src: device buffer of 2 * 8 * 64 fragments
// (bf16: 16 bytes each, 16 KB; fp8: 32 bytes each, 32 KB) of valid operand
// values; out: device buffer of nblocks * 256 floats. Returns 0, 1 for bad
// arguments, 2 when the launch fails.
extern "C" int mfma_probe_launch(int fp8, int64_t nblocks, int iters, const void* src, void* out, void* stream) {
  if (nblocks <= 0 || nblocks >= (int64_t)1 << 31 || iters <= 0 || !src || !out) return 1;
  const dim3 grid((unsigned)nblocks), block(256);
  if (fp8)
    hipLaunchKernelGGL(probe::mfma_ceiling_kernel<true>, grid, block, 0, (hipStream_t)stream, (const int*)src,
                       (float*)out, iters);
  else
    hipLaunchKernelGGL(probe::mfma_ceiling_kernel<false>, grid, block, 0, (hipStream_t)stream, (const int*)src,
                       (float*)out, iters);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// As mfma_probe_launch, for mfma_softmax_kernel: the same MFMAs, each followed
// by its share of the attention tile's softmax VALU instructions.
extern "C" int mfma_softmax_probe_launch(int fp8, int64_t nblocks, int iters, const void* src, void* out,
                                         void* stream) {
  if (nblocks <= 0 || nblocks >= (int64_t)1 << 31 || iters <= 0 || !src || !out) return 1;
  const dim3 grid((unsigned)nblocks), block(256);
  if (fp8)
    hipLaunchKernelGGL(probe::mfma_softmax_kernel<true>, grid, block, 0, (hipStream_t)stream, (const int*)src,
                       (float*)out, iters);
  else
    hipLaunchKernelGGL(probe::mfma_softmax_kernel<false>, grid, block, 0, (hipStream_t)stream, (const int*)src,
                       (float*)out, iters);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Launches nblocks workgroups of 4 waves of valu_rate_kernel<kind> (kind 0:
// exp2 only, 1: fma only, 2: both) on `stream`, each wave issuing iters * 8
// instructions of each form it runs; out: device buffer of nblocks * 256
// floats. Returns 0, 1 for bad arguments, 2 when the launch fails.
extern "C" int valu_rate_probe_launch(int kind, int64_t nblocks, int iters, void* out, void* stream) {
  if (kind < 0 || kind > 2 || nblocks <= 0 || nblocks >= (int64_t)1 << 31 || iters <= 0 || !out) return 1;
  const dim3 grid((unsigned)nblocks), block(256);
  if (kind == 0)
    hipLaunchKernelGGL(probe::valu_rate_kernel<0>, grid, block, 0, (hipStream_t)stream, (float*)out, iters);
  else if (kind == 1)
    hipLaunchKernelGGL(probe::valu_rate_kernel<1>, grid, block, 0, (hipStream_t)stream, (float*)out, iters);
  else
    hipLaunchKernelGGL(probe::valu_rate_kernel<2>, grid, block, 0, (hipStream_t)stream, (float*)out, iters);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Compute units and peak shader clock (kHz) of the current device, for the
// dense peak CUs x clock x {4096 bf16, 8192 fp8} flops per clock per CU.
// Returns 0, or 2 when the runtime does not answer.
extern "C" int mfma_probe_device(int* cus, int* clock_khz) {
  int dev = 0;
  if (!cus || !clock_khz) return 1;
  if (hipGetDevice(&dev) != hipSuccess) return 2;
  if (hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 2;
  if (hipDeviceGetAttribute(clock_khz, hipDeviceAttributeClockRate, dev) != hipSuccess) return 2;
  return 0;
}
