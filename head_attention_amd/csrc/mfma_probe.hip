// MFMA-only throughput probe for gfx950 (MI355X), a measurement aid for the
// benchmark, not part of the attention boundary: it shows what the matrix
// cores sustain on this device under the attention kernels' own MFMA forms
// (bf16 32x32x16 and fp8 32x32x64 with unit scales) when nothing else runs.
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
        acc[j & 3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[j], b[(3 * j + 1) & (kFrags - 1)], acc[j & 3],
                                                                     0, 0, 0, 127, 0, 127);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int k = 0; k < 16; ++k) s += acc[i][k];
  out[gw * 64 + lane] = s;   // keeps the MFMAs live
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
