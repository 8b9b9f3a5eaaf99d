// Device helpers shared by the forward and backward attention kernels for
// gfx950: vector types, buffer descriptors, the direct global->LDS copy, and
// cross-half-wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hat {

typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(8))) short i16x8;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
#define LDS_AS __attribute__((address_space(3)))

// Buffer descriptor word 3 for raw (untyped, unswizzled) buffer access on gfx950.
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

__device__ __forceinline__ i32x4 rsrc_words(const void* base, uint32_t bytes) {
  const unsigned long long a = (unsigned long long)base;
  return i32x4{(int)(unsigned)a, (int)((unsigned)(a >> 32) & 0xFFFFu), (int)bytes, kRsrcWord3};
}

// Direct global->LDS copy of 16 bytes per lane: lane l writes LDS bytes
// [lds_base + 16 l, +16) from buffer offset voff (out-of-range offsets read as
// zero). Written as asm so that the compiler does not make later LDS reads of
// other ring slots wait for it; the kernel waits on vmcnt itself before the
// barrier that publishes a slot. The copy takes its LDS address from m0, a
// register the compiler reserves: the asm saves m0 and puts it back once the
// load has been issued (the load reads m0 at issue).
__device__ __forceinline__ void dma16(const i32x4 rsrc, int voff, unsigned lds_base) {
  unsigned saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
               "s_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(voff), "s"(rsrc), "s"(lds_base) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Exchange a value with the lane 32 away and combine: returns f(x, x^32) on every lane.
__device__ __forceinline__ float xor32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// acc + lo + hi of a packed bf16 pair (dot product with (1, 1), fp32 accumulate).
__device__ __forceinline__ float sum_bf16x2(unsigned pair, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), __builtin_bit_cast(bf16x2, 0x3F803F80u),
                                         acc, false);
}

__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  bf16x2 v = __builtin_convertvector(f32x2{a, b}, bf16x2);
  return __builtin_bit_cast(unsigned, v);
}

}  // namespace hat
