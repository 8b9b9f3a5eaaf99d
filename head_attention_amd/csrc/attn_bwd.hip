// Attention backward (dQ, dK, dV) for gfx950 (MI355X, CDNA4), bf16.
//
// The method: the gradients of the attention forward with respect to Q, K and
// V, the dQ / dK / dV that the page "feat(attention): add strict bitwise ROCm
// path" checks next to out and lse (Latest status) and whose deterministic
// and non-deterministic timings it compares (section "What the strict
// contract costs"). With s = scale * Q K^T over the allowed keys, P =
// softmax(s) recomputed from the forward's LSE, and D_i = dO_i . O_i:
//     dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D),
//     dQ = scale * dS K,   dK = scale * dS^T Q.
// O is the output the caller passes (the forward's bf16 out): where a row's P
// is nearly one key, dP - D is a small difference of larger numbers and the
// rounding of that O decides it.
//
// Design (gfx950 first):
//  * Deterministic by construction: no atomics, every sum in a fixed order,
//    and workspace O(rows) rather than O(Sq * Skv). Two kernels share the
//    work. The dQ kernel is shaped like the forward: a workgroup holds 256
//    query rows (8 waves x 32), streams K and V tiles of 64 keys through an
//    LDS ring, recomputes S^T = K Q^T and dP^T = V dO^T, forms dS^T and
//    accumulates dQ^T += K^T dS^T. It also writes each row's statistics
//    {LSE * log2(e), D} for the second kernel. The dK/dV kernel holds 256
//    keys (8 waves x 32): its K fragments in registers and its V rows in LDS,
//    and streams Q and dO tiles of 64 rows (with their statistics) through
//    the ring, computing S = Q K^T and dP = dO V^T, then dV^T += dO^T P and
//    dK^T += Q^T dS. The recomputation of S and dP in the dQ kernel is the
//    price of determinism without O(Sq * Skv) memory.
//  * Every product runs on v_mfma_f32_32x32x16_bf16 with fp32 accumulation;
//    P and dS are rounded to bf16 as MFMA operands. A lane owns one row
//    (dQ kernel: a query; dK/dV kernel: a key), so the scores it produces are
//    already the B operand of the next product, with the same consistent row
//    permutation as in the forward's P V step.
//  * Tiles that are read both as rows and through the transposing
//    ds_read_b64_tr_b16 use an XOR swizzle that is bank-conflict free for both
//    access patterns.
//  * Key chunks: key j sits at position j + kv_start (causal: allowed for
//    query i iff j + kv_start <= i). Given the full softmax's O and LSE, the
//    call for one chunk yields that chunk's dK, dV and its share of dQ.
//  * Grouped KV heads: a dK/dV workgroup either loops over every query head of
//    its KV head (sums in registers), or, when that leaves too few workgroups
//    for the chip, takes one query head and writes fp32 partials that a small
//    kernel sums over the group in head order.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <type_traits>
#include <algorithm>

#include "attn.h"
#include "device_common.h"

namespace hat {
namespace bwd {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;   // rows a workgroup owns (queries in dQ, keys in dK/dV)
constexpr int kBN = 64;            // rows per streamed tile
constexpr float kLog2e = 1.4426950408889634f;

struct Params {
  const char* q;
  const char* k;
  const char* v;
  const char* o;
  const char* dout;
  const float* lse;
  char* dq;
  char* dk;
  char* dv;
  float* stats;   // [B * Hq * Sq] x {LSE * log2(e) (+inf for a row without keys), D}
  float* dk32;    // per-query-head fp32 partials [B, Hq, Skv, D] (null: write dk/dv directly)
  float* dv32;
  int B, Hq, Hkv, Sq, Skv, group, hpw, n_qtiles, n_kblocks;
  int kv_start;   // key j sits at position j + kv_start (causal: allowed for query i iff j + kv_start <= i)
  float c;        // scale * log2(e)
  float scale;
};

template <int D>
struct BTile {
  static constexpr int ROWB = 2 * D;           // bytes per row
  static constexpr int CH = ROWB / 16;         // 16-byte chunks per row
  static constexpr int RP = 256 / ROWB;        // rows per 256 bytes
  static constexpr int BYTES = kBN * ROWB;     // one 64-row tile
  static constexpr int NINSTR = BYTES / 1024;  // 64-lane x 16-byte copies per tile
  // Tiles read both as 16-row MFMA operands and through the transposing reads.
  __device__ static __forceinline__ int dswz(int r) {
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  }
  // Tiles read as rows only.
  __device__ static __forceinline__ int rswz(int r) { return (r / RP) & (CH - 1); }
};

// Operand addresses. A row's byte offset r * ROWB has no bits in the chunk
// field (bits 4 .. 4 + log2(CH) - 1), so the swizzled address of logical chunk
// lc splits into a per-lane base XOR a constant:
//   r * ROWB + ((lc ^ swz(r)) << 4) = (r * ROWB | ((lc0 ^ swz(r)) << 4)) ^ ((lc - lc0) << 4)
// whenever lc - lc0 only sets bits that lc0 leaves clear. Row blocks that are
// multiples of 16 rows share swz and differ by an immediate offset.

// Per-lane base of the 16-byte row reads of row n (+ multiples of 16 rows):
// logical chunk 2 dc + g sits at base ^ (dc << 5).
template <int D>
__device__ __forceinline__ int row_base(int n, int g, int swz) {
  return n * (2 * D) | ((g ^ swz) << 4);
}

// Per-lane base of the transposing reads for rows row1 = 4 g + rr (+ 8 second)
// (+ multiples of 16 rows) and columns 16 dgrp + 4 ss: column block db sits at
// base ^ (db << 6).
template <int D>
__device__ __forceinline__ int tr_base(int g, int rr, int dgrp, int ss, int second) {
  using T = BTile<D>;
  const int row1 = 4 * g + rr + 8 * second;
  return row1 * T::ROWB + (((2 * dgrp + (ss >> 1)) ^ T::dswz(row1)) << 4) + 8 * (ss & 1);
}

__device__ __forceinline__ bf16x8 lds_b128(const LDS_AS char* a) { return *(const LDS_AS bf16x8*)a; }

// A operand of a product whose reduction runs over a tile's rows (two
// transposing reads: rows row1 + {0..3} and row1 + 8 + {0..3}), in the row
// order of pack8() below.
__device__ __forceinline__ bf16x8 tr_pair(const LDS_AS char* a1, const LDS_AS char* a2) {
  const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)a1);
  const i16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)a2);
  return __builtin_bit_cast(bf16x8, i16x8{v1[0], v1[1], v1[2], v1[3], v2[0], v2[1], v2[2], v2[3]});
}

// Elements 8*half .. 8*half+7 of an MFMA result as the bf16 B operand of the next product.
__device__ __forceinline__ bf16x8 pack8(const f32x16& x, int half) {
  const u32x4 pk = u32x4{pack_bf16(x[8 * half + 0], x[8 * half + 1]), pack_bf16(x[8 * half + 2], x[8 * half + 3]),
                         pack_bf16(x[8 * half + 4], x[8 * half + 5]), pack_bf16(x[8 * half + 6], x[8 * half + 7])};
  return __builtin_bit_cast(bf16x8, pk);
}

__device__ __forceinline__ i32x4 sgpr_rsrc(const i32x4 r) {
  return i32x4{__builtin_amdgcn_readfirstlane(r[0]), __builtin_amdgcn_readfirstlane(r[1]),
               __builtin_amdgcn_readfirstlane(r[2]), __builtin_amdgcn_readfirstlane(r[3])};
}

// ---------------------------------------------------------------------------
// dQ kernel (and the row statistics)
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kThreads) attn_bwd_dq_kernel(const Params p) {
  using T = BTile<D>;
  constexpr int ROWB = T::ROWB;
  constexpr int NDB = D / 32;
  constexpr int NKB = kBN / 32;
  constexpr int S = 4;                                     // ring depth
  __shared__ __attribute__((aligned(1024))) char smem_raw[S * 2 * T::BYTES];   // [slot][K, V]
  LDS_AS char* smem = (LDS_AS char*)smem_raw;

  const int BH = p.B * p.Hq;
  const int bid = (int)blockIdx.x;
  int bh, qt;
  if (CAUSAL) {  // longest rows first
    qt = p.n_qtiles - 1 - bid / BH;
    bh = bid % BH;
  } else {
    bh = bid / p.n_qtiles;
    qt = bid % p.n_qtiles;
  }
  const int b = bh / p.Hq, h = bh % p.Hq, hk = h / p.group;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 5, n = lane & 31;
  const int Sq = p.Sq, Skv = p.Skv, kv_start = p.kv_start;
  const float c = p.c, scale = p.scale;   // locals: lambdas must not capture the kernel argument
  const int q0 = qt * kBM, qw = q0 + wave * 32, qi = qw + n;

  const size_t qrow0 = (size_t)bh * (size_t)Sq;
  const size_t krow0 = (size_t)(b * p.Hkv + hk) * (size_t)Skv;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + qrow0 * ROWB, (uint32_t)Sq * ROWB);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(p.o + qrow0 * ROWB, (uint32_t)Sq * ROWB);
  const __amdgpu_buffer_rsrc_t rdo = make_rsrc(p.dout + qrow0 * ROWB, (uint32_t)Sq * ROWB);
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(p.lse + qrow0, (uint32_t)Sq * 4);
  const i32x4 rk = rsrc_words(p.k + krow0 * ROWB, (uint32_t)Skv * ROWB);
  const i32x4 rv = rsrc_words(p.v + krow0 * ROWB, (uint32_t)Skv * ROWB);

  const int rows_end = min(q0 + kBM, Sq);
  const int kv_end = CAUSAL ? min(Skv, max(0, rows_end - kv_start)) : Skv;
  const int ntot = (kv_end + kBN - 1) / kBN;
  const bool wave_live = qw < Sq;
  const int w_kv_end = CAUSAL ? min(Skv, max(0, min(qw + 32, Sq) - kv_start)) : Skv;
  const int w_ntiles = wave_live ? (w_kv_end + kBN - 1) / kBN : 0;

  // Q and dO rows as B operands (rows >= Sq read as zero); D_i = dO_i . O_i.
  bf16x8 qf[D / 16], df[D / 16];
  float dsum = 0.f;
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc) {
    const int off = qi * ROWB + (16 * dc + 8 * g) * 2;
    qf[dc] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
    df[dc] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rdo, off, 0, 0));
    const bf16x8 of = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(ro, off, 0, 0));
#pragma unroll
    for (int j = 0; j < 8; ++j) dsum = __builtin_fmaf((float)df[dc][j], (float)of[j], dsum);
  }
  const float delta = xor32_sum(dsum);
  const float lse = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl, qi * 4, 0, 0));
  const float lse2 = lse == -INFINITY ? INFINITY : lse * kLog2e;   // keyless row: P = 0
  if (g == 0) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.stats + 2 * qrow0, (uint32_t)Sq * 8);
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(lse2), __float_as_uint(delta)}, rs, qi * 8, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the row loads landed before any copy is queued

  for (int i = threadIdx.x; i < S * 2 * T::BYTES / 16; i += kThreads)
    *(LDS_AS u32x4*)(smem + i * 16) = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();

  const unsigned smem_addr = (unsigned)(uintptr_t)smem;
  constexpr int PW = 2 * T::NINSTR / kWaves;
  static_assert(PW >= 1 && PW * kWaves == 2 * T::NINSTR, "tile copies must split evenly over waves");
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  // The K and V descriptors, made wave-uniform once here (lane reads are
  // convergent operations, which the compiler keeps inside the loop).
  const i32x4 rkw = sgpr_rsrc(rk), rvw = sgpr_rsrc(rv);
  auto issue = [&](int u) __attribute__((always_inline)) {
    const int key0 = u * kBN, slot = u % S;
#pragma unroll
    for (int j = 0; j < PW; ++j) {
      const int ins = wv * PW + j;
      const bool isv = ins >= T::NINSTR;
      const int c0 = (isv ? ins - T::NINSTR : ins) * 64;
      const int cidx = c0 + lane;
      const int r = cidx / T::CH, pc = cidx % T::CH;
      const int goff = (key0 + r) * ROWB + (pc ^ T::dswz(r)) * 16;
      const unsigned dst = __builtin_amdgcn_readfirstlane(smem_addr + (slot * 2 + (isv ? 1 : 0)) * T::BYTES + c0 * 16);
      dma16(isv ? rvw : rkw, goff, dst);
    }
  };

  f32x16 acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = f32x16{};
  const int l16 = lane & 15, dgrp = (lane >> 4) & 1, rr = l16 >> 2, ss = l16 & 3;

#pragma unroll
  for (int u = 0; u < S - 1; ++u)
    if (u < ntot) issue(u);
  auto sync = [&](int u) __attribute__((always_inline)) {
    if (u + 2 < ntot) wait_vmcnt<2 * PW>();
    else if (u + 1 < ntot) wait_vmcnt<PW>();
    else wait_vmcnt<0>();
    __syncthreads();
    if (u + S - 1 < ntot) issue(u + S - 1);
  };
  const int rb = row_base<D>(n, g, T::dswz(n));
  const int tb0 = tr_base<D>(g, rr, dgrp, ss, 0), tb1 = tr_base<D>(g, rr, dgrp, ss, 1);
  auto step = [&](int u, auto masked_c) __attribute__((always_inline)) {
    const LDS_AS char* ks = smem + ((u % S) * 2 + 0) * T::BYTES;
    const LDS_AS char* vs = ks + T::BYTES;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      // S^T = K Q^T and dP^T = V dO^T for 32 keys
      f32x16 s = f32x16{}, dp = f32x16{};
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int dc = 0; dc < D / 16; ++dc) {
        const int off = (rb ^ (dc << 5)) + 32 * kb * ROWB;
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_b128(ks + off), qf[dc], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_b128(vs + off), df[dc], dp, 0, 0, 0);
      }
      // operand reads four MFMAs ahead of their use, in a region of their own
      // (each read right before its MFMA otherwise)
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < 2 * (D / 16) - 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (decltype(masked_c)::value) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = u * kBN + 32 * kb + 8 * (i >> 2) + 4 * g + (i & 3);
          const bool ok = key < Skv && (!CAUSAL || key + kv_start <= qi);
          s[i] = ok ? s[i] : -INFINITY;
        }
      }
      // dS^T = P^T (dP^T - D), P^T = exp2(c s - LSE log2 e)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, -lse2));
        s[i] = pv * (dp[i] - delta);
      }
      // dQ^T += K^T dS^T over the block's two 16-key groups
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const bf16x8 dsf = pack8(s, half);
        const int roff = (32 * kb + 16 * half) * ROWB;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              tr_pair(ks + roff + (tb0 ^ (db << 6)), ks + roff + (tb1 ^ (db << 6))), dsf, acc[db], 0, 0, 0);
      }
    }
  };
  const int first_masked = CAUSAL ? min(Skv / kBN, max(0, qw - kv_start + 1) / kBN) : Skv / kBN;
  int u = 0;
  for (; u < min(first_masked, ntot); ++u) {
    sync(u);
    if (u < w_ntiles) step(u, std::false_type{});
  }
  for (; u < ntot; ++u) {
    sync(u);
    if (u < w_ntiles) step(u, std::true_type{});
  }

  if (!wave_live) return;
  const __amdgpu_buffer_rsrc_t rdq = make_rsrc(p.dq + qrow0 * ROWB, (uint32_t)Sq * ROWB);
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const u32x2 w = u32x2{pack_bf16(acc[db][4 * ii + 0] * scale, acc[db][4 * ii + 1] * scale),
                            pack_bf16(acc[db][4 * ii + 2] * scale, acc[db][4 * ii + 3] * scale)};
      const int col = 32 * db + 8 * ii + 4 * g;
      __builtin_amdgcn_raw_buffer_store_b64(w, rdq, (qi * D + col) * 2, 0, 0);
    }
}

// ---------------------------------------------------------------------------
// dK / dV kernel
// ---------------------------------------------------------------------------
template <int D>
struct DkdvCfg {
  static constexpr int S = D == 128 ? 2 : 4;                  // ring depth
  static constexpr int STAGE = 2 * BTile<D>::BYTES + 1024;    // Q tile, dO tile, 128 rows of statistics
  static constexpr int VBYTES = kBM * BTile<D>::ROWB;         // the workgroup's V rows
  static constexpr int LDS = VBYTES + S * STAGE;
};

template <int N>
__device__ __forceinline__ void wait_ahead(int ahead) {
  if (ahead >= 2) wait_vmcnt<2 * N>();
  else if (ahead == 1) wait_vmcnt<N>();
  else wait_vmcnt<0>();
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kThreads) attn_bwd_dkdv_kernel(const Params p) {
  using T = BTile<D>;
  using C = DkdvCfg<D>;
  constexpr int ROWB = T::ROWB;
  constexpr int NDB = D / 32;
  constexpr int S = C::S;
  __shared__ __attribute__((aligned(1024))) char smem_raw[C::LDS];
  LDS_AS char* smem = (LDS_AS char*)smem_raw;
  LDS_AS char* vsm = smem;                    // V rows of the workgroup
  LDS_AS char* ring = smem + C::VBYTES;

  const int nhg = p.Hq / p.hpw;               // query-head groups per batch entry
  const int BHG = p.B * nhg;
  const int bid = (int)blockIdx.x;
  int bhg, kbk;
  if (CAUSAL) {  // the first key blocks see the most queries: run them first
    kbk = bid / BHG;
    bhg = bid % BHG;
  } else {
    bhg = bid / p.n_kblocks;
    kbk = bid % p.n_kblocks;
  }
  const int b = bhg / nhg, h0 = (bhg % nhg) * p.hpw, hk = h0 / p.group;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 5, n = lane & 31;
  const int Sq = p.Sq, Skv = p.Skv, Hq = p.Hq, kv_start = p.kv_start;
  const float c = p.c, scale = p.scale;   // locals: lambdas must not capture the kernel argument
  const char* const gq = p.q;
  const char* const gdo = p.dout;
  const float* const gstats = p.stats;
  const int k0 = kbk * kBM, kw = k0 + 32 * wave, kj = kw + n;

  const size_t krow0 = (size_t)(b * p.Hkv + hk) * (size_t)Skv;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + krow0 * ROWB, (uint32_t)Skv * ROWB);
  const i32x4 rvw = rsrc_words(p.v + krow0 * ROWB, (uint32_t)Skv * ROWB);

  // K rows as B operands of S = Q K^T (keys >= Skv read as zero).
  bf16x8 kf[D / 16];
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc)
    kf[dc] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, kj * ROWB + (16 * dc + 8 * g) * 2, 0, 0));
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)

  for (int i = threadIdx.x; i < S * C::STAGE / 16; i += kThreads)
    *(LDS_AS u32x4*)(ring + i * 16) = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();

  const unsigned smem_addr = (unsigned)(uintptr_t)smem;
  const unsigned ring_addr = smem_addr + C::VBYTES;
  const int wv = __builtin_amdgcn_readfirstlane(wave);

  // V rows of the workgroup into LDS, once (the oldest copies of every wave).
  constexpr int VPW = C::VBYTES / 1024 / kWaves;
  static_assert(VPW * kWaves * 1024 == C::VBYTES, "V copies must split evenly over waves");
#pragma unroll
  for (int j = 0; j < VPW; ++j) {
    const int c0 = (wv * VPW + j) * 64;
    const int cidx = c0 + lane;
    const int r = cidx / T::CH, pc = cidx % T::CH;
    dma16(sgpr_rsrc(rvw), (k0 + r) * ROWB + (pc ^ T::rswz(r)) * 16,
          __builtin_amdgcn_readfirstlane(smem_addr + c0 * 16));
  }

  // Query tiles: for each of the workgroup's query heads, tiles [qt_begin, nqt).
  const int nqt = (Sq + kBN - 1) / kBN;
  const int qt_begin = CAUSAL ? min(nqt, (k0 + kv_start) / kBN) : 0;
  const int per_head = nqt - qt_begin;
  const int ntot = per_head * p.hpw;
  // This wave: tiles before w_qt_begin hold no row >= its first key; from
  // w_qt_full on every row is >= its last key.
  const int w_qt_begin = CAUSAL ? (kw + kv_start) / kBN : 0;
  const int w_qt_full = CAUSAL ? (kw + kv_start + 31 + kBN - 1) / kBN : 0;

  constexpr int PW = 2 * T::NINSTR / kWaves;
  static_assert(PW >= 1 && PW * kWaves == 2 * T::NINSTR, "tile copies must split evenly over waves");
  auto issue = [&](int u) __attribute__((always_inline)) {
    // head and tile of step u, made wave-uniform right after the division (which
    // runs on the vector ALU), so that the descriptors below stay scalar
    const int hh = __builtin_amdgcn_readfirstlane(u / per_head);
    const int qt = qt_begin + __builtin_amdgcn_readfirstlane(u - hh * per_head);
    const size_t qrow0 = (size_t)(b * Hq + h0 + hh) * (size_t)Sq;
    const unsigned base = ring_addr + (u % S) * C::STAGE;
#pragma unroll
    for (int j = 0; j < PW; ++j) {
      const int ins = wv * PW + j;
      const bool isdo = ins >= T::NINSTR;
      const int c0 = (isdo ? ins - T::NINSTR : ins) * 64;
      const int cidx = c0 + lane;
      const int r = cidx / T::CH, pc = cidx % T::CH;
      const i32x4 rs = rsrc_words((isdo ? gdo : gq) + qrow0 * ROWB, (uint32_t)Sq * ROWB);
      dma16(sgpr_rsrc(rs), (qt * kBN + r) * ROWB + (pc ^ T::dswz(r)) * 16,
            __builtin_amdgcn_readfirstlane(base + (isdo ? T::BYTES : 0) + c0 * 16));
    }
    if (wv == 0) {   // statistics of rows qt*64 .. +127 (the second half unused)
      const i32x4 rs = rsrc_words(gstats + 2 * qrow0, (uint32_t)Sq * 8);
      dma16(sgpr_rsrc(rs), qt * kBN * 8 + lane * 16, __builtin_amdgcn_readfirstlane(base + 2 * T::BYTES));
    }
  };
#pragma unroll
  for (int u = 0; u < S - 1; ++u)
    if (u < ntot) issue(u);
  auto sync = [&](int u) __attribute__((always_inline)) {
    const int ahead = min(S - 2, ntot - 1 - u);
    if (wv == 0) wait_ahead<PW + 1>(ahead);
    else wait_ahead<PW>(ahead);
    __syncthreads();
    if (u + S - 1 < ntot) issue(u + S - 1);
  };

  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) {
    dk[i] = f32x16{};
    dv[i] = f32x16{};
  }
  const int l16 = lane & 15, dgrp = (lane >> 4) & 1, rr = l16 >> 2, ss = l16 & 3;
  const int rb = row_base<D>(n, g, T::dswz(n));                         // Q / dO rows
  const int vb = row_base<D>(32 * wave + n, g, T::rswz(32 * wave + n));  // V rows
  const int tb0 = tr_base<D>(g, rr, dgrp, ss, 0), tb1 = tr_base<D>(g, rr, dgrp, ss, 1);

  auto step = [&](int u, int qt, auto masked_c) __attribute__((always_inline)) {
    const LDS_AS char* qs = ring + (u % S) * C::STAGE;
    const LDS_AS char* dos = qs + T::BYTES;
    const LDS_AS char* st = qs + 2 * T::BYTES;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      // S = Q K^T and dP = dO V^T for 32 query rows x this wave's 32 keys
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int dc = 0; dc < D / 16; ++dc) {
        const int off = (rb ^ (dc << 5)) + 32 * qb * ROWB;
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_b128(qs + off), kf[dc], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_b128(dos + off), lds_b128(vsm + (vb ^ (dc << 5))), dp, 0, 0, 0);
      }
      // causal: row 32 qb + 8 j + 4 g + t of the tile sees this lane's key iff 8 j + t >= thr
      [[maybe_unused]] const int thr = kj + kv_start - (qt * kBN + 32 * qb + 4 * g);
      // P = exp2(c s - LSE log2 e) and dS = P (dP - D), in place, with the
      // statistics of this lane's rows 32 qb + 8 j + 4 g + (0..3)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 a = *(const LDS_AS f32x4*)(st + (32 * qb + 8 * j + 4 * g) * 8);
        const f32x4 e = *(const LDS_AS f32x4*)(st + (32 * qb + 8 * j + 4 * g) * 8 + 16);
        const float l2[4] = {a[0], a[2], e[0], e[2]};
        const float dl[4] = {a[1], a[3], e[1], e[3]};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int i = 4 * j + t;
          float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, -l2[t]));
          if constexpr (decltype(masked_c)::value) pv = 8 * j + t >= thr ? pv : 0.f;
          s[i] = pv;
          dp[i] = pv * (dp[i] - dl[t]);
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS over the block's two 16-row groups
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const bf16x8 pf = pack8(s, half);
        const bf16x8 dsf = pack8(dp, half);
        const int roff = (32 * qb + 16 * half) * ROWB;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int o0 = roff + (tb0 ^ (db << 6)), o1 = roff + (tb1 ^ (db << 6));
          dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_pair(dos + o0, dos + o1), pf, dv[db], 0, 0, 0);
          dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_pair(qs + o0, qs + o1), dsf, dk[db], 0, 0, 0);
        }
      }
      // keep the two halves apart: interleaving them doubles the live scores
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  int u = 0;
  for (int hh = 0; hh < p.hpw; ++hh) {
    int qt = qt_begin;
    if constexpr (CAUSAL) {
      for (; qt < min(w_qt_full, nqt); ++qt, ++u) {
        sync(u);
        if (qt >= w_qt_begin) step(u, qt, std::true_type{});
      }
    }
    for (; qt < nqt; ++qt, ++u) {
      sync(u);
      step(u, qt, std::false_type{});
    }
  }
  wait_vmcnt<0>();   // no copy may still be writing LDS when the workgroup ends

  if (p.dk32 == nullptr) {
    const __amdgpu_buffer_rsrc_t rdk = make_rsrc(p.dk + krow0 * ROWB, (uint32_t)Skv * ROWB);
    const __amdgpu_buffer_rsrc_t rdv = make_rsrc(p.dv + krow0 * ROWB, (uint32_t)Skv * ROWB);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int col = 32 * db + 8 * ii + 4 * g;
        const u32x2 wk = u32x2{pack_bf16(dk[db][4 * ii + 0] * scale, dk[db][4 * ii + 1] * scale),
                               pack_bf16(dk[db][4 * ii + 2] * scale, dk[db][4 * ii + 3] * scale)};
        const u32x2 wvv = u32x2{pack_bf16(dv[db][4 * ii + 0], dv[db][4 * ii + 1]),
                                pack_bf16(dv[db][4 * ii + 2], dv[db][4 * ii + 3])};
        __builtin_amdgcn_raw_buffer_store_b64(wk, rdk, (kj * D + col) * 2, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b64(wvv, rdv, (kj * D + col) * 2, 0, 0);
      }
  } else {
    const size_t prow0 = (size_t)(b * p.Hq + h0) * (size_t)Skv;
    const __amdgpu_buffer_rsrc_t rdk = make_rsrc(p.dk32 + prow0 * D, (uint32_t)Skv * D * 4);
    const __amdgpu_buffer_rsrc_t rdv = make_rsrc(p.dv32 + prow0 * D, (uint32_t)Skv * D * 4);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int col = 32 * db + 8 * ii + 4 * g;
        const u32x4 wk = u32x4{__float_as_uint(dk[db][4 * ii + 0] * scale), __float_as_uint(dk[db][4 * ii + 1] * scale),
                               __float_as_uint(dk[db][4 * ii + 2] * scale), __float_as_uint(dk[db][4 * ii + 3] * scale)};
        const u32x4 wvv = u32x4{__float_as_uint(dv[db][4 * ii + 0]), __float_as_uint(dv[db][4 * ii + 1]),
                                __float_as_uint(dv[db][4 * ii + 2]), __float_as_uint(dv[db][4 * ii + 3])};
        __builtin_amdgcn_raw_buffer_store_b128(wk, rdk, (kj * D + col) * 4, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(wvv, rdv, (kj * D + col) * 4, 0, 0);
      }
  }
}

// Sum of the per-query-head partials over each KV head's group, in head order.
template <int D>
__global__ void __launch_bounds__(256) attn_bwd_group_sum_kernel(const float* __restrict__ dk32,
                                                                 const float* __restrict__ dv32, char* dk, char* dv,
                                                                 int Hkv, int group, int Skv, long long total4) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;   // one 4-element column group
  if (idx >= total4) return;
  const long long row = idx / (D / 4);
  const int c4 = (int)(idx % (D / 4));
  const long long key = row % Skv, bhk = row / Skv;
  const long long b = bhk / Hkv, hk = bhk % Hkv;
  f32x4 sk = f32x4{0.f, 0.f, 0.f, 0.f}, sv = sk;
  for (int j = 0; j < group; ++j) {
    const long long off = (((b * Hkv + hk) * group + j) * Skv + key) * D + 4 * c4;
    sk += *(const f32x4*)(dk32 + off);
    sv += *(const f32x4*)(dv32 + off);
  }
  const long long o = (row * D + 4 * c4) * 2;
  *(u32x2*)(dk + o) = u32x2{pack_bf16(sk[0], sk[1]), pack_bf16(sk[2], sk[3])};
  *(u32x2*)(dv + o) = u32x2{pack_bf16(sv[0], sv[1]), pack_bf16(sv[2], sv[3])};
}

typedef void (*kernel_fn)(Params);

}  // namespace bwd
}  // namespace hat

using namespace hat::bwd;

// Heads per dK/dV workgroup: the whole group (no partials) when that still
// gives at least two workgroups per CU of a 256-CU chip, else one.
static int64_t bwd_heads_per_wg(int64_t B, int64_t Hq, int64_t Hkv, int64_t Skv) {
  const int64_t group = Hq / Hkv;
  if (group <= 1) return 1;
  const int64_t nkb = (Skv + kBM - 1) / kBM;
  return B * Hkv * nkb >= 512 ? group : 1;
}

static int64_t bwd_stats_bytes(int64_t B, int64_t Hq, int64_t Sq) {
  return (B * Hq * Sq * 8 + 255) / 256 * 256;
}

static int64_t bwd_workspace(int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Skv, int64_t D) {
  int64_t bytes = bwd_stats_bytes(B, Hq, Sq);
  if (Hkv > 0 && bwd_heads_per_wg(B, Hq, Hkv, Skv) < Hq / Hkv) bytes += 2 * B * Hq * Skv * D * 4;
  return bytes;
}

extern "C" int64_t attn_bwd_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Skv, int64_t D) {
  if (B < 0 || Hq < 0 || Hkv < 0 || Sq < 0 || Skv < 0 || (D != 64 && D != 128)) return -1;
  if (Hq > 0 && (Hkv == 0 || Hq % Hkv != 0)) return -1;
  if (Hq == 0) return 0;
  return bwd_workspace(B, Hq, Hkv, Sq, Skv, D);
}

static attn_status_t bwd_launch(const void* q, const void* k, const void* v, const void* out, const void* dout,
                                const float* lse, void* dq, void* dk, void* dv,
                                int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Skv, int64_t D,
                                float scale, int causal, attn_dtype_t dtype, int64_t kv_start,
                                void* workspace, int64_t workspace_bytes, void* stream) {
  if (dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
  if (D != 64 && D != 128) return ATTN_ERR_HEAD_DIM;
  if (B < 0 || Hq < 0 || Hkv < 0 || Sq < 0 || Skv < 0 || kv_start < 0) return ATTN_ERR_SHAPE;
  if (Hq > 0 && (Hkv == 0 || Hq % Hkv != 0)) return ATTN_ERR_SHAPE;
  if (!(scale > 0.f) || !isfinite(scale)) return ATTN_ERR_SCALE;
  const bool any_q = B > 0 && Hq > 0 && Sq > 0;
  const bool any_kv = B > 0 && Hkv > 0 && Skv > 0;
  if (!any_q && !any_kv) return ATTN_OK;
  if (any_q && (!q || !out || !dout || !lse || !dq)) return ATTN_ERR_NULL;
  if (any_kv && (!k || !v || !dk || !dv)) return ATTN_ERR_NULL;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out | (uintptr_t)dout | (uintptr_t)dq |
       (uintptr_t)dk | (uintptr_t)dv) & 15)
    return ATTN_ERR_ALIGN;
  if ((uintptr_t)lse & 3) return ATTN_ERR_ALIGN;
  const int64_t lim = (int64_t)1 << 31;
  const int64_t rowb = 2 * D;
  if ((Sq + kBM) * rowb >= lim || (Skv + kBM) * rowb >= lim || (Skv + kBM) * D * 4 >= lim || (Sq + kBM) * 8 >= lim)
    return ATTN_ERR_OVERFLOW;
  if (kv_start + Skv + kBM >= ((int64_t)1 << 30)) return ATTN_ERR_OVERFLOW;   // key positions stay below 2^30
  const int64_t need = bwd_workspace(B, Hq, Hkv, Sq, Skv, D);
  if (need > 0 && (!workspace || ((uintptr_t)workspace & 255) || workspace_bytes < need)) return ATTN_ERR_WORKSPACE;
  const int64_t n_qtiles = (Sq + kBM - 1) / kBM, n_kblocks = (Skv + kBM - 1) / kBM;
  const int64_t hpw = bwd_heads_per_wg(B, Hq, Hkv, Skv);
  const int64_t grid_q = B * Hq * n_qtiles, grid_k = B * (Hq / hpw) * n_kblocks;
  if (grid_q >= lim || grid_k >= lim || B * Hq * Sq >= lim || B * Hkv * Skv * D >= lim) return ATTN_ERR_OVERFLOW;

  Params p;
  p.q = (const char*)q;
  p.k = (const char*)k;
  p.v = (const char*)v;
  p.o = (const char*)out;
  p.dout = (const char*)dout;
  p.lse = lse;
  p.dq = (char*)dq;
  p.dk = (char*)dk;
  p.dv = (char*)dv;
  p.stats = (float*)workspace;
  const bool partial = hpw < Hq / Hkv;
  p.dk32 = partial ? (float*)((char*)workspace + bwd_stats_bytes(B, Hq, Sq)) : nullptr;
  p.dv32 = partial ? p.dk32 + B * Hq * Skv * D : nullptr;
  p.B = (int)B;
  p.Hq = (int)Hq;
  p.Hkv = (int)Hkv;
  p.Sq = (int)Sq;
  p.Skv = any_kv ? (int)Skv : 0;
  p.group = (int)(Hq / Hkv);
  p.hpw = (int)hpw;
  p.n_qtiles = (int)n_qtiles;
  p.n_kblocks = (int)n_kblocks;
  p.kv_start = (int)kv_start;
  p.c = scale * kLog2e;
  p.scale = scale;
  const hipStream_t st = (hipStream_t)stream;

  // dQ first: it also writes the row statistics the dK/dV kernel reads.
  if (any_q) {
    kernel_fn fq = D == 128 ? (causal ? attn_bwd_dq_kernel<128, true> : attn_bwd_dq_kernel<128, false>)
                            : (causal ? attn_bwd_dq_kernel<64, true> : attn_bwd_dq_kernel<64, false>);
    hipLaunchKernelGGL(fq, dim3((unsigned)grid_q), dim3(kThreads), 0, st, p);
    if (hipGetLastError() != hipSuccess) return ATTN_ERR_HIP;
  }
  if (any_kv) {
    kernel_fn fk = D == 128 ? (causal ? attn_bwd_dkdv_kernel<128, true> : attn_bwd_dkdv_kernel<128, false>)
                            : (causal ? attn_bwd_dkdv_kernel<64, true> : attn_bwd_dkdv_kernel<64, false>);
    hipLaunchKernelGGL(fk, dim3((unsigned)grid_k), dim3(kThreads), 0, st, p);
    if (hipGetLastError() != hipSuccess) return ATTN_ERR_HIP;
    if (partial) {
      const long long total4 = (long long)(B * Hkv * Skv * D / 4);
      const unsigned blocks = (unsigned)((total4 + 255) / 256);
      if (D == 128)
        hipLaunchKernelGGL(attn_bwd_group_sum_kernel<128>, dim3(blocks), dim3(256), 0, st, p.dk32, p.dv32,
                           p.dk, p.dv, p.Hkv, p.group, p.Skv, total4);
      else
        hipLaunchKernelGGL(attn_bwd_group_sum_kernel<64>, dim3(blocks), dim3(256), 0, st, p.dk32, p.dv32,
                           p.dk, p.dv, p.Hkv, p.group, p.Skv, total4);
      if (hipGetLastError() != hipSuccess) return ATTN_ERR_HIP;
    }
  }
  return ATTN_OK;
}

extern "C" attn_status_t attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                                  const float* lse, void* dq, void* dk, void* dv,
                                  int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Skv, int64_t D,
                                  float scale, int causal, attn_dtype_t dtype,
                                  void* workspace, int64_t workspace_bytes, void* stream) {
  return bwd_launch(q, k, v, out, dout, lse, dq, dk, dv, B, Hq, Hkv, Sq, Skv, D, scale, causal, dtype, 0,
                    workspace, workspace_bytes, stream);
}

extern "C" attn_status_t attn_bwd_chunk(const void* q, const void* k, const void* v, const void* out,
                                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                        int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Skv, int64_t D,
                                        float scale, int causal, attn_dtype_t dtype, int64_t kv_start,
                                        void* workspace, int64_t workspace_bytes, void* stream) {
  return bwd_launch(q, k, v, out, dout, lse, dq, dk, dv, B, Hq, Hkv, Sq, Skv, D, scale, causal, dtype, kv_start,
                    workspace, workspace_bytes, stream);
}
