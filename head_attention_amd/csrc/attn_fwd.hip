// Fused attention forward with per-row LSE for gfx950 (MI355X, CDNA4).
//
// The method is the flash-style attention forward the pages turn on: the SDPA
// forward with log-sum-exp of the page "[Proposal] ROCm (AMD Instinct) support
// for the core attention and distributed init" ("Where it breaks on ROCm"),
// and the bf16 / fp8 (per-tensor q/k/v descale) forward of the page "F8 fmha
// ASM gfx950" (Test Result section), whose fp8 kernel runs the 32x32x64 fp8
// MFMA for head dim 128 (Technical Details section). Grouped KV heads follow
// the 32/8-head layout and the causal prefill of the page "feat(attention):
// add strict bitwise ROCm path" (ROCm Validation, Benchmark results).
//
// Design (gfx950 first; nothing here is translated from another kernel):
//  * One workgroup = 8 wavefronts = 256 query rows of one (batch, head); each
//    wave owns 32 rows. The grid covers B * Hq * ceil(Sq / 256) workgroups.
//    A grid small enough to leave half the CUs idle uses workgroups of 4
//    wavefronts (128 rows) instead, twice as many of them.
//  * K and V stream through LDS in tiles of 64 keys, in a ring of kStages
//    slots filled kStages-1 tiles ahead by buffer_load ... lds (global -> LDS
//    without VGPRs); one workgroup barrier per tile publishes a tile and
//    retires the oldest slot. Out-of-range key rows read as zero through the
//    buffer descriptor's range check.
//  * Scores are computed transposed, S^T = K Q^T, on 32x32 MFMAs (bf16
//    32x32x16, or fp8 32x32x64): each lane then owns one query row's scores,
//    so row max / row sum are in-register work plus one permlane32 swap.
//  * O^T += V^T P^T keeps P in the registers the score MFMA produced; V^T
//    operands come from LDS with the transposing reads ds_read_b64_tr_b16
//    (bf16) and ds_read_b64_tr_b8 (fp8). The key order inside a tile is
//    permuted consistently between P and V, which leaves the sum unchanged.
//  * Online softmax in base 2 with a checked running max m (of
//    scale*log2(e)*s): p = exp2(c*s - m) is formed with the current m, and
//    as long as every p of a tile stays at most 2^8 (a lane's partial row
//    sum bounds its own p) the tile needs no row max at all. Otherwise, and
//    for a row's first tile, m becomes the exact running max, O and l are
//    rescaled by exp2(m_old - m_new) and p is formed again (a wave-uniform
//    branch, rarely taken). p <= 2^8 is well inside bf16 and fp32 range.
//    Each lane adds its fp32 partial row sum of a tile into an fp64 l, so
//    that rows over millions of keys keep the tail of their sum.
//  * fp8: p carries a factor 2^kPre (folded into the exp2 offset), so that
//    e4m3fn P is at most 2^8 and keeps full precision for the typical
//    p ~ 1e-2; l sums the same scaled, unrounded fp32 values, and the
//    epilogue divides by l and multiplies by v_descale, so the factor cancels.
//  * Causal: a workgroup only loads the key tiles its rows can see; within
//    them a wave skips tiles entirely above its rows and masks only tiles that
//    cross its diagonal. Causal grids run the longest query tiles first.
//  * Local attention (window sides and sink keys; the window_size_left /
//    window_size_right arguments of the page "F8 fmha ASM gfx950", Test
//    Result section): a workgroup loads only the sink tiles and the tiles its
//    rows' windows cover (one or two runs of the tile sequence); each wave
//    takes the tiles that are wholly inside its rows' windows or sinks in
//    loops without mask code and decides skip / whole / masked only for the
//    tiles around them.
//  * Key splits (split-KV): workgroups of one query tile may take disjoint
//    whole-tile key ranges, each written as a normalised fp32 partial with
//    its LSE; merge_splits_kernel combines them by LSE on the device.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <type_traits>
#include <algorithm>

#include "attn.h"
#include "device_common.h"

namespace hat {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;   // query rows per workgroup
constexpr int kBN = 64;            // keys per K/V tile
constexpr int kStages = 4;         // LDS ring depth (K/V tiles in flight)

struct Params {
  const char* q;
  const char* k;
  const char* v;
  char* o;
  float* lse;
  int B, Hq, Hkv, Sq, Skv, group, n_qtiles, kv_start;
  float c;  // scale * log2(e)
  const float* qd;
  const float* kd;
  const float* vd;
  // Key splits: workgroup blockIdx.x / (B * Hq * n_qtiles) takes keys
  // [split * split_len, + split_len). With o32 set, each split writes its
  // normalised fp32 O and its LSE to o32 / lse32, rows [split * part_rows, +
  // part_rows) holding global rows [part_row0, part_row0 + part_rows).
  // Tail mode (n_full >= 0, non-causal): workgroups [0, n_full) take whole
  // query tiles 0 .. n_full-1 and write out / lse directly; the later ones
  // take the nsplit key splits of each remaining (tail) tile.
  int nsplit, split_len;
  float* o32;
  float* lse32;
  int n_full, part_rows, part_row0;
  // Local attention (instances with WIN): key position j (absolute, i.e.
  // local key + kv_start) is allowed for query i iff i - wl <= j <= i + wr, or
  // j < sink; causal additionally requires j <= i. Unbounded sides hold 2^30.
  int wl, wr, sink;
};

// LDS layout of one K or V tile: kBN rows of ROWB bytes, 16-byte chunks permuted
// within a row by an XOR swizzle so that the MFMA operand reads hit distinct banks.
template <int D, bool FP8>
struct Tile {
  static constexpr int ELT = FP8 ? 1 : 2;
  static constexpr int ROWB = D * ELT;        // bytes per key row
  static constexpr int CH = ROWB / 16;        // 16-byte chunks per row
  static constexpr int RP = 256 / ROWB;       // rows per 256 bytes
  static constexpr int BYTES = kBN * ROWB;
  static constexpr int NINSTR = BYTES / 1024; // 64-lane x 16-byte loads per tile and matrix
  // K operand reads: 16 consecutive rows, same logical chunk -> distinct banks.
  __device__ static __forceinline__ int kswz(int r) { return (r / RP) & (CH - 1); }
  // V operand reads (transposing): bf16 reads 4 rows x 32 bytes per 16 lanes,
  // fp8 reads rows {0..3, 8..11} (+4 for the upper half-wave) x 16 bytes.
  __device__ static __forceinline__ int vswz(int r) {
    if constexpr (!FP8) {
      if constexpr (D == 128) return (r & 3) << 2;
      else return ((r >> 1) & 1) << 2;
    } else {
      if constexpr (D == 128) return (((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2);
      else return ((r >> 3) & 1) << 1;
    }
  }
};

template <int D, bool CAUSAL, bool FP8, bool WIN, int NW>
__global__ void __launch_bounds__(64 * NW) attn_fwd_kernel(const Params p) {
  constexpr int kW = NW;            // waves per workgroup (8, or 4 for grids that leave CUs idle)
  constexpr int kThr = 64 * NW;
  constexpr int kRows = 32 * NW;    // query rows per workgroup
  using T = Tile<D, FP8>;
  constexpr int ROWB = T::ROWB;
  constexpr int NDB = D / 32;                       // 32-wide output column blocks
  constexpr int NKB = kBN / 32;                     // 32-key blocks per tile
  constexpr float kPre = FP8 ? 4.f : 0.f;           // fp8: p carries a factor 2^kPre
  __shared__ __attribute__((aligned(1024))) char smem_raw[kStages * 2 * T::BYTES];  // [slot][K, V]
  LDS_AS char* smem = (LDS_AS char*)smem_raw;

  const int BH = p.B * p.Hq;
  int split, bid;
  if (p.n_full >= 0) {
    if ((int)blockIdx.x < p.n_full) {
      split = -1;   // whole tile, direct output
      bid = (int)blockIdx.x;
    } else {
      const int r = (int)blockIdx.x - p.n_full;
      split = r % p.nsplit;
      bid = p.n_full + r / p.nsplit;
    }
  } else {
    const int per_split = BH * p.n_qtiles;
    split = (int)(blockIdx.x / per_split);
    bid = (int)(blockIdx.x % per_split);
  }
  int bh, qt;
  if (CAUSAL) {  // longest rows first
    qt = p.n_qtiles - 1 - bid / BH;
    bh = bid % BH;
  } else {
    bh = bid / p.n_qtiles;
    qt = bid % p.n_qtiles;
  }
  // This workgroup's keys: [s0, s0 + Skv) of the head; causal positions shift by s0.
  const int s0 = split < 0 ? 0 : split * p.split_len;
  const int Skv = split < 0 ? p.Skv : max(0, min(p.Skv - s0, p.split_len));
  const int kv_start = p.kv_start + s0;
  const int b = bh / p.Hq, h = bh % p.Hq, hk = h / p.group;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 5, n = lane & 31;
  const int q0 = qt * kRows, qw = q0 + wave * 32, qi = qw + n;

  const size_t qrow0 = (size_t)(b * p.Hq + h) * (size_t)p.Sq;
  const size_t krow0 = (size_t)(b * p.Hkv + hk) * (size_t)p.Skv + (size_t)(Skv > 0 ? s0 : 0);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + qrow0 * ROWB, (uint32_t)p.Sq * ROWB);
  const i32x4 rk = rsrc_words(p.k + krow0 * ROWB, (uint32_t)Skv * ROWB);
  const i32x4 rv = rsrc_words(p.v + krow0 * ROWB, (uint32_t)Skv * ROWB);
  const unsigned smem_addr = (unsigned)(uintptr_t)smem;

  float c = p.c, oscale = 1.f;
  if constexpr (FP8) {
    const float qd = p.qd ? *p.qd : 1.f, kd = p.kd ? *p.kd : 1.f, vd = p.vd ? *p.vd : 1.f;
    c *= qd * kd;
    oscale = vd;
  }

  // Key tiles this workgroup needs, and those this wave needs.
  const int rows_end = min(q0 + kRows, p.Sq);
  const int kv_end = CAUSAL ? min(Skv, max(0, rows_end - kv_start)) : Skv;
  const int ntiles = (kv_end + kBN - 1) / kBN;
  const bool wave_live = qw < p.Sq;
  const int w_kv_end = CAUSAL ? min(Skv, max(0, min(qw + 32, p.Sq) - kv_start)) : Skv;
  const int w_ntiles = wave_live ? (w_kv_end + kBN - 1) / kBN : 0;

  // The key tiles this workgroup loads, in order: u = 0 .. ntot-1 is tile
  // tile_of(u). One run [0, ntiles) without a window; with one, up to two runs:
  // the sink tiles from 0, then the tiles the rows' windows cover.
  const int wl = p.wl, wr = p.wr, sink = p.sink;
  int tA0 = 0, nA = ntiles, tB0 = 0, nB = 0;
  if constexpr (WIN) {
    const int q1 = rows_end;
    const int cap = CAUSAL ? q1 - 1 : 0x7fffffff;                 // last key position any row may see
    const int wlo = q0 - wl <= kv_start ? 0 : q0 - wl - kv_start;
    const int whi = min(Skv - 1, min(q1 - 1 + wr, cap) - kv_start);
    const int shi = min(Skv - 1, min(sink - 1, cap) - kv_start);
    const int b0 = wlo / kBN, b1 = whi >= wlo ? whi / kBN + 1 : b0;  // window tiles [b0, b1)
    const int a1 = shi >= 0 ? shi / kBN + 1 : 0;                      // sink tiles [0, a1)
    if (a1 == 0) { tA0 = b0; nA = b1 - b0; }
    else if (b1 > b0 && b0 <= a1) { tA0 = 0; nA = max(a1, b1); }
    else { tA0 = 0; nA = a1; tB0 = b0; nB = b1 - b0; }
  }
  const int ntot = nA + nB;
  auto tile_of = [&](int u) __attribute__((always_inline)) { return u < nA ? tA0 + u : tB0 + (u - nA); };

  // Q fragments (B operand of S^T = K Q^T); rows >= Sq read as zero.
  bf16x8 qf16[FP8 ? 1 : D / 16];
  i32x8 qf8[FP8 ? D / 64 : 1];
  if constexpr (!FP8) {
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc) {
      u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rq, qi * ROWB + (16 * dc + 8 * g) * 2, 0, 0);
      qf16[dc] = __builtin_bit_cast(bf16x8, x);
    }
  } else {
#pragma unroll
    for (int dc = 0; dc < D / 64; ++dc) {
      u32x4 x0 = __builtin_amdgcn_raw_buffer_load_b128(rq, qi * ROWB + 64 * dc + 32 * g, 0, 0);
      u32x4 x1 = __builtin_amdgcn_raw_buffer_load_b128(rq, qi * ROWB + 64 * dc + 32 * g + 16, 0, 0);
      qf8[dc] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                      (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
    }
  }

  // Q has landed before any copy is queued behind it: the compiler's own
  // memory-counter waits for Q then never wait for the copies.
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)

  // Clear the ring once, so that tail rows never expose uninitialised LDS.
  for (int i = threadIdx.x; i < kStages * 2 * T::BYTES / 16; i += kThr)
    *(LDS_AS u32x4*)(smem + i * 16) = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();

  // Global -> LDS for tile t into slot t % kStages: the 2*NINSTR 1-KB pieces
  // (K first, then V) are split evenly, piece w*PW .. w*PW+PW-1 to wave w. LDS
  // is written lane-linearly, so the swizzle is applied to the global address
  // each lane fetches.
  constexpr int PW = 2 * T::NINSTR / kW;   // pieces per wave per tile
  static_assert(PW >= 1 && PW * kW == 2 * T::NINSTR, "tile pieces must split evenly over waves");
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  // The K and V buffer descriptors, made wave-uniform once here: lane reads
  // are convergent operations, which the compiler keeps inside the loop.
  const i32x4 rkw = i32x4{__builtin_amdgcn_readfirstlane(rk[0]), __builtin_amdgcn_readfirstlane(rk[1]),
                          __builtin_amdgcn_readfirstlane(rk[2]), __builtin_amdgcn_readfirstlane(rk[3])};
  const i32x4 rvw = i32x4{__builtin_amdgcn_readfirstlane(rv[0]), __builtin_amdgcn_readfirstlane(rv[1]),
                          __builtin_amdgcn_readfirstlane(rv[2]), __builtin_amdgcn_readfirstlane(rv[3])};
  auto issue = [&](int u) __attribute__((always_inline)) {
    const int key0 = tile_of(u) * kBN;
    const int slot = u % kStages;
#pragma unroll
    for (int j = 0; j < PW; ++j) {
      const int ins = wv * PW + j;
      const bool isv = ins >= T::NINSTR;
      const int c0 = (isv ? ins - T::NINSTR : ins) * 64;
      const int cidx = c0 + lane;
      const int r = cidx / T::CH, pc = cidx % T::CH;
      const int lc = pc ^ (isv ? T::vswz(r) : T::kswz(r));
      const int goff = (key0 + r) * ROWB + lc * 16;
      const unsigned dst = __builtin_amdgcn_readfirstlane(smem_addr + (slot * 2 + (isv ? 1 : 0)) * T::BYTES + c0 * 16);
      dma16(isv ? rvw : rkw, goff, dst);
    }
  };

  f32x16 o[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) o[i] = f32x16{};
  // l, the lane's share of the row sum, gathers one fp32 partial per tile in
  // fp64: once m has reached a dominant key, the remaining tiles each add about
  // one fp32 ulp of l, and over 10^5 tiles those roundings would bias l.
  float m = -INFINITY;
  double l = 0.0;

  // Per-lane constant parts of the LDS operand addresses.
  // K operand (A of S^T): row 32*kb + n, logical chunk per dc.
  const int krow = n;
  // V operand (A of O^T), transposing reads.
  const int l16 = lane & 15, dgrp = (lane >> 4) & 1;

  // Tiles 0 .. kStages-2 in flight before the loop; iteration t waits for its
  // own copies of tile t (the copies of later tiles may still be in flight),
  // then the barrier publishes tile t and retires slot (t-1) % kStages, which
  // is refilled with tile t + kStages - 1.
#pragma unroll
  for (int u = 0; u < kStages - 1; ++u)
    if (u < ntot) issue(u);
  // Tile u of the sequence: wait for this wave's copies of it, barrier, queue
  // tile u + kStages - 1 into the slot every wave is done with.
  auto sync = [&](int u) __attribute__((always_inline)) {
    if (u + 2 < ntot) wait_vmcnt<2 * PW>();
    else if (u + 1 < ntot) wait_vmcnt<PW>();
    else wait_vmcnt<0>();
    __syncthreads();
    if (u + kStages - 1 < ntot) issue(u + kStages - 1);
  };
  [[maybe_unused]] int pkeep[kBN / 64][8] = {};   // fp8: last P words, reused as conversion targets
  constexpr std::integral_constant<int, -1> kAnySlot{};
  // The tile's scores, softmax and P V for this wave. Masked tiles take the
  // element mask; the others are compiled without it, so no mask work is ever
  // speculated on them.
  // slot_c: the tile's ring slot as a compile-time constant (its LDS operand
  // reads then take immediate offsets), or kAnySlot for u % kStages.
  auto step = [&](int u, auto masked_c, auto slot_c) __attribute__((always_inline)) {
    const int t = tile_of(u);
    constexpr int kSlot = decltype(slot_c)::value;
    const int slot = kSlot >= 0 ? kSlot : u % kStages;
    const LDS_AS char* ks = smem + (slot * 2 + 0) * T::BYTES;
    const LDS_AS char* vs = smem + (slot * 2 + 1) * T::BYTES;

    // ---- S^T = K Q^T ----
    f32x16 s[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      s[kb] = f32x16{};
      const int r = 32 * kb + krow;
      const LDS_AS char* krowp = ks + r * ROWB;
      if constexpr (!FP8) {
#pragma unroll
        for (int dc = 0; dc < D / 16; ++dc) {
          const int lc = 2 * dc + g;
          const bf16x8 kf = *(const LDS_AS bf16x8*)(krowp + ((lc ^ T::kswz(r)) * 16));
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf16[dc], s[kb], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int dc = 0; dc < D / 64; ++dc) {
          const int lc = 4 * dc + 2 * g;
          const i32x4 k0 = *(const LDS_AS i32x4*)(krowp + ((lc ^ T::kswz(r)) * 16));
          const i32x4 k1 = *(const LDS_AS i32x4*)(krowp + (((lc + 1) ^ T::kswz(r)) * 16));
          const i32x8 kf = i32x8{k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]};
          s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf, qf8[dc], s[kb], 0, 0, 0, 127, 0, 127);
        }
      }
    }

    // ---- mask: keys past Skv, and (causal) keys after the query ----
    if constexpr (decltype(masked_c)::value) {
      const int key0 = t * kBN;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + 32 * kb + 8 * (i >> 2) + 4 * g + (i & 3);
          const int kp = key + kv_start;
          bool ok = key < Skv && (!CAUSAL || kp <= qi);
          if constexpr (WIN) ok = ok && ((kp >= qi - wl && kp <= qi + wr) || kp < sink);
          s[kb][i] = ok ? s[kb][i] : -INFINITY;
        }
    }

    // ---- online softmax (base 2) with a checked running max. p = exp2(c s - m)
    // is formed with the current m; while every p of the tile stays at most
    // 2^8 (a lane's partial row sum bounds its p) m is good enough and no row
    // max is needed. Otherwise (or while m is still -inf) m becomes the exact
    // running max, O and l are rescaled, and p is formed again.
    f32x16 sraw[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) sraw[kb] = s[kb];
    float moff = kPre - (m == -INFINITY ? 0.f : m);
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i], c, moff));
        s[kb][i] = pv;
        rs += pv;
      }
    if (__any(m == -INFINITY || !(rs <= 256.f))) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sraw[kb][i]);
      const float mnew = fmaxf(m, xor32_max(mx) * c);
      const float alpha = mnew > m ? __builtin_amdgcn_exp2f(m - mnew) : 1.f;   // 0 when m was -inf
      l *= (double)alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db] *= alpha;
      m = mnew;
      moff = kPre - (m == -INFINITY ? 0.f : m);
      rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sraw[kb][i], c, moff));
          s[kb][i] = pv;
          rs += pv;
        }
    }
    l += (double)rs;

    // ---- O^T += V^T P^T ----
    if constexpr (!FP8) {
      const int rr = l16 >> 2, ss = l16 & 3;
#pragma unroll
      for (int kg = 0; kg < kBN / 16; ++kg) {  // 16-key groups
        const int kb = kg >> 1, half = kg & 1;
        bf16x8 pf;
        {
          const u32x4 pk = u32x4{pack_bf16(s[kb][8 * half + 0], s[kb][8 * half + 1]),
                                 pack_bf16(s[kb][8 * half + 2], s[kb][8 * half + 3]),
                                 pack_bf16(s[kb][8 * half + 4], s[kb][8 * half + 5]),
                                 pack_bf16(s[kb][8 * half + 6], s[kb][8 * half + 7])};
          pf = __builtin_bit_cast(bf16x8, pk);
        }
        const int key1 = 32 * kb + 16 * half + 4 * g + rr;   // keys key1, key1+8
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int col = 32 * db + 16 * dgrp + 4 * ss;
          const int lc = col >> 3, hb = (col & 7) * 2;
          const LDS_AS char* a1 = vs + key1 * ROWB + ((lc ^ T::vswz(key1)) * 16) + hb;
          const LDS_AS char* a2 = vs + (key1 + 8) * ROWB + ((lc ^ T::vswz(key1 + 8)) * 16) + hb;
          const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)a1);
          const i16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)a2);
          const i16x8 vv = i16x8{v1[0], v1[1], v1[2], v1[3], v2[0], v2[1], v2[2], v2[3]};
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv), pf, o[db], 0, 0, 0);
        }
      }
    } else {
      const int rr = l16 >> 1, hh = l16 & 1;
#pragma unroll
      for (int kq = 0; kq < kBN / 64; ++kq) {  // 64-key groups (one fp8 MFMA deep)
        int pw[8];
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          const int j = 4 * w, kb = 2 * kq + (j >> 4), i = j & 15;
          // the first conversion writes the low half-word only; the previous
          // tile's word is passed as the high half (overwritten next) so that no
          // register has to be cleared for it
          int x = __builtin_amdgcn_cvt_pk_fp8_f32(s[kb][i], s[kb][i + 1], pkeep[kq][w], false);
          x = __builtin_amdgcn_cvt_pk_fp8_f32(s[kb][i + 2], s[kb][i + 3], x, true);
          pw[w] = x;
          pkeep[kq][w] = x;
        }
        const i32x8 pf = i32x8{pw[0], pw[1], pw[2], pw[3], pw[4], pw[5], pw[6], pw[7]};
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int lc = 2 * db + dgrp;
          int vw[8];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int key = 64 * kq + 32 * (u >> 1) + 16 * (u & 1) + 8 * (rr >> 2) + 4 * g + (rr & 3);
            const LDS_AS char* a = vs + key * ROWB + ((lc ^ T::vswz(key)) * 16) + 8 * hh;
            const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS i32x2*)a);
            vw[2 * u] = x[0];
            vw[2 * u + 1] = x[1];
          }
          const i32x8 vf = i32x8{vw[0], vw[1], vw[2], vw[3], vw[4], vw[5], vw[6], vw[7]};
          o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pf, o[db], 0, 0, 0, 127, 0, 127);
        }
      }
    }
  };
  if constexpr (!WIN) {
    const int first_masked = CAUSAL ? min(Skv / kBN, max(0, qw - kv_start + 1) / kBN) : Skv / kBN;
    const int n_plain = min(first_masked, ntot);
    int u = 0;
    if constexpr (FP8) {
      // fp8: the unmasked tiles in groups of kStages, each with its ring slot
      // as a compile-time constant, so that the LDS operand reads take their
      // slot as an immediate offset and no per-tile address arithmetic is left
      // in this VALU-bound loop (about 2 % faster; the bf16 loop is not limited
      // by it, and its slots lie beyond the reads' immediate-offset range).
      static_assert(kStages == 4, "the unrolled fp8 loop assumes a ring of four slots");
      for (; u + kStages <= n_plain; u += kStages) {
        auto one = [&](auto slot_c) __attribute__((always_inline)) {
          const int uu = u + decltype(slot_c)::value;
          sync(uu);
          if (uu < w_ntiles) step(uu, std::false_type{}, slot_c);
        };
        one(std::integral_constant<int, 0>{});
        one(std::integral_constant<int, 1>{});
        one(std::integral_constant<int, 2>{});
        one(std::integral_constant<int, 3>{});
      }
    }
    for (; u < n_plain; ++u) {
      sync(u);
      if (u < w_ntiles) step(u, std::false_type{}, kAnySlot);
    }
    for (; u < ntot; ++u) {
      sync(u);
      if (u < w_ntiles) step(u, std::true_type{}, kAnySlot);
    }
  } else {
    // Per tile and wave: skip it (no key of it is allowed for any of the
    // wave's rows), take it whole, or mask it. The whole tiles of a wave form
    // at most two runs of the tile sequence (inside the sink keys; inside
    // every row's window), which get a loop of their own without mask code;
    // the tiles around them are skipped or masked (the masked step gives a
    // whole tile the same bits, and one step variant per loop keeps these
    // loops' register pressure down).
    const int r_lo = qw, r_hi = min(qw + 31, p.Sq - 1);
    const int cap = CAUSAL ? r_hi : 0x7fffffff;
    auto general = [&](int u) __attribute__((always_inline)) {
      sync(u);
      if (!wave_live) return;
      const int t = tile_of(u);
      const int k_lo = t * kBN + kv_start, k_hi = k_lo + kBN - 1;
      const bool any = t * kBN < Skv && ((k_hi >= r_lo - wl && k_lo <= min(r_hi + wr, cap)) || (k_lo < sink && k_lo <= cap));
      if (!any) return;
      step(u, std::true_type{}, kAnySlot);
    };
    // First position in the sequence whose tile index is >= x.
    auto seq_lb = [&](int x) __attribute__((always_inline)) {
      if (x <= tA0) return 0;
      if (x < tA0 + nA) return x - tA0;
      if (nB == 0 || x <= tB0) return nA;
      if (x < tB0 + nB) return nA + x - tB0;
      return ntot;
    };
    auto fdiv = [](int a) { return a >= 0 ? a / kBN : -((-a + kBN - 1) / kBN); };   // floor(a / kBN)
    const int t_full = Skv / kBN - 1;                            // last tile with no key past Skv
    const int hi_lim = CAUSAL ? r_lo : min(r_lo + wr, 0x3fffffff);
    const int ts_hi = min(t_full, fdiv(min(sink - 1, CAUSAL ? r_lo : 0x3fffffff) - kv_start - (kBN - 1)));
    const int tw_lo = max(0, -fdiv(-(r_hi - wl - kv_start)));    // ceil
    const int tw_hi = min(t_full, fdiv(hi_lim - kv_start - (kBN - 1)));
    int us0 = 0, us1 = 0, uw0 = 0, uw1 = 0;
    if (wave_live) {
      if (ts_hi >= 0) us1 = seq_lb(ts_hi + 1);
      if (tw_hi >= tw_lo) {
        uw0 = seq_lb(tw_lo);
        uw1 = seq_lb(tw_hi + 1);
      }
      if (uw1 <= uw0) uw0 = uw1 = us1;                           // no window run
      if (uw0 <= us1) {                                           // the runs touch: one run
        us1 = max(us1, uw1);
        uw0 = uw1 = us1;
      }
    }
    int u = 0;
    for (; u < us0; ++u) general(u);
    for (; u < us1; ++u) {
      sync(u);
      step(u, std::false_type{}, kAnySlot);
    }
    for (; u < uw0; ++u) general(u);
    for (; u < uw1; ++u) {
      sync(u);
      step(u, std::false_type{}, kAnySlot);
    }
    for (; u < ntot; ++u) general(u);
  }


  // ---- epilogue: O = O_acc * oscale / l (bf16), LSE = ln2 * (m + log2 l) ----
  if (!wave_live) return;
  const int qi_full = qi;
  const float ltot = xor32_sum((float)l);
  const float inv = ltot > 0.f ? oscale / ltot : 0.f;
  const float lse = ltot > 0.f ? (m + __log2f(ltot) - kPre) * 0.69314718055994531f : -INFINITY;
  if (p.o32 == nullptr || split < 0) {
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(p.o + qrow0 * (size_t)(D * 2), (uint32_t)p.Sq * D * 2);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const u32x2 w = u32x2{pack_bf16(o[db][4 * ii + 0] * inv, o[db][4 * ii + 1] * inv),
                              pack_bf16(o[db][4 * ii + 2] * inv, o[db][4 * ii + 3] * inv)};
        const int col = 32 * db + 8 * ii + 4 * g;
        __builtin_amdgcn_raw_buffer_store_b64(w, ro, (qi * D + col) * 2, 0, 0);
      }
    if (g == 0) {
      const __amdgpu_buffer_rsrc_t rl = make_rsrc(p.lse + qrow0, (uint32_t)p.Sq * 4);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse), rl, qi * 4, 0, 0);
    }
  } else {
    // one key split: normalised fp32 O and the split's LSE, for the merge kernel;
    // rows of this tile from its first row q0 (rows >= Sq fall outside the range)
    const size_t prow0 = (size_t)split * (size_t)p.part_rows + (qrow0 + (size_t)q0 - (size_t)p.part_row0);
    const int qi = qi_full - q0;
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(p.o32 + prow0 * D, (uint32_t)(p.Sq - q0) * D * 4);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const u32x4 w = u32x4{__float_as_uint(o[db][4 * ii + 0] * inv), __float_as_uint(o[db][4 * ii + 1] * inv),
                              __float_as_uint(o[db][4 * ii + 2] * inv), __float_as_uint(o[db][4 * ii + 3] * inv)};
        const int col = 32 * db + 8 * ii + 4 * g;
        __builtin_amdgcn_raw_buffer_store_b128(w, ro, (qi * D + col) * 4, 0, 0);
      }
    if (g == 0) {
      const __amdgpu_buffer_rsrc_t rl = make_rsrc(p.lse32 + prow0, (uint32_t)(p.Sq - q0) * 4);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse), rl, qi * 4, 0, 0);
    }
  }
}

// Merge of the key splits of attn_fwd_splitkv: for each row, L = ln sum_s
// e^(L_s) and O = sum_s e^(L_s - L) O_s (fp32, bf16 out); rows whose splits
// are all empty (L_s = -inf) get O = 0 and L = -inf. Sixteen lanes per row,
// eight columns each (D = 128) or four (D = 64).
template <int D>
__global__ void __launch_bounds__(256) merge_splits_kernel(const float* __restrict__ o32, const float* __restrict__ lse32,
                                                           char* __restrict__ out, float* __restrict__ lse,
                                                           long long rows, int nsplit) {
  constexpr int PER = D / 16;                    // columns per lane
  const long long row = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int part = threadIdx.x & 15;
  if (row >= rows) return;
  float mx = -INFINITY;
  for (int sp = 0; sp < nsplit; ++sp) mx = fmaxf(mx, lse32[(long long)sp * rows + row]);
  float acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = 0.f;
  float tot = 0.f;
  if (mx != -INFINITY) {
    constexpr float kLog2e = 1.4426950408889634f;
    for (int sp = 0; sp < nsplit; ++sp) {
      const float w = __builtin_amdgcn_exp2f((lse32[(long long)sp * rows + row] - mx) * kLog2e);   // 0 for an empty split
      tot += w;
      const float* src = o32 + ((long long)sp * rows + row) * D + part * PER;
#pragma unroll
      for (int j = 0; j < PER; j += 4) {
        const f32x4 x = *(const f32x4*)(src + j);
        acc[j] += w * x[0];
        acc[j + 1] += w * x[1];
        acc[j + 2] += w * x[2];
        acc[j + 3] += w * x[3];
      }
    }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  unsigned pk[PER / 2];
#pragma unroll
  for (int j = 0; j < PER / 2; ++j) pk[j] = pack_bf16(acc[2 * j] * inv, acc[2 * j + 1] * inv);
  if constexpr (PER == 8)
    *(u32x4*)(out + (row * D + part * PER) * 2) = u32x4{pk[0], pk[1], pk[2], pk[3]};
  else
    *(u32x2*)(out + (row * D + part * PER) * 2) = u32x2{pk[0], pk[1]};
  if (part == 0) lse[row] = tot > 0.f ? mx + __logf(tot) : -INFINITY;
}

typedef void (*kernel_fn)(Params);

template <int D, bool FP8, int NW>
kernel_fn pick_nw(bool causal, bool win) {
  if (win) return causal ? attn_fwd_kernel<D, true, FP8, true, NW> : attn_fwd_kernel<D, false, FP8, true, NW>;
  return causal ? attn_fwd_kernel<D, true, FP8, false, NW> : attn_fwd_kernel<D, false, FP8, false, NW>;
}

template <int D, bool FP8>
kernel_fn pick(bool causal, bool win, int nw) {
  return nw == 4 ? pick_nw<D, FP8, 4>(causal, win) : pick_nw<D, FP8, 8>(causal, win);
}

}  // namespace hat

using namespace hat;

static constexpr int64_t kMaxSplits = 256;

// Compute units of the current device (queried once per device).
static int device_cus() {
  static int cache[64] = {0};
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64 && cache[dev] > 0) return cache[dev];
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (dev < 64) cache[dev] = cus;
  return cus;
}

static int64_t splitkv_bytes(int64_t B, int64_t Hq, int64_t Sq, int64_t D, int64_t nsplit) {
  return nsplit <= 1 ? 0 : nsplit * B * Hq * Sq * (D + 1) * 4;
}

static attn_status_t launch(const void* q, const void* k, const void* v, void* out, float* lse,
                            int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Skv, int64_t D,
                            float scale, int causal, attn_dtype_t dtype,
                            const float* qd, const float* kd, const float* vd, int64_t kv_start,
                            int64_t nsplit, void* workspace, int64_t workspace_bytes, void* stream,
                            int64_t window_left = -1, int64_t window_right = -1, int64_t sink = 0,
                            bool tail_only = false) {
  if (dtype != ATTN_BF16 && dtype != ATTN_FP8_E4M3FN) return ATTN_ERR_DTYPE;
  if (D != 64 && D != 128) return ATTN_ERR_HEAD_DIM;
  if (B < 0 || Hq < 0 || Hkv < 0 || Sq < 0 || Skv < 0 || kv_start < 0) return ATTN_ERR_SHAPE;
  if (window_left < -1 || window_right < -1 || sink < 0) return ATTN_ERR_SHAPE;
  if (Hq > 0 && (Hkv == 0 || Hq % Hkv != 0)) return ATTN_ERR_SHAPE;
  if (!(scale > 0.f) || !isfinite(scale)) return ATTN_ERR_SCALE;
  const int64_t elt = dtype == ATTN_BF16 ? 2 : 1;
  const int64_t rowb = D * elt;
  const bool any_q = B > 0 && Hq > 0 && Sq > 0;
  const bool any_kv = B > 0 && Hkv > 0 && Skv > 0;
  if (!any_q) return ATTN_OK;  // nothing to compute
  if (!q || !out || !lse) return ATTN_ERR_NULL;
  if (any_kv && (!k || !v)) return ATTN_ERR_NULL;
  if (((uintptr_t)q | (uintptr_t)out | (uintptr_t)k | (uintptr_t)v) & 15) return ATTN_ERR_ALIGN;
  if ((uintptr_t)lse & 3) return ATTN_ERR_ALIGN;
  // Per-head slices are addressed with 32-bit offsets (plus one tile of slack).
  const int64_t lim = (int64_t)1 << 31;
  if ((Sq + kBM) * D * 2 >= lim || (Skv + kBN) * rowb >= lim || Sq + kBM >= lim) return ATTN_ERR_OVERFLOW;
  // Key positions stay below 2^30, so position arithmetic (with the unbounded
  // window sides held as 2^30) never leaves int range.
  if (kv_start + Skv + kBN >= ((int64_t)1 << 30)) return ATTN_ERR_OVERFLOW;
  if (nsplit < 1 || nsplit > kMaxSplits) return ATTN_ERR_SHAPE;
  // Key splits are whole tiles; fewer tiles than splits leaves fewer splits.
  const int64_t ktiles = any_kv ? (Skv + kBN - 1) / kBN : 0;
  const int64_t per = ktiles > 0 ? (ktiles + nsplit - 1) / nsplit : 1;
  const int64_t nsp = ktiles > 0 ? (ktiles + per - 1) / per : 1;
  const bool win = window_left >= 0 || window_right >= 0 || sink > 0;
  // Tail mode: only the query tiles of the grid's last, partly filled round of
  // workgroups are split (non-causal, no window).
  const bool tail = tail_only && nsp > 1 && !causal && !win;
  // Workgroups of 8 waves (256 query rows); 4 waves (128 rows) when an unsplit
  // grid of 256-row tiles fills at most half the CUs, so that the doubled grid
  // of half-size workgroups still runs in one round.
  const int nw = nsp == 1 && 2 * B * Hq * ((Sq + kBM - 1) / kBM) <= (int64_t)device_cus() ? 4 : 8;
  const int64_t n_qtiles = (Sq + 32 * nw - 1) / (32 * nw);
  const int64_t rows = B * Hq * Sq;
  const int64_t ntiles = B * Hq * n_qtiles;
  int64_t n_full = -1, part_rows = rows, part_row0 = 0, grid = ntiles * nsp;
  if (tail) {
    const int64_t cus = device_cus();
    n_full = ntiles / cus * cus;
    if (n_full == 0 || n_full == ntiles) return ATTN_ERR_SHAPE;
    part_row0 = (n_full / n_qtiles) * Sq + (n_full % n_qtiles) * (32 * nw);
    part_rows = rows - part_row0;
    grid = n_full + (ntiles - n_full) * nsp;
  }
  if (nsp > 1) {
    if (!workspace) return ATTN_ERR_WORKSPACE;
    if ((uintptr_t)workspace & 15) return ATTN_ERR_WORKSPACE;
    if (workspace_bytes < nsp * part_rows * (D + 1) * 4) return ATTN_ERR_WORKSPACE;
    if ((Sq + kBM) * D * 4 >= lim) return ATTN_ERR_OVERFLOW;
  }
  if (B * Hq >= lim || grid >= lim || (rows + 16) / 16 >= lim) return ATTN_ERR_OVERFLOW;

  Params p;
  p.q = (const char*)q;
  p.k = (const char*)k;
  p.v = (const char*)v;
  p.o = (char*)out;
  p.lse = lse;
  p.B = (int)B;
  p.Hq = (int)Hq;
  p.Hkv = (int)Hkv;
  p.Sq = (int)Sq;
  p.Skv = any_kv ? (int)Skv : 0;
  p.group = (int)(Hq / Hkv);
  p.n_qtiles = (int)n_qtiles;
  p.kv_start = (int)kv_start;
  p.c = scale * 1.4426950408889634f;
  p.qd = dtype == ATTN_FP8_E4M3FN ? qd : nullptr;
  p.kd = dtype == ATTN_FP8_E4M3FN ? kd : nullptr;
  p.vd = dtype == ATTN_FP8_E4M3FN ? vd : nullptr;
  p.nsplit = (int)nsp;
  p.split_len = nsp > 1 ? (int)(per * kBN) : (int)Skv;
  p.o32 = nsp > 1 ? (float*)workspace : nullptr;
  p.lse32 = nsp > 1 ? (float*)workspace + nsp * part_rows * D : nullptr;
  p.n_full = (int)n_full;
  p.part_rows = (int)part_rows;
  p.part_row0 = (int)part_row0;
  constexpr int64_t kUnbounded = (int64_t)1 << 30;
  p.wl = (int)(window_left < 0 ? kUnbounded : std::min(window_left, kUnbounded));
  p.wr = (int)(window_right < 0 ? kUnbounded : std::min(window_right, kUnbounded));
  p.sink = (int)std::min(sink, kUnbounded);

  kernel_fn fn;
  if (dtype == ATTN_BF16) fn = D == 128 ? pick<128, false>(causal, win, nw) : pick<64, false>(causal, win, nw);
  else fn = D == 128 ? pick<128, true>(causal, win, nw) : pick<64, true>(causal, win, nw);
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(64 * nw), 0, (hipStream_t)stream, p);
  if (hipGetLastError() != hipSuccess) return ATTN_ERR_HIP;
  if (nsp > 1) {
    const unsigned mgrid = (unsigned)((part_rows + 15) / 16);
    char* out_part = (char*)out + part_row0 * D * 2;
    float* lse_part = lse + part_row0;
    if (D == 128)
      hipLaunchKernelGGL(merge_splits_kernel<128>, dim3(mgrid), dim3(256), 0, (hipStream_t)stream,
                         p.o32, p.lse32, out_part, lse_part, (long long)part_rows, (int)nsp);
    else
      hipLaunchKernelGGL(merge_splits_kernel<64>, dim3(mgrid), dim3(256), 0, (hipStream_t)stream,
                         p.o32, p.lse32, out_part, lse_part, (long long)part_rows, (int)nsp);
    if (hipGetLastError() != hipSuccess) return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

// Key splits for a grid that leaves compute units idle: none when the query
// tiles already occupy at least 85 % of the last round of workgroups (the
// chip is power-bound, so idle CUs cost little); else the fewest splits, each
// of at least 16 key tiles, that bring the rounds to 90 % occupancy (merge
// traffic and per-workgroup start-up grow with the split count). A grid of
// less than one round that 16 splits cannot bring to 90 % (a few query tiles
// against many keys) takes the count up to kMaxSplits with the least
// estimated time, rounds * (key tiles per split + 2 tiles of workgroup
// start-up) + 3 tiles for the merge launch, or the fewest within 3 % of it.
// (A grid of one round or more is left to tail_splits.)
static int64_t auto_full_splits(int64_t B, int64_t Hq, int64_t Sq, int64_t Skv) {
  const int64_t cus = device_cus();
  const int64_t nwg = B * Hq * ((Sq + kBM - 1) / kBM);
  const int64_t ktiles = (Skv + kBN - 1) / kBN;
  auto occupancy = [&](int64_t sp) {
    const int64_t w = nwg * sp;
    return (double)w / (double)(cus * ((w + cus - 1) / cus));
  };
  if (nwg <= 0 || ktiles <= 0 || occupancy(1) >= 0.85) return 1;
  for (int64_t sp = 2; sp <= 16 && ktiles / sp >= 16; ++sp)
    if (occupancy(sp) >= 0.9) return sp;
  if (nwg >= cus) return 1;
  const int64_t maxsp = std::min<int64_t>(kMaxSplits, ktiles / 16);
  auto cost = [&](int64_t sp) {
    return (double)((nwg * sp + cus - 1) / cus) * (double)((ktiles + sp - 1) / sp + 2) + (sp > 1 ? 3.0 : 0.0);
  };
  double best = cost(1);
  for (int64_t sp = 2; sp <= maxsp; ++sp) best = std::min(best, cost(sp));
  for (int64_t sp = 1; sp <= maxsp; ++sp)
    if (cost(sp) <= 1.03 * best) return sp;
  return 1;
}

// Tail splits: when whole rounds of 256-row query tiles fill every CU and a
// last round is left partly empty, split only that round's tiles into k key
// ranges, k in 2..8 (each at least 16 key tiles), so that the k-times more,
// k-times shorter workgroups finish sooner than one more whole round: the k
// minimising ceil(tail * k / CUs) / k, if that is at most 0.85 of a round.
// Returns 0 when no such k exists.
static int64_t tail_splits(int64_t B, int64_t Hq, int64_t Sq, int64_t Skv) {
  const int64_t cus = device_cus();
  const int64_t ntiles = B * Hq * ((Sq + kBM - 1) / kBM);
  const int64_t ntail = ntiles % cus;
  if (ntiles < cus || ntail == 0) return 0;
  const int64_t ktiles = (Skv + kBN - 1) / kBN;
  int64_t best = 0;
  double best_t = 0.85 + 1e-9;
  for (int64_t k = 2; k <= 8 && ktiles / k >= 16; ++k) {
    const double t = (double)((ntail * k + cus - 1) / cus) / (double)k;
    if (t < best_t - 1e-9) {
      best = k;
      best_t = t;
    }
  }
  return best;
}

// The split count attn_fwd_splitkv uses for n_splits = 0: the whole-grid split
// when one helps, else a tail split (non-causal calls only), else 1.
static int64_t auto_splits(int64_t B, int64_t Hq, int64_t Sq, int64_t Skv) {
  const int64_t f = auto_full_splits(B, Hq, Sq, Skv);
  if (f > 1) return f;
  const int64_t t = tail_splits(B, Hq, Sq, Skv);
  return t >= 2 ? t : 1;
}

extern "C" attn_status_t attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                                  int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Skv, int64_t D,
                                  float scale, int causal, attn_dtype_t dtype,
                                  const float* q_descale, const float* k_descale, const float* v_descale,
                                  void* stream) {
  return launch(q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, scale, causal, dtype, q_descale, k_descale,
                v_descale, 0, 1, nullptr, 0, stream);
}

extern "C" attn_status_t attn_fwd_chunk(const void* q, const void* k, const void* v, void* out, float* lse,
                                        int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Skv, int64_t D,
                                        float scale, int causal, attn_dtype_t dtype,
                                        const float* q_descale, const float* k_descale,
                                        const float* v_descale, int64_t kv_start, void* stream) {
  return launch(q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, scale, causal, dtype, q_descale, k_descale,
                v_descale, kv_start, 1, nullptr, 0, stream);
}

extern "C" attn_status_t attn_fwd_window(const void* q, const void* k, const void* v, void* out, float* lse,
                                         int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Skv, int64_t D,
                                         float scale, int causal, attn_dtype_t dtype,
                                         const float* q_descale, const float* k_descale, const float* v_descale,
                                         int64_t kv_start, int64_t window_left, int64_t window_right, int64_t sink,
                                         void* stream) {
  return launch(q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, scale, causal, dtype, q_descale, k_descale,
                v_descale, kv_start, 1, nullptr, 0, stream, window_left, window_right, sink);
}

extern "C" int64_t attn_splitkv_auto_splits(int64_t B, int64_t Hq, int64_t Sq, int64_t Skv, int64_t D) {
  if (B < 0 || Hq < 0 || Sq < 0 || Skv < 0 || (D != 64 && D != 128)) return -1;
  return auto_splits(B, Hq, Sq, Skv);
}

extern "C" int64_t attn_splitkv_workspace_bytes(int64_t B, int64_t Hq, int64_t Sq, int64_t D, int64_t n_splits) {
  if (B < 0 || Hq < 0 || Sq < 0 || (D != 64 && D != 128) || n_splits < 0 || n_splits > kMaxSplits) return -1;
  return splitkv_bytes(B, Hq, Sq, D, n_splits);
}

extern "C" attn_status_t attn_fwd_splitkv(const void* q, const void* k, const void* v, void* out, float* lse,
                                          int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Skv, int64_t D,
                                          float scale, int causal, attn_dtype_t dtype,
                                          const float* q_descale, const float* k_descale, const float* v_descale,
                                          int64_t n_splits, void* workspace, int64_t workspace_bytes, void* stream) {
  if (n_splits < 0) return ATTN_ERR_SHAPE;
  bool tail_only = false;
  if (n_splits == 0) {
    n_splits = 1;
    if (B > 0 && Hq > 0 && Sq > 0 && Skv > 0) {
      n_splits = auto_full_splits(B, Hq, Sq, Skv);
      if (n_splits <= 1 && !causal) {
        const int64_t t = tail_splits(B, Hq, Sq, Skv);
        if (t >= 2) {
          n_splits = t;
          tail_only = true;
        }
      }
    }
  }
  return launch(q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, scale, causal, dtype, q_descale, k_descale,
                v_descale, 0, n_splits, workspace, workspace_bytes, stream, -1, -1, 0, tail_only);
}
