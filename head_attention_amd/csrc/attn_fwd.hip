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
//    A grid small enough to leave half the CUs idle uses workgroups of 128
//    rows instead, twice as many of them: for bf16 without a window 8
//    wavefronts in which two share each 32 rows and take alternate key tiles
//    (merged through LDS at the end), otherwise 4 wavefronts.
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
//    cross its diagonal. Causal grids run the longest query tiles first; a
//    causal grid of key-split workgroups (one round) pairs an early and a late
//    64-row block in each workgroup instead, so that all take about as long.
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
#include <mutex>

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

// The fp8 product of the page "F8 fmha ASM gfx950" (Technical Details: the
// 32x32x64 fp8 MFMA for head dim 128): e4m3fn operands, fp32 accumulate, no
// block scales. The builtin is the scaled form; with both scale operands 0 and
// no op_sel the compiler emits the unscaled v_mfma_f32_32x32x64_f8f6f4, a
// shorter instruction that holds no VGPR for a scale (the scaled form with
// unit scales issued as the longer encoding and pinned a register to 127).
__device__ __forceinline__ f32x16 mfma_e4m3(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

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

template <int D, bool CAUSAL, bool FP8, bool WIN, int NW, int KS>
__global__ void __launch_bounds__(64 * NW) attn_fwd_kernel(const Params p) {
  constexpr int kW = NW;            // waves per workgroup (8, or 4 for grids that leave CUs idle)
  constexpr int kThr = 64 * NW;
  // KS (key split, bf16 without a window; 0 = none): KS waves own the same 32
  // rows and share its key tiles, two tiles per barrier step, and their (m,
  // l, O) are merged through LDS at the end. KS = 2: waves w and w + NW/2
  // (causal: 2r and 2r + 1) take alternate tiles. KS = 4: waves 2j + r (j =
  // 0..3) of row group r each take one 32-key half of one of the step's two
  // tiles (tile j / 2, half j % 2). A workgroup then covers 32 NW / KS rows
  // at two waves per SIMD, for grids too small to fill the CUs.
  static_assert(KS == 0 || KS == 2 || KS == 4, "key split factors 2 and 4");
  static_assert(!KS || (!FP8 && !WIN && NW == 8), "the key split is a bf16 8-wave mode");
  constexpr int kRG = KS ? NW / KS : NW;  // waves with distinct query rows
  constexpr int kRows = 32 * kRG;         // query rows per workgroup
  constexpr bool FOLD = KS == 2 && CAUSAL;   // folded causal grid (below)
  using T = Tile<D, FP8>;
  constexpr int ROWB = T::ROWB;
  constexpr int NDB = D / 32;                       // 32-wide output column blocks
  constexpr int NKB = kBN / 32;                     // 32-key blocks per tile
  constexpr float kPre = FP8 ? 4.f : 0.f;           // fp8: p carries a factor 2^kPre
  // The software-pipelined tile loop (fp8 head dim 128 without a window)
  // synchronises every kSync tiles, over rings of 2 kSync slots for K and V.
  constexpr bool PIPE = FP8 && !WIN && D == 128 && T::NINSTR % NW == 0;
  constexpr int kSync = 4;
  constexpr int kLds = PIPE ? 2 * (2 * kSync) * T::BYTES : kStages * 2 * T::BYTES;
  __shared__ __attribute__((aligned(1024))) char smem_raw[kLds];  // PIPE: [K ring][V ring]; else [slot][K, V]
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
    int gb = (int)blockIdx.x;
    if constexpr (!CAUSAL) {
      // Workgroups go to the eight XCDs round-robin (workgroup i to XCD i % 8)
      // and each XCD has an L2 of its own: give XCD x one contiguous range of
      // the grid's work instead, so that the workgroups an XCD runs at a time
      // share their key/value head. (Causal grids keep their longest-first
      // order, which balances them.)
      const int n = (int)gridDim.x, q8 = n >> 3, rem = n & 7, x = gb & 7, r = gb >> 3;
      gb = x < rem ? x * (q8 + 1) + r : rem * (q8 + 1) + (x - rem) * q8 + r;
    }
    split = gb / per_split;
    bid = gb % per_split;
  }
  int bh, qt;
  if (CAUSAL) {  // longest rows first (folded: the workgroups whose later block reaches furthest)
    qt = FOLD ? bid / BH : p.n_qtiles - 1 - bid / BH;
    // Within one query-tile row of the grid, workgroup r goes to XCD r % 8:
    // when the heads split evenly over the XCDs, give XCD x the contiguous
    // heads [x BH/8, (x+1) BH/8), which share key/value heads under grouped
    // heads (and the batch entry).
    const int r = bid % BH;
    bh = (BH & 7) == 0 ? (r & 7) * (BH >> 3) + (r >> 3) : r;
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
  // KS and causal: the grid is folded. Workgroup qt takes the 64-row blocks qt
  // (row groups 0, 1) and J-1-qt (row groups 2, 3) of the head's J blocks, so
  // that every workgroup holds about the same number of visible (query, key)
  // pairs and the grid's one round ends together instead of waiting on the
  // last rows' workgroup. The two key halves of a row group are waves 2r', 2r'+1
  // (r' = row group mod 2), so that waves w and w + 4, which share a SIMD, hold
  // one row group of each block. When J is odd the middle workgroup's second
  // block is its first, and row groups 2, 3 stay idle.
  const int rw = !KS ? wave : KS == 4 ? wave & 1 : FOLD ? ((wave >> 2) << 1) | ((wave >> 1) & 1) : wave % kRG;   // the wave's 32-row group
  // KS: its share of the keys, 0 .. KS-1 (KS = 2: tiles kh, kh + 2, ...)
  [[maybe_unused]] const int kh = !KS ? 0 : KS == 4 ? wave >> 1 : FOLD ? wave & 1 : wave / kRG;
  const int g = lane >> 5, n = lane & 31;
  const int nblk = (p.Sq + 63) >> 6;   // FOLD: the head's 64-row blocks
  const int q0 = FOLD ? 64 * (nblk - 1 - qt) : qt * kRows;   // FOLD: the second (later) block
  const int qw = FOLD ? 64 * (rw < 2 ? qt : nblk - 1 - qt) + 32 * (rw & 1) : q0 + rw * 32, qi = qw + n;
  const bool fold_dup = FOLD && rw >= 2 && nblk - 1 - qt == qt;

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
  // c is negative only through an fp8 descale of that sign; then the largest
  // c*s belongs to the smallest s, and a masked key holds +inf (c*s = -inf).
  const bool cneg = FP8 && c < 0.f;
  const float smask = cneg ? INFINITY : -INFINITY;

  // Key tiles this workgroup needs, and those this wave needs.
  const int rows_end = min(q0 + (FOLD ? 64 : kRows), p.Sq);
  const int kv_end = CAUSAL ? min(Skv, max(0, rows_end - kv_start)) : Skv;
  const int ntiles = (kv_end + kBN - 1) / kBN;
  const bool wave_live = qw < p.Sq && !fold_dup;
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

  // Wait for Q, then clear all of LDS once (both rings) when the last key
  // tile is ragged, so that its missing rows never expose uninitialised LDS.
  // With whole tiles only, every byte the loop reads is written by a tile
  // copy first, and the clear is skipped (the condition is the workgroup's
  // own). The wait is the compiler's own instruction, so its memory-counter
  // bookkeeping knows that Q has landed, and none of its later waits waits
  // for a copy queued behind Q.
  const bool ragged = Skv % kBN != 0;
  auto q_wait_and_clear = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    if (ragged)
      for (int i = threadIdx.x; i < kLds / 16; i += kThr)
        *(LDS_AS u32x4*)(smem + i * 16) = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
  };
  if constexpr (!KS) q_wait_and_clear();

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
  // The key-split loop waits for every copy in flight before its first tile
  // anyway: with whole tiles only (no clear), it queues its first two tiles
  // right behind the Q loads, and one wait covers both (a memory latency less
  // at each workgroup's start, which these one-round grids see whole). The
  // other loops first wait for tile 0 alone and queue their copies after Q
  // has landed (queued before, they made the many-round grids 2-4 % slower).
  if constexpr (KS) {
    auto first = [&]() __attribute__((always_inline)) {
      if (ntot > 0) issue(0);
      if (ntot > 1) issue(1);
    };
    if (!ragged) first();
    q_wait_and_clear();
    if (ragged) first();
  }

  f32x16 o[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) o[i] = f32x16{};
  // l, the lane's share of the row sum, gathers one fp32 partial per tile in
  // fp64: once m has reached a dominant key, the remaining tiles each add about
  // one fp32 ulp of l, and over 10^5 tiles those roundings would bias l.
  float m = -INFINITY;
  double l = 0.0;
  // bf16: dl gathers sum(bf16(p) - p), so that l + dl is the sum of the very
  // P values the P V product consumes. O is divided by that sum: a key that
  // carries most of a row's weight then cancels exactly, whatever the rounding
  // of its p. The LSE keeps the unrounded l.
  [[maybe_unused]] float dl = 0.f;

  // Per-lane constant parts of the LDS operand addresses.
  // K operand (A of S^T): row 32*kb + n, logical chunk per dc.
  const int krow = n;
  // V operand (A of O^T), transposing reads.
  const int l16 = lane & 15, dgrp = (lane >> 4) & 1;

  // Tiles 0 .. kStages-2 in flight before the loop; iteration t waits for its
  // own copies of tile t (the copies of later tiles may still be in flight),
  // then the barrier publishes tile t and retires slot (t-1) % kStages, which
  // is refilled with tile t + kStages - 1.
  if constexpr (!PIPE && !KS) {
#pragma unroll
    for (int u = 0; u < kStages - 1; ++u)
      if (u < ntot) issue(u);
  }
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
  // nkb_c: the 32-key blocks taken, kb0 .. kb0 + NB - 1 (NB = NKB: the whole
  // tile, kb0 = 0; NB = 1: a half tile, bf16 only). The LDS swizzles do not
  // depend on the block, so a half only shifts the rows read.
  auto stepk = [&](int u, auto masked_c, auto slot_c, auto nkb_c, int kb0) __attribute__((always_inline)) {
    constexpr int NB = decltype(nkb_c)::value;
    static_assert(NB == NKB || (NB == 1 && !FP8), "half tiles are a bf16 form");
    const int t = tile_of(u);
    constexpr int kSlot = decltype(slot_c)::value;
    const int slot = kSlot >= 0 ? kSlot : u % kStages;
    const LDS_AS char* ks = smem + (slot * 2 + 0) * T::BYTES;
    const LDS_AS char* vs = smem + (slot * 2 + 1) * T::BYTES;

    // ---- S^T = K Q^T ----
    f32x16 s[NB];
#pragma unroll
    for (int kk = 0; kk < NB; ++kk) {
      const int kb = kb0 + kk;
      s[kk] = f32x16{};
      const int r = 32 * kb + krow;
      const LDS_AS char* krowp = ks + r * ROWB;
      if constexpr (!FP8) {
#pragma unroll
        for (int dc = 0; dc < D / 16; ++dc) {
          const int lc = 2 * dc + g;
          const bf16x8 kf = *(const LDS_AS bf16x8*)(krowp + ((lc ^ T::kswz(r)) * 16));
          s[kk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf16[dc], s[kk], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int dc = 0; dc < D / 64; ++dc) {
          const int lc = 4 * dc + 2 * g;
          const i32x4 k0 = *(const LDS_AS i32x4*)(krowp + ((lc ^ T::kswz(r)) * 16));
          const i32x4 k1 = *(const LDS_AS i32x4*)(krowp + (((lc + 1) ^ T::kswz(r)) * 16));
          const i32x8 kf = i32x8{k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]};
          s[kk] = mfma_e4m3(kf, qf8[dc], s[kk]);
        }
      }
    }

    if constexpr (!FP8) {
      // K operand reads four MFMAs ahead of their use, in a region of their
      // own, instead of each read right before its MFMA.
      constexpr int NM = NB * (D / 16);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < NM - 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- mask: keys past Skv, and (causal) keys after the query ----
    if constexpr (decltype(masked_c)::value) {
      const int key0 = t * kBN;
#pragma unroll
      for (int kk = 0; kk < NB; ++kk)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + 32 * (kb0 + kk) + 8 * (i >> 2) + 4 * g + (i & 3);
          const int kp = key + kv_start;
          bool ok = key < Skv && (!CAUSAL || kp <= qi);
          if constexpr (WIN) ok = ok && ((kp >= qi - wl && kp <= qi + wr) || kp < sink);
          s[kk][i] = ok ? s[kk][i] : smask;
        }
    }

    // ---- online softmax (base 2) with a checked running max. p = exp2(c s - m)
    // is formed with the current m; while every p of the tile stays at most
    // 2^8 m is good enough and no row max is needed. The check is on the
    // lane's partial sums over each 32-key block (16 p each, bounding every
    // one of them): while no score exceeds m every p is at most 2^kPre and
    // those sums at most 2^8, so only a tile that raises the max can fail it.
    // Otherwise (or while m is still -inf) the tile's row max is taken and, if
    // it exceeds m in any row, m becomes the exact running max, O and l are
    // rescaled, and p is formed again.
    f32x16 sraw[NB];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) sraw[kb] = s[kb];
    float moff = kPre - (m == -INFINITY ? 0.f : m);
    float rk[NB];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i], c, moff));
        s[kb][i] = pv;
        rk[kb] = i == 0 ? pv : rk[kb] + pv;
      }
    float rs = rk[0], rx = rk[0];
#pragma unroll
    for (int kb = 1; kb < NB; ++kb) {
      rs += rk[kb];
      rx = fmaxf(rx, rk[kb]);
    }
    if (__any(m == -INFINITY || !(rx <= 256.f))) {
      float mx = -INFINITY;   // max of s, or of -s when c < 0
      if (!cneg) {
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sraw[kb][i]);
      } else {
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, -sraw[kb][i]);
      }
      const float mnew = fmaxf(m, xor32_max(mx) * fabsf(c));
      // If no row's max grew (say every row is still fully masked), the pass
      // above stands.
      if (__any(mnew > m)) {
        const float alpha = mnew > m ? __builtin_amdgcn_exp2f(m - mnew) : 1.f;   // 0 when m was -inf
        l *= (double)alpha;
        if constexpr (!FP8) dl *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[db] *= alpha;
        m = mnew;
        moff = kPre - (m == -INFINITY ? 0.f : m);
        rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sraw[kb][i], c, moff));
            s[kb][i] = pv;
            rs += pv;
          }
      }
    }
    l += (double)rs;

    // ---- O^T += V^T P^T ----
    if constexpr (!FP8) {
      const int rr = l16 >> 2, ss = l16 & 3;
      float dr = -rs;   // becomes sum(bf16(p)) - sum(p) over this tile
#pragma unroll
      for (int kg = 0; kg < 2 * NB; ++kg) {  // 16-key groups
        const int kb = kg >> 1, half = kg & 1;
        bf16x8 pf;
        {
          const u32x4 pk = u32x4{pack_bf16(s[kb][8 * half + 0], s[kb][8 * half + 1]),
                                 pack_bf16(s[kb][8 * half + 2], s[kb][8 * half + 3]),
                                 pack_bf16(s[kb][8 * half + 4], s[kb][8 * half + 5]),
                                 pack_bf16(s[kb][8 * half + 6], s[kb][8 * half + 7])};
          pf = __builtin_bit_cast(bf16x8, pk);
#pragma unroll
          for (int w = 0; w < 4; ++w) dr = sum_bf16x2(pk[w], dr);
        }
        const int key1 = 32 * (kb0 + kb) + 16 * half + 4 * g + rr;   // keys key1, key1+8
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
      dl += dr;
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
          o[db] = mfma_e4m3(vf, pf, o[db]);
        }
      }
    }
  };
  auto step = [&](int u, auto masked_c, auto slot_c) __attribute__((always_inline)) {
    stepk(u, masked_c, slot_c, std::integral_constant<int, NKB>{}, 0);
  };
  if constexpr (PIPE) {
    // ---- software-pipelined tile loop ----
    // Iteration u (0 .. ntot) runs S(u+1) = K(u+1) Q^T and O += V(u-1)^T
    // P(u-1) on the MFMAs while the VALU turns S(u) into P(u): the three are
    // independent, so the wave's softmax instructions issue between its MFMAs
    // instead of after them. K(x) lives in K slot x % NS and V(x) in V slot
    // x % NS (NS = 2 kSync); the workgroup synchronises every kSync
    // iterations (one barrier per kSync * 64 keys), queueing K kSync+1 to
    // 2 kSync tiles and V kSync-1 to 2 kSync-2 tiles ahead, so that a slot is
    // refilled only after every wave has read it. S and P are double
    // buffered: S(u) lives in S[u & 1], P(u) in P[u & 1].
    constexpr int NS = 2 * kSync;
    static_assert(NS == 8, "the steady loop below is unrolled over eight ring slots");
    constexpr int PWK = T::NINSTR / kW;   // K pieces (and V pieces) per wave per tile
    int gk[PWK], gv[PWK];
    unsigned lk[PWK];
#pragma unroll
    for (int j = 0; j < PWK; ++j) {
      const int c0 = (wv * PWK + j) * 64, cidx = c0 + lane, r = cidx / T::CH, pc = cidx % T::CH;
      gk[j] = r * ROWB + ((pc ^ T::kswz(r)) * 16);
      gv[j] = r * ROWB + ((pc ^ T::vswz(r)) * 16);
      lk[j] = __builtin_amdgcn_readfirstlane(smem_addr + c0 * 16);
    }
    // LDS: the K ring (kStages tiles) and then the V ring, so that every slot
    // of either ring lies within the reads' 16-bit immediate offsets.
    constexpr int KRING = 0, VRING = NS * T::BYTES;
    auto issue_k = [&](int t, int slot) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < PWK; ++j) dma16(rkw, t * (kBN * ROWB) + gk[j], lk[j] + KRING + slot * T::BYTES);
    };
    auto issue_v = [&](int t, int slot) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < PWK; ++j) dma16(rvw, t * (kBN * ROWB) + gv[j], lk[j] + VRING + slot * T::BYTES);
    };
    // Iteration u = kSync U synchronises: each wave waits for its own copies
    // (those queued kSync iterations earlier; nothing else is in flight then),
    // and the barrier publishes them and retires every slot read in
    // iterations u-kSync .. u-1; then K(u+kSync+1 .. u+2kSync) and
    // V(u+kSync-1 .. u+2kSync-2) are queued for the next kSync iterations.
    // Iterations u .. u+kSync-1 read K(u+1 .. u+kSync) and V(u-1 ..
    // u+kSync-2), all published at u.
    auto psync = [&](int u) __attribute__((always_inline)) {
      wait_vmcnt<0>();
      __syncthreads();
#pragma unroll
      for (int j = 1; j <= kSync; ++j)
        if (u + kSync + j < ntot) issue_k(u + kSync + j, (u + kSync + j) % NS);
#pragma unroll
      for (int j = 0; j < kSync; ++j)
        if (u + kSync - 1 + j < ntot) issue_v(u + kSync - 1 + j, (u + kSync - 1 + j) % NS);
    };

    static_assert(FP8, "the pipelined loop is the fp8 loop");
    // Per-lane LDS operand offsets (rows 32 apart, and keys 16 apart, share
    // the swizzle, so tiles and key groups add immediate offsets): K row n,
    // 16-byte chunk 4 dc + 2 g + h; V (transposing reads) key kv0 + 16 i for
    // i = 0..3, chunk 2 db + dgrp.
    constexpr int NKO = 2 * (D / 64);
    int koff[NKO];
    int voff[NDB];
#pragma unroll
    for (int dc = 0; dc < D / 64; ++dc)
#pragma unroll
      for (int h = 0; h < 2; ++h) koff[2 * dc + h] = krow * ROWB + (((4 * dc + 2 * g + h) ^ T::kswz(krow)) * 16);
    {
      const int rr = l16 >> 1, hh = l16 & 1;
      const int kv0 = 8 * (rr >> 2) + 4 * g + (rr & 3);
#pragma unroll
      for (int db = 0; db < NDB; ++db) voff[db] = kv0 * ROWB + (((2 * db + dgrp) ^ T::vswz(kv0)) * 16) + 8 * hh;
    }

    // moff = kPre - m (kPre while m is -inf), changed only by a re-base; lf
    // gathers the row-sum partials of up to four tiles in fp32 before they
    // enter the fp64 l.
    float moff = kPre;
    float lf = 0.f;
    auto flush = [&]() __attribute__((always_inline)) {
      l += (double)lf;
      lf = 0.f;
    };
    constexpr int NPW = 8;   // P words per lane and tile (e4m3fn x4)
    f32x16 S[2][NKB];
    int P[2][NPW];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int w = 0; w < NPW; ++w) P[b][w] = 0;

    auto kload8 = [&](int slot, int kb, int dc) __attribute__((always_inline)) {
      const LDS_AS char* kp = smem + KRING + slot * T::BYTES + kb * 32 * ROWB;
      const i32x4 k0 = *(const LDS_AS i32x4*)(kp + koff[2 * dc]);
      const i32x4 k1 = *(const LDS_AS i32x4*)(kp + koff[2 * dc + 1]);
      return i32x8{k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]};
    };
    // The V ring starts at 64 KB, beyond the 16-bit offset field of an LDS
    // read: its base goes into the address registers once (opaque to the
    // compiler, which would otherwise OR ring, slot and key-group constants
    // into a fresh register for every read), leaving offsets below 64 KB.
    int vbase[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      vbase[db] = VRING + voff[db];
      asm volatile("" : "+v"(vbase[db]));
    }
    auto vload8 = [&](int slot, int db) __attribute__((always_inline)) {
      const LDS_AS char* vp = smem + vbase[db] + slot * T::BYTES;
      int vw[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS i32x2*)(vp + i * 16 * ROWB));
        vw[2 * i] = x[0];
        vw[2 * i + 1] = x[1];
      }
      return i32x8{vw[0], vw[1], vw[2], vw[3], vw[4], vw[5], vw[6], vw[7]};
    };
    auto mfma8 = [](i32x8 a, i32x8 b, f32x16 c) __attribute__((always_inline)) {
      return mfma_e4m3(a, b, c);
    };
    // S(next) = K Q^T and O += V^T P(prev), MFMAs alternating between the two
    // products; do_qk / do_pv drop either (edge iterations).
    auto mma = [&](f32x16 (&sn)[NKB], const int (&pp)[NPW], int kslot, int vslot, bool do_qk, bool do_pv)
        __attribute__((always_inline)) {
      static_assert(NKB == 2 && NDB == 4, "hd128 tile shapes");
      if (do_qk) { sn[0] = f32x16{}; sn[1] = f32x16{}; }
      const i32x8 pf = i32x8{pp[0], pp[1], pp[2], pp[3], pp[4], pp[5], pp[6], pp[7]};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kb = i & 1, dc = i >> 1;
        if (do_qk) sn[kb] = mfma8(kload8(kslot, kb, dc), qf8[dc], sn[kb]);
        if (do_pv) o[i] = mfma8(vload8(vslot, i), pf, o[i]);
      }
    };
    // Softmax of one tile: P from S (e4m3fn scaled by 2^kPre), with the
    // checked running max; the pack happens before the check and is redone if
    // the tile re-bases.
    // keep(): called on the rare re-base path only; the steady loop passes one
    // that uses the next tile's scores there, which keeps their MFMAs ahead of
    // the branch (inside the interleaved region) instead of sunk past it.
    auto softmax = [&](f32x16 (&sc)[NKB], int (&pw)[NPW], auto masked_c, int t, auto sched_c, auto keep)
        __attribute__((always_inline)) {
      if constexpr (decltype(masked_c)::value) {
        const int key0 = t * kBN;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = key0 + 32 * kb + 8 * (i >> 2) + 4 * g + (i & 3);
            const bool ok = key < Skv && (!CAUSAL || key + kv_start <= qi);
            sc[kb][i] = ok ? sc[kb][i] : smask;
          }
      }
      // rs: the tile's unrounded row-sum share; rx: the larger of its two 32-key
      // block shares (the size check)
      auto expo = [&](float moff, float& rs, float& rx) __attribute__((always_inline)) {
        float r0 = 0.f, r1 = 0.f;
        float gs[8];   // sums of four; a tree from these needs no zero start
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          const int kb = w >> 2, i = 4 * (w & 3);
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][i + 0], c, moff));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][i + 1], c, moff));
          const float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][i + 2], c, moff));
          const float p3 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][i + 3], c, moff));
          gs[w] = (p0 + p1) + (p2 + p3);
          if (w == 3) r0 = (gs[0] + gs[1]) + (gs[2] + gs[3]);
          if (w == 7) r1 = (gs[4] + gs[5]) + (gs[6] + gs[7]);
          // the first conversion writes the low half-word only; the word of two
          // tiles back is passed as the kept half so that nothing is cleared
          int x = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, pw[w], false);
          pw[w] = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, x, true);
        }
        rs = r0 + r1;
        rx = fmaxf(r0, r1);
      };
      float rs, rx;
      expo(moff, rs, rx);
      if constexpr (decltype(sched_c)::value) {
        // Interleave: the 8 MFMAs of mma() one by one, each followed by the
        // LDS operand reads (2 or 4) of the MFMA two places later and its share
        // of the softmax: 10 VALU and 4 exp2 (v_exp_f32 is a transcendental,
        // mask 0x400, which the VALU mask 0x002 does not take; counted apart
        // they stay spread over the slots instead of gathering in the first
        // ones). The first MFMA waits on the K reads queued at the top of the
        // iteration, so 12 VALU and 4 exp2 go ahead of it; the last two slots
        // take what is left (6 + 2 and 4 + 2 of the 82 + 32).
#define HAT_SLOT(nds, nv, nt)                            \
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     \
  __builtin_amdgcn_sched_group_barrier(0x100, nds, 0);   \
  __builtin_amdgcn_sched_group_barrier(0x002, nv, 0);    \
  __builtin_amdgcn_sched_group_barrier(0x400, nt, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);
        __builtin_amdgcn_sched_group_barrier(0x400, 4, 0);
        HAT_SLOT(2, 10, 4) HAT_SLOT(4, 10, 4) HAT_SLOT(2, 10, 4) HAT_SLOT(4, 10, 4)
        HAT_SLOT(2, 10, 4) HAT_SLOT(4, 10, 4) HAT_SLOT(0, 6, 2) HAT_SLOT(0, 4, 2)
#undef HAT_SLOT
      }
      // In steady iterations tile 0 has given every row a finite m, so only
      // the size check remains; the edges also re-base while m is -inf.
      const bool need = decltype(sched_c)::value ? !(rx <= 256.f) : (m == -INFINITY || !(rx <= 256.f));
      if (__any(need)) {
        keep();
        // the scores pass through an empty asm here, so that the row max below
        // cannot be speculated ahead of the branch into the common path
        asm volatile("" : "+v"(sc[0]), "+v"(sc[1]));
        float mx = -INFINITY;   // max of s, or of -s when c < 0
        if (!cneg) {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[kb][i]);
        } else {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, -sc[kb][i]);
        }
        const float mnew = fmaxf(m, xor32_max(mx) * fabsf(c));
        // no row's max grew (say every row still fully masked): the pack stands
        if (__any(mnew > m)) {
          const float alpha = mnew > m ? __builtin_amdgcn_exp2f(m - mnew) : 1.f;   // 0 when m was -inf
          l *= (double)alpha;
          lf *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db) o[db] *= alpha;
          m = mnew;
          moff = kPre - (m == -INFINITY ? 0.f : m);
          expo(moff, rs, rx);
        }
      }
      lf += rs;
    };

    // The wave's bounds, made provably wave-uniform so that the loops below
    // branch on scalars: its tile count, its first masked tile, and the end
    // of its steady iterations (1 .. ss_end-1 run every part unmasked).
    const int w_nt = __builtin_amdgcn_readfirstlane(w_ntiles);
    const int w_fm = __builtin_amdgcn_readfirstlane(CAUSAL ? min(Skv / kBN, max(0, qw - kv_start + 1) / kBN)
                                                           : Skv / kBN);
    const int ss_end = min(w_nt - 1, w_fm);
    // One iteration with its parts decided at run time (the edges of the loop).
    auto edge = [&](int u, f32x16 (&sc)[NKB], f32x16 (&sn)[NKB], int (&pc)[NPW], const int (&pp)[NPW])
        __attribute__((always_inline)) {
      if (u % kSync == 0) psync(u);
      mma(sn, pp, (u + 1) % NS, (u + NS - 1) % NS, u + 1 < w_nt, u >= 1 && u <= w_nt);
      __builtin_amdgcn_sched_barrier(0);   // edges are rare: not interleaved, fewer live registers
      auto none = []() __attribute__((always_inline)) {};
      if (u < w_nt) {
        if (u >= w_fm) softmax(sc, pc, std::true_type{}, u, std::false_type{}, none);
        else softmax(sc, pc, std::false_type{}, u, std::false_type{}, none);
        flush();
      }
    };
    // A steady iteration: every part runs, unmasked, interleaved.
    auto steady = [&](int u, f32x16 (&sc)[NKB], f32x16 (&sn)[NKB], int (&pc)[NPW], const int (&pp)[NPW], int kslot,
                      int vslot, auto sync_c) __attribute__((always_inline)) {
      if constexpr (decltype(sync_c)::value) psync(u);
      mma(sn, pp, kslot, vslot, true, true);
      auto keep = [&]() __attribute__((always_inline)) { asm volatile("" ::"v"(sn[0]), "v"(sn[1])); };
      softmax(sc, pc, std::false_type{}, u, std::true_type{}, keep);
    };

    // A steady iteration whose ring slots and synchronisation are decided at
    // run time (the short runs after the eight-at-a-time loop).
    auto steady_rt = [&](int u, f32x16 (&sc)[NKB], f32x16 (&sn)[NKB], int (&pc)[NPW], const int (&pp)[NPW])
        __attribute__((always_inline)) {
      if (u % kSync == 0) psync(u);
      mma(sn, pp, (u + 1) % NS, (u + NS - 1) % NS, true, true);
      auto keep = [&]() __attribute__((always_inline)) { asm volatile("" ::"v"(sn[0]), "v"(sn[1])); };
      softmax(sc, pc, std::false_type{}, u, std::true_type{}, keep);
    };

    // Prologue: K(0 .. kSync) and V(0 .. kSync-2), then S(0); iteration 0
    // queues the next ones.
#pragma unroll
    for (int x = 0; x <= kSync; ++x)
      if (x < ntot) issue_k(x, x);
#pragma unroll
    for (int x = 0; x <= kSync - 2; ++x)
      if (x < ntot) issue_v(x, x);
    wait_vmcnt<0>();
    __syncthreads();
    if (w_nt > 0) mma(S[0], P[1], 0, 0, true, false);
    if (ntot > 0) {
      edge(0, S[0], S[1], P[0], P[1]);
      int u = 1;
      // Steady iterations eight at a time (u = 1 mod 8 at the top), so that the
      // ring slots, buffers and barriers are compile-time constants.
      constexpr std::false_type no{};
      constexpr std::true_type yes{};
      for (; u + 7 < ss_end; u += 8) {
        steady(u + 0, S[1], S[0], P[1], P[0], 2, 0, no);
        steady(u + 1, S[0], S[1], P[0], P[1], 3, 1, no);
        steady(u + 2, S[1], S[0], P[1], P[0], 4, 2, no);
        steady(u + 3, S[0], S[1], P[0], P[1], 5, 3, yes);   // u + 3 = 0 mod 4
        steady(u + 4, S[1], S[0], P[1], P[0], 6, 4, no);
        steady(u + 5, S[0], S[1], P[0], P[1], 7, 5, no);
        steady(u + 6, S[1], S[0], P[1], P[0], 0, 6, no);
        steady(u + 7, S[0], S[1], P[0], P[1], 1, 7, yes);   // u + 7 = 0 mod 8
        flush();
      }
      // Fewer than eight steady iterations left (all of a short key range):
      // two at a time, interleaved as above, with the ring slots and the
      // synchronisation decided at run time (u stays odd).
      for (; u + 1 < ss_end; u += 2) {
        steady_rt(u, S[1], S[0], P[1], P[0]);
        steady_rt(u + 1, S[0], S[1], P[0], P[1]);
        flush();
      }
      // The rest (u is odd here), two at a time with compile-time buffers.
      for (; u <= ntot; u += 2) {
        edge(u, S[1], S[0], P[1], P[0]);
        if (u + 1 > ntot) break;
        edge(u + 1, S[0], S[1], P[0], P[1]);
      }
    }
  } else if constexpr (KS) {
    // Tiles 2v and 2v+1 (slots 2v % kStages and (2v+1) % kStages) at step v:
    // KS = 2, by the waves of key share 0 and 1; KS = 4, tile 2v + kh / 2 by
    // the two waves kh of that tile, each taking its half kh % 2 of the keys.
    // Step v's barrier retires the slots of step v-1, which take tiles 2v+2
    // and 2v+3. Every wave runs ceil(ntot/2) steps (ntot is the workgroup's),
    // so the barriers pair up.
    const int first_masked = CAUSAL ? min(Skv / kBN, max(0, qw - kv_start + 1) / kBN) : Skv / kBN;
    const int n_plain = min(first_masked, ntot);
    const int kt = KS == 4 ? kh >> 1 : kh;          // the wave's tile of each step
    [[maybe_unused]] const int kb0 = kh & 1;        // KS = 4: its half of that tile
    auto kstep = [&](int u, auto masked_c) __attribute__((always_inline)) {
      if constexpr (KS == 4) stepk(u, masked_c, kAnySlot, std::integral_constant<int, 1>{}, kb0);
      else step(u, masked_c, kAnySlot);
    };
    auto ksync = [&](int v) __attribute__((always_inline)) {
      wait_vmcnt<0>();
      __syncthreads();
      if (2 * v + 2 < ntot) issue(2 * v + 2);
      if (2 * v + 3 < ntot) issue(2 * v + 3);
    };
    int v = 0;
    for (; 2 * v + 1 < n_plain; ++v) {   // both tiles of the step unmasked for this wave's rows
      ksync(v);
      if (2 * v + kt < w_ntiles) kstep(2 * v + kt, std::false_type{});
    }
    for (; 2 * v < ntot; ++v) {
      ksync(v);
      const int u = 2 * v + kt;
      // (KS = 4: a half holding no key the wave's rows may see is skipped)
      if (u < ntot && u < w_ntiles && (KS != 4 || kBN * u + 32 * kb0 < w_kv_end)) kstep(u, std::true_type{});
    }
    // Merge: key shares 1 .. KS-1 hand their m, l, dl and O (lane by lane: the
    // same rows and columns) to share 0 through LDS; share 0 then writes the
    // output.
    wait_vmcnt<0>();
    __syncthreads();   // every ring read done
    constexpr int NF = NDB * 16 + 4;   // floats per lane: O, m, dl, l (two words)
    constexpr int NP = KS - 1;         // partials per row group
    static_assert(kRG * NP * NF * 64 * 4 <= kLds, "merge buffer fits the ring");
    LDS_AS float* xb0 = (LDS_AS float*)smem + rw * NP * NF * 64 + lane;
    if (kh != 0) {
      LDS_AS float* xb = xb0 + (kh - 1) * NF * 64;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) xb[(db * 16 + i) * 64] = o[db][i];
      const u32x2 lw = __builtin_bit_cast(u32x2, l);
      xb[(NF - 4) * 64] = m;
      xb[(NF - 3) * 64] = dl;
      xb[(NF - 2) * 64] = __uint_as_float(lw[0]);
      xb[(NF - 1) * 64] = __uint_as_float(lw[1]);
    }
    __syncthreads();
    if (kh != 0) return;
    if constexpr (KS == 2) {
      LDS_AS float* xb = xb0;
      const float m1 = xb[(NF - 4) * 64], dl1 = xb[(NF - 3) * 64];
      const double l1 = __builtin_bit_cast(double, u32x2{__float_as_uint(xb[(NF - 2) * 64]),
                                                         __float_as_uint(xb[(NF - 1) * 64])});
      const float mm = fmaxf(m, m1);
      const float a0 = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mm);
      const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] = o[db][i] * a0 + xb[(db * 16 + i) * 64] * a1;
      l = l * (double)a0 + l1 * (double)a1;
      dl = dl * a0 + dl1 * a1;
      m = mm;
    } else {   // KS = 4: the three partners' partials, under the largest of the four maxima
      float mj[NP], aj[NP];
      float mm = m;
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        mj[j] = xb0[(j * NF + NF - 4) * 64];
        mm = fmaxf(mm, mj[j]);
      }
      const float a0 = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mm);
#pragma unroll
      for (int j = 0; j < NP; ++j) aj[j] = mj[j] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mj[j] - mm);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float acc = o[db][i] * a0;
#pragma unroll
          for (int j = 0; j < NP; ++j) acc += xb0[(j * NF + db * 16 + i) * 64] * aj[j];
          o[db][i] = acc;
        }
      double lacc = l * (double)a0;
      float dacc = dl * a0;
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        const double lj = __builtin_bit_cast(double, u32x2{__float_as_uint(xb0[(j * NF + NF - 2) * 64]),
                                                           __float_as_uint(xb0[(j * NF + NF - 1) * 64])});
        lacc += lj * (double)aj[j];
        dacc += xb0[(j * NF + NF - 3) * 64] * aj[j];
      }
      l = lacc;
      dl = dacc;
      m = mm;
    }
  } else if constexpr (!WIN) {
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
  const float lp = FP8 ? ltot : xor32_sum((float)l + dl);   // sum of the P the MFMAs consumed
  const float inv = ltot > 0.f ? oscale / lp : 0.f;
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

// Persistent form of the classic tile loop, for grids of many query tiles
// with short key ranges (non-causal, no window, no key splits): a grid of at
// most one workgroup per CU, each walking one contiguous range of the
// B * Hq * n_qtiles query tiles of 256 rows. The K/V ring runs on across the
// range (step s = query tile t0 + s / nk, key tile s % nk; copies three steps
// ahead), so the next tile's first copies are in flight while the current
// one finishes, and the next tile's Q loads go out before the current tile's
// O stores. A workgroup per query tile instead pays its Q load, ring fill and
// O store in turn on every tile. Per tile the arithmetic is the classic
// loop's (QK^T, checked running max, P V), so the bf16 bits equal
// attn_fwd_kernel's with 8 waves and no key split. The tile step is written
// out here for the non-causal case rather than shared with attn_fwd_kernel's,
// so that the code of that kernel's measured instances stays as it is.
template <int D, bool FP8>
__global__ void __launch_bounds__(512) attn_fwd_persist_kernel(const Params p) {
  constexpr int kW = 8, kThr = 512;
  using T = Tile<D, FP8>;
  constexpr int ROWB = T::ROWB;
  constexpr int NDB = D / 32;
  constexpr int NKB = kBN / 32;
  constexpr float kPre = FP8 ? 4.f : 0.f;
  constexpr int kLds = kStages * 2 * T::BYTES;
  __shared__ __attribute__((aligned(1024))) char smem_raw[kLds];
  LDS_AS char* smem = (LDS_AS char*)smem_raw;
  const unsigned smem_addr = (unsigned)(uintptr_t)smem;

  // This workgroup's query tiles [t0, t1): XCD x (workgroups reach the XCDs
  // round-robin) gets one contiguous share of the grid, cut into equal ranges.
  const long long ntq = (long long)p.B * p.Hq * p.n_qtiles;
  int L = (int)blockIdx.x;
  {
    const int n = (int)gridDim.x, q8 = n >> 3, rem = n & 7, x = L & 7, r = L >> 3;
    L = x < rem ? x * (q8 + 1) + r : rem * (q8 + 1) + (x - rem) * q8 + r;
  }
  const int t0 = (int)(ntq * L / gridDim.x), t1 = (int)(ntq * (L + 1) / gridDim.x);
  const int Skv = p.Skv;
  const int nk = (Skv + kBN - 1) / kBN;   // key tiles per query tile
  const int n_whole = Skv / kBN;          // the unmasked ones
  const int nsteps = (t1 - t0) * nk;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 5, n = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(wave);

  float c = p.c, oscale = 1.f;
  if constexpr (FP8) {
    const float qd = p.qd ? *p.qd : 1.f, kd = p.kd ? *p.kd : 1.f, vd = p.vd ? *p.vd : 1.f;
    c *= qd * kd;
    oscale = vd;
  }
  const bool cneg = FP8 && c < 0.f;
  const float smask = cneg ? INFINITY : -INFINITY;

  // Copies of step s into slot s % kStages (pieces split over the waves as in
  // attn_fwd_kernel; the buffer range of the step's head zero-fills rows past
  // Skv).
  constexpr int PW = 2 * T::NINSTR / kW;
  static_assert(PW >= 1 && PW * kW == 2 * T::NINSTR, "tile pieces must split evenly over waves");
  auto issue = [&](int s) __attribute__((always_inline)) {
    const int tq = __builtin_amdgcn_readfirstlane(t0 + s / nk);
    const int u = __builtin_amdgcn_readfirstlane(s - (s / nk) * nk);
    const int bh = tq / p.n_qtiles, b = bh / p.Hq, hk = (bh % p.Hq) / p.group;
    const size_t krow0 = (size_t)(b * p.Hkv + hk) * (size_t)Skv;
    const i32x4 rk = rsrc_words(p.k + krow0 * ROWB, (uint32_t)Skv * ROWB);
    const i32x4 rv = rsrc_words(p.v + krow0 * ROWB, (uint32_t)Skv * ROWB);
    const i32x4 rkw = i32x4{__builtin_amdgcn_readfirstlane(rk[0]), __builtin_amdgcn_readfirstlane(rk[1]),
                            __builtin_amdgcn_readfirstlane(rk[2]), __builtin_amdgcn_readfirstlane(rk[3])};
    const i32x4 rvw = i32x4{__builtin_amdgcn_readfirstlane(rv[0]), __builtin_amdgcn_readfirstlane(rv[1]),
                            __builtin_amdgcn_readfirstlane(rv[2]), __builtin_amdgcn_readfirstlane(rv[3])};
    const int key0 = u * kBN;
    const int slot = s % kStages;
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

  // Q of query tile tq: this wave's 32 rows (rows >= Sq read as zero).
  bf16x8 qf16[FP8 ? 1 : D / 16];
  i32x8 qf8[FP8 ? D / 64 : 1];
  auto load_q = [&](int tq) __attribute__((always_inline)) {
    const int bh = tq / p.n_qtiles, qt = tq - bh * p.n_qtiles;
    const size_t qrow0 = (size_t)bh * (size_t)p.Sq;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + qrow0 * ROWB, (uint32_t)p.Sq * ROWB);
    const int qi = qt * kBM + wave * 32 + n;
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
  };

  if (t0 < t1) load_q(t0);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): Q has landed before any copy is queued
  if (Skv % kBN != 0)
    for (int i = threadIdx.x; i < kLds / 16; i += kThr)
      *(LDS_AS u32x4*)(smem + i * 16) = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s)
    if (s < nsteps) issue(s);

  // Step s: wait for this wave's copies of it (those of the next two steps may
  // still be in flight), barrier, queue step s + kStages - 1.
  auto sync = [&](int s) __attribute__((always_inline)) {
    if (s + 2 < nsteps) wait_vmcnt<2 * PW>();
    else if (s + 1 < nsteps) wait_vmcnt<PW>();
    else wait_vmcnt<0>();
    __syncthreads();
    if (s + kStages - 1 < nsteps) issue(s + kStages - 1);
  };

  f32x16 o[NDB];
  float m;
  double l;
  [[maybe_unused]] float dl;
  [[maybe_unused]] int pkeep[kBN / 64][8] = {};
  const int krow = n;
  const int l16 = lane & 15, dgrp = (lane >> 4) & 1;

  // One key tile (key tile u in ring slot `slot`) for this wave's rows.
  auto step = [&](int u, int slot, auto masked_c) __attribute__((always_inline)) {
    const LDS_AS char* ks = smem + (slot * 2 + 0) * T::BYTES;
    const LDS_AS char* vs = smem + (slot * 2 + 1) * T::BYTES;
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
          s[kb] = mfma_e4m3(kf, qf8[dc], s[kb]);
        }
      }
    }
    if constexpr (decltype(masked_c)::value) {   // keys past Skv
      const int key0 = u * kBN;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + 32 * kb + 8 * (i >> 2) + 4 * g + (i & 3);
          s[kb][i] = key < Skv ? s[kb][i] : smask;
        }
    }
    // online softmax with the checked running max, as in attn_fwd_kernel
    f32x16 sraw[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) sraw[kb] = s[kb];
    float moff = kPre - (m == -INFINITY ? 0.f : m);
    float rk[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i], c, moff));
        s[kb][i] = pv;
        rk[kb] = i == 0 ? pv : rk[kb] + pv;
      }
    float rs = rk[0], rx = rk[0];
#pragma unroll
    for (int kb = 1; kb < NKB; ++kb) {
      rs += rk[kb];
      rx = fmaxf(rx, rk[kb]);
    }
    if (__any(m == -INFINITY || !(rx <= 256.f))) {
      float mx = -INFINITY;
      if (!cneg) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sraw[kb][i]);
      } else {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, -sraw[kb][i]);
      }
      const float mnew = fmaxf(m, xor32_max(mx) * fabsf(c));
      if (__any(mnew > m)) {
        const float alpha = mnew > m ? __builtin_amdgcn_exp2f(m - mnew) : 1.f;
        l *= (double)alpha;
        if constexpr (!FP8) dl *= alpha;
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
    }
    l += (double)rs;
    // O^T += V^T P^T
    if constexpr (!FP8) {
      const int rr = l16 >> 2, ss = l16 & 3;
      float dr = -rs;
#pragma unroll
      for (int kg = 0; kg < kBN / 16; ++kg) {
        const int kb = kg >> 1, half = kg & 1;
        bf16x8 pf;
        {
          const u32x4 pk = u32x4{pack_bf16(s[kb][8 * half + 0], s[kb][8 * half + 1]),
                                 pack_bf16(s[kb][8 * half + 2], s[kb][8 * half + 3]),
                                 pack_bf16(s[kb][8 * half + 4], s[kb][8 * half + 5]),
                                 pack_bf16(s[kb][8 * half + 6], s[kb][8 * half + 7])};
          pf = __builtin_bit_cast(bf16x8, pk);
#pragma unroll
          for (int w = 0; w < 4; ++w) dr = sum_bf16x2(pk[w], dr);
        }
        const int key1 = 32 * kb + 16 * half + 4 * g + rr;
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
      dl += dr;
    } else {
      const int rr = l16 >> 1, hh = l16 & 1;
#pragma unroll
      for (int kq = 0; kq < kBN / 64; ++kq) {
        int pw[8];
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          const int j = 4 * w, kb = 2 * kq + (j >> 4), i = j & 15;
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
          for (int uu = 0; uu < 4; ++uu) {
            const int key = 64 * kq + 32 * (uu >> 1) + 16 * (uu & 1) + 8 * (rr >> 2) + 4 * g + (rr & 3);
            const LDS_AS char* a = vs + key * ROWB + ((lc ^ T::vswz(key)) * 16) + 8 * hh;
            const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS i32x2*)a);
            vw[2 * uu] = x[0];
            vw[2 * uu + 1] = x[1];
          }
          const i32x8 vf = i32x8{vw[0], vw[1], vw[2], vw[3], vw[4], vw[5], vw[6], vw[7]};
          o[db] = mfma_e4m3(vf, pf, o[db]);
        }
      }
    }
  };

  int s = 0;
  for (int tq = t0; tq < t1; ++tq) {
    const int bh = tq / p.n_qtiles, qt = tq - bh * p.n_qtiles;
    const int qw = qt * kBM + wave * 32, qi = qw + n;
    const bool live = qw < p.Sq;
#pragma unroll
    for (int i = 0; i < NDB; ++i) o[i] = f32x16{};
    m = -INFINITY;
    l = 0.0;
    if constexpr (!FP8) dl = 0.f;
    int u = 0;
    for (; u < n_whole; ++u, ++s) {
      sync(s);
      if (live) step(u, s % kStages, std::false_type{});
    }
    for (; u < nk; ++u, ++s) {
      sync(s);
      if (live) step(u, s % kStages, std::true_type{});
    }
    // the next tile's Q, queued ahead of this tile's O stores
    if (tq + 1 < t1) load_q(tq + 1);
    if (live) {
      const float ltot = xor32_sum((float)l);
      const float lp = FP8 ? ltot : xor32_sum((float)l + dl);
      const float inv = ltot > 0.f ? oscale / lp : 0.f;
      const float lse = ltot > 0.f ? (m + __log2f(ltot) - kPre) * 0.69314718055994531f : -INFINITY;
      const size_t qrow0 = (size_t)bh * (size_t)p.Sq;
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
  if (win)
    return causal ? attn_fwd_kernel<D, true, FP8, true, NW, 0> : attn_fwd_kernel<D, false, FP8, true, NW, 0>;
  return causal ? attn_fwd_kernel<D, true, FP8, false, NW, 0> : attn_fwd_kernel<D, false, FP8, false, NW, 0>;
}

// ks: the bf16 key-split factor (8 waves; 2: 128 rows, 4: 64 rows), 0 for
// none; nw otherwise.
template <int D, bool FP8>
kernel_fn pick(bool causal, bool win, int nw, int ks) {
  if constexpr (!FP8) {
    if (ks == 4) return causal ? attn_fwd_kernel<D, true, false, false, 8, 4> : attn_fwd_kernel<D, false, false, false, 8, 4>;
    if (ks == 2) return causal ? attn_fwd_kernel<D, true, false, false, 8, 2> : attn_fwd_kernel<D, false, false, false, 8, 2>;
  }
  return nw == 4 ? pick_nw<D, FP8, 4>(causal, win) : pick_nw<D, FP8, 8>(causal, win);
}

}  // namespace hat

using namespace hat;

static constexpr int64_t kMaxSplits = 256;
// Longest key range (in 64-key tiles) that runs on persistent workgroups.
static constexpr int64_t kPersistMaxKeyTiles = 8;

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
  // bf16 without a window runs 8-wave key-split workgroups instead: of 64
  // rows (four waves per row group, each on half of one of a step's two key
  // tiles) when that grid still fits one round of the CUs, else of 128 rows
  // (two waves per row group taking alternate tiles). Measured at D128
  // causal: 64-row workgroups take 14-16 % off a grid that fits one round;
  // in two rounds they are 8 % slower than one round of 128-row workgroups
  // (their short steps expose the copies' latency).
  const int ks = nw == 4 && dtype == ATTN_BF16 && !win
                     ? (B * Hq * ((Sq + 63) / 64) <= (int64_t)device_cus() ? 4 : 2) : 0;
  const int64_t rows_wg = ks ? 32 * 8 / ks : 32 * nw;   // query rows per workgroup
  const int64_t n_qtiles = (Sq + rows_wg - 1) / rows_wg;
  const int64_t rows = B * Hq * Sq;
  const int64_t ntiles = B * Hq * n_qtiles;
  int64_t n_full = -1, part_rows = rows, part_row0 = 0, grid = ntiles * nsp;
  if (tail) {
    const int64_t cus = device_cus();
    n_full = ntiles / cus * cus;
    if (n_full == 0 || n_full == ntiles) return ATTN_ERR_SHAPE;
    part_row0 = (n_full / n_qtiles) * Sq + (n_full % n_qtiles) * rows_wg;
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
  // Grids of at least two rounds over short key ranges (non-causal, no window,
  // no key splits) run persistent workgroups instead, one per CU at most, each
  // walking a range of query tiles: per-tile start-up and O stores then
  // overlap the neighbouring tiles' work.
  const int64_t cus = device_cus();
  const bool pers = !causal && !win && nsp == 1 && nw == 8 && ktiles <= kPersistMaxKeyTiles && ntiles >= 2 * cus;
  if (pers) {
    grid = cus;
    fn = dtype == ATTN_BF16 ? (D == 128 ? attn_fwd_persist_kernel<128, false> : attn_fwd_persist_kernel<64, false>)
                            : (D == 128 ? attn_fwd_persist_kernel<128, true> : attn_fwd_persist_kernel<64, true>);
  } else if (dtype == ATTN_BF16) {
    fn = D == 128 ? pick<128, false>(causal, win, nw, ks) : pick<64, false>(causal, win, nw, ks);
  } else {
    fn = D == 128 ? pick<128, true>(causal, win, nw, 0) : pick<64, true>(causal, win, nw, 0);
  }
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(ks || pers ? 512 : 64 * nw), 0, (hipStream_t)stream, p);
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

// ---- attn_fwd_splitkv_static: the split partials in a static device array ----
//
// For callers that cannot allocate device memory (code under stream capture,
// tight serving loops, harnesses that forbid allocation): the split-KV
// forward with its fp32 partials in `scratch`, a file-scope device array of
// kStaticScratchBytes that every GPU the library runs on holds until the
// process ends. Host code never uses the array's name as an address (on the
// host it only names the symbol): each device's address comes from
// hipGetSymbolAddress, taken once per device with that device current and kept.
static constexpr int64_t kStaticScratchBytes = ATTN_SPLITKV_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[64];

static void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

extern "C" attn_status_t attn_fwd_splitkv_static(const void* q, const void* k, const void* v, void* out, float* lse,
                                                 int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Skv,
                                                 int64_t D, float scale, int causal, attn_dtype_t dtype,
                                                 const float* q_descale, const float* k_descale,
                                                 const float* v_descale, int64_t n_splits, void* stream) {
  void* ws = scratch_on_current_device();
  if (ws == nullptr) return ATTN_ERR_HIP;
  // The partials need not start at any value: every split writes all of its
  // rows before the merge kernel (same stream) reads them. Launch checks the
  // split count's need against the array's size (ATTN_ERR_WORKSPACE beyond it).
  return attn_fwd_splitkv(q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, scale, causal, dtype, q_descale, k_descale,
                          v_descale, n_splits, ws, kStaticScratchBytes, stream);
}
