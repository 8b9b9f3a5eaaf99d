/*
 * attn.h — C ABI of the MI355X (gfx950) fused attention forward with LSE, its
 * key-chunk, local-attention and split-KV forms, the deterministic backward,
 * and the host-side LSE merge.
 *
 * The operation is the fused scaled-dot-product attention forward that also
 * returns the per-row log-sum-exp, as used through the flash/efficient SDPA
 * kernels on the page "[Proposal] ROCm (AMD Instinct) support for the core
 * attention and distributed init" (section "Where it breaks on ROCm" and the
 * follow-up on compute_log_sumexp) and as the fmha_v3_fwd call on the page
 * "F8 fmha ASM gfx950" (Test Result section: softmax_scale, is_causal,
 * return_softmax_lse, out, q/k/v_descale):
 *
 *     O[b,h,i,:] = sum_j softmax_j(scale * q_i . k_j  [masked]) * v_j
 *     LSE[b,h,i] = ln sum_j exp(scale * q_i . k_j)      (allowed j only)
 *
 * with query head h reading KV head h / (Hq / Hkv) (grouped KV heads, as in
 * the 32/8-head layout on the page "feat(attention): add strict bitwise ROCm
 * path", ROCm Validation section). The (out, lse) pair is what that page's
 * attention boundary returns, and what a later merge of key chunks needs.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers are DEVICE pointers unless the name or comment says host. The
 * caller owns every buffer; the library never allocates, frees or
 * synchronises. Work is enqueued on `stream` (a hipStream_t; NULL = the
 * default stream) and the call returns at once. Calls are stateless and
 * re-entrant; identical inputs give bitwise-identical outputs.
 *
 * Layouts (all contiguous, row-major):
 *   q, out : [B, Hq,  Sq,  D]     k, v : [B, Hkv, Skv, D]     lse : [B, Hq, Sq] fp32
 * Element types: q, k, v are bf16 (ATTN_BF16) or OCP FP8 e4m3fn codes
 * (ATTN_FP8_E4M3FN); out is always bf16 (round to nearest even); lse is fp32
 * in natural log and includes the softmax scale.
 *
 * Errors: every argument is checked before anything is enqueued; on any
 * error nothing is launched and an ATTN_ERR_* code is returned. There is no
 * fallback to another implementation.
 */
#ifndef HEAD_ATTENTION_AMD_ATTN_H
#define HEAD_ATTENTION_AMD_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Size in bytes of the static device array attn_fwd_splitkv_static keeps its split
 * partials in (one per GPU). */
#define ATTN_SPLITKV_STATIC_SCRATCH_BYTES ((int64_t)64 << 20)

typedef enum {
  ATTN_BF16 = 0,        /* q, k, v hold bf16 */
  ATTN_FP8_E4M3FN = 1   /* q, k, v hold e4m3fn codes; real value = decode(code) * descale */
} attn_dtype_t;

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,      /* a required pointer is NULL */
  ATTN_ERR_SHAPE = 2,     /* a negative size, Hkv = 0 with Hq > 0, Hq % Hkv != 0, kv_start < 0,
                             n_splits outside 0..256, a window side < -1 or sink < 0 */
  ATTN_ERR_HEAD_DIM = 3,  /* D is not 64 or 128 */
  ATTN_ERR_DTYPE = 4,     /* unknown attn_dtype_t */
  ATTN_ERR_ALIGN = 5,     /* q, k, v or out not 16-byte aligned, or lse not 4-byte aligned */
  ATTN_ERR_OVERFLOW = 6,  /* one head's slice, padded by one tile, reaches 2^31 bytes
                             ((Sq + 256) * D * 2 for q/out, (Skv + 64) * D * elt for k/v:
                             D128 allows Sq <= 8388351 and Skv <= 8388543 in bf16,
                             16777151 in fp8), kv_start + Skv reaches 2^30, or the grid
                             is too large */
  ATTN_ERR_SCALE = 7,     /* scale is not finite or not > 0 */
  ATTN_ERR_HIP = 8,       /* the kernel launch failed */
  ATTN_ERR_WORKSPACE = 9  /* attn_fwd_splitkv / attn_bwd: workspace NULL, misaligned, or too small */
} attn_status_t;

/*
 * attn_fwd — O and LSE of the attention forward.
 *
 *   q, k, v      device inputs, layouts above, type `dtype`.
 *   out          device bf16 output [B, Hq, Sq, D].
 *   lse          device fp32 output [B, Hq, Sq].
 *   B, Hq, Hkv   batch, query heads, KV heads (Hq % Hkv == 0).
 *   Sq, Skv      query and key lengths. Zero is allowed: Sq = 0 (or B = 0,
 *                Hq = 0) enqueues nothing; Skv = 0 writes O = 0, LSE = -inf.
 *   D            head dimension, 64 or 128.
 *   scale        softmax scale (finite, > 0), e.g. 1/sqrt(D).
 *   causal       nonzero: key j is allowed for query i iff j <= i (top-left).
 *   q/k/v_descale  fp8 only: device pointers to one fp32 each; NULL means 1.
 *                Ignored for bf16. Read on the device, so the host cannot check
 *                them: any finite value is accepted, of either sign (a negative
 *                q_descale * k_descale makes the largest score the one of the
 *                smallest code product, and the kernel takes its row max that
 *                way); a NaN or infinite descale gives NaN or infinite out and
 *                lse.
 *   stream       hipStream_t to enqueue on.
 *
 * A row with no allowed key gets O = 0 and LSE = -inf.
 */
attn_status_t attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                       int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Skv, int64_t D,
                       float scale, int causal, attn_dtype_t dtype,
                       const float* q_descale, const float* k_descale, const float* v_descale,
                       void* stream);

/*
 * attn_fwd_chunk — attn_fwd over one chunk of keys that starts at absolute
 * key position kv_start (>= 0): with causal, key j of the chunk is allowed for
 * query i iff j + kv_start <= i. With kv_start = 0 it equals attn_fwd. The
 * (out, lse) of several chunks over disjoint key ranges combine with
 * attn_merge_lse2_host (two chunks) into the attention over their union, the
 * out/LSE merge the page "feat(attention): add strict bitwise ROCm path"
 * performs across context-parallel ranks (Summary table, CP communication).
 */
attn_status_t attn_fwd_chunk(const void* q, const void* k, const void* v, void* out, float* lse,
                             int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Skv, int64_t D,
                             float scale, int causal, attn_dtype_t dtype,
                             const float* q_descale, const float* k_descale, const float* v_descale,
                             int64_t kv_start, void* stream);

/*
 * attn_fwd_window — attn_fwd_chunk with local (sliding-window) attention and
 * attention sinks, the window_size_left / window_size_right arguments of the
 * fmha_v3_fwd call on the page "F8 fmha ASM gfx950" (Test Result section) and
 * the window / sink configurations of the page "[Proposal] ROCm (AMD
 * Instinct) support for the core attention and distributed init". With key
 * position j = (key index + kv_start), key j is allowed for query i iff
 *     (window_left < 0  or j >= i - window_left) and
 *     (window_right < 0 or j <= i + window_right),  or  j < sink,
 * and, with causal, also j <= i. window_left / window_right = -1 means that
 * side is unbounded; sink = 0 means no sink keys. All -1, -1, 0 is
 * attn_fwd_chunk. Key tiles no row of a workgroup can see are not read.
 * Errors as attn_fwd_chunk; ATTN_ERR_SHAPE for window sides < -1 or sink < 0.
 */
attn_status_t attn_fwd_window(const void* q, const void* k, const void* v, void* out, float* lse,
                              int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Skv, int64_t D,
                              float scale, int causal, attn_dtype_t dtype,
                              const float* q_descale, const float* k_descale, const float* v_descale,
                              int64_t kv_start, int64_t window_left, int64_t window_right, int64_t sink,
                              void* stream);

/*
 * attn_merge_lse2_host — merge two partial results on the HOST: the out/LSE
 * combination of attention over two key chunks that the page "feat(attention):
 * add strict bitwise ROCm path" performs across context-parallel ranks (Summary
 * table: the boundary returns (out, lse); Q/K/V all-gather then Out/LSE
 * reduce-scatter), here as a plain host routine run after the two chunk calls.
 *
 *   o1, o2, o_out  host bf16 bit patterns [B, H, S, D]
 *   lse1, lse2, lse_out  host fp32 [B, H, S] (natural log)
 *
 * For each row: L = ln(e^L1 + e^L2), O = e^(L1-L) O1 + e^(L2-L) O2, computed
 * in fp32 and rounded to bf16 (nearest even). Both L1 and L2 = -inf gives
 * O = 0, L = -inf. Output buffers may alias the inputs element for element.
 * Returns ATTN_ERR_NULL / ATTN_ERR_SHAPE on bad arguments; runs synchronously.
 */
attn_status_t attn_merge_lse2_host(const uint16_t* o1, const float* lse1,
                                   const uint16_t* o2, const float* lse2,
                                   uint16_t* o_out, float* lse_out,
                                   int64_t B, int64_t H, int64_t S, int64_t D);

/*
 * attn_fwd_splitkv — attn_fwd with the keys split over n_splits workgroup
 * sets, for shapes whose B * Hq * ceil(Sq / 256) query tiles leave the GPU's
 * compute units idle (few heads, short Sq against a long Skv). Each split
 * computes the (O, LSE) of its key range — the chunk semantics of
 * attn_fwd_chunk — into the caller's workspace as fp32, and a second kernel on
 * the same stream merges them by LSE into out (bf16) and lse, the N-way form
 * of the out/LSE merge on the page "feat(attention): add strict bitwise ROCm
 * path" (Summary table, CP communication). Results equal attn_fwd's up to
 * fp32 rounding of the partial sums.
 *
 *   n_splits        >= 1 splits of whole 64-key tiles (fewer are used when Skv
 *                   has fewer tiles); 1 is attn_fwd itself (no workspace is
 *                   read). 0 lets the library choose: a split of every query
 *                   tile when the grid leaves compute units idle, else, for
 *                   non-causal calls whose whole rounds of query tiles fill
 *                   every compute unit, a split of only the query tiles of the
 *                   last, partly filled round (the other rows are written
 *                   exactly as attn_fwd writes them), else none. At most 256.
 *   workspace       device buffer of at least attn_splitkv_workspace_bytes(B,
 *                   Hq, Sq, D, n) bytes, n = n_splits, or for n_splits = 0
 *                   n = attn_splitkv_auto_splits(...), 16-byte aligned, owned by the
 *                   caller; its contents on entry do not matter and are
 *                   overwritten. It may be NULL when one split is used.
 *   workspace_bytes its size in bytes.
 * Other arguments, layouts and errors as attn_fwd; ATTN_ERR_WORKSPACE when a
 * workspace is needed and is missing, misaligned or too small. Two calls that
 * overlap in time must not share a workspace.
 */
attn_status_t attn_fwd_splitkv(const void* q, const void* k, const void* v, void* out, float* lse,
                               int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Skv, int64_t D,
                               float scale, int causal, attn_dtype_t dtype,
                               const float* q_descale, const float* k_descale, const float* v_descale,
                               int64_t n_splits, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * attn_fwd_splitkv_static — attn_fwd_splitkv without a workspace argument, for
 * callers that cannot allocate device memory (code under stream/graph
 * capture, tight serving loops, harnesses that forbid allocation). The split
 * partials live in a static device array of ATTN_SPLITKV_STATIC_SCRATCH_BYTES
 * (64 MiB) that each GPU the library runs on holds until the process ends; the
 * call itself allocates nothing. The caller still passes inputs and outputs.
 * Arguments and results as attn_fwd_splitkv (n_splits = 0: the library's
 * choice); ATTN_ERR_WORKSPACE when the chosen split count needs more than the
 * array holds (attn_splitkv_workspace_bytes > 64 MiB; nothing is launched),
 * ATTN_ERR_HIP when the array's device address cannot be obtained. Every call
 * on one GPU shares that GPU's array: calls that overlap in time on one GPU
 * (different streams, or different threads) race and must not be issued.
 */
attn_status_t attn_fwd_splitkv_static(const void* q, const void* k, const void* v, void* out, float* lse,
                                      int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Skv, int64_t D,
                                      float scale, int causal, attn_dtype_t dtype,
                                      const float* q_descale, const float* k_descale, const float* v_descale,
                                      int64_t n_splits, void* stream);

/* Bytes of workspace attn_fwd_splitkv needs for n_splits (0 when n_splits <= 1;
 * n_splits * B * Hq * Sq * (D + 1) * 4), or -1 on invalid arguments. */
int64_t attn_splitkv_workspace_bytes(int64_t B, int64_t Hq, int64_t Sq, int64_t D, int64_t n_splits);

/* The split count attn_fwd_splitkv uses for n_splits = 0 on the current
 * device, for sizing its workspace. With T = B * Hq * ceil(Sq / 256) query
 * tiles of 256 rows (split calls always use 256-row tiles) and every split
 * at least 16 key tiles:
 *   - when T leaves more than 15 % of its last round over the compute units
 *     idle, the fewest splits of every tile, at most 16, that reach 90 %;
 *     if none does and T is below one round (a few query tiles against many
 *     keys), the count up to 256 with the least estimated time,
 *     rounds * (key tiles per split + 2) + 3 for the merge, or the fewest
 *     within 3 % of that;
 *   - else, when T is at least one round and the last round is partly empty,
 *     the k in 2..8 that splits only that round's tiles into the least time,
 *     ceil(tail * k / CUs) / k rounds, if that is at most 0.85 of a round
 *     (used by non-causal calls only; a causal call then runs unsplit);
 *   - else 1.
 * -1 on invalid arguments. Queries the current HIP device. */
int64_t attn_splitkv_auto_splits(int64_t B, int64_t Hq, int64_t Sq, int64_t Skv, int64_t D);

/*
 * attn_bwd — gradients of the attention forward (bf16): dQ, dK, dV, the
 * tensors the page "feat(attention): add strict bitwise ROCm path" checks next
 * to out and lse (Latest status) and whose deterministic backward it times
 * (section "What the strict contract costs"). With P the forward's softmax
 * (recomputed from q, k and lse) and D_i = sum_d dout[i,d] * out[i,d]:
 *     dv = P^T dout,   dS = P * (dout v^T - D),
 *     dq = scale * dS k,   dk = scale * dS^T q,
 * summed over the query heads of each KV head for dk and dv.
 *
 *   q, out, dout, dq  [B, Hq, Sq, D] bf16 (out and lse as attn_fwd returned
 *                     them for the same q, k, v, scale and causal)
 *   k, v, dk, dv      [B, Hkv, Skv, D] bf16
 *   lse               [B, Hq, Sq] fp32 (natural log, scale included)
 *   causal            top-left: key j is allowed for query i iff j <= i
 *   dtype             ATTN_BF16 only (ATTN_ERR_DTYPE otherwise)
 *   workspace         device buffer of at least attn_bwd_workspace_bytes(...)
 *                     bytes, 256-byte aligned, owned by the caller; its
 *                     contents on entry do not matter. It may be NULL when
 *                     that size is 0.
 * dq, dk, dv are written in full (zeros where nothing contributes); rows with
 * lse = -inf contribute nothing. The result is deterministic: no atomics,
 * every sum in a fixed order, so identical inputs give identical bits, and a
 * batch entry's gradients do not depend on the other entries. Two calls that
 * overlap in time must not share a workspace. Errors as attn_fwd;
 * ATTN_ERR_WORKSPACE when the workspace is missing, misaligned or too small.
 */
attn_status_t attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                       const float* lse, void* dq, void* dk, void* dv,
                       int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Skv, int64_t D,
                       float scale, int causal, attn_dtype_t dtype,
                       void* workspace, int64_t workspace_bytes, void* stream);

/*
 * attn_bwd_chunk — attn_bwd for one key chunk of a longer key sequence, the
 * backward of attn_fwd_chunk: key j of k / v sits at position j + kv_start
 * (>= 0) and, with causal, is allowed for query i iff j + kv_start <= i. out
 * and lse must be those of the attention over ALL keys (the merged result of
 * the chunks, as after the out/LSE merge on the page "feat(attention): add
 * strict bitwise ROCm path", Summary table), so that P and D are the full
 * softmax's. Then dk and dv are this chunk's gradients and dq is the chunk's
 * contribution: the full dQ is the sum of dq over the chunks. kv_start = 0 is
 * attn_bwd. Errors as attn_bwd; ATTN_ERR_SHAPE for kv_start < 0,
 * ATTN_ERR_OVERFLOW when kv_start + Skv reaches 2^30.
 */
attn_status_t attn_bwd_chunk(const void* q, const void* k, const void* v, const void* out, const void* dout,
                             const float* lse, void* dq, void* dk, void* dv,
                             int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Skv, int64_t D,
                             float scale, int causal, attn_dtype_t dtype, int64_t kv_start,
                             void* workspace, int64_t workspace_bytes, void* stream);

/* Bytes of workspace attn_bwd and attn_bwd_chunk need: 8 per query row (its LSE and D), plus
 * fp32 partial dK and dV per query head (8 * B * Hq * Skv * D) when grouped KV
 * heads are split over workgroups; -1 on invalid arguments. */
int64_t attn_bwd_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Skv, int64_t D);

/* Static, human-readable name of a status code (never NULL). Every entry point
 * fails closed with one of these codes rather than falling back to another
 * path, the refusal the page "feat(attention): add strict bitwise ROCm path"
 * asks of an unsupported request (Summary and Changes sections). */
const char* attn_status_string(attn_status_t s);

#ifdef __cplusplus
}
#endif

#endif /* HEAD_ATTENTION_AMD_ATTN_H */
