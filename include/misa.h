/*
 * misa.h -- C ABI of the MISA indexer library for AMD Instinct MI355X (gfx950).
 *
 * MISA (Mixture of Indexer Sparse Attention) replaces the DeepSeek Sparse
 * Attention (DSA) token indexer: a block-pooled router picks, per query, the
 * h most useful of the H indexer heads, and only those heads score the
 * query's causal prefix before the top-k token selection.  Source: the MISA
 * summary page ("MISA: Mixture of Indexer Sparse Attention for Long-Context
 * LLM Inference"), Eq. (1)-(2) in "Introduction and Theoretical Foundation",
 * Eq. (4), (7)-(10) in "Methodology" 1, Eq. (11)-(12) in "Methodology" 2.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer is a DEVICE pointer owned by the caller.  The library never
 *    allocates or frees device memory; scratch space is the caller's `ws`
 *    buffer of `ws_bytes` bytes (size it with misa_workspace_bytes()).
 *  - Arrays are dense row-major with the shapes given below and 16-byte
 *    aligned base addresses.  Element types: q and k are `shape->qk_dtype`
 *    (fp32, bf16, or OCP fp8 e4m3fn); w, scales, pooled keys, E and scores
 *    are fp32; indices are int32.
 *  - Sequence b holds L keys; its T queries sit at positions L-T .. L-1, and
 *    query t sees the causal prefix of keys 0 .. L-T+t (its own position
 *    included), n_t = L-T+t+1 keys.  Decode is T = 1.
 *  - fp8 inputs carry one fp32 scale per query token, q_scale [batch, T], and
 *    one per key token, k_scale [batch, L]: value = code * scale, scale > 0.
 *    For fp32/bf16 inputs the scale pointers are ignored and may be NULL.
 *  - Calls are asynchronous on `stream` (NULL = the default stream).  Argument
 *    checks run on the host before anything is launched; a failed check
 *    returns its status and launches nothing.  A launch failure returns
 *    MISA_ERR_HIP.  The library keeps no mutable global state: calls on
 *    different streams are independent when their workspaces are distinct.
 *    The only state carried between calls lives in the caller's `ws` (see
 *    misa_decode_step); no result ever depends on it.
 *  - Limits of this build: d = 128; 1 <= H <= 64; 1 <= h <= min(H, 16);
 *    1 <= k <= k' <= 8192; B >= 1; 1 <= T <= L < 2^31; batch*T*max(L,k')
 *    < 2^40.  Violations return MISA_ERR_UNSUPPORTED (a limit of this build)
 *    or MISA_ERR_INVALID_ARG (an argument no build accepts).
 *  - Selected-token outputs have SET semantics: the order of the k slots is
 *    unspecified; when n_t < k the trailing slots hold index -1 and score
 *    -INFINITY.  Among tokens with bit-identical fp32 scores the lower token
 *    index is kept.
 */
#ifndef MISA_H
#define MISA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MISA_OK = 0,
  MISA_ERR_INVALID_ARG = -1, /* a null/misaligned pointer or an impossible size */
  MISA_ERR_UNSUPPORTED = -2, /* a valid request outside this build's limits   */
  MISA_ERR_WORKSPACE = -3,   /* ws is NULL or smaller than required            */
  MISA_ERR_HIP = -4          /* a HIP launch or runtime call failed            */
} misa_status;

typedef enum {
  MISA_F32 = 0,
  MISA_BF16 = 1,
  MISA_FP8_E4M3 = 2 /* OCP e4m3fn: bias 7, max 448, no infinities */
} misa_dtype;

/* Problem shape.  H is the number of indexer heads (H^I on the page), d the
 * head dimension, B the router block size, qk_dtype a misa_dtype. */
typedef struct {
  int32_t batch, L, T, H, d, B;
  int32_t qk_dtype;
} misa_shape;

/* Bytes of workspace that suffice for every entry point below called with
 * this shape and these h, k, k' (pass kprime = k when MISA-dagger is unused).
 * Returns 0 for an invalid shape. */
size_t misa_workspace_bytes(const misa_shape* shape, int32_t h, int32_t k, int32_t kprime);

/* Eq. (4): pooled[b, m, :] = mean of k[b, s, :] over the block
 * s in [m*B, min((m+1)*B, L)), for m < M = ceil(L/B).  The last block may be
 * partial (mean over its actual members).  fp8 keys are dequantised first.
 *   k        [batch, L, d]   qk_dtype
 *   k_scale  [batch, L]      fp32 (fp8 only)
 *   pooled   [batch, M, d]   fp32, written
 * In decode the pooled keys are a cache: call once per sequence and again
 * only for blocks that changed (see misa_pool_keys_range). */
misa_status misa_pool_keys(const misa_shape* shape, const void* k, const float* k_scale,
                           float* pooled, hipStream_t stream);

/* Eq. (4) restricted to blocks [block_begin, block_begin + block_count) of
 * every sequence: the incremental update of the decode cache when new keys
 * land in the last block.  Same layouts as misa_pool_keys; other blocks of
 * `pooled` are left untouched.  block_begin + block_count must be <= M. */
misa_status misa_pool_keys_range(const misa_shape* shape, int32_t block_begin, int32_t block_count,
                                 const void* k, const float* k_scale, float* pooled,
                                 hipStream_t stream);

/* Eq. (7)-(8), the block-pooled router.  For query t with n_t = L-T+t+1:
 *   E[b,t,j] = (1/M_t) * sum_{m < M_t} |w[b,t,j] * ReLU(q[b,t,j,:] . p_m)|,
 * M_t = ceil(n_t/B), where p_m = pooled[b,m,:] for the floor(n_t/B) blocks
 * lying wholly in the prefix and, when B does not divide n_t, the last p_m is
 * the mean of keys floor(n_t/B)*B .. n_t-1 (computed here from k).  Then
 * heads[b,t,:] = the h heads of largest E (ties: lower head), ascending.
 *   q        [batch, T, H, d]  qk_dtype      q_scale [batch, T] (fp8 only)
 *   w        [batch, T, H]     fp32
 *   pooled   [batch, M, d]     fp32 (from misa_pool_keys)
 *   k        [batch, L, d]     qk_dtype      k_scale [batch, L] (fp8 only)
 *   heads    [batch, T, h]     int32, written (ascending)
 *   E_out    [batch, T, H]     fp32, written if non-NULL */
misa_status misa_route(const misa_shape* shape, int32_t h, const void* q, const float* q_scale,
                       const float* w, const float* pooled, const void* k, const float* k_scale,
                       int32_t* heads, float* E_out, void* ws, size_t ws_bytes, hipStream_t stream);

/* Eq. (9)-(10) (Eq. (11) when called with k = k'):
 *   I[b,t,s] = sum_{j in heads[b,t,:]} w[b,t,j] * ReLU(q[b,t,j,:] . k[b,s,:])
 * for s in 0 .. n_t-1, then idx[b,t,:] = the k tokens of largest I.
 *   heads      [batch, T, h]  int32 head ids in [0, H) (e.g. from misa_route)
 *   idx        [batch, T, k]  int32, written (set semantics, -1 padding)
 *   scores_out [batch, T, k]  fp32 I of each idx slot, written if non-NULL */
misa_status misa_score_topk(const misa_shape* shape, int32_t h, int32_t k, const void* q,
                            const float* q_scale, const float* w, const void* kk,
                            const float* k_scale, const int32_t* heads, int32_t* idx,
                            float* scores_out, void* ws, size_t ws_bytes, hipStream_t stream);

/* Eq. (12), the fine stage of MISA-dagger: for every candidate s in
 * cand[b,t,:] (entries < 0 are padding and ignored), the full-head score
 *   I[b,t,s] = sum_{j < H} w[b,t,j] * ReLU(q[b,t,j,:] . k[b,s,:]),
 * then idx[b,t,:] = the k candidates of largest I.  Candidates must be
 * distinct token positions within query t's prefix.  Key rows are gathered
 * in list order, so a list sorted by token position runs faster (prefill
 * lists of misa_score_topk come out that way, apart from the few entries of
 * the threshold bin at their end); the result does not depend on the order.
 *   cand       [batch, T, kprime]  int32 (e.g. idx of misa_score_topk with k')
 *   idx        [batch, T, k]       int32, written
 *   scores_out [batch, T, k]       fp32, written if non-NULL */
misa_status misa_rerank(const misa_shape* shape, int32_t kprime, int32_t k, const void* q,
                        const float* q_scale, const float* w, const void* kk, const float* k_scale,
                        const int32_t* cand, int32_t* idx, float* scores_out, void* ws,
                        size_t ws_bytes, hipStream_t stream);

/* One decode step of MISA (T = 1; bf16 or fp8 only): Eq. (4) for the block
 * holding the newest key, then Eq. (7)-(8) and Eq. (9)-(10) -- the results of
 *   misa_pool_keys_range(shape, M-1, 1, ...); misa_route(...); misa_score_topk(...)
 * in two kernel launches (three when batch < 8).
 *   pooled   [batch, M, d]  fp32, read and written: blocks 0 .. M-2 must hold
 *            their Eq. (4) means (the cache kept by misa_pool_keys); block
 *            M-1 (keys (M-1)*B .. L-1, possibly partial) is recomputed from k
 *            and written.
 *   heads    [batch, h]     int32, written (ascending)
 *   E_out    [batch, H]     fp32, written if non-NULL
 *   idx, scores_out [batch, k] as misa_score_topk.
 * Other arguments and layouts as misa_route and misa_score_topk.  T != 1 or
 * fp32 inputs return MISA_ERR_UNSUPPORTED.
 *
 * State in `ws` (batch >= 8, the single-kernel form): the G workgroups of a
 * sequence share their router partial sums through `ws`, using one 64-bit
 * arrival word per sequence that this call's select kernel re-arms for the
 * NEXT call on the same `ws`.  A call whose `ws` is fresh (first call), was
 * used in between by another entry point, or was sized for another shape
 * finds no armed word: every workgroup then computes all router partials
 * itself (same additions in the same order, so the same result bits) and
 * the call is slower (about the router cost times G).  An armed word whose
 * peers are late makes a workgroup poll it up to 65536 times (with short
 * sleeps) before it takes the same local path, so one call never waits on
 * another.  Two calls that overlap on one `ws` race and are not allowed. */
misa_status misa_decode_step(const misa_shape* shape, int32_t h, int32_t k, const void* q,
                             const float* q_scale, const float* w, float* pooled, const void* kk,
                             const float* k_scale, int32_t* heads, float* E_out, int32_t* idx,
                             float* scores_out, void* ws, size_t ws_bytes, hipStream_t stream);

/* misa_decode_step for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments (minus ws), checks and results as
 * misa_decode_step; the workspace is a fixed device array inside the library,
 * MISA_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, which each GPU the library
 * runs on holds until the process ends.  Nothing is allocated by the call
 * (no hipMalloc, no allocating library routine).
 *   - A shape whose decode workspace exceeds the array returns
 *     MISA_ERR_UNSUPPORTED and launches nothing.  The need is batch * L * 4
 *     bytes of scores, about 9 MB of digit histograms when batch >= 8 (34 KB
 *     per sequence below that) and about 17 KB per sequence: batch 32 x
 *     L 32768 takes 13.6 MB, batch 8 x L 131072 13.1 MB, batch 64 x
 *     L 131072 43.9 MB, batch 1 x L 2^20 4.3 MB.
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents (including the router arrival words documented at
 *     misa_decode_step).  Calls that overlap in time on one GPU -- on
 *     different streams, or from different threads -- race and give wrong
 *     results: serialise them.
 *   - The first call on each device looks up the array's device address
 *     (hipGetSymbolAddress, no allocation); a failure returns MISA_ERR_HIP. */
#define MISA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
misa_status misa_decode_step_noalloc(const misa_shape* shape, int32_t h, int32_t k, const void* q,
                                     const float* q_scale, const float* w, float* pooled,
                                     const void* kk, const float* k_scale, int32_t* heads,
                                     float* E_out, int32_t* idx, float* scores_out,
                                     hipStream_t stream);

/* Eq. (1)-(2), the dense DSA indexer baseline: Eq. (9)-(10) with every head
 * j < H, no router.  Layouts as misa_score_topk. */
misa_status dsa_index_dense(const misa_shape* shape, int32_t k, const void* q,
                            const float* q_scale, const float* w, const void* kk,
                            const float* k_scale, int32_t* idx, float* scores_out, void* ws,
                            size_t ws_bytes, hipStream_t stream);

/* MISA x HISA ("Methodology" 1, "Key distinction from HISA"; "Theoretical
 * and Practical Implications", "Scalability"): the Eq. (7) affinities
 * A = w * ReLU(q . p) reduced across the heads instead of the blocks pick the
 * query's top-m blocks, and the routed scoring of Eq. (9) runs only over their
 * tokens.  For query t (n_t = L-T+t+1, the same causal blocks as misa_route):
 *   G[b,t,blk] = sum_{j < H} w[b,t,j] * ReLU(q[b,t,j,:] . p_blk),  blk < M_t
 *   the m blocks of largest G (ties: lower block; all M_t when M_t <= m)
 *   I[b,t,s] = sum_{j in heads[b,t,:]} w[b,t,j] * ReLU(q[b,t,j,:] . k[b,s,:])
 *              for the tokens s <= L-T+t of those blocks
 *   idx[b,t,:] = the k of those tokens with the largest I (ties: lower token;
 *                -1 / -INFINITY padding when they are fewer than k).
 *   pooled            [batch, M, d]  fp32 (misa_pool_keys)
 *   heads             [batch, T, h]  int32 (misa_route)
 *   blocks_out        [batch, T, m]  int32, written if non-NULL: the blocks,
 *                     ascending, -1 padding
 *   block_scores_out  [batch, T, m]  fp32, written if non-NULL: G of each slot
 *   idx, scores_out   [batch, T, k]  as misa_score_topk
 * Limits: bf16 or fp8 inputs, h <= 16, k <= 8192, m * B <= 8192, one
 * sequence's keys below 2 GiB; otherwise MISA_ERR_UNSUPPORTED (h > H, m < 1,
 * k < 1 or a NULL/misaligned input: MISA_ERR_INVALID_ARG).  ws must hold
 * misa_hisa_workspace_bytes(shape, h, m, k) bytes (0 for invalid arguments);
 * it carries nothing from one call to the next. */
size_t misa_hisa_workspace_bytes(const misa_shape* shape, int32_t h, int32_t m, int32_t k);
misa_status misa_hisa_score_topk(const misa_shape* shape, int32_t h, int32_t m, int32_t k,
                                 const void* q, const float* q_scale, const float* w,
                                 const float* pooled, const void* kk, const float* k_scale,
                                 const int32_t* heads, int32_t* blocks_out,
                                 float* block_scores_out, int32_t* idx, float* scores_out,
                                 void* ws, size_t ws_bytes, hipStream_t stream);

/* A static, human-readable name of a status code. */
const char* misa_status_string(misa_status status);

#ifdef __cplusplus
}
#endif

#endif /* MISA_H */
