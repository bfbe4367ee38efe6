// C ABI of the MISA indexer (declared in include/misa.h): argument checks on
// the host, workspace sizing, and dispatch to the kernels on the caller's
// stream.  Nothing here allocates device memory.
#include "misa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "launch.hpp"

namespace {

using misa::Shape;

constexpr int32_t kMaxTopk = 8192;
constexpr int32_t kMaxRouted = 16;
constexpr int32_t kMaxHeads = 64;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Validates the shape; on success fills `out`.
misa_status check_shape(const misa_shape* sh, Shape& out) {
  if (!sh) return MISA_ERR_INVALID_ARG;
  if (sh->batch < 1 || sh->L < 1 || sh->T < 1 || sh->T > sh->L || sh->H < 1 || sh->d < 1 ||
      sh->B < 1)
    return MISA_ERR_INVALID_ARG;
  if (sh->qk_dtype < MISA_F32 || sh->qk_dtype > MISA_FP8_E4M3) return MISA_ERR_INVALID_ARG;
  if (sh->d != 128 || sh->H > kMaxHeads) return MISA_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(sh->batch) * sh->T * sh->L >= (int64_t{1} << 40))
    return MISA_ERR_UNSUPPORTED;
  out = Shape{sh->batch, sh->L, sh->T, sh->H, sh->d, sh->B, sh->qk_dtype};
  return MISA_OK;
}

misa_status check_inputs(const Shape& s, const void* q, const float* q_scale, const float* w,
                         const void* k, const float* k_scale) {
  if (!q || !w || !k || !aligned16(q) || !aligned16(w) || !aligned16(k))
    return MISA_ERR_INVALID_ARG;
  if (s.dtype == MISA_FP8_E4M3 &&
      (!q_scale || !k_scale || !aligned16(q_scale) || !aligned16(k_scale)))
    return MISA_ERR_INVALID_ARG;
  return MISA_OK;
}

misa_status check_out(const void* p, bool required) {
  if (!p) return required ? MISA_ERR_INVALID_ARG : MISA_OK;
  return aligned16(p) ? MISA_OK : MISA_ERR_INVALID_ARG;
}

misa_status check_topk(int32_t k) {
  if (k < 1) return MISA_ERR_INVALID_ARG;
  if (k > kMaxTopk) return MISA_ERR_UNSUPPORTED;
  return MISA_OK;
}

misa_status check_ws(const void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return MISA_OK;
  if (!ws || ws_bytes < need) return MISA_ERR_WORKSPACE;
  if (!aligned16(ws)) return MISA_ERR_INVALID_ARG;
  return MISA_OK;
}

misa_status from_hip(hipError_t e) { return e == hipSuccess ? MISA_OK : MISA_ERR_HIP; }

#define MISA_TRY(expr)                   \
  do {                                   \
    const misa_status st_ = (expr);      \
    if (st_ != MISA_OK) return st_;      \
  } while (0)

// Argument checks of the decode step (both forms); fills `s` on success.
misa_status check_decode_step(const misa_shape* shape, int32_t h, int32_t k, const void* q,
                              const float* q_scale, const float* w, const float* pooled,
                              const void* kk, const float* k_scale, const int32_t* heads,
                              const float* E_out, const int32_t* idx, const float* scores_out,
                              Shape& s) {
  MISA_TRY(check_shape(shape, s));
  if (h < 1 || h > s.H) return MISA_ERR_INVALID_ARG;
  if (h > kMaxRouted || s.T != 1 || s.dtype == MISA_F32) return MISA_ERR_UNSUPPORTED;
  MISA_TRY(check_topk(k));
  MISA_TRY(check_inputs(s, q, q_scale, w, kk, k_scale));
  MISA_TRY(check_out(pooled, true));
  MISA_TRY(check_out(heads, true));
  MISA_TRY(check_out(E_out, false));
  MISA_TRY(check_out(idx, true));
  MISA_TRY(check_out(scores_out, false));
  if (s.batch > 65535) return MISA_ERR_UNSUPPORTED;
  return MISA_OK;
}

}  // namespace

extern "C" {

size_t misa_workspace_bytes(const misa_shape* shape, int32_t h, int32_t k, int32_t kprime) {
  Shape s;
  if (check_shape(shape, s) != MISA_OK) return 0;
  const int32_t kp = std::max(k, kprime);
  size_t need = misa::route_ws_bytes(s);
  // Score workspace for both selection sizes: the prefill candidate
  // capacity is not monotone in k (a larger k can take a lower sampling
  // margin), so the smaller k may need more than the larger.
  for (const int32_t kk : {k, kp}) {
    if (kk < 1) continue;
    need = std::max(need, misa::score_ws_bytes(s, std::max<int32_t>(h, 1), kk));
    need = std::max(need, misa::score_ws_bytes(s, s.H, kk));
  }
  need = std::max(need, misa::rerank_ws_bytes(s, kp));
  if (s.T == 1 && s.dtype != MISA_F32) need = std::max(need, misa::decode_ws_bytes(s));
  return need;
}

misa_status misa_pool_keys_range(const misa_shape* shape, int32_t block_begin,
                                 int32_t block_count, const void* k, const float* k_scale,
                                 float* pooled, hipStream_t stream) {
  Shape s;
  MISA_TRY(check_shape(shape, s));
  if (block_begin < 0 || block_count < 0 ||
      static_cast<int64_t>(block_begin) + block_count > s.M())
    return MISA_ERR_INVALID_ARG;
  if (!k || !aligned16(k)) return MISA_ERR_INVALID_ARG;
  if (s.dtype == MISA_FP8_E4M3 && (!k_scale || !aligned16(k_scale))) return MISA_ERR_INVALID_ARG;
  MISA_TRY(check_out(pooled, true));
  if (block_count > 65535 * 256 || s.batch > 65535) return MISA_ERR_UNSUPPORTED;
  return from_hip(misa::launch_pool(s, block_begin, block_count, k, k_scale, pooled, stream));
}

misa_status misa_pool_keys(const misa_shape* shape, const void* k, const float* k_scale,
                           float* pooled, hipStream_t stream) {
  Shape s;
  MISA_TRY(check_shape(shape, s));
  return misa_pool_keys_range(shape, 0, static_cast<int32_t>(s.M()), k, k_scale, pooled, stream);
}

misa_status misa_route(const misa_shape* shape, int32_t h, const void* q, const float* q_scale,
                       const float* w, const float* pooled, const void* k, const float* k_scale,
                       int32_t* heads, float* E_out, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  Shape s;
  MISA_TRY(check_shape(shape, s));
  if (h < 1 || h > s.H) return MISA_ERR_INVALID_ARG;
  if (h > kMaxRouted) return MISA_ERR_UNSUPPORTED;
  MISA_TRY(check_inputs(s, q, q_scale, w, k, k_scale));
  if (!pooled || !aligned16(pooled)) return MISA_ERR_INVALID_ARG;
  MISA_TRY(check_out(heads, true));
  MISA_TRY(check_out(E_out, false));
  MISA_TRY(check_ws(ws, ws_bytes, misa::route_ws_bytes(s)));
  if (s.batch > 65535) return MISA_ERR_UNSUPPORTED;
  return from_hip(
      misa::launch_route(s, h, q, q_scale, w, pooled, k, k_scale, heads, E_out, ws, stream));
}

misa_status misa_score_topk(const misa_shape* shape, int32_t h, int32_t k, const void* q,
                            const float* q_scale, const float* w, const void* kk,
                            const float* k_scale, const int32_t* heads, int32_t* idx,
                            float* scores_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  Shape s;
  MISA_TRY(check_shape(shape, s));
  if (h < 1 || h > s.H) return MISA_ERR_INVALID_ARG;
  if (h > kMaxRouted) return MISA_ERR_UNSUPPORTED;
  MISA_TRY(check_topk(k));
  MISA_TRY(check_inputs(s, q, q_scale, w, kk, k_scale));
  if (!heads || !aligned16(heads)) return MISA_ERR_INVALID_ARG;
  MISA_TRY(check_out(idx, true));
  MISA_TRY(check_out(scores_out, false));
  MISA_TRY(check_ws(ws, ws_bytes, misa::score_ws_bytes(s, h, k)));
  if (s.batch > 65535 || s.T > 65535) return MISA_ERR_UNSUPPORTED;
  return from_hip(misa::launch_score_topk(s, h, heads, k, q, q_scale, w, kk, k_scale, idx,
                                          scores_out, ws, stream));
}

misa_status misa_decode_step(const misa_shape* shape, int32_t h, int32_t k, const void* q,
                             const float* q_scale, const float* w, float* pooled, const void* kk,
                             const float* k_scale, int32_t* heads, float* E_out, int32_t* idx,
                             float* scores_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  Shape s;
  MISA_TRY(check_decode_step(shape, h, k, q, q_scale, w, pooled, kk, k_scale, heads, E_out, idx,
                             scores_out, s));
  MISA_TRY(check_ws(ws, ws_bytes, misa::decode_ws_bytes(s)));
  return from_hip(misa::launch_decode_step(s, h, k, q, q_scale, w, pooled, kk, k_scale, heads,
                                           E_out, idx, scores_out, ws, stream));
}

misa_status misa_decode_step_noalloc(const misa_shape* shape, int32_t h, int32_t k,
                                     const void* q, const float* q_scale, const float* w,
                                     float* pooled, const void* kk, const float* k_scale,
                                     int32_t* heads, float* E_out, int32_t* idx,
                                     float* scores_out, hipStream_t stream) {
  Shape s;
  MISA_TRY(check_decode_step(shape, h, k, q, q_scale, w, pooled, kk, k_scale, heads, E_out, idx,
                             scores_out, s));
  static_assert(misa::kStaticScratchBytes == MISA_NOALLOC_SCRATCH_BYTES, "header limit");
  if (misa::decode_ws_bytes(s) > misa::kStaticScratchBytes) return MISA_ERR_UNSUPPORTED;
  void* ws = nullptr;
  MISA_TRY(from_hip(misa::static_scratch(&ws)));
  return from_hip(misa::launch_decode_step(s, h, k, q, q_scale, w, pooled, kk, k_scale, heads,
                                           E_out, idx, scores_out, ws, stream));
}


misa_status dsa_index_dense(const misa_shape* shape, int32_t k, const void* q,
                            const float* q_scale, const float* w, const void* kk,
                            const float* k_scale, int32_t* idx, float* scores_out, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  Shape s;
  MISA_TRY(check_shape(shape, s));
  MISA_TRY(check_topk(k));
  MISA_TRY(check_inputs(s, q, q_scale, w, kk, k_scale));
  MISA_TRY(check_out(idx, true));
  MISA_TRY(check_out(scores_out, false));
  MISA_TRY(check_ws(ws, ws_bytes, misa::score_ws_bytes(s, s.H, k)));
  if (s.batch > 65535 || s.T > 65535) return MISA_ERR_UNSUPPORTED;
  return from_hip(misa::launch_score_topk(s, s.H, nullptr, k, q, q_scale, w, kk, k_scale, idx,
                                          scores_out, ws, stream));
}

misa_status misa_rerank(const misa_shape* shape, int32_t kprime, int32_t k, const void* q,
                        const float* q_scale, const float* w, const void* kk, const float* k_scale,
                        const int32_t* cand, int32_t* idx, float* scores_out, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
  Shape s;
  MISA_TRY(check_shape(shape, s));
  MISA_TRY(check_topk(k));
  if (kprime < k) return MISA_ERR_INVALID_ARG;
  if (kprime > kMaxTopk) return MISA_ERR_UNSUPPORTED;
  MISA_TRY(check_inputs(s, q, q_scale, w, kk, k_scale));
  if (!cand || !aligned16(cand)) return MISA_ERR_INVALID_ARG;
  MISA_TRY(check_out(idx, true));
  MISA_TRY(check_out(scores_out, false));
  MISA_TRY(check_ws(ws, ws_bytes, misa::rerank_ws_bytes(s, kprime)));
  if (s.batch > 65535 || s.T > 65535) return MISA_ERR_UNSUPPORTED;
  return from_hip(misa::launch_rerank(s, kprime, k, q, q_scale, w, kk, k_scale, cand, idx,
                                      scores_out, ws, stream));
}

size_t misa_hisa_workspace_bytes(const misa_shape* shape, int32_t h, int32_t m, int32_t k) {
  Shape s;
  if (check_shape(shape, s) != MISA_OK || h < 1 || m < 1 || k < 1) return 0;
  if (check_topk(k) != MISA_OK) return 0;
  return misa::hisa_ws_bytes(s, m, k);
}

misa_status misa_hisa_score_topk(const misa_shape* shape, int32_t h, int32_t m, int32_t k,
                                 const void* q, const float* q_scale, const float* w,
                                 const float* pooled, const void* kk, const float* k_scale,
                                 const int32_t* heads, int32_t* blocks_out,
                                 float* block_scores_out, int32_t* idx, float* scores_out,
                                 void* ws, size_t ws_bytes, hipStream_t stream) {
  Shape s;
  MISA_TRY(check_shape(shape, s));
  if (h < 1 || h > s.H || m < 1) return MISA_ERR_INVALID_ARG;
  if (h > kMaxRouted) return MISA_ERR_UNSUPPORTED;
  MISA_TRY(check_topk(k));
  MISA_TRY(check_inputs(s, q, q_scale, w, kk, k_scale));
  if (!pooled || !aligned16(pooled) || !heads || !aligned16(heads)) return MISA_ERR_INVALID_ARG;
  MISA_TRY(check_out(blocks_out, false));
  MISA_TRY(check_out(block_scores_out, false));
  MISA_TRY(check_out(idx, true));
  MISA_TRY(check_out(scores_out, false));
  if (!misa::hisa_supported(s, m) || s.batch > 65535 || s.T > 65535) return MISA_ERR_UNSUPPORTED;
  MISA_TRY(check_ws(ws, ws_bytes, misa::hisa_ws_bytes(s, m, k)));
  return from_hip(misa::launch_hisa_score_topk(s, h, heads, m, k, q, q_scale, w, pooled, kk,
                                               k_scale, blocks_out, block_scores_out, idx,
                                               scores_out, ws, stream));
}

const char* misa_status_string(misa_status status) {
  switch (status) {
    case MISA_OK: return "MISA_OK";
    case MISA_ERR_INVALID_ARG: return "MISA_ERR_INVALID_ARG";
    case MISA_ERR_UNSUPPORTED: return "MISA_ERR_UNSUPPORTED";
    case MISA_ERR_WORKSPACE: return "MISA_ERR_WORKSPACE";
    case MISA_ERR_HIP: return "MISA_ERR_HIP";
  }
  return "MISA_ERR_UNKNOWN";
}

}  // extern "C"
