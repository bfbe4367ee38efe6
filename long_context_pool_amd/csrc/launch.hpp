// Host-side launchers of the MISA kernels (internal; the public ABI is misa.h).
// Each returns the hipError_t of its launch(es).  Arguments were validated by
// the caller (api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace misa {

struct Shape {
  int32_t batch, L, T, H, d, B, dtype;
  int64_t M() const { return (static_cast<int64_t>(L) + B - 1) / B; }
};

hipError_t launch_pool(const Shape& s, int32_t block_begin, int32_t block_count, const void* k,
                       const float* k_scale, float* pooled, hipStream_t st);

// Router: E and top-h heads.  ws must hold route_ws_bytes(s).
size_t route_ws_bytes(const Shape& s);
hipError_t launch_route(const Shape& s, int32_t h, const void* q, const float* q_scale,
                        const float* w, const float* pooled, const void* k, const float* k_scale,
                        int32_t* heads, float* E_out, void* ws, hipStream_t st);

// Router on the matrix cores (bf16/fp8 inputs); no workspace.
bool route_mfma_supported(const Shape& s);
size_t route_mfma_ws_bytes(const Shape& s);
hipError_t launch_route_mfma(const Shape& s, int32_t h, const void* q, const float* q_scale,
                             const float* w, const float* pooled, const void* k,
                             const float* k_scale, int32_t* heads, float* E_out, void* ws,
                             hipStream_t st);

// Decode router (T == 1) on the vector ALU: chunked partial sums + finalize.
size_t route_decode_ws_bytes(const Shape& s);
hipError_t launch_route_decode(const Shape& s, int32_t h, const void* q, const float* q_scale,
                               const float* w, const float* pooled, const void* k,
                               const float* k_scale, int32_t* heads, float* E_out, void* ws,
                               hipStream_t st);

// Token scoring + top-k over each query's causal prefix.  heads == nullptr
// scores with all H heads (dense DSA); otherwise with the nh listed heads.
size_t score_ws_bytes(const Shape& s, int32_t nh, int32_t k);
hipError_t launch_score_topk(const Shape& s, int32_t nh, const int32_t* heads, int32_t k,
                             const void* q, const float* q_scale, const float* w, const void* kk,
                             const float* k_scale, int32_t* idx, float* scores_out, void* ws,
                             hipStream_t st);

// Decode (T == 1, bf16/fp8) token scoring + top-k: MFMA key streaming, then a
// per-sequence select.  ws must hold decode_ws_bytes(s).
size_t decode_ws_bytes(const Shape& s);
hipError_t launch_decode_score_topk(const Shape& s, int32_t nh, const int32_t* heads, int32_t k,
                                    const void* q, const float* q_scale, const float* w,
                                    const void* kk, const float* k_scale, int32_t* idx,
                                    float* scores_out, void* ws, hipStream_t st);

// Multi-query decode (2 <= T <= 8 queries at the end of each sequence,
// bf16/fp8, nh <= 16): every key read once for all T queries, then a row
// histogram and the decode select per (sequence, query).  ws must hold
// decode_mq_ws_bytes(s).
bool decode_mq_supported(const Shape& s, int32_t nh);
size_t decode_mq_ws_bytes(const Shape& s);
hipError_t launch_decode_mq_score_topk(const Shape& s, int32_t nh, const int32_t* heads, int32_t k,
                                       const void* q, const float* q_scale, const float* w,
                                       const void* kk, const float* k_scale, int32_t* idx,
                                       float* scores_out, void* ws, hipStream_t st);

// Fused decode step (T == 1, bf16/fp8): refresh the pooled key of the block
// holding key L-1, route (E, top-h) and score + top-k; two kernels.  ws must
// hold decode_ws_bytes(s).
hipError_t launch_decode_step(const Shape& s, int32_t h, int32_t k, const void* q,
                              const float* q_scale, const float* w, float* pooled, const void* kk,
                              const float* k_scale, int32_t* heads, float* E_out, int32_t* idx,
                              float* scores_out, void* ws, hipStream_t st);

// Prefill (T > 1, bf16/fp8) token scoring + top-k on 32x32 MFMA tiles with
// sampled thresholds, certified candidate selection and a repair path.
bool prefill_supported(const Shape& s);
size_t prefill_ws_bytes(const Shape& s, int32_t nh, int32_t k);
hipError_t launch_prefill_score_topk(const Shape& s, int32_t nh, const int32_t* heads, int32_t k,
                                     const void* q, const float* q_scale, const float* w,
                                     const void* kk, const float* k_scale, int32_t* idx,
                                     float* scores_out, void* ws, hipStream_t st);

// MISA-dagger fine stage.
size_t rerank_ws_bytes(const Shape& s, int32_t kprime);
hipError_t launch_rerank(const Shape& s, int32_t kprime, int32_t k, const void* q,
                         const float* q_scale, const float* w, const void* kk, const float* k_scale,
                         const int32_t* cand, int32_t* idx, float* scores_out, void* ws,
                         hipStream_t st);

// The re-rank with a list of heads per query (heads [batch*T, nh]; nullptr:
// every head) -- the routed scoring over a candidate list.  m > 0: `cand`
// holds m blocks per query ([batch*T, m]) whose B tokens each are the first
// m B of the kprime candidates (the rest padding); needs a head list of at
// most 16.  Head lists and blocks: bf16/fp8 keys within a buffer
// descriptor's reach only.
hipError_t launch_rerank_heads(const Shape& s, int32_t kprime, int32_t k, const void* q,
                               const float* q_scale, const float* w, const void* kk,
                               const float* k_scale, const int32_t* cand, int32_t m,
                               const int32_t* heads, int32_t nh, int32_t* idx, float* scores_out,
                               void* ws, hipStream_t st);

// Pooled keys -> bf16 hi and lo planes [batch*M, 128] (the router's B
// operand).
hipError_t launch_pooled_split(const Shape& s, const float* pooled, uint16_t* hi, uint16_t* lo,
                               hipStream_t st);

// MISA x HISA: block scores G (Eq. (7) affinities summed over heads), the
// top-m blocks, and the routed top-k over their tokens.
bool hisa_supported(const Shape& s, int32_t m);
size_t hisa_ws_bytes(const Shape& s, int32_t m, int32_t k);
hipError_t launch_hisa_score_topk(const Shape& s, int32_t nh, const int32_t* heads, int32_t m,
                                  int32_t k, const void* q, const float* q_scale, const float* w,
                                  const float* pooled, const void* kk, const float* k_scale,
                                  int32_t* blocks_out, float* block_scores_out, int32_t* idx,
                                  float* scores_out, void* ws, hipStream_t st);

inline size_t align_up(size_t x, size_t a = 256) { return (x + a - 1) / a * a; }

// The fixed device scratch of the no-allocation decode step: its size, and
// this device's address of it (looked up on the first call on each device).
constexpr size_t kStaticScratchBytes = size_t{64} << 20;
hipError_t static_scratch(void** ptr);

}  // namespace misa
