// Eq. (12) of the MISA summary page ("Methodology" 2, MISA-dagger fine
// stage): every candidate token kept by the routed pass is re-scored with all
// H heads (the Eq. (1) score) and the k best candidates are kept.
//
// A score kernel writes one fp32 score per (query, candidate) into the
// workspace (one thread per candidate, the query's H rows staged in LDS); a
// block radix select per query then picks the k winners among the valid
// (non-negative) candidates.
#include "common.hpp"
#include "launch.hpp"
#include "topk.hpp"

namespace misa {

namespace {

constexpr int kRerankThreads = 256;
constexpr int kTopkThreads = 1024;
constexpr int kMaxHeads = 64;

template <int DT>
__global__ __launch_bounds__(kRerankThreads) void rerank_score_kernel(
    const void* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    const void* __restrict__ k, const float* __restrict__ k_scale,
    const int32_t* __restrict__ cand, int32_t kprime, float* __restrict__ out, int32_t L,
    int32_t T, int32_t H) {
  __shared__ float qs[kMaxHeads][kD];
  __shared__ float wsh[kMaxHeads];
  const int t = blockIdx.y;
  const int64_t seq = blockIdx.z;
  const int64_t r = seq * T + t;
  const float sq = (DT == kFP8) ? q_scale[r] : 1.f;
  for (int e = threadIdx.x; e < H * kD; e += kRerankThreads)
    qs[e / kD][e % kD] = load_elem<DT>(q, r * H * kD + e) * sq;
  if (threadIdx.x < H) wsh[threadIdx.x] = w[r * H + threadIdx.x];
  __syncthreads();
  const int64_t c = static_cast<int64_t>(blockIdx.x) * kRerankThreads + threadIdx.x;
  if (c >= kprime) return;
  const int32_t s = cand[r * kprime + c];
  const int64_t pos = static_cast<int64_t>(L) - T + t;
  if (s < 0 || s > pos) {  // padding, or outside the query's prefix: ignored
    out[r * kprime + c] = -__builtin_inff();
    return;
  }
  float kr[kD];
  const float sk = (DT == kFP8) ? k_scale[seq * L + s] : 1.f;
#pragma unroll
  for (int i = 0; i < kD; ++i) kr[i] = load_elem<DT>(k, (seq * L + s) * kD + i) * sk;
  float acc = 0.f;
  for (int j = 0; j < H; ++j) {
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < kD; ++i) dot += qs[j][i] * kr[i];
    acc += wsh[j] * fmaxf(dot, 0.f);
  }
  out[r * kprime + c] = acc;
}

__global__ __launch_bounds__(kTopkThreads) void topk_list_kernel(const float* __restrict__ sc,
                                                                 const int32_t* __restrict__ cand,
                                                                 int32_t kprime, int32_t L,
                                                                 int32_t T, int32_t k,
                                                                 int32_t* __restrict__ idx,
                                                                 float* __restrict__ scores_out) {
  __shared__ TopkFastSmem sm;
  const int64_t r = static_cast<int64_t>(blockIdx.y) * T + blockIdx.x;
  const int64_t pos = static_cast<int64_t>(L) - T + blockIdx.x;
  const float* srow = sc + r * kprime;
  const int32_t* crow = cand + r * kprime;
  block_topk_fast<kTopkThreads>(
      kprime, k, [=](int64_t i) { return crow[i] >= 0 && crow[i] <= pos; },
      [=](int64_t i) { return srow[i]; }, [=](int64_t i) { return crow[i]; }, idx + r * k,
      scores_out ? scores_out + r * k : nullptr, sm);
}

}  // namespace

size_t rerank_ws_bytes(const Shape& s, int32_t kprime) {
  return align_up(static_cast<size_t>(s.batch) * s.T * kprime * sizeof(float));
}

hipError_t launch_rerank(const Shape& s, int32_t kprime, int32_t k, const void* q,
                         const float* q_scale, const float* w, const void* kk, const float* k_scale,
                         const int32_t* cand, int32_t* idx, float* scores_out, void* ws,
                         hipStream_t st) {
  float* sc = static_cast<float*>(ws);
  dim3 g1((kprime + kRerankThreads - 1) / kRerankThreads, s.T, s.batch);
  switch (s.dtype) {
    case kF32:
      rerank_score_kernel<kF32><<<g1, kRerankThreads, 0, st>>>(q, q_scale, w, kk, k_scale, cand,
                                                               kprime, sc, s.L, s.T, s.H);
      break;
    case kBF16:
      rerank_score_kernel<kBF16><<<g1, kRerankThreads, 0, st>>>(q, q_scale, w, kk, k_scale, cand,
                                                                kprime, sc, s.L, s.T, s.H);
      break;
    default:
      rerank_score_kernel<kFP8><<<g1, kRerankThreads, 0, st>>>(q, q_scale, w, kk, k_scale, cand,
                                                               kprime, sc, s.L, s.T, s.H);
      break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2(s.T, s.batch);
  topk_list_kernel<<<g2, kTopkThreads, 0, st>>>(sc, cand, kprime, s.L, s.T, k, idx, scores_out);
  return hipGetLastError();
}

}  // namespace misa
