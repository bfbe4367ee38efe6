// Eq. (9)-(10) (routed heads) and Eq. (1)-(2) (all heads, dense DSA) of the
// MISA summary page: token scores over each query's causal prefix followed by
// the top-k selection.
//
// Portable path: a score kernel writes every query's fp32 score row into the
// workspace (one thread per key, the query's head rows staged in LDS), then a
// block radix select per row picks the k winners.
#include "common.hpp"
#include "launch.hpp"
#include "topk.hpp"

namespace misa {

namespace {

constexpr int kScoreThreads = 256;
constexpr int kTopkThreads = 1024;
constexpr int kMaxHeads = 64;

template <int DT>
__global__ __launch_bounds__(kScoreThreads) void score_rows_kernel(
    const void* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    const void* __restrict__ k, const float* __restrict__ k_scale,
    const int32_t* __restrict__ heads, int32_t nh, float* __restrict__ rows, int32_t L, int32_t T,
    int32_t H) {
  __shared__ float qs[kMaxHeads][kD];
  __shared__ float wsh[kMaxHeads];
  const int t = blockIdx.y;
  const int64_t seq = blockIdx.z;
  const int64_t r = seq * T + t;
  const int64_t pos = static_cast<int64_t>(L) - T + t;
  const int64_t s0 = static_cast<int64_t>(blockIdx.x) * kScoreThreads;
  if (s0 > pos) return;
  const float sq = (DT == kFP8) ? q_scale[r] : 1.f;
  for (int e = threadIdx.x; e < nh * kD; e += kScoreThreads) {
    const int a = e / kD;
    int j = heads ? heads[r * nh + a] : a;
    j = (j >= 0 && j < H) ? j : 0;
    qs[a][e % kD] = load_elem<DT>(q, (r * H + j) * kD + e % kD) * sq;
  }
  if (threadIdx.x < nh) {
    const int j = heads ? heads[r * nh + threadIdx.x] : threadIdx.x;
    // A head id outside [0, H) contributes nothing.
    wsh[threadIdx.x] = (j >= 0 && j < H) ? w[r * H + j] : 0.f;
  }
  __syncthreads();
  const int64_t s = s0 + threadIdx.x;
  if (s > pos) return;
  float kr[kD];
  const float sk = (DT == kFP8) ? k_scale[seq * L + s] : 1.f;
#pragma unroll
  for (int i = 0; i < kD; ++i) kr[i] = load_elem<DT>(k, (seq * L + s) * kD + i) * sk;
  float acc = 0.f;
  for (int a = 0; a < nh; ++a) {
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < kD; ++i) dot += qs[a][i] * kr[i];
    acc += wsh[a] * fmaxf(dot, 0.f);
  }
  rows[r * static_cast<int64_t>(L) + s] = acc;
}

// Top-k over the materialised score row of query t (its first n_t entries).
__global__ __launch_bounds__(kTopkThreads) void topk_rows_kernel(const float* __restrict__ rows,
                                                                 int32_t L, int32_t T, int32_t k,
                                                                 int32_t* __restrict__ idx,
                                                                 float* __restrict__ scores_out) {
  __shared__ TopkFastSmem sm;
  const int t = blockIdx.x;
  const int64_t r = static_cast<int64_t>(blockIdx.y) * T + t;
  const int64_t n = static_cast<int64_t>(L) - T + t + 1;
  const float* row = rows + r * static_cast<int64_t>(L);
  block_topk_fast<kTopkThreads>(
      n, k, [](int64_t) { return true; }, [=](int64_t i) { return row[i]; },
      [](int64_t i) { return static_cast<int32_t>(i); }, idx + r * k,
      scores_out ? scores_out + r * k : nullptr, sm);
}

}  // namespace

size_t score_ws_bytes(const Shape& s, int32_t nh, int32_t k) {
  if (s.T == 1 && s.dtype != kF32) return decode_ws_bytes(s);
  if (decode_mq_supported(s, nh)) return decode_mq_ws_bytes(s);
  if (prefill_supported(s)) return prefill_ws_bytes(s, nh, k);
  return align_up(static_cast<size_t>(s.batch) * s.T * s.L * sizeof(float));
}

hipError_t launch_score_topk(const Shape& s, int32_t nh, const int32_t* heads, int32_t k,
                             const void* q, const float* q_scale, const float* w, const void* kk,
                             const float* k_scale, int32_t* idx, float* scores_out, void* ws,
                             hipStream_t st) {
  if (s.T == 1 && s.dtype != kF32)
    return launch_decode_score_topk(s, nh, heads, k, q, q_scale, w, kk, k_scale, idx, scores_out,
                                    ws, st);
  if (decode_mq_supported(s, nh))
    return launch_decode_mq_score_topk(s, nh, heads, k, q, q_scale, w, kk, k_scale, idx, scores_out,
                                       ws, st);
  if (prefill_supported(s))
    return launch_prefill_score_topk(s, nh, heads, k, q, q_scale, w, kk, k_scale, idx, scores_out,
                                     ws, st);
  float* rows = static_cast<float*>(ws);
  dim3 g1((s.L + kScoreThreads - 1) / kScoreThreads, s.T, s.batch);
  switch (s.dtype) {
    case kF32:
      score_rows_kernel<kF32><<<g1, kScoreThreads, 0, st>>>(q, q_scale, w, kk, k_scale, heads, nh,
                                                            rows, s.L, s.T, s.H);
      break;
    case kBF16:
      score_rows_kernel<kBF16><<<g1, kScoreThreads, 0, st>>>(q, q_scale, w, kk, k_scale, heads, nh,
                                                             rows, s.L, s.T, s.H);
      break;
    default:
      score_rows_kernel<kFP8><<<g1, kScoreThreads, 0, st>>>(q, q_scale, w, kk, k_scale, heads, nh,
                                                            rows, s.L, s.T, s.H);
      break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2(s.T, s.batch);
  topk_rows_kernel<<<g2, kTopkThreads, 0, st>>>(rows, s.L, s.T, k, idx, scores_out);
  return hipGetLastError();
}

}  // namespace misa
