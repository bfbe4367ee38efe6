// Eq. (7)-(8) of the MISA summary page ("Methodology" 1) for decode: one query
// per sequence, its whole prefix of L keys, M = L/B (+1 partial) blocks.
//
// The work (H heads x M blocks x d) is small but must be spread over the chip:
// workgroup (chunk c, sequence) takes 32 pooled blocks, stages them in LDS and
// each thread dots its head row (fp32 registers; bf16/fp8 codes are exact in
// fp32) with its share of the blocks -- exact fp32 products, no rounding of the
// pooled keys.  The per-chunk ReLU sums go to the workspace; a one-wave
// finalize kernel per sequence adds them in chunk order, adds the partial
// last block (mean of the keys after the last complete block), forms
// E_j = |w_j| * s * sum / M_t (s = fp8 query scale, else 1) and picks the
// top-h heads.
#include "common.hpp"
#include "launch.hpp"
#include "route_common.hpp"

namespace misa {

namespace {

constexpr int kChunk = 32;         // pooled blocks per workgroup
constexpr int kRDThreads = 256;    // 4 waves; thread t: head t%64, blocks t/64 + 4i
constexpr int kMaxH = 64;

template <int DT>
__global__ __launch_bounds__(kRDThreads) void route_decode_partial_kernel(
    const void* __restrict__ q, const float* __restrict__ pooled, float* __restrict__ part,
    int32_t H, int64_t M, int64_t full, int32_t nchunks) {
  __shared__ __attribute__((aligned(16))) float ps[kChunk][kD];
  __shared__ float red[kRDThreads / kWave][kMaxH];
  const int c = blockIdx.x;
  const int64_t seq = blockIdx.y;
  const int j = threadIdx.x & (kMaxH - 1);
  const int sub = threadIdx.x / kMaxH;
  const int64_t b0 = static_cast<int64_t>(c) * kChunk;
  const int nb = static_cast<int>(min<int64_t>(kChunk, full - b0));
  // Stage the chunk's pooled keys (fp32) in LDS.
  for (int e = threadIdx.x; e < kChunk * kD / 4; e += kRDThreads) {
    const int b = e / (kD / 4);
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (b < nb) v = reinterpret_cast<const float4*>(pooled + (seq * M + b0 + b) * kD)[e % (kD / 4)];
    reinterpret_cast<float4*>(&ps[b][0])[e % (kD / 4)] = v;
  }
  // This thread's head row in registers (vector loads, widened to fp32).
  float qr[kD];
  load_head_row<DT>(q, (seq * H + (j < H ? j : 0)) * kD, qr);
  __syncthreads();
  float acc = 0.f;
  for (int b = sub; b < nb; b += kRDThreads / kMaxH) acc += relu(dot_lds_row(qr, &ps[b][0]));
  red[sub][j] = acc;
  __syncthreads();
  if (threadIdx.x < kMaxH) {
    float sum = red[0][threadIdx.x];
#pragma unroll
    for (int u = 1; u < kRDThreads / kMaxH; ++u) sum += red[u][threadIdx.x];
    part[(seq * nchunks + c) * kMaxH + threadIdx.x] = sum;
  }
}

template <int DT>
__global__ __launch_bounds__(kWave) void route_decode_finalize_kernel(
    const void* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    const void* __restrict__ k, const float* __restrict__ k_scale, const float* __restrict__ part,
    int32_t* __restrict__ heads, float* __restrict__ E_out, int32_t L, int32_t H, int32_t B,
    int32_t h, int32_t nchunks) {
  __shared__ float kp[kD];
  __shared__ float rowsum[1][64];
  __shared__ float partial[64];
  const int lane = lane_id();
  const int64_t seq = blockIdx.x;
  const int64_t r = seq;  // T == 1
  const int64_t n = L;
  const int64_t full = n / B;
  const int64_t Mt = (n + B - 1) / B;
  // Chunk partials, 8 loads in flight at a time, added in chunk order.
  float sum = 0.f;
  for (int c0 = 0; c0 < nchunks; c0 += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = c0 + u < nchunks ? part[(seq * nchunks + c0 + u) * kMaxH + lane] : 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) sum += v[u];
  }
  rowsum[0][lane] = sum;
  const bool has_partial = Mt > full;
  if (has_partial) {
    for (int u = 0; u < 2; ++u) {
      const int dim = lane + kWave * u;
      float acc = 0.f;
      for (int64_t s = full * B; s < n; ++s) {
        float x = load_elem<DT>(k, (seq * L + s) * kD + dim);
        if constexpr (DT == kFP8) x *= k_scale[seq * L + s];
        acc += x;
      }
      kp[dim] = acc / static_cast<float>(n - full * B);
    }
    __syncthreads();
    float dot = 0.f;
    if (lane < H)
      for (int i = 0; i < kD; ++i) dot += load_elem<DT>(q, (r * H + lane) * kD + i) * kp[i];
    partial[lane] = fmaxf(dot, 0.f);
  }
  __syncthreads();
  const float sq = (DT == kFP8) ? q_scale[r] : 1.f;
  finalize_query(rowsum, 1, has_partial ? partial : nullptr, H, h, w, sq, r, Mt, heads, E_out);
}

}  // namespace

int32_t route_decode_chunks(const Shape& s) {
  const int64_t full = static_cast<int64_t>(s.L) / s.B;
  const int64_t nch = (full + kChunk - 1) / kChunk;
  return static_cast<int32_t>(nch < 1 ? 1 : nch);
}

size_t route_decode_ws_bytes(const Shape& s) {
  return align_up(static_cast<size_t>(s.batch) * route_decode_chunks(s) * kMaxH * sizeof(float));
}

hipError_t launch_route_decode(const Shape& s, int32_t h, const void* q, const float* q_scale,
                               const float* w, const float* pooled, const void* k,
                               const float* k_scale, int32_t* heads, float* E_out, void* ws,
                               hipStream_t st) {
  const int32_t nch = route_decode_chunks(s);
  const int64_t full = static_cast<int64_t>(s.L) / s.B;
  float* part = static_cast<float*>(ws);
  dim3 g1(nch, s.batch);
  switch (s.dtype) {
    case kF32:
      route_decode_partial_kernel<kF32><<<g1, kRDThreads, 0, st>>>(q, pooled, part, s.H, s.M(), full, nch);
      route_decode_finalize_kernel<kF32><<<s.batch, kWave, 0, st>>>(q, q_scale, w, k, k_scale, part, heads, E_out, s.L, s.H, s.B, h, nch);
      break;
    case kBF16:
      route_decode_partial_kernel<kBF16><<<g1, kRDThreads, 0, st>>>(q, pooled, part, s.H, s.M(), full, nch);
      route_decode_finalize_kernel<kBF16><<<s.batch, kWave, 0, st>>>(q, q_scale, w, k, k_scale, part, heads, E_out, s.L, s.H, s.B, h, nch);
      break;
    default:
      route_decode_partial_kernel<kFP8><<<g1, kRDThreads, 0, st>>>(q, pooled, part, s.H, s.M(), full, nch);
      route_decode_finalize_kernel<kFP8><<<s.batch, kWave, 0, st>>>(q, q_scale, w, k, k_scale, part, heads, E_out, s.L, s.H, s.B, h, nch);
      break;
  }
  return hipGetLastError();
}

}  // namespace misa
