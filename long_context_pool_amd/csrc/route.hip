// Eq. (7)-(8) of the MISA summary page ("Methodology" 1): the block-pooled
// router.  For query t (prefix of n_t keys) and head j
//   E_{t,j} = |w_{t,j}| * (1/M_t) * sum_{m < M_t} ReLU(q_{t,j} . p_m),
// which equals the page's mean of |A_{t,j,m}| because |w*ReLU(x)| = |w|*ReLU(x).
// The M_t = ceil(n_t/B) pooled keys p_m are the Eq. (4) block means for the
// blocks inside the prefix plus, when B does not divide n_t, the mean of the
// partial last block's keys (the query never sees a key beyond its position).
// The top-h heads by E (ties to the lower head) are written in ascending order.
//
// One workgroup (4 waves) per query: the query's H rows are staged in LDS as
// fp32, each thread owns one head and a 1/NSUB slice of the blocks, partials
// are combined in fixed order, and wave 0 picks the top-h heads with h rounds
// of a wave-wide arg-max.
#include "common.hpp"
#include "launch.hpp"

namespace misa {

namespace {

constexpr int kRouteThreads = 256;
constexpr int kMaxHeads = 64;

template <int DT>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    const void* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    const float* __restrict__ pooled, const void* __restrict__ k, const float* __restrict__ k_scale,
    int32_t* __restrict__ heads, float* __restrict__ E_out, int32_t L, int32_t T, int32_t H,
    int32_t B, int64_t M, int32_t h) {
  __shared__ float qs[kMaxHeads][kD + 1];
  __shared__ float kp[kD];
  __shared__ float part[kRouteThreads];
  __shared__ float Es[kMaxHeads];

  const int t = blockIdx.x;
  const int64_t seq = blockIdx.y;
  const int64_t r = seq * T + t;
  const int64_t pos = static_cast<int64_t>(L) - T + t;
  const int64_t n = pos + 1;
  const int64_t full = n / B;
  const int64_t Mt = (n + B - 1) / B;

  const float sq = (DT == kFP8) ? q_scale[r] : 1.f;
  const int64_t qrow = r * H * kD;
  for (int e = threadIdx.x; e < H * kD; e += kRouteThreads)
    qs[e / kD][e % kD] = load_elem<DT>(q, qrow + e) * sq;
  if (Mt > full && threadIdx.x < kD) {
    float acc = 0.f;
    for (int64_t s = full * B; s <= pos; ++s) {
      float x = load_elem<DT>(k, (seq * L + s) * kD + threadIdx.x);
      if constexpr (DT == kFP8) x *= k_scale[seq * L + s];
      acc += x;
    }
    kp[threadIdx.x] = acc / static_cast<float>(n - full * B);
  }
  __syncthreads();

  const int nsub = kRouteThreads / H;
  const int j = threadIdx.x % H;
  const int sub = threadIdx.x / H;
  float acc = 0.f;
  if (sub < nsub) {
    for (int64_t b = sub; b < full; b += nsub) {
      const float* pb = pooled + (seq * M + b) * kD;
      float dot = 0.f;
#pragma unroll 8
      for (int i = 0; i < kD; ++i) dot += qs[j][i] * pb[i];
      acc += fmaxf(dot, 0.f);
    }
    if (sub == 0 && Mt > full) {
      float dot = 0.f;
#pragma unroll 8
      for (int i = 0; i < kD; ++i) dot += qs[j][i] * kp[i];
      acc += fmaxf(dot, 0.f);
    }
  }
  part[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x < H) {
    float sum = part[threadIdx.x];
    for (int u = 1; u < nsub; ++u) sum += part[u * H + threadIdx.x];
    const float e = fabsf(w[r * H + threadIdx.x]) * sum / static_cast<float>(Mt);
    Es[threadIdx.x] = e;
    if (E_out) E_out[r * H + threadIdx.x] = e;
  }
  __syncthreads();

  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const float v = lane < H ? Es[lane] : -2.f;
    bool taken = false;
    for (int round = 0; round < h; ++round) {
      float bv = taken ? -1.f : v;
      int bi = lane;
#pragma unroll
      for (int o = kWave / 2; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(bv, o, kWave);
        const int oi = __shfl_xor(bi, o, kWave);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
      }
      if (bi == lane) taken = true;
    }
    const uint64_t mask = __ballot(taken);
    if (taken) heads[r * h + lanes_below(mask)] = lane;
  }
}

}  // namespace

size_t route_ws_bytes(const Shape& s) {
  if (s.T == 1) return route_decode_ws_bytes(s);
  return route_mfma_supported(s) ? route_mfma_ws_bytes(s) : 0;
}

hipError_t launch_route(const Shape& s, int32_t h, const void* q, const float* q_scale,
                        const float* w, const float* pooled, const void* k, const float* k_scale,
                        int32_t* heads, float* E_out, void* ws, hipStream_t st) {
  if (s.T == 1)
    return launch_route_decode(s, h, q, q_scale, w, pooled, k, k_scale, heads, E_out, ws, st);
  if (route_mfma_supported(s))
    return launch_route_mfma(s, h, q, q_scale, w, pooled, k, k_scale, heads, E_out, ws, st);
  dim3 grid(s.T, s.batch);
  switch (s.dtype) {
    case kF32:
      route_kernel<kF32><<<grid, kRouteThreads, 0, st>>>(q, q_scale, w, pooled, k, k_scale, heads,
                                                         E_out, s.L, s.T, s.H, s.B, s.M(), h);
      break;
    case kBF16:
      route_kernel<kBF16><<<grid, kRouteThreads, 0, st>>>(q, q_scale, w, pooled, k, k_scale, heads,
                                                          E_out, s.L, s.T, s.H, s.B, s.M(), h);
      break;
    default:
      route_kernel<kFP8><<<grid, kRouteThreads, 0, st>>>(q, q_scale, w, pooled, k, k_scale, heads,
                                                         E_out, s.L, s.T, s.H, s.B, s.M(), h);
      break;
  }
  return hipGetLastError();
}

}  // namespace misa
