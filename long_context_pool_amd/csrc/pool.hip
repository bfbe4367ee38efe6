// Eq. (4) of the MISA summary page ("Methodology" 1, block-pooled router):
// each block of B consecutive keys is summarised by the mean of its members.
//
// One workgroup of 4 waves per (block, sequence).  Lane l of every wave owns
// dims 2l and 2l+1; wave w sums rows s0+w, s0+w+4, ...  in fp32 (fp8 codes are
// scaled by their per-token scale first); the four wave partials are added
// in fixed order, so the result is deterministic.  Bandwidth-bound: one read
// of the keys, d*4 bytes written per block.
#include "common.hpp"
#include "launch.hpp"

namespace misa {

namespace {

constexpr int kPoolThreads = 256;

template <int DT>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(const void* __restrict__ k,
                                                            const float* __restrict__ k_scale,
                                                            float* __restrict__ pooled, int32_t L,
                                                            int32_t B, int32_t block_begin,
                                                            int64_t M) {
  __shared__ float part[kPoolThreads / kWave][kD];
  const int64_t blk = block_begin + blockIdx.x;
  const int64_t seq = blockIdx.y;
  const int64_t s0 = blk * B;
  const int64_t s1 = min<int64_t>(s0 + B, L);
  const int lane = lane_id();
  const int wv = threadIdx.x / kWave;
  float a0 = 0.f, a1 = 0.f;
  for (int64_t s = s0 + wv; s < s1; s += kPoolThreads / kWave) {
    const int64_t row = (seq * L + s) * kD;
    float x0 = load_elem<DT>(k, row + 2 * lane);
    float x1 = load_elem<DT>(k, row + 2 * lane + 1);
    if constexpr (DT == kFP8) {
      const float sc = k_scale[seq * L + s];
      x0 *= sc;
      x1 *= sc;
    }
    a0 += x0;
    a1 += x1;
  }
  part[wv][2 * lane] = a0;
  part[wv][2 * lane + 1] = a1;
  __syncthreads();
  if (threadIdx.x < kD) {
    float acc = part[0][threadIdx.x];
#pragma unroll
    for (int w = 1; w < kPoolThreads / kWave; ++w) acc += part[w][threadIdx.x];
    pooled[(seq * M + blk) * kD + threadIdx.x] = acc / static_cast<float>(s1 - s0);
  }
}

}  // namespace

hipError_t launch_pool(const Shape& s, int32_t block_begin, int32_t block_count, const void* k,
                       const float* k_scale, float* pooled, hipStream_t st) {
  if (block_count <= 0) return hipSuccess;
  dim3 grid(block_count, s.batch);
  switch (s.dtype) {
    case kF32:
      pool_kernel<kF32><<<grid, kPoolThreads, 0, st>>>(k, k_scale, pooled, s.L, s.B, block_begin, s.M());
      break;
    case kBF16:
      pool_kernel<kBF16><<<grid, kPoolThreads, 0, st>>>(k, k_scale, pooled, s.L, s.B, block_begin, s.M());
      break;
    default:
      pool_kernel<kFP8><<<grid, kPoolThreads, 0, st>>>(k, k_scale, pooled, s.L, s.B, block_begin, s.M());
      break;
  }
  return hipGetLastError();
}

}  // namespace misa
