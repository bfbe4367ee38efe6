// Eq. (4) of the MISA summary page ("Methodology" 1, block-pooled router):
// each block of B consecutive keys is summarised by the mean of its members.
//
// One workgroup per (block, sequence).  The block's rows are read 64 at a
// time (thread t: row t/4, 32 consecutive dims, one vector load run), widened
// to fp32 (fp8 codes times their per-token scale) into an LDS tile, and
// thread d < 128 adds column d in row order, so the sum is deterministic.
// Bandwidth-bound: one read of the keys, d*4 bytes written per block.
#include "common.hpp"
#include "launch.hpp"

namespace misa {

namespace {

constexpr int kPoolThreads = 256;
constexpr int kPoolRows = 64;  // rows per chunk: thread t loads row t/4, dims [32(t%4), +32)

template <int DT>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(const void* __restrict__ k,
                                                            const float* __restrict__ k_scale,
                                                            float* __restrict__ pooled, int32_t L,
                                                            int32_t B, int32_t block_begin,
                                                            int64_t M) {
  __shared__ float tile[kPoolRows][kD + 4];
  const int64_t blk = block_begin + blockIdx.x;
  const int64_t seq = blockIdx.y;
  const int64_t s0 = blk * B;
  const int64_t s1 = min<int64_t>(s0 + B, L);
  const int lr = threadIdx.x >> 2;
  const int dc = (threadIdx.x & 3) * 32;
  float acc = 0.f;  // thread t < 128: sum of dim t over the block
  for (int64_t c0 = s0; c0 < s1; c0 += kPoolRows) {
    const int64_t s = c0 + lr;
    float x[32];
    if (s < s1) {
      const int64_t base = (seq * L + s) * kD + dc;
      const float sc = (DT == kFP8) ? k_scale[seq * L + s] : 1.f;
      if constexpr (DT == kF32) {
        const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(k) + base);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float4 v = src[u];
          x[4 * u] = v.x; x[4 * u + 1] = v.y; x[4 * u + 2] = v.z; x[4 * u + 3] = v.w;
        }
      } else if constexpr (DT == kBF16) {
        const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(k) + base);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint4 v = src[u];
          const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[8 * u + 2 * e] = __uint_as_float(wd[e] << 16);
            x[8 * u + 2 * e + 1] = __uint_as_float(wd[e] & 0xFFFF0000u);
          }
        }
      } else {
        const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(k) + base);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const uint4 v = src[u];
          const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 16; ++e) x[16 * u + e] = fp8_to_f32((wd[e / 4] >> (8 * (e % 4))) & 0xFF) * sc;
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 32; ++e) x[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 32; ++e) tile[lr][dc + e] = x[e];
    __syncthreads();
    if (threadIdx.x < kD) {
      const int rows = static_cast<int>(min<int64_t>(kPoolRows, s1 - c0));
      for (int rr = 0; rr < rows; ++rr) acc += tile[rr][threadIdx.x];  // fixed row order
    }
    __syncthreads();
  }
  if (threadIdx.x < kD) pooled[(seq * M + blk) * kD + threadIdx.x] = acc / static_cast<float>(s1 - s0);
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
