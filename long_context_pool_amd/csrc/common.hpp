// Device helpers shared by the MISA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace misa {

constexpr int kWave = 64;
constexpr int kD = 128;  // head dimension supported by this build

enum DType : int32_t { kF32 = 0, kBF16 = 1, kFP8 = 2 };

// ---------------------------------------------------------------- element loads

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// OCP e4m3fn byte -> fp32 through the gfx950 hardware converter (this target's
// fp8 conversions use the OCP encoding).
__device__ __forceinline__ float fp8_to_f32(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(byte), 0);
}

// Load element i of a row in dtype DT as fp32.
template <int DT>
__device__ __forceinline__ float load_elem(const void* base, int64_t i) {
  if constexpr (DT == kF32) {
    return static_cast<const float*>(base)[i];
  } else if constexpr (DT == kBF16) {
    return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[i]);
  } else {
    return fp8_to_f32(static_cast<const uint8_t*>(base)[i]);
  }
}

template <int DT>
constexpr int elem_bytes() {
  return DT == kF32 ? 4 : (DT == kBF16 ? 2 : 1);
}

// ReLU as one v_med3_f32: clamp(x, 0, 3e38) equals max(x, 0) for every finite
// score (fmaxf adds a NaN-quieting v_max per element).
__device__ __forceinline__ float relu(float x) { return __builtin_amdgcn_fmed3f(x, 0.f, 3.0e38f); }

// ---------------------------------------------------------------- ordering keys

// Order-preserving map fp32 -> u32 (larger float <=> larger key); -0 maps like +0.
// Host-callable too (the top-k key intervals are checked exhaustively on the CPU).
__host__ __device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------- wave / block scans

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Number of set bits of a 64-bit lane mask strictly below this lane.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0));
}

__device__ __forceinline__ int wave_inclusive_sum(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(v, o, kWave);
    if (lane >= o) v += y;
  }
  return v;
}

// Block-wide exclusive prefix sum of `v` in thread order; `total` receives the
// block sum.  `tmp` is LDS scratch of NT/64 ints.  Contains __syncthreads().
template <int NT>
__device__ __forceinline__ int block_exclusive_sum(int v, int* tmp, int& total) {
  constexpr int NW = NT / kWave;
  const int lane = lane_id();
  const int wid = threadIdx.x / kWave;
  const int inc = wave_inclusive_sum(v);
  if (lane == kWave - 1) tmp[wid] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int c = tmp[i];
    base += (i < wid) ? c : 0;
    tot += c;
  }
  __syncthreads();
  total = tot;
  return base + inc - v;
}

}  // namespace misa
