// Thin wrappers over the gfx950 MFMA builtins used by the scoring kernels.
//
// Lane layouts (wave64; l = lane):
//  16x16x32 bf16 : lane supplies A[row l%16][k 8*(l/16)+i], B[k 8*(l/16)+i][col l%16], i<8;
//                  acc reg r holds C[row 4*(l/16)+r][col l%16].
//  32x32x16 bf16 : A[row l%32][k 8*(l/32)+i], B[k 8*(l/32)+i][col l%32], i<8;
//                  acc reg r holds C[row 8*(r/4) + 4*(l/32) + r%4][col l%32].
//  16x16x128 fp8 : A[row l%16][k 32*(l/16)+i], i<32 (OCP e4m3fn bytes); C as 16x16x32.
//  32x32x64 fp8  : A[row l%32][k 32*(l/32)+i], i<32; C as 32x32x16.
// Since a dot product does not depend on the order of its terms, every kernel
// assigns head-dimension elements to (lane group, k-step) so that each lane
// reads one contiguous run of its key row; A and B use the same assignment.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace misa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) int i32x8;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x4 mfma16_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// fp8 (e4m3fn) x fp8 with unit block scales (e8m0 127 = 2^0).
__device__ __forceinline__ f32x4 mfma16_fp8(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
__device__ __forceinline__ f32x16 mfma32_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Split an fp32 quad into bf16 hi (RNE) and lo (RNE of the remainder) pairs.
__device__ __forceinline__ void split_bf16(float4 x, uint32_t& h0, uint32_t& h1, uint32_t& l0,
                                           uint32_t& l1) {
  const uint32_t a = f32_to_bf16_bits(x.x), b = f32_to_bf16_bits(x.y);
  const uint32_t c = f32_to_bf16_bits(x.z), d = f32_to_bf16_bits(x.w);
  h0 = a | (b << 16);
  h1 = c | (d << 16);
  l0 = f32_to_bf16_bits(x.x - __uint_as_float(a << 16)) |
       (f32_to_bf16_bits(x.y - __uint_as_float(b << 16)) << 16);
  l1 = f32_to_bf16_bits(x.z - __uint_as_float(c << 16)) |
       (f32_to_bf16_bits(x.w - __uint_as_float(d << 16)) << 16);
}

}  // namespace misa
