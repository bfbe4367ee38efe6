// Helpers shared by the router kernels (Eq. (7)-(8) of the MISA summary page).
#pragma once

#include "common.hpp"

namespace misa {

// One head row of q (kD elements from element offset `off`) widened to fp32
// in registers with 16-byte loads; fp8 codes are not scaled.
template <int DT>
__device__ __forceinline__ void load_head_row(const void* q, int64_t off, float (&qr)[kD]) {
  if constexpr (DT == kF32) {
    const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(q) + off);
#pragma unroll
    for (int u = 0; u < kD / 4; ++u) {
      const float4 v = src[u];
      qr[4 * u] = v.x; qr[4 * u + 1] = v.y; qr[4 * u + 2] = v.z; qr[4 * u + 3] = v.w;
    }
  } else if constexpr (DT == kBF16) {
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(q) + off);
#pragma unroll
    for (int u = 0; u < kD / 8; ++u) {
      const uint4 v = src[u];
      const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qr[8 * u + 2 * e] = __uint_as_float(wd[e] << 16);
        qr[8 * u + 2 * e + 1] = __uint_as_float(wd[e] & 0xFFFF0000u);
      }
    }
  } else {
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(q) + off);
#pragma unroll
    for (int u = 0; u < kD / 16; ++u) {
      const uint4 v = src[u];
      const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 16; ++e) qr[16 * u + e] = fp8_to_f32((wd[e / 4] >> (8 * (e % 4))) & 0xFF);
    }
  }
}

// q . p for a register row qr and an LDS row p (kD floats, broadcast reads),
// in four interleaved partial sums so the FMAs do not form one serial chain.
__device__ __forceinline__ float dot_lds_row(const float (&qr)[kD], const float* p) {
  const float4* pb = reinterpret_cast<const float4*>(p);
  float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f;
#pragma unroll
  for (int i = 0; i < kD / 4; ++i) {
    const float4 v = pb[i];
    d0 = fmaf(qr[4 * i], v.x, d0);
    d1 = fmaf(qr[4 * i + 1], v.y, d1);
    d2 = fmaf(qr[4 * i + 2], v.z, d2);
    d3 = fmaf(qr[4 * i + 3], v.w, d3);
  }
  return (d0 + d1) + (d2 + d3);
}

// Top-h of Eq. (8) by one wave: lane j < H holds E_j (>= 0); h rounds of a
// wave arg-max (ties to the lower head) mark the winners, which are written
// to heads[0..h) in ascending head order.
__device__ __forceinline__ void wave_top_heads(float e, int H, int h, int32_t* heads) {
  const int lane = lane_id();
  if (lane >= H) e = -2.f;
  bool taken = false;
  for (int round = 0; round < h; ++round) {
    float bv = taken ? -1.f : e;
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
  if (taken) heads[lanes_below(mask)] = lane;
}

// The same selection as wave_top_heads by ranks: lane l counts the lanes
// whose E beats its own (larger, or equal with a lower head) and is taken
// when fewer than h do.  64 independent compares per lane instead of h
// dependent arg-max rounds.
__device__ __forceinline__ void wave_top_heads_rank(float e, int H, int h, int32_t* heads) {
  const int lane = lane_id();
  if (lane >= H) e = -2.f;
  int rank = 0;
#pragma unroll 8
  for (int j = 0; j < kWave; ++j) {
    const float ej = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(e), j));
    rank += (ej > e || (ej == e && j < lane)) ? 1 : 0;
  }
  const bool taken = lane < H && rank < h;
  const uint64_t mask = __ballot(taken);
  if (taken) heads[lanes_below(mask)] = lane;
}

// One wave: E for its query from nparts row-sum slices (LDS, added in order)
// plus the partial-block term, then top-h.
__device__ __forceinline__ void finalize_query(const float (*rowsum)[64], int nparts,
                                               const float* partial, int H, int h, const float* w,
                                               float sq, int64_t r, int64_t Mt, int32_t* heads,
                                               float* E_out) {
  const int lane = lane_id();
  float e = -2.f;
  if (lane < H) {
    float sum = rowsum[0][lane];
    for (int p = 1; p < nparts; ++p) sum += rowsum[p][lane];
    sum += partial ? partial[lane] : 0.f;
    e = fabsf(w[r * H + lane]) * sq * sum / static_cast<float>(Mt);
    if (E_out) E_out[r * H + lane] = e;
  }
  wave_top_heads_rank(e, H, h, heads + r * h);
}

}  // namespace misa
