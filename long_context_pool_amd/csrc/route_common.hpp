// Helpers shared by the router kernels (Eq. (7)-(8) of the MISA summary page).
#pragma once

#include "common.hpp"

namespace misa {

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
  wave_top_heads(e, H, h, heads + r * h);
}

}  // namespace misa
