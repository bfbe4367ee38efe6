// Scoring one query against a stream of keys on 16x16 MFMA tiles, Eq. (9) /
// Eq. (1) of the MISA summary page: I_s = sum_j w_j * ReLU(q_j . k_s).
//
// The query's scored head rows are the A operand (16-row tiles, rows past the
// head count are zero); 16 keys form one output tile.  A row (d = 128) is cut
// into 16-byte pieces; in load step i, lane group g = l/16 of lane l takes
// piece 4*i + g of key l%16, so each load instruction reads 64 contiguous
// bytes of each of 16 keys (measured faster than one contiguous 64-byte run
// per lane).  The MFMA k index is therefore a permutation of the head
// dimension, the same for A and B, which leaves every dot product unchanged.
// The ReLU * w head sum is taken on the accumulators and finished with a
// 4-lane reduction.
#pragma once

#include "common.hpp"
#include "mfma.hpp"

namespace misa {

template <int DT, int NRT>
struct RowScorer {
  bf16x8 a16[NRT][4];
  i32x8 a8[NRT];
  float wl[NRT][4];

  // One query: qrows = its H head rows (kD elements each, `pitch` elements
  // apart, any address space), wrow = its H weights, sq = its fp8 scale (1
  // otherwise); the nh scored heads are hsel[0..nh) (or 0..nh-1 when hsel is
  // null); ids outside [0, H) score nothing.
  __device__ __forceinline__ void init_rows(const void* qrows, const float* wrow, float sq,
                                            const int32_t* hsel, int nh, int H, int pitch = kD) {
    const int lane = lane_id();
    const int col = lane & 15;
    const int qq = lane >> 4;
    auto head_of = [&](int row) -> int {
      if (row >= nh) return -1;
      const int j = hsel ? hsel[row] : row;
      return (j >= 0 && j < H) ? j : -1;
    };
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = head_of(rt * 16 + 4 * qq + i);
        wl[rt][i] = (j >= 0) ? wrow[j] * sq : 0.f;
      }
      const int j = head_of(rt * 16 + col);
      const int64_t qoff = static_cast<int64_t>(j < 0 ? 0 : j) * pitch;
      if constexpr (DT == kBF16) {
        const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(qrows) + qoff);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) a16[rt][ks] = as_bf16x8(j < 0 ? make_uint4(0, 0, 0, 0) : src[4 * ks + qq]);
      } else {
        const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(qrows) + qoff);
        const uint4 lo = j < 0 ? make_uint4(0, 0, 0, 0) : src[qq];
        const uint4 hi = j < 0 ? make_uint4(0, 0, 0, 0) : src[4 + qq];
        a8[rt] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
    }
  }

  // Query row r (= seq*T + t) of q [rows, H, kD] with nh scored heads:
  // heads[hr*nh + i] (or i when heads is null); hr < 0 means hr = r.
  __device__ __forceinline__ void init(const void* q, const float* q_scale, const float* w,
                                       const int32_t* heads, int nh, int64_t r, int H,
                                       int64_t hr = -1) {
    if (hr < 0) hr = r;
    const void* qrows = (DT == kBF16)
        ? static_cast<const void*>(static_cast<const uint16_t*>(q) + r * H * kD)
        : static_cast<const void*>(static_cast<const uint8_t*>(q) + r * H * kD);
    init_rows(qrows, w + r * H, (DT == kFP8) ? q_scale[r] : 1.f, heads ? heads + hr * nh : nullptr,
              nh, H);
  }

  // Key operands of 64 keys: 4 groups of 16 keys, 4 (bf16) or 2 (fp8)
  // 16-byte pieces per lane.
  using Keys = uint4[4][DT == kBF16 ? 4 : 2];

  // Loads keys [s0, s0+64) of `krows` (row s at krows + s*kD elements), valid
  // below s_end; invalid keys load row s_safe (which every caller guarantees
  // to exist) and are zeroed.
  __device__ __forceinline__ static void load64(const void* krows, int64_t s0, int64_t s_end,
                                                int64_t s_safe, Keys& kb) {
    const int lane = lane_id();
    const int col = lane & 15;
    const int qq = lane >> 4;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int64_t s = s0 + 16 * g + col;
      const bool ok = s < s_end;
      const int64_t row = (ok ? s : s_safe) * kD;
      if constexpr (DT == kBF16) {
        const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(krows) + row);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kb[g][ks] = ok ? src[4 * ks + qq] : make_uint4(0, 0, 0, 0);
      } else {
        const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(krows) + row);
        kb[g][0] = ok ? src[qq] : make_uint4(0, 0, 0, 0);
        kb[g][1] = ok ? src[4 + qq] : make_uint4(0, 0, 0, 0);
      }
    }
  }

  // Scores of 64 loaded keys; returns the score of key s0 + lane (unscaled by
  // the fp8 key scale).  Zeroed keys score 0.
  __device__ __forceinline__ float compute64(const Keys& kb) const {
    const int lane = lane_id();
    const int qq = lane >> 4;
    float res = 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float part = 0.f;
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (DT == kBF16) {
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) acc = mfma16_bf16(a16[rt][ks], as_bf16x8(kb[g][ks]), acc);
        } else {
          const i32x8 b8{(int)kb[g][0].x, (int)kb[g][0].y, (int)kb[g][0].z, (int)kb[g][0].w,
                         (int)kb[g][1].x, (int)kb[g][1].y, (int)kb[g][1].z, (int)kb[g][1].w};
          acc = mfma16_fp8(a8[rt], b8, acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) part += wl[rt][i] * relu(acc[i]);
      }
      // Sum the four lane groups holding rows 0-3, 4-7, 8-11, 12-15.
      part += __shfl_xor(part, 16, kWave);
      part += __shfl_xor(part, 32, kWave);
      if (qq == g) res = part;  // lane group g keeps key group g: lane l <-> key s0 + l
    }
    return res;
  }

  // Scores of keys [s0, s0+64): load64 then compute64.
  __device__ __forceinline__ float score64(const void* krows, int64_t s0, int64_t s_end,
                                           int64_t s_safe) const {
    Keys kb;
    load64(krows, s0, s_end, s_safe, kb);
    return compute64(kb);
  }
};

}  // namespace misa
