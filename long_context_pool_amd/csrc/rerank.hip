// Eq. (12) of the MISA summary page ("Methodology" 2, MISA-dagger fine
// stage): every candidate token kept by the routed pass is re-scored with all
// H heads (the Eq. (1) score) and the k best candidates are kept.
//
// bf16 / fp8: the query's H head rows are the A operand of 32x32 MFMA tiles
// (held in registers); each 32-candidate column tile gathers its key rows
// straight into B registers (lane l: candidate l%32, head-dim elements
// [64*(l/32), +64) -- one contiguous run per lane).  The ReLU * w head sum is
// taken on the accumulators.  With many query rows, one workgroup per query
// keeps its k' scores in LDS and selects in place; with few rows (decode) the
// candidates of a query are spread over many workgroups, scores go to the
// workspace and a select kernel per query follows.
// fp32: one thread per candidate (query rows staged in LDS), then the select.
#include "common.hpp"
#include "launch.hpp"
#include "mfma.hpp"
#include "topk.hpp"

namespace misa {

namespace {

constexpr int kRerankThreads = 256;
constexpr int kTopkThreads = 1024;
constexpr int kMaxHeads = 64;

template <int DT>
__global__ __launch_bounds__(kRerankThreads) void rerank_score_kernel(
    const void* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    const void* __restrict__ k, const float* __restrict__ k_scale,
    const int32_t* __restrict__ cand, int32_t kprime, float* __restrict__ out, int32_t L,
    int32_t T, int32_t H) {
  __shared__ float qs[kMaxHeads][kD];
  __shared__ float wsh[kMaxHeads];
  const int t = blockIdx.y;
  const int64_t seq = blockIdx.z;
  const int64_t r = seq * T + t;
  const float sq = (DT == kFP8) ? q_scale[r] : 1.f;
  for (int e = threadIdx.x; e < H * kD; e += kRerankThreads)
    qs[e / kD][e % kD] = load_elem<DT>(q, r * H * kD + e) * sq;
  if (threadIdx.x < H) wsh[threadIdx.x] = w[r * H + threadIdx.x];
  __syncthreads();
  const int64_t c = static_cast<int64_t>(blockIdx.x) * kRerankThreads + threadIdx.x;
  if (c >= kprime) return;
  const int32_t s = cand[r * kprime + c];
  const int64_t pos = static_cast<int64_t>(L) - T + t;
  if (s < 0 || s > pos) {  // padding, or outside the query's prefix: ignored
    out[r * kprime + c] = -__builtin_inff();
    return;
  }
  float kr[kD];
  const float sk = (DT == kFP8) ? k_scale[seq * L + s] : 1.f;
#pragma unroll
  for (int i = 0; i < kD; ++i) kr[i] = load_elem<DT>(k, (seq * L + s) * kD + i) * sk;
  float acc = 0.f;
  for (int j = 0; j < H; ++j) {
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < kD; ++i) dot += qs[j][i] * kr[i];
    acc += wsh[j] * fmaxf(dot, 0.f);
  }
  out[r * kprime + c] = acc;
}

__global__ __launch_bounds__(kTopkThreads) void topk_list_kernel(const float* __restrict__ sc,
                                                                 const int32_t* __restrict__ cand,
                                                                 int32_t kprime, int32_t L,
                                                                 int32_t T, int32_t k,
                                                                 int32_t* __restrict__ idx,
                                                                 float* __restrict__ scores_out) {
  __shared__ TopkFastSmem sm;
  const int64_t r = static_cast<int64_t>(blockIdx.y) * T + blockIdx.x;
  const int64_t pos = static_cast<int64_t>(L) - T + blockIdx.x;
  const float* srow = sc + r * kprime;
  const int32_t* crow = cand + r * kprime;
  block_topk_fast<kTopkThreads>(
      kprime, k, [=](int64_t i) { return crow[i] >= 0 && crow[i] <= pos; },
      [=](int64_t i) { return srow[i]; }, [=](int64_t i) { return crow[i]; }, idx + r * k,
      scores_out ? scores_out + r * k : nullptr, sm);
}

constexpr int kRRThreads = 256;
constexpr int kRRWaves = kRRThreads / kWave;
constexpr int kMaxKprime = 8192;

// Per-wave state: the query's head rows (A) and per-lane row weights.
template <int DT, int RT>
struct CandScorer {
  bf16x8 a16[RT][8];
  i32x8 a8[RT][2];
  float wl[RT][16];

  __device__ __forceinline__ void init(const void* q, const float* q_scale, const float* w,
                                       int64_t r, int H) {
    const int lane = lane_id();
    const int hf = lane >> 5;
    const float sq = (DT == kFP8) ? q_scale[r] : 1.f;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int j = rt * 32 + (lane & 31);
      const int64_t qoff = (r * H + (j < H ? j : 0)) * kD;
      if constexpr (DT == kBF16) {
        const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(q) + qoff + 64 * hf);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) a16[rt][ks] = as_bf16x8(j < H ? src[ks] : make_uint4(0, 0, 0, 0));
      } else {
        const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(q) + qoff + 64 * hf);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const uint4 lo = j < H ? src[2 * ks] : make_uint4(0, 0, 0, 0);
          const uint4 hi = j < H ? src[2 * ks + 1] : make_uint4(0, 0, 0, 0);
          a8[rt][ks] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = rt * 32 + 8 * (i / 4) + 4 * hf + (i % 4);
        wl[rt][i] = row < H ? w[r * H + row] * sq : 0.f;
      }
    }
  }

  // Score of this lane's column candidate whose key row starts at krow
  // (always a valid row; the caller masks invalid candidates).
  __device__ __forceinline__ float score(const void* krow) const {
    const int hf = lane_id() >> 5;
    f32x16 acc[RT];
    if constexpr (DT == kBF16) {
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(krow) + 64 * hf);
      uint4 b[8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) b[ks] = src[ks];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          acc[rt] = mfma32_bf16(a16[rt][ks], as_bf16x8(b[ks]), ks == 0 ? f32x16{} : acc[rt]);
    } else {
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(krow) + 64 * hf);
      uint4 b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) b[u] = src[u];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const i32x8 bb{(int)b[2 * ks].x, (int)b[2 * ks].y, (int)b[2 * ks].z, (int)b[2 * ks].w,
                       (int)b[2 * ks + 1].x, (int)b[2 * ks + 1].y, (int)b[2 * ks + 1].z, (int)b[2 * ks + 1].w};
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[rt] = mfma32_fp8(a8[rt][ks], bb, ks == 0 ? f32x16{} : acc[rt]);
      }
    }
    float part = 0.f;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 16; ++i) part += wl[rt][i] * relu(acc[rt][i]);
    return part + __shfl_xor(part, 32, kWave);  // rows 4hf..: the other half-wave
  }
};

template <int DT>
__device__ __forceinline__ const void* key_row(const void* k, int64_t row) {
  if constexpr (DT == kBF16) return static_cast<const uint16_t*>(k) + row * kD;
  else return static_cast<const uint8_t*>(k) + row * kD;
}

// One workgroup per query row: scores of all k' candidates in LDS, then the
// top-k among the valid ones.
template <int DT, int RT>
__global__ __launch_bounds__(kRRThreads) void rerank_fused_kernel(
    const void* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    const void* __restrict__ k, const float* __restrict__ k_scale,
    const int32_t* __restrict__ cand, int32_t kprime, int32_t k_top, int32_t L, int32_t T,
    int32_t H, int32_t* __restrict__ idx, float* __restrict__ scores_out) {
  __shared__ float sc[kMaxKprime];
  __shared__ TopkFastSmem sm;
  const int64_t r = blockIdx.x;
  const int64_t seq = r / T;
  const int64_t pos = static_cast<int64_t>(L) - T + (r % T);
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int32_t* crow = cand + r * kprime;
  CandScorer<DT, RT> cs;
  cs.init(q, q_scale, w, r, H);
  const int ntile = (kprime + 31) / 32;
  for (int ct = wave; ct < ntile; ct += kRRWaves) {
    const int c = ct * 32 + (lane & 31);
    const int32_t s = c < kprime ? crow[c] : -1;
    const bool ok = s >= 0 && s <= pos;
    const int64_t row = seq * L + (ok ? s : 0);
    float v = cs.score(key_row<DT>(k, row));
    if constexpr (DT == kFP8) v *= k_scale[row];
    if (lane < 32 && c < kprime) sc[c] = v;
  }
  __syncthreads();
  block_topk_fast<kRRThreads>(
      kprime, k_top, [=](int64_t c) { return crow[c] >= 0 && crow[c] <= pos; },
      [=](int64_t c) { return sc[c]; }, [=](int64_t c) { return crow[c]; }, idx + r * k_top,
      scores_out ? scores_out + r * k_top : nullptr, sm);
}

// Few query rows: workgroup (chunk, row) scores 32 candidates per wave and
// writes them to the workspace; topk_list_kernel selects afterwards.
template <int DT, int RT>
__global__ __launch_bounds__(kRRThreads) void rerank_split_kernel(
    const void* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    const void* __restrict__ k, const float* __restrict__ k_scale,
    const int32_t* __restrict__ cand, int32_t kprime, int32_t L, int32_t T, int32_t H,
    float* __restrict__ out) {
  const int64_t r = blockIdx.y;
  const int64_t seq = r / T;
  const int64_t pos = static_cast<int64_t>(L) - T + (r % T);
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  CandScorer<DT, RT> cs;
  cs.init(q, q_scale, w, r, H);
  const int c = (blockIdx.x * kRRWaves + wave) * 32 + (lane & 31);
  const int32_t s = c < kprime ? cand[r * kprime + c] : -1;
  const bool ok = s >= 0 && s <= pos;
  const int64_t row = seq * L + (ok ? s : 0);
  float v = cs.score(key_row<DT>(k, row));
  if constexpr (DT == kFP8) v *= k_scale[row];
  if (lane < 32 && c < kprime) out[r * kprime + c] = ok ? v : -__builtin_inff();
}

}  // namespace

size_t rerank_ws_bytes(const Shape& s, int32_t kprime) {
  return align_up(static_cast<size_t>(s.batch) * s.T * kprime * sizeof(float));
}

hipError_t launch_rerank(const Shape& s, int32_t kprime, int32_t k, const void* q,
                         const float* q_scale, const float* w, const void* kk, const float* k_scale,
                         const int32_t* cand, int32_t* idx, float* scores_out, void* ws,
                         hipStream_t st) {
  const int64_t rows = static_cast<int64_t>(s.batch) * s.T;
  float* sc = static_cast<float*>(ws);
  if (s.dtype != kF32) {
    const bool two = s.H > 32;
    if (rows >= 64) {
#define RF(DT, RT) rerank_fused_kernel<DT, RT><<<static_cast<unsigned>(rows), kRRThreads, 0, st>>>(q, q_scale, w, kk, k_scale, cand, kprime, k, s.L, s.T, s.H, idx, scores_out)
      if (s.dtype == kBF16) { if (two) RF(kBF16, 2); else RF(kBF16, 1); }
      else { if (two) RF(kFP8, 2); else RF(kFP8, 1); }
#undef RF
      return hipGetLastError();
    }
    dim3 g((kprime + kRRWaves * 32 - 1) / (kRRWaves * 32), static_cast<unsigned>(rows));
#define RS(DT, RT) rerank_split_kernel<DT, RT><<<g, kRRThreads, 0, st>>>(q, q_scale, w, kk, k_scale, cand, kprime, s.L, s.T, s.H, sc)
    if (s.dtype == kBF16) { if (two) RS(kBF16, 2); else RS(kBF16, 1); }
    else { if (two) RS(kFP8, 2); else RS(kFP8, 1); }
#undef RS
  } else {
    dim3 g1((kprime + kRerankThreads - 1) / kRerankThreads, s.T, s.batch);
    rerank_score_kernel<kF32><<<g1, kRerankThreads, 0, st>>>(q, q_scale, w, kk, k_scale, cand,
                                                             kprime, sc, s.L, s.T, s.H);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2(s.T, s.batch);
  topk_list_kernel<<<g2, kTopkThreads, 0, st>>>(sc, cand, kprime, s.L, s.T, k, idx, scores_out);
  return hipGetLastError();
}

}  // namespace misa
