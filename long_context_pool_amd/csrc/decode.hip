// Decode (one query per sequence) token scoring, Eq. (9) / Eq. (1) of the MISA
// summary page, followed by the top-k of Eq. (10) / (2).
//
// Decode is HBM-bound: every key of the sequence is read once (d*e bytes per
// key) whether h or H heads score it.  The score kernel streams keys with
// 16-byte loads straight into MFMA B operands: the query's scored head rows
// are the A operand (16-row tiles, rows past the head count are zero), 16 keys
// form one 16x16 output tile, and the ReLU * w head sum is done on the
// accumulators followed by a 4-lane reduction.  Each wave streams a contiguous
// run of keys and writes their scores (L fp32 per sequence) to the workspace.
//
// Selection without extra passes over the scores: while scoring, each
// workgroup counts its scores by their 13-bit order-preserving key digit
// (LDS histogram, flushed to the sequence's global histogram with atomics).
// The select kernel then knows, before touching the scores, the digit b* that
// holds the k-th best and how many scores lie above it; one pass over the row
// writes the tokens above b* and gathers those at b* into LDS, where the k-th
// is resolved exactly (pairwise rank, or radix select for long lists).
#include "common.hpp"
#include "launch.hpp"
#include "mfma.hpp"
#include "row_scorer.hpp"
#include "topk.hpp"

namespace misa {

namespace {

#ifndef MISA_DECODE_THREADS
#define MISA_DECODE_THREADS 256
#endif
#ifndef MISA_DECODE_KEYS_PER_WAVE
#define MISA_DECODE_KEYS_PER_WAVE 256
#endif
constexpr int kDecThreads = MISA_DECODE_THREADS;
constexpr int kDecWaves = kDecThreads / kWave;
constexpr int kSelThreads = 1024;
constexpr int kDigitShift = 19;                   // key >> 19: sign, exponent, 4 mantissa bits
constexpr int kDigits = 1 << (32 - kDigitShift);  // 8192
constexpr int kCandCap = 8192;

__device__ __forceinline__ uint32_t key_digit(float v) { return float_key(v) >> kDigitShift; }

template <int DT, int NRT>
__global__ __launch_bounds__(kDecThreads) void decode_score_kernel(
    const void* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    const void* __restrict__ k, const float* __restrict__ k_scale,
    const int32_t* __restrict__ heads, int32_t nh, float* __restrict__ rows,
    uint32_t* __restrict__ ghist, int32_t L, int32_t H, int32_t keys_per_wave) {
  __shared__ uint32_t hist[kDigits];
  for (int b = threadIdx.x; b < kDigits; b += kDecThreads) hist[b] = 0;
  __syncthreads();
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int64_t r = blockIdx.y;  // sequence (T == 1)
  RowScorer<DT, NRT> sc;
  sc.init(q, q_scale, w, heads, nh, r, H);
  const void* krows = (DT == kBF16) ? static_cast<const void*>(static_cast<const uint16_t*>(k) + r * L * kD)
                                    : static_cast<const void*>(static_cast<const uint8_t*>(k) + r * L * kD);
  const int64_t s_begin = (static_cast<int64_t>(blockIdx.x) * kDecWaves + wave) * keys_per_wave;
  const int64_t s_end = min<int64_t>(s_begin + keys_per_wave, L);
  for (int64_t s0 = s_begin; s0 < s_end; s0 += 64) {
    const float res = sc.score64(krows, s0, s_end, s_begin);
    const int64_t s = s0 + lane;
    if (s < s_end) {
      float v = res;
      if constexpr (DT == kFP8) v *= k_scale[r * L + s];
      rows[r * L + s] = v;
      atomicAdd(&hist[key_digit(v)], 1u);
    }
  }
  __syncthreads();
  uint32_t* gh = ghist + r * kDigits;
  for (int b = threadIdx.x; b < kDigits; b += kDecThreads) {
    const uint32_t c = hist[b];
    if (c) atomicAdd(&gh[b], c);
  }
}

__global__ void hist_clear_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = 0;
}

struct SelSmem {
  TopkSmem base;
  float cand_score[kCandCap];
  int32_t cand_idx[kCandCap];
  int wtmp[32];
  int sel_digit, sel_above, sel_count;
  int cnt_hi, cnt_at;
};

// Top-k of sequence r's score row given its digit histogram (see header).
__global__ __launch_bounds__(kSelThreads) void select_hist_kernel(
    const float* __restrict__ rows, const uint32_t* __restrict__ ghist, int32_t L, int32_t k,
    int32_t* __restrict__ idx_out, float* __restrict__ scores_out) {
  __shared__ SelSmem sm;
  const int64_t r = blockIdx.x;
  const int64_t n = L;
  const float* row = rows + r * n;
  int32_t* out_idx = idx_out + r * k;
  float* out_score = scores_out ? scores_out + r * k : nullptr;
  const int lane = lane_id();
  const int wid = threadIdx.x / kWave;
  if (n <= k) {
    for (int64_t i = threadIdx.x; i < k; i += kSelThreads) {
      out_idx[i] = i < n ? static_cast<int32_t>(i) : -1;
      if (out_score) out_score[i] = i < n ? row[i] : -__builtin_inff();
    }
    return;
  }
  // Digit b* holding the k-th best: suffix scan of the histogram.
  {
    constexpr int BPT = kDigits / kSelThreads;
    const uint32_t* gh = ghist + r * kDigits;
    int local[BPT];
    int lsum = 0;
#pragma unroll
    for (int c = 0; c < BPT; ++c) {
      local[c] = static_cast<int>(gh[kDigits - 1 - (threadIdx.x * BPT + c)]);
      lsum += local[c];
    }
    int total;
    int run = block_exclusive_sum<kSelThreads>(lsum, sm.wtmp, total);
#pragma unroll
    for (int c = 0; c < BPT; ++c) {
      if (run < k && run + local[c] >= k) {
        sm.sel_digit = kDigits - 1 - (threadIdx.x * BPT + c);
        sm.sel_above = run;
        sm.sel_count = local[c];
      }
      run += local[c];
    }
    if (threadIdx.x == 0) {
      sm.cnt_hi = 0;
      sm.cnt_at = 0;
    }
    __syncthreads();
  }
  const uint32_t bstar = static_cast<uint32_t>(sm.sel_digit);
  const int above = sm.sel_above;
  const int bcount = sm.sel_count;
  if (bcount > kCandCap) {
    block_topk<kSelThreads>(
        n, k, [](int64_t) { return true; }, [=](int64_t i) { return float_key(row[i]); },
        [](int64_t i) { return static_cast<int32_t>(i); }, [=](int64_t i) { return row[i]; },
        out_idx, out_score, sm.base);
    return;
  }
  // One pass: digits above b* -> output, digit b* -> LDS list.  Each wave
  // owns a contiguous range; positions come from wave ballots + LDS counters.
  constexpr int NW = kSelThreads / kWave;
  const int64_t CW = ((n + NW - 1) / NW + kWave - 1) / kWave * kWave;
  const int64_t wend = min<int64_t>((wid + 1) * CW, n);
  constexpr int kBatch = 16;  // loads in flight per lane before they are used
  for (int64_t b0 = wid * CW; b0 < wend; b0 += kBatch * kWave) {
    float vb[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t i = b0 + u * kWave + lane;
      vb[u] = i < wend ? row[i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t i = b0 + u * kWave + lane;
      const bool ok = i < wend;
      const float v = vb[u];
      const uint32_t dg = key_digit(v);
      const bool hi = ok && dg > bstar;
      const bool at = ok && dg == bstar;
      const uint64_t mh = __ballot(hi);
      const uint64_t ma = __ballot(at);
      if (mh) {
        int base = 0;
        if (lane == 0) base = atomicAdd(&sm.cnt_hi, __popcll(mh));
        base = __shfl(base, 0, kWave);
        if (hi) {
          const int p = base + lanes_below(mh);
          if (p < k) {
            out_idx[p] = static_cast<int32_t>(i);
            if (out_score) out_score[p] = v;
          }
        }
      }
      if (ma) {
        int base = 0;
        if (lane == 0) base = atomicAdd(&sm.cnt_at, __popcll(ma));
        base = __shfl(base, 0, kWave);
        if (at) {
          const int p = base + lanes_below(ma);
          if (p < kCandCap) {
            sm.cand_score[p] = v;
            sm.cand_idx[p] = static_cast<int32_t>(i);
          }
        }
      }
    }
  }
  __syncthreads();
  // The (k - above) best of the b* list (set semantics: any order).
  const int need = k - above;
  if (bcount <= kRankMax) {
    if (threadIdx.x < bcount) {
      const uint32_t key = float_key(sm.cand_score[threadIdx.x]);
      const int32_t id = sm.cand_idx[threadIdx.x];
      int rank = 0;
      for (int j = 0; j < bcount; ++j) {
        const uint32_t kj = float_key(sm.cand_score[j]);
        rank += (kj > key || (kj == key && sm.cand_idx[j] < id)) ? 1 : 0;
      }
      if (rank < need) {
        out_idx[above + rank] = id;
        if (out_score) out_score[above + rank] = sm.cand_score[threadIdx.x];
      }
    }
    return;
  }
  const float* cs = sm.cand_score;
  const int32_t* ci = sm.cand_idx;
  block_topk<kSelThreads>(
      bcount, need, [](int64_t) { return true; }, [=](int64_t j) { return float_key(cs[j]); },
      [=](int64_t j) { return ci[j]; }, [=](int64_t j) { return cs[j]; }, out_idx + above,
      out_score ? out_score + above : nullptr, sm.base);
}

template <int DT, int NRT>
void launch_dec(const Shape& s, int32_t nh, const int32_t* heads, const void* q, const float* qs,
                const float* w, const void* kk, const float* ks, float* rows, uint32_t* ghist,
                hipStream_t st) {
  const int kpw = MISA_DECODE_KEYS_PER_WAVE;
  dim3 grid((s.L + kDecWaves * kpw - 1) / (kDecWaves * kpw), s.batch);
  decode_score_kernel<DT, NRT><<<grid, kDecThreads, 0, st>>>(q, qs, w, kk, ks, heads, nh, rows,
                                                             ghist, s.L, s.H, kpw);
}

template <int DT>
void launch_dec_dt(const Shape& s, int32_t nh, const int32_t* heads, const void* q,
                   const float* qs, const float* w, const void* kk, const float* ks, float* rows,
                   uint32_t* ghist, hipStream_t st) {
  if (nh <= 16) launch_dec<DT, 1>(s, nh, heads, q, qs, w, kk, ks, rows, ghist, st);
  else if (nh <= 32) launch_dec<DT, 2>(s, nh, heads, q, qs, w, kk, ks, rows, ghist, st);
  else launch_dec<DT, 4>(s, nh, heads, q, qs, w, kk, ks, rows, ghist, st);
}

}  // namespace

size_t decode_ws_bytes(const Shape& s) {
  return align_up(static_cast<size_t>(s.batch) * s.L * sizeof(float)) +
         align_up(static_cast<size_t>(s.batch) * kDigits * sizeof(uint32_t));
}

hipError_t launch_decode_score_topk(const Shape& s, int32_t nh, const int32_t* heads, int32_t k,
                                    const void* q, const float* q_scale, const float* w,
                                    const void* kk, const float* k_scale, int32_t* idx,
                                    float* scores_out, void* ws, hipStream_t st) {
  float* rows = static_cast<float*>(ws);
  uint32_t* ghist = reinterpret_cast<uint32_t*>(
      static_cast<char*>(ws) + align_up(static_cast<size_t>(s.batch) * s.L * sizeof(float)));
  const int64_t nh_bins = static_cast<int64_t>(s.batch) * kDigits;
  hist_clear_kernel<<<static_cast<unsigned>((nh_bins + 1023) / 1024), 256, 0, st>>>(ghist, nh_bins);
  if (s.dtype == kBF16) launch_dec_dt<kBF16>(s, nh, heads, q, q_scale, w, kk, k_scale, rows, ghist, st);
  else launch_dec_dt<kFP8>(s, nh, heads, q, q_scale, w, kk, k_scale, rows, ghist, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  select_hist_kernel<<<s.batch, kSelThreads, 0, st>>>(rows, ghist, s.L, k, idx, scores_out);
  return hipGetLastError();
}

}  // namespace misa
