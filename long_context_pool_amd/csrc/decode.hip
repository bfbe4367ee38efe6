// Decode (one query per sequence): token scoring, Eq. (9) / Eq. (1) of the
// MISA summary page, and the top-k of Eq. (10) / (2); plus the fused decode
// step (router of Eq. (7)-(8) + scoring + top-k).
//
// Decode is HBM-bound: every key of the sequence is read once (d*e bytes per
// key) whether h or H heads score it.  The score kernel streams keys with
// 16-byte loads straight into MFMA B operands (RowScorer: the query's scored
// head rows are the A operand, 16 keys per 16x16 output tile, ReLU * w head
// sum on the accumulators) and writes the scores (L fp32 per sequence) to the
// workspace.  While scoring, each workgroup counts its scores by a histogram
// digit (a monotone map of the score to 8192 bins; LDS histogram, flushed to
// the sequence's global histogram with atomics), so after the score kernel
// the digit b* holding the k-th best score of every sequence is known without
// another pass:
//   compact  (many workgroups per sequence): every workgroup finds b* from the
//            histogram, writes its tokens of digits above b* straight to the
//            output and appends those of digit b* to a short list (one packed
//            atomic counter per sequence reserves both ranges);
//   resolve  (one workgroup per sequence): the (k - above) best of the b*
//            list, exactly.
// Kernel boundaries order these steps: no workgroup waits for another inside
// a kernel (a device-wide release fence per workgroup costs far more than a
// launch here).
//
// The fused step starts with a router kernel: workgroup (chunk, sequence)
// sums ReLU(q_j . p_b) over 32 pooled blocks in fp32 (the last block's pooled
// key -- the block holding the newest key -- is recomputed from the keys and
// written back to the cache, the per-step pooling of Eq. (4)); every score
// workgroup then finishes the router for its sequence (E and top-h, Eq. (7)-
// (8)) before scoring, so no separate route launch is needed.
#include "common.hpp"
#include "launch.hpp"
#include "mfma.hpp"
#include "route_common.hpp"
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
constexpr int kDigits = 8192;
constexpr int kCandCap = 2048;                    // LDS list of the threshold digit
constexpr int kChunk = 32;                        // pooled blocks per router workgroup
constexpr int kMaxH = 64;

// Histogram digit of a score: a monotone (non-decreasing) map of fp32 values
// to [0, kDigits) that spends its bins where top-k thresholds live.  Bin 0
// holds every negative value, bin 1 zero (and subnormals); positive values
// with binary exponent in a 63-binade window get 128 bins per binade (7
// mantissa bits: bins 0.8% wide), values below or above the window share the
// window's first or last bin.  A 13-bit prefix of the order-preserving key
// would spend 7/8 of its bins on exponents that scores never reach and leave
// bins 6% wide.
constexpr int kExpLo = 127 - 31;  // window: values in [2^-31, 2^32)
constexpr int kExpBins = 63;
__device__ __forceinline__ uint32_t key_digit(float v) {
  const uint32_t u = __float_as_uint(v);
  const int e = static_cast<int>((u >> 23) & 0xFFu);
  if (u >> 31) return 0u;
  if (e == 0) return 1u;
  if (e < kExpLo) return 2u;
  if (e >= kExpLo + kExpBins) return 2u + ((kExpBins - 1) << 7) + 127u;
  return 2u + (static_cast<uint32_t>(e - kExpLo) << 7) + ((u >> 16) & 0x7Fu);
}
static_assert(2 + (kExpBins << 7) <= kDigits, "digit range");

// The digit b* of the k-th largest score of a row from its digit histogram
// gh[kDigits] (total n > k): *digit, *above = count in higher digits, *count =
// count at b*.  All threads call; the results are in LDS on return.
template <int NT>
__device__ __forceinline__ void find_digit(const uint32_t* gh, int k, int* scan_tmp, int* digit,
                                           int* above, int* count) {
  constexpr int BPT = kDigits / NT;
  int local[BPT];
  int lsum = 0;
  // Thread t owns digits kDigits-1-t*BPT downwards (highest digits first).
  const uint4* src = reinterpret_cast<const uint4*>(gh + kDigits - (threadIdx.x + 1) * BPT);
#pragma unroll
  for (int c = 0; c < BPT / 4; ++c) {
    const uint4 v = src[BPT / 4 - 1 - c];
    local[4 * c] = static_cast<int>(v.w);
    local[4 * c + 1] = static_cast<int>(v.z);
    local[4 * c + 2] = static_cast<int>(v.y);
    local[4 * c + 3] = static_cast<int>(v.x);
  }
#pragma unroll
  for (int c = 0; c < BPT; ++c) lsum += local[c];
  int total;
  int run = block_exclusive_sum<NT>(lsum, scan_tmp, total);
#pragma unroll
  for (int c = 0; c < BPT; ++c) {
    if (run < k && run + local[c] >= k) {
      *digit = kDigits - 1 - (threadIdx.x * BPT + c);
      *above = run;
      *count = local[c];
    }
    run += local[c];
  }
  __syncthreads();
}

struct DecodeArgs {
  const void* q;
  const float* q_scale;
  const float* w;
  const void* k;
  const float* k_scale;
  const int32_t* heads;  // scored heads [batch, nh] (nullptr: all heads) -- unfused
  int32_t nh;
  // Fused router: per-chunk partial ReLU sums [batch, nchunks, 64].
  const float* route_part;
  int32_t nchunks;
  int32_t h;
  int32_t* heads_out;
  float* E_out;
  int64_t Mt;
  // Score rows [batch, L] and digit histograms [batch, kDigits].
  float* rows;
  uint32_t* ghist;
  int32_t L, H, keys_per_wave;
};

template <int DT, int NRT, bool FUSED>
__global__ __launch_bounds__(kDecThreads) void decode_score_kernel(DecodeArgs a) {
  __shared__ uint32_t hist[kDigits];
  __shared__ int32_t sh_heads[16];
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int64_t r = blockIdx.y;  // sequence (T == 1)
  for (int b = threadIdx.x; b < kDigits; b += kDecThreads) hist[b] = 0;
  const int32_t* heads = a.heads;
  int64_t hrow = r;
  if constexpr (FUSED) {
    // Finish the router for this sequence: E_j and the top-h heads.
    if (wave == 0) {
      float sum = 0.f;
      for (int c0 = 0; c0 < a.nchunks; c0 += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          v[u] = c0 + u < a.nchunks ? a.route_part[(r * a.nchunks + c0 + u) * kMaxH + lane] : 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) sum += v[u];
      }
      float e = -2.f;
      if (lane < a.H) {
        const float sq = (DT == kFP8) ? a.q_scale[r] : 1.f;
        e = fabsf(a.w[r * a.H + lane]) * sq * sum / static_cast<float>(a.Mt);
        if (blockIdx.x == 0 && a.E_out) a.E_out[r * a.H + lane] = e;
      }
      wave_top_heads(e, a.H, a.h, sh_heads);
    }
    __syncthreads();
    if (blockIdx.x == 0 && threadIdx.x < a.h) a.heads_out[r * a.h + threadIdx.x] = sh_heads[threadIdx.x];
    heads = sh_heads;
    hrow = 0;
  }
  __syncthreads();
  RowScorer<DT, NRT> sc;
  sc.init(a.q, a.q_scale, a.w, heads, a.nh, r, a.H, hrow);
  const void* krows = (DT == kBF16) ? static_cast<const void*>(static_cast<const uint16_t*>(a.k) + r * a.L * kD)
                                    : static_cast<const void*>(static_cast<const uint8_t*>(a.k) + r * a.L * kD);
  const int64_t s_begin = (static_cast<int64_t>(blockIdx.x) * kDecWaves + wave) * a.keys_per_wave;
  const int64_t s_end = min<int64_t>(s_begin + a.keys_per_wave, a.L);
  float* row = a.rows + r * a.L;
  for (int64_t s0 = s_begin; s0 < s_end; s0 += 64) {
    const float res = sc.score64(krows, s0, s_end, s_begin);
    const int64_t s = s0 + lane;
    if (s < s_end) {
      float v = res;
      if constexpr (DT == kFP8) v *= a.k_scale[r * a.L + s];
      row[s] = v;
      atomicAdd(&hist[key_digit(v)], 1u);
    }
  }
  __syncthreads();
  uint32_t* gh = a.ghist + r * kDigits;
  for (int b = threadIdx.x; b < kDigits; b += kDecThreads) {
    const uint32_t c = hist[b];
    if (c) atomicAdd(&gh[b], c);
  }
}

// Top-k of one row in one workgroup (rows of at most PER * kSelThreads
// scores): the row is read once into registers (PER scores per thread,
// coalesced) together with the histogram, tokens of digits above b* go
// straight to the output and those of digit b* to an LDS list (positions
// from one block scan), and the list is resolved exactly.  Everything is a
// short chain of dependent steps: this kernel is latency-bound.
constexpr int kSelThreads = 1024;

struct SelectSmem {
  alignas(16) float cand_score[kCandCap];
  alignas(16) int32_t cand_idx[kCandCap];
  ResolveSmem rs;
  TopkSmem base;
  int scan_tmp[32];
  int digit, above, count;
};

template <int PER>
__global__ __launch_bounds__(kSelThreads) void decode_select_kernel(
    const float* __restrict__ rows, const uint32_t* __restrict__ ghist, int32_t* __restrict__ idx,
    float* __restrict__ scores_out, int32_t L, int32_t k) {
  __shared__ SelectSmem sm;
  const int64_t r = blockIdx.x;
  const float* row = rows + r * L;
  int32_t* out = idx + r * k;
  float* out_s = scores_out ? scores_out + r * k : nullptr;
  if (L <= k) {
    for (int i = threadIdx.x; i < k; i += kSelThreads) {
      out[i] = i < L ? i : -1;
      if (out_s) out_s[i] = i < L ? row[i] : -__builtin_inff();
    }
    return;
  }
  // Loads are clamped to the row (L >= 1) and masked below, so the register
  // array is written without branches.
  float v[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) v[j] = row[min(j * kSelThreads + static_cast<int>(threadIdx.x), L - 1)];
  find_digit<kSelThreads>(ghist + r * kDigits, k, sm.scan_tmp, &sm.digit, &sm.above, &sm.count);
  const uint32_t bstar = static_cast<uint32_t>(sm.digit);
  const int above = sm.above;
  const int bcount = sm.count;
  if (bcount > kCandCap) {
    block_topk<kSelThreads>(
        L, k, [](int64_t) { return true; }, [=](int64_t i) { return float_key(row[i]); },
        [](int64_t i) { return static_cast<int32_t>(i); }, [=](int64_t i) { return row[i]; }, out,
        out_s, sm.base);
    return;
  }
  uint64_t mh = 0, ma = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = j * kSelThreads + threadIdx.x;
    const uint32_t dg = key_digit(v[j]);
    mh |= (i < L && dg > bstar) ? (uint64_t{1} << j) : 0u;
    ma |= (i < L && dg == bstar) ? (uint64_t{1} << j) : 0u;
  }
  // Packed counts: above-b* in the low 16 bits (row total < k <= 8192),
  // at-b* in the high 16 bits (row total <= kCandCap).
  int total;
  const int off = block_exclusive_sum<kSelThreads>(__popcll(mh) | (__popcll(ma) << 16), sm.scan_tmp,
                                                   total);
  int ph = off & 0xFFFF;
  int pa = off >> 16;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = j * kSelThreads + threadIdx.x;
    if ((mh >> j) & 1u) {
      if (ph < k) {
        out[ph] = i;
        if (out_s) out_s[ph] = v[j];
      }
      ++ph;
    } else if ((ma >> j) & 1u) {
      if (pa < kCandCap) {
        sm.cand_score[pa] = v[j];
        sm.cand_idx[pa] = i;
      }
      ++pa;
    }
  }
  __syncthreads();
  if (resolve_list<kSelThreads>(sm.cand_score, sm.cand_idx, bcount, k - above, out + above,
                                out_s ? out_s + above : nullptr, sm.rs))
    return;
  __syncthreads();
  const float* cs = sm.cand_score;
  const int32_t* ci = sm.cand_idx;
  block_topk<kSelThreads>(
      bcount, k - above, [](int64_t) { return true; }, [=](int64_t j) { return float_key(cs[j]); },
      [=](int64_t j) { return ci[j]; }, [=](int64_t j) { return cs[j]; }, out + above,
      out_s ? out_s + above : nullptr, sm.base);
}

// Top-k step 1: tokens of digits above b* -> output, digit b* -> the list.
// Workgroup (chunk, sequence) takes kCompactChunk consecutive scores.
constexpr int kCompactThreads = 256;
constexpr int kCompactPer = 16;  // scores per thread
constexpr int kCompactChunk = kCompactThreads * kCompactPer;

struct SelState {
  int digit, above, count, pad;
};

__global__ __launch_bounds__(kCompactThreads) void decode_compact_kernel(
    const float* __restrict__ rows, const uint32_t* __restrict__ ghist, uint32_t* __restrict__ cnt,
    SelState* __restrict__ sel, float* __restrict__ cand_s, int32_t* __restrict__ cand_i,
    int32_t* __restrict__ idx, float* __restrict__ scores_out, int32_t L, int32_t k) {
  __shared__ int scan_tmp[32];
  __shared__ int s_digit, s_above, s_count;
  __shared__ uint32_t s_base;
  if (L <= k) return;
  const int64_t r = blockIdx.y;
  const float* row = rows + r * L;
  const int c0 = blockIdx.x * kCompactChunk;
  // Scores first (independent of b*), so their loads overlap the scan.
  float v[kCompactPer];  // clamped loads; tokens past L are masked below
#pragma unroll
  for (int j = 0; j < kCompactPer; ++j)
    v[j] = row[min(c0 + j * kCompactThreads + static_cast<int>(threadIdx.x), L - 1)];
  find_digit<kCompactThreads>(ghist + r * kDigits, k, scan_tmp, &s_digit, &s_above, &s_count);
  const uint32_t bstar = static_cast<uint32_t>(s_digit);
  const int count = s_count;
  if (blockIdx.x == 0 && threadIdx.x == 0) sel[r] = SelState{s_digit, s_above, count, 0};
  if (count > kCandCap) return;  // the resolve kernel selects from the whole row
  uint32_t mh = 0, ma = 0;
#pragma unroll
  for (int j = 0; j < kCompactPer; ++j) {
    const int i = c0 + j * kCompactThreads + threadIdx.x;
    const uint32_t dg = key_digit(v[j]);
    mh |= (i < L && dg > bstar) ? (1u << j) : 0u;
    ma |= (i < L && dg == bstar) ? (1u << j) : 0u;
  }
  // Packed counts: above-b* in the low 16 bits (their row total is below
  // k <= 8192), at-b* in the high 16 bits (row total <= kCandCap).
  const int packed = __popc(mh) | (__popc(ma) << 16);
  int total;
  const int off = block_exclusive_sum<kCompactThreads>(packed, scan_tmp, total);
  if (threadIdx.x == 0) s_base = atomicAdd(&cnt[r], static_cast<uint32_t>(total));
  __syncthreads();
  const uint32_t base = s_base + static_cast<uint32_t>(off);
  int ph = static_cast<int>(base & 0xFFFFu);
  int pa = static_cast<int>(base >> 16);
  int32_t* out = idx + r * k;
  float* out_s = scores_out ? scores_out + r * k : nullptr;
  float* ls = cand_s + r * kCandCap;
  int32_t* li = cand_i + r * kCandCap;
#pragma unroll
  for (int j = 0; j < kCompactPer; ++j) {
    const int i = c0 + j * kCompactThreads + threadIdx.x;
    if ((mh >> j) & 1u) {
      if (ph < k) {
        out[ph] = i;
        if (out_s) out_s[ph] = v[j];
      }
      ++ph;
    } else if ((ma >> j) & 1u) {
      if (pa < kCandCap) {
        ls[pa] = v[j];
        li[pa] = i;
      }
      ++pa;
    }
  }
}

// Top-k step 2, one workgroup per sequence: the (k - above) best of the b*
// list (or, when b* holds more than kCandCap tokens, the whole row).
constexpr int kResolveThreads = 256;

struct ResolveAll {
  alignas(16) float cand_score[kCandCap];
  alignas(16) int32_t cand_idx[kCandCap];
  ResolveSmem rs;
  TopkSmem base;
};

__global__ __launch_bounds__(kResolveThreads) void decode_resolve_kernel(
    const float* __restrict__ rows, const SelState* __restrict__ sel,
    const float* __restrict__ cand_s, const int32_t* __restrict__ cand_i,
    int32_t* __restrict__ idx, float* __restrict__ scores_out, int32_t L, int32_t k) {
  __shared__ ResolveAll sm;
  const int64_t r = blockIdx.x;
  const float* row = rows + r * L;
  int32_t* out = idx + r * k;
  float* out_s = scores_out ? scores_out + r * k : nullptr;
  if (L <= k) {
    for (int i = threadIdx.x; i < k; i += kResolveThreads) {
      out[i] = i < L ? i : -1;
      if (out_s) out_s[i] = i < L ? row[i] : -__builtin_inff();
    }
    return;
  }
  const SelState st = sel[r];
  const int above = st.above;
  const int bcount = st.count;
  if (bcount > kCandCap) {
    block_topk<kResolveThreads>(
        L, k, [](int64_t) { return true; }, [=](int64_t i) { return float_key(row[i]); },
        [](int64_t i) { return static_cast<int32_t>(i); }, [=](int64_t i) { return row[i]; }, out,
        out_s, sm.base);
    return;
  }
  for (int t = threadIdx.x; t < bcount; t += kResolveThreads) {
    sm.cand_score[t] = cand_s[r * kCandCap + t];
    sm.cand_idx[t] = cand_i[r * kCandCap + t];
  }
  __syncthreads();
  if (resolve_list<kResolveThreads>(sm.cand_score, sm.cand_idx, bcount, k - above, out + above,
                                    out_s ? out_s + above : nullptr, sm.rs))
    return;
  __syncthreads();
  const float* cs = sm.cand_score;
  const int32_t* ci = sm.cand_idx;
  block_topk<kResolveThreads>(
      bcount, k - above, [](int64_t) { return true; }, [=](int64_t j) { return float_key(cs[j]); },
      [=](int64_t j) { return ci[j]; }, [=](int64_t j) { return cs[j]; }, out + above,
      out_s ? out_s + above : nullptr, sm.base);
}

__global__ void clear_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = 0;
}

// Fused step, kernel 1: router partial sums over 32 pooled blocks per
// workgroup; the workgroup holding the newest key's block recomputes that
// block's mean from the keys and writes it to the cache.  Also zeroes the
// digit histograms and compaction counters of the top-k kernels.
template <int DT>
__global__ __launch_bounds__(256) void step_route_kernel(
    const void* __restrict__ q, float* __restrict__ pooled, const void* __restrict__ k,
    const float* __restrict__ k_scale, float* __restrict__ part, uint32_t* __restrict__ zero,
    int64_t nzero, int32_t L, int32_t H, int32_t B, int64_t M, int32_t nchunks) {
  __shared__ __attribute__((aligned(16))) float ps[kChunk][kD];
  __shared__ float red[4][kMaxH];
  __shared__ float lastp[32][kD];
  {
    const int64_t g = static_cast<int64_t>(blockIdx.y) * gridDim.x + blockIdx.x;
    const int64_t G = static_cast<int64_t>(gridDim.x) * gridDim.y;
    for (int64_t i = g * 256 + threadIdx.x; i < nzero; i += G * 256) zero[i] = 0;
  }
  const int c = blockIdx.x;
  const int64_t seq = blockIdx.y;
  const int j = threadIdx.x & (kMaxH - 1);
  const int sub = threadIdx.x / kMaxH;
  const int64_t b0 = static_cast<int64_t>(c) * kChunk;
  const int nb = static_cast<int>(min<int64_t>(kChunk, M - b0));
  const int64_t blast = M - 1;  // the block holding key L-1
  for (int e = threadIdx.x; e < kChunk * kD / 4; e += 256) {
    const int b = e / (kD / 4);
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (b < nb && b0 + b != blast)
      v = reinterpret_cast<const float4*>(pooled + (seq * M + b0 + b) * kD)[e % (kD / 4)];
    reinterpret_cast<float4*>(&ps[b][0])[e % (kD / 4)] = v;
  }
  if (blast >= b0 && blast < b0 + nb) {
    // Mean of keys [blast*B, L): thread t takes 16-byte piece t % P of key
    // rows t / P + KPR * u; a round's loads are all in flight together and
    // the per-dimension partial sums of the KPR key slots meet in LDS.
    constexpr int EB = (DT == kBF16) ? 2 : 1;  // bytes per element
    constexpr int P = kD * EB / 16;            // pieces per key row
    constexpr int EPP = 16 / EB;               // elements per piece
    constexpr int KPR = 256 / P;               // key slots
    constexpr int U = 4;
    const int piece = threadIdx.x % P;
    const int slot = threadIdx.x / P;
    const int64_t s0 = blast * B;
    const int nl = static_cast<int>(L - s0);
    const uint8_t* kb = static_cast<const uint8_t*>(k) + (seq * L + s0) * kD * EB;
    float acc[EPP];
#pragma unroll
    for (int e = 0; e < EPP; ++e) acc[e] = 0.f;
    for (int r0 = 0; r0 < nl; r0 += KPR * U) {
      uint4 v[U];
      float sc[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int key = r0 + slot + KPR * u;
        v[u] = make_uint4(0, 0, 0, 0);
        sc[u] = 0.f;
        if (key < nl) {
          v[u] = reinterpret_cast<const uint4*>(kb + static_cast<int64_t>(key) * kD * EB)[piece];
          if constexpr (DT == kFP8) sc[u] = k_scale[seq * L + s0 + key];
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t wd[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
        if constexpr (DT == kBF16) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[2 * e] += __uint_as_float(wd[e] << 16);
            acc[2 * e + 1] += __uint_as_float(wd[e] & 0xFFFF0000u);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[e] += fp8_to_f32((wd[e / 4] >> (8 * (e % 4))) & 0xFF) * sc[u];
        }
      }
    }
#pragma unroll
    for (int e = 0; e < EPP; ++e) lastp[slot][piece * EPP + e] = acc[e];
    __syncthreads();
    if (threadIdx.x < kD) {
      float sum = 0.f;
#pragma unroll
      for (int sl = 0; sl < KPR; ++sl) sum += lastp[sl][threadIdx.x];
      const float m = sum / static_cast<float>(nl);
      ps[blast - b0][threadIdx.x] = m;
      pooled[(seq * M + blast) * kD + threadIdx.x] = m;
    }
  }
  float qr[kD];
  load_head_row<DT>(q, (seq * H + (j < H ? j : 0)) * kD, qr);
  __syncthreads();
  float acc = 0.f;
  for (int b = sub; b < nb; b += 4) acc += relu(dot_lds_row(qr, &ps[b][0]));
  red[sub][j] = acc;
  __syncthreads();
  if (threadIdx.x < kMaxH)
    part[(seq * nchunks + c) * kMaxH + threadIdx.x] =
        red[0][threadIdx.x] + red[1][threadIdx.x] + red[2][threadIdx.x] + red[3][threadIdx.x];
}

template <int DT, bool FUSED>
void launch_score(const Shape& s, const DecodeArgs& a, hipStream_t st) {
  dim3 grid((s.L + kDecWaves * a.keys_per_wave - 1) / (kDecWaves * a.keys_per_wave), s.batch);
  if (a.nh <= 16) decode_score_kernel<DT, 1, FUSED><<<grid, kDecThreads, 0, st>>>(a);
  else if (a.nh <= 32) decode_score_kernel<DT, 2, FUSED><<<grid, kDecThreads, 0, st>>>(a);
  else decode_score_kernel<DT, 4, FUSED><<<grid, kDecThreads, 0, st>>>(a);
}

struct DecodeWs {
  float* rows;
  uint32_t* ghist;  // [batch, kDigits], followed by
  uint32_t* cnt;    // [batch] packed compaction counters (zeroed together)
  SelState* sel;
  float* cand_s;
  int32_t* cand_i;
  float* part;
  size_t total;
};

DecodeWs decode_layout(const Shape& s, void* ws) {
  const uintptr_t base = reinterpret_cast<uintptr_t>(ws);
  const size_t nb = static_cast<size_t>(s.batch);
  DecodeWs d{};
  size_t off = 0;
  d.rows = reinterpret_cast<float*>(base + off);
  off += align_up(nb * s.L * sizeof(float));
  d.ghist = reinterpret_cast<uint32_t*>(base + off);
  d.cnt = reinterpret_cast<uint32_t*>(base + off) + nb * kDigits;
  off += align_up((nb * kDigits + nb) * sizeof(uint32_t));
  d.sel = reinterpret_cast<SelState*>(base + off);
  off += align_up(nb * sizeof(SelState));
  d.cand_s = reinterpret_cast<float*>(base + off);
  off += align_up(nb * kCandCap * sizeof(float));
  d.cand_i = reinterpret_cast<int32_t*>(base + off);
  off += align_up(nb * kCandCap * sizeof(int32_t));
  d.part = reinterpret_cast<float*>(base + off);
  const int64_t nch = (s.M() + kChunk - 1) / kChunk;
  off += align_up(nb * nch * kMaxH * sizeof(float));
  d.total = off;
  return d;
}

void launch_select(const Shape& s, const DecodeWs& d, int32_t k, int32_t* idx, float* scores_out,
                   hipStream_t st) {
#ifndef MISA_DECODE_SELECT_SPLIT
  if (s.L <= 32 * kSelThreads) {
    decode_select_kernel<32><<<s.batch, kSelThreads, 0, st>>>(d.rows, d.ghist, idx, scores_out, s.L, k);
    return;
  }
#endif
  dim3 g((s.L + kCompactChunk - 1) / kCompactChunk, s.batch);
  decode_compact_kernel<<<g, kCompactThreads, 0, st>>>(d.rows, d.ghist, d.cnt, d.sel, d.cand_s,
                                                       d.cand_i, idx, scores_out, s.L, k);
  decode_resolve_kernel<<<s.batch, kResolveThreads, 0, st>>>(d.rows, d.sel, d.cand_s, d.cand_i, idx,
                                                             scores_out, s.L, k);
}

}  // namespace

size_t decode_ws_bytes(const Shape& s) { return decode_layout(s, nullptr).total; }

hipError_t launch_decode_score_topk(const Shape& s, int32_t nh, const int32_t* heads, int32_t k,
                                    const void* q, const float* q_scale, const float* w,
                                    const void* kk, const float* k_scale, int32_t* idx,
                                    float* scores_out, void* ws, hipStream_t st) {
  const DecodeWs d = decode_layout(s, ws);
  const int64_t nz = static_cast<int64_t>(s.batch) * kDigits + s.batch;
  clear_kernel<<<static_cast<unsigned>((nz + 1023) / 1024), 256, 0, st>>>(d.ghist, nz);
  DecodeArgs a{q, q_scale, w, kk, k_scale, heads, nh, nullptr, 0, 0, nullptr, nullptr, 0,
               d.rows, d.ghist, s.L, s.H, MISA_DECODE_KEYS_PER_WAVE};
  if (s.dtype == kBF16) launch_score<kBF16, false>(s, a, st);
  else launch_score<kFP8, false>(s, a, st);
  launch_select(s, d, k, idx, scores_out, st);
  return hipGetLastError();
}

hipError_t launch_decode_step(const Shape& s, int32_t h, int32_t k, const void* q,
                              const float* q_scale, const float* w, float* pooled, const void* kk,
                              const float* k_scale, int32_t* heads, float* E_out, int32_t* idx,
                              float* scores_out, void* ws, hipStream_t st) {
  const DecodeWs d = decode_layout(s, ws);
  const int64_t M = s.M();
  const int32_t nch = static_cast<int32_t>((M + kChunk - 1) / kChunk);
  const int64_t nz = static_cast<int64_t>(s.batch) * kDigits + s.batch;
  dim3 g1(nch, s.batch);
  if (s.dtype == kBF16)
    step_route_kernel<kBF16><<<g1, 256, 0, st>>>(q, pooled, kk, k_scale, d.part, d.ghist, nz, s.L,
                                                 s.H, s.B, M, nch);
  else
    step_route_kernel<kFP8><<<g1, 256, 0, st>>>(q, pooled, kk, k_scale, d.part, d.ghist, nz, s.L,
                                                s.H, s.B, M, nch);
  DecodeArgs a{q, q_scale, w, kk, k_scale, nullptr, h, d.part, nch, h, heads, E_out, M,
               d.rows, d.ghist, s.L, s.H, MISA_DECODE_KEYS_PER_WAVE};
  if (s.dtype == kBF16) launch_score<kBF16, true>(s, a, st);
  else launch_score<kFP8, true>(s, a, st);
  launch_select(s, d, k, idx, scores_out, st);
  return hipGetLastError();
}

}  // namespace misa
