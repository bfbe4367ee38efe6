// Decode (one query per sequence): token scoring, Eq. (9) / Eq. (1) of the
// MISA summary page, and the top-k of Eq. (10) / (2); plus the fused decode
// step (router of Eq. (7)-(8) + scoring + top-k).
//
// Decode is HBM-bound: every key of the sequence is read once (d*e bytes per
// key) whether h or H heads score it.  The scorers stream keys with 16-byte
// loads straight into MFMA B operands (RowScorer: the query's scored head
// rows are the A operand, 16 keys per 16x16 output tile, ReLU * w head sum on
// the accumulators) and write the scores (L fp32 per sequence) to the
// workspace.  While scoring, each workgroup counts its scores by a histogram
// digit (a monotone map of the score to 8192 bins), so after scoring the
// digit b* holding the k-th best score of every sequence is known without
// another pass.  The select kernel (many workgroups per sequence) finds b*
// from the histograms, writes its tokens of digits above b* straight to the
// output and appends those of digit b* to a short list; the last workgroup
// of the sequence to arrive takes the (k - above) best of that list.
//
// The fused step has two forms:
//  - batch >= 8: one kernel (decode_step_kernel) with G workgroups per
//    sequence; each computes one chunk of the router sums, the chunks are
//    exchanged through the workspace (or recomputed locally, bit-identically,
//    when a peer is late), then every workgroup picks the heads and scores
//    its key range;
//  - smaller batches: a router-partials kernel (step_route_kernel, which
//    also re-pools the newest block) and the score kernel, which finishes
//    the router (E and top-h) in its prologue.
// Both are followed by the select kernel.
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
#ifndef MISA_DECODE_PREFETCH
#define MISA_DECODE_PREFETCH 1
#endif
constexpr int kDecThreads = MISA_DECODE_THREADS;
constexpr int kDecPrefetch = MISA_DECODE_PREFETCH;  // 64-key groups in flight per wave
constexpr int kDecWaves = kDecThreads / kWave;
constexpr int kCandCap = 2048;  // LDS list of the threshold digit
constexpr uint64_t kSyncMagic = 0x4D4953415354ull;  // 48-bit tag of a re-armed router arrival word

// Wait until this wave's vector-memory operations have completed.
__device__ __forceinline__ void vmcnt_zero_wait() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

constexpr int kChunk = 32;      // pooled blocks per router workgroup
constexpr int kMaxH = 64;

// Per-row histogram record: kDigits fine bins, then kCoarse coarse bins
// (coarse bin c = fine bins [32c, 32c + 32)).
constexpr int kCoarse = 256;
constexpr int kFinePerCoarse = kDigits / kCoarse;
constexpr int kHistWords = kDigits + kCoarse;

// Coarse bin count owned by thread t (< kCoarse): coarse bin kCoarse-1-t, so
// threads run from the highest scores down; summed over the row's G
// histogram records (kHistWords apart).  Issued before the caller's other
// loads so that it is not queued behind them.
// Sum of word p[g * kHistWords] over g < G, eight loads in flight at a time.
__device__ __forceinline__ int sum_records(const uint32_t* p, int G) {
  int c = 0, g = 0;
  for (; g + 8 <= G; g += 8) {
    uint32_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[static_cast<int64_t>(g + u) * kHistWords];
#pragma unroll
    for (int u = 0; u < 8; ++u) c += static_cast<int>(v[u]);
  }
  for (; g < G; ++g) c += static_cast<int>(p[static_cast<int64_t>(g) * kHistWords]);
  return c;
}

__device__ __forceinline__ int load_coarse(const uint32_t* gh, int G = 1) {
  return threadIdx.x < kCoarse ? sum_records(gh + kDigits + kCoarse - 1 - threadIdx.x, G) : 0;
}

// The digit b* of the k-th largest score of a row (n > k scores) from its G
// histogram records at gh: *digit, *above = count in higher digits, *count =
// count at b*.  c = load_coarse(gh, G).  All threads call; results are in LDS
// on return.
template <int NT>
__device__ __forceinline__ void find_digit(const uint32_t* gh, int c, int k, int* scan_tmp,
                                           int* sel_coarse, int* digit, int* above, int* count,
                                           int G = 1) {
  static_assert(NT >= kCoarse, "one coarse bin per thread");
  int total;
  const int run = block_exclusive_sum<NT>(c, scan_tmp, total);  // count in higher coarse bins
  if (threadIdx.x < kCoarse && run < k && run + c >= k) {
    sel_coarse[0] = kCoarse - 1 - static_cast<int>(threadIdx.x);
    sel_coarse[1] = run;
  }
  __syncthreads();
  if (threadIdx.x < kWave) {
    const int cb = sel_coarse[0];
    const int base = sel_coarse[1];
    const int lane = threadIdx.x;
    // Lane l < 32 owns fine bin 32cb + 31 - l.
    const int f = lane < kFinePerCoarse ? sum_records(gh + cb * kFinePerCoarse + kFinePerCoarse - 1 - lane, G) : 0;
    const int inc = wave_inclusive_sum(f);
    const int ex = inc - f;
    if (lane < kFinePerCoarse && base + ex < k && base + inc >= k) {
      *digit = cb * kFinePerCoarse + kFinePerCoarse - 1 - lane;
      *above = base + ex;
      *count = f;
    }
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
  // Score rows [batch, L] and histogram records [batch, kHistWords].
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
  const void* krows = (DT == kBF16) ? static_cast<const void*>(static_cast<const uint16_t*>(a.k) + r * a.L * kD)
                                    : static_cast<const void*>(static_cast<const uint8_t*>(a.k) + r * a.L * kD);
  const int64_t s_begin = (static_cast<int64_t>(blockIdx.x) * kDecWaves + wave) * a.keys_per_wave;
  const int64_t s_end = min<int64_t>(s_begin + a.keys_per_wave, a.L);
  // The first 64 keys are loaded before the prologue (histogram clear,
  // router finish, query rows) so that their latency overlaps it.
  typename RowScorer<DT, NRT>::Keys kb;
  if (s_begin < s_end) RowScorer<DT, NRT>::load64(krows, s_begin, s_end, s_begin, kb);
  RowScorer<DT, NRT> sc;
  if constexpr (FUSED) {
    // Finish the router for this sequence (E_j and the top-h heads, Eq. (7)-
    // (8)) while the keys load.  Every load of the prologue is issued at
    // once: the query's head rows and weights are staged in LDS (in the
    // histogram area, cleared afterwards), so the scorer's operands do not
    // wait for the head choice to be fetched from HBM.
    constexpr int EB = (DT == kBF16) ? 2 : 1;
    constexpr int QPIECES = kMaxH * kD * EB / 16;  // 16-byte pieces of all head rows
    static_assert(QPIECES * 16 + kMaxH * 4 <= kDigits * 4, "staging fits the histogram area");
    uint8_t* q_lds = reinterpret_cast<uint8_t*>(hist);
    float* w_lds = reinterpret_cast<float*>(q_lds + QPIECES * 16);
    const uint4* qsrc = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.q) + r * a.H * kD * EB);
    const int qpieces = a.H * kD * EB / 16;
    uint4 qv[(QPIECES + kDecThreads - 1) / kDecThreads];
#pragma unroll
    for (int u = 0; u < (QPIECES + kDecThreads - 1) / kDecThreads; ++u) {
      const int pc = u * kDecThreads + threadIdx.x;
      qv[u] = pc < qpieces ? qsrc[pc] : make_uint4(0, 0, 0, 0);
    }
    const int hd = threadIdx.x & (kMaxH - 1);
    const int grp = threadIdx.x / kMaxH;
    constexpr int NG = kDecThreads / kMaxH;
    const float wv = (threadIdx.x < kMaxH && hd < a.H) ? a.w[r * a.H + hd] : 0.f;
    const float sq = (DT == kFP8) ? a.q_scale[r] : 1.f;
    // Chunk partials: group g sums chunks g, g + NG, ... (all loads at once).
    constexpr int kMaxPer = 16;
    float pv[kMaxPer];
#pragma unroll
    for (int u = 0; u < kMaxPer; ++u) {
      const int c = grp + NG * u;
      pv[u] = c < a.nchunks ? a.route_part[(r * a.nchunks + c) * kMaxH + hd] : 0.f;
    }
    float psum = 0.f;
#pragma unroll
    for (int u = 0; u < kMaxPer; ++u) psum += pv[u];
    for (int c = grp + NG * kMaxPer; c < a.nchunks; c += NG) psum += a.route_part[(r * a.nchunks + c) * kMaxH + hd];
    __shared__ float red[NG][kMaxH];
    red[grp][hd] = psum;
#pragma unroll
    for (int u = 0; u < (QPIECES + kDecThreads - 1) / kDecThreads; ++u) {
      const int pc = u * kDecThreads + threadIdx.x;
      if (pc < QPIECES) reinterpret_cast<uint4*>(q_lds)[pc] = qv[u];
    }
    if (threadIdx.x < kMaxH) w_lds[threadIdx.x] = wv;
    __syncthreads();
    if (wave == 0) {
      float sum = 0.f;
#pragma unroll
      for (int g = 0; g < NG; ++g) sum += red[g][lane];
      float e = -2.f;
      if (lane < a.H) {
        e = fabsf(wv) * sq * sum / static_cast<float>(a.Mt);
        if (blockIdx.x == 0 && a.E_out) a.E_out[r * a.H + lane] = e;
      }
      wave_top_heads(e, a.H, a.h, sh_heads);
    }
    __syncthreads();
    if (blockIdx.x == 0 && threadIdx.x < a.h) a.heads_out[r * a.h + threadIdx.x] = sh_heads[threadIdx.x];
    sc.init_rows(q_lds, w_lds, sq, sh_heads, a.nh, a.H);
    __syncthreads();  // the staging area becomes the histogram
  } else {
    sc.init(a.q, a.q_scale, a.w, a.heads, a.nh, r, a.H);
  }
  for (int b = threadIdx.x; b < kDigits; b += kDecThreads) hist[b] = 0;
  __syncthreads();
  float* row = a.rows + r * a.L;
  auto emit = [&](float res, int64_t s0) {
    const int64_t s = s0 + lane;
    if (s < s_end) {
      float v = res;
      if constexpr (DT == kFP8) v *= a.k_scale[r * a.L + s];
      row[s] = v;
      atomicAdd(&hist[key_digit(v)], 1u);
    }
  };
  if constexpr (kDecPrefetch == 1) {
    for (int64_t s0 = s_begin; s0 < s_end; s0 += 64) {
      if (s0 != s_begin) RowScorer<DT, NRT>::load64(krows, s0, s_end, s_begin, kb);
      emit(sc.compute64(kb), s0);
    }
  } else {
    // Two 64-key groups per wave: one is scored while the other loads.
    typename RowScorer<DT, NRT>::Keys kb1;
    if (s_begin + 64 < s_end) RowScorer<DT, NRT>::load64(krows, s_begin + 64, s_end, s_begin, kb1);
    for (int64_t s0 = s_begin; s0 < s_end; s0 += 128) {
      const float r0 = sc.compute64(kb);
      if (s0 + 128 < s_end) RowScorer<DT, NRT>::load64(krows, s0 + 128, s_end, s_begin, kb);
      emit(r0, s0);
      if (s0 + 64 < s_end) {
        const float r1 = sc.compute64(kb1);
        if (s0 + 192 < s_end) RowScorer<DT, NRT>::load64(krows, s0 + 192, s_end, s_begin, kb1);
        emit(r1, s0 + 64);
      }
    }
  }
  __syncthreads();
  uint32_t* gh = a.ghist + r * kHistWords;
  for (int b = threadIdx.x; b < kDigits; b += kDecThreads) {
    const uint32_t c = hist[b];
    if (c) atomicAdd(&gh[b], c);
  }
  for (int cb = threadIdx.x; cb < kCoarse; cb += kDecThreads) {
    uint32_t c = 0;
#pragma unroll
    for (int u = 0; u < kFinePerCoarse; ++u) c += hist[cb * kFinePerCoarse + (u + cb) % kFinePerCoarse];
    if (c) atomicAdd(&gh[kDigits + cb], c);
  }
}

// Top-k after scoring, one kernel: workgroup (chunk, sequence) takes
// kCompactChunk consecutive scores, finds b* from the histogram records,
// writes its tokens of digits above b* straight to the output and appends
// those of digit b* to a short list (one packed atomic counter per sequence
// reserves both ranges).  The last workgroup of the sequence to finish (an
// arrival counter, zeroed by the kernel before) then takes the (k - above)
// best of the list, exactly.  The list is written and read with
// device-coherent accesses, and each workgroup's writes are complete before
// it is counted.  When b* holds more than kCandCap tokens, workgroup 0 alone
// selects from the whole row.
constexpr int kCompactThreads = 256;
constexpr int kCompactPer = 16;  // scores per thread
constexpr int kCompactChunk = kCompactThreads * kCompactPer;
static_assert(kCompactThreads <= kCandCap, "speculative list loads stay inside the list");

struct SelectSmem {
  alignas(16) float cand_score[kCandCap];
  alignas(16) int32_t cand_idx[kCandCap];
  ResolveSmem rs;
  TopkSmem base;
  int scan_tmp[32];
  int s_coarse[2];
  int s_digit, s_above, s_count, s_last;
  uint32_t s_base;
};

__global__ __launch_bounds__(kCompactThreads) void decode_select_kernel(
    const float* __restrict__ rows, const uint32_t* __restrict__ ghist, uint32_t* __restrict__ cnt,
    uint32_t* __restrict__ done, float* __restrict__ cand_s, int32_t* __restrict__ cand_i,
    int32_t* __restrict__ idx, float* __restrict__ scores_out, int32_t L, int32_t k, int32_t G,
    uint64_t* __restrict__ rsync, int32_t T) {
  __shared__ SelectSmem sm;
  const int64_t r = blockIdx.y;
  // Re-arm the next step's router exchange (this kernel follows the step
  // kernel, so every arrival of this call has been counted).
  if (rsync && blockIdx.x == 0 && threadIdx.x == 0) rsync[r] = kSyncMagic << 16;
  const float* row = rows + r * L;
  // Row r = (sequence, query t < T): the query's prefix is keys [0, n).
  const int32_t n = L - T + 1 + static_cast<int32_t>(r % T);
  int32_t* out = idx + r * k;
  float* out_s = scores_out ? scores_out + r * k : nullptr;
  if (n <= k) {
    if (blockIdx.x == 0)
      for (int i = threadIdx.x; i < k; i += kCompactThreads) {
        out[i] = i < n ? i : -1;
        if (out_s) out_s[i] = i < n ? row[i] : -__builtin_inff();
      }
    return;
  }
  const int c0 = blockIdx.x * kCompactChunk;
  const uint32_t* gh = ghist + r * G * kHistWords;
  const int coarse = load_coarse(gh, G);
  // Scores first (independent of b*), so their loads overlap the scan.
  float v[kCompactPer];  // clamped loads; tokens past n are masked below
#pragma unroll
  for (int j = 0; j < kCompactPer; ++j)
    v[j] = row[min(c0 + j * kCompactThreads + static_cast<int>(threadIdx.x), n - 1)];
  find_digit<kCompactThreads>(gh, coarse, k, sm.scan_tmp, sm.s_coarse, &sm.s_digit, &sm.s_above,
                              &sm.s_count, G);
  const uint32_t bstar = static_cast<uint32_t>(sm.s_digit);
  const int count = sm.s_count;
  const int above = sm.s_above;
  if (count > kCandCap) {
    if (blockIdx.x == 0)
      block_topk<kCompactThreads>(
          n, k, [](int64_t) { return true; }, [=](int64_t i) { return float_key(row[i]); },
          [](int64_t i) { return static_cast<int32_t>(i); }, [=](int64_t i) { return row[i]; }, out,
          out_s, sm.base);
    return;
  }
  const uint32_t lo = digit_lo_key(bstar), hi = digit_hi_key(bstar);
  uint32_t mh = 0, ma = 0;
#pragma unroll
  for (int j = 0; j < kCompactPer; ++j) {
    const int i = c0 + j * kCompactThreads + threadIdx.x;
    const uint32_t key = float_key(v[j]);
    mh |= (i < n && key > hi) ? (1u << j) : 0u;
    ma |= (i < n && key >= lo && key <= hi) ? (1u << j) : 0u;
  }
  // Packed counts: above-b* in the low 16 bits (their row total is below
  // k <= 8192), at-b* in the high 16 bits (row total <= kCandCap).
  const int packed = __popc(mh) | (__popc(ma) << 16);
  int total;
  const int off = block_exclusive_sum<kCompactThreads>(packed, sm.scan_tmp, total);
  if (threadIdx.x == 0) sm.s_base = atomicAdd(&cnt[r], static_cast<uint32_t>(total));
  __syncthreads();
  const uint32_t base = sm.s_base + static_cast<uint32_t>(off);
  int ph = static_cast<int>(base & 0xFFFFu);
  int pa = static_cast<int>(base >> 16);
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
        __hip_atomic_store(reinterpret_cast<uint32_t*>(ls + pa), __float_as_uint(v[j]), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(li + pa, i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      ++pa;
    }
  }
  // Arrival: this workgroup's list entries are complete before it counts.
  vmcnt_zero_wait();
  __syncthreads();
  if (threadIdx.x == 0) sm.s_last = atomicAdd(&done[r], 1u) == gridDim.x - 1 ? 1 : 0;
  __syncthreads();
  if (!sm.s_last) return;
  // The last workgroup: the (k - above) best of the list (all of its loads
  // in flight at once).
  {
    constexpr int PER = kCandCap / kCompactThreads;
    uint32_t vs[PER];
    int32_t vi[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int t = static_cast<int>(threadIdx.x) + u * kCompactThreads;
      vs[u] = t < count ? __hip_atomic_load(reinterpret_cast<const uint32_t*>(ls + t), __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT)
                        : 0u;
      vi[u] = t < count ? __hip_atomic_load(li + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int t = static_cast<int>(threadIdx.x) + u * kCompactThreads;
      if (t < count) {
        sm.cand_score[t] = __uint_as_float(vs[u]);
        sm.cand_idx[t] = vi[u];
      }
    }
  }
  __syncthreads();
  if (resolve_list<kCompactThreads>(sm.cand_score, sm.cand_idx, count, k - above, out + above,
                                    out_s ? out_s + above : nullptr, sm.rs))
    return;
  __syncthreads();
  const float* cs = sm.cand_score;
  const int32_t* ci = sm.cand_idx;
  block_topk<kCompactThreads>(
      count, k - above, [](int64_t) { return true; }, [=](int64_t j) { return float_key(cs[j]); },
      [=](int64_t j) { return ci[j]; }, [=](int64_t j) { return cs[j]; }, out + above,
      out_s ? out_s + above : nullptr, sm.base);
}

__global__ void clear_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = 0;
}

// Fused step, kernel 1: router partial sums.  Workgroup (c, sequence) with
// c < nmain sums ReLU(q_j . p_b) over pooled blocks [32c, 32c+32) of the
// cached blocks 0 .. M-2; workgroup (nmain, sequence) recomputes the mean of
// the newest block M-1 (keys (M-1)B .. L-1) from the keys, writes it to the
// cache and forms its ReLU(q_j . p) term.  Partial j of slot c goes to
// part[(seq*(nmain+1) + c)*64 + j].  Every workgroup also zeroes a share of
// the digit histograms and compaction counters of the top-k kernels.
template <int DT>
__global__ __launch_bounds__(256) void step_route_kernel(
    const void* __restrict__ q, float* __restrict__ pooled, const void* __restrict__ k,
    const float* __restrict__ k_scale, float* __restrict__ part, uint32_t* __restrict__ zero,
    int64_t nzero, int32_t L, int32_t H, int32_t B, int64_t M, int32_t nmain) {
  __shared__ __attribute__((aligned(16))) float ps[kD];
  __shared__ float lastp[32][kD];
  {
    const int64_t g = static_cast<int64_t>(blockIdx.y) * gridDim.x + blockIdx.x;
    const int64_t G = static_cast<int64_t>(gridDim.x) * gridDim.y;
    for (int64_t i = g * 256 + threadIdx.x; i < nzero; i += G * 256) zero[i] = 0;
  }
  const int c = blockIdx.x;
  const int64_t seq = blockIdx.y;
  float* out = part + (seq * (nmain + 1) + c) * kMaxH;
  if (c == nmain) {
    // Mean of keys [(M-1)B, L): thread t takes 16-byte piece t % P of key
    // rows t / P + KPR * u; a round's loads are all in flight together and
    // the per-dimension partial sums of the KPR key slots meet in LDS.
    constexpr int EB = (DT == kBF16) ? 2 : 1;  // bytes per element
    constexpr int P = kD * EB / 16;            // pieces per key row
    constexpr int EPP = 16 / EB;               // elements per piece
    constexpr int KPR = 256 / P;               // key slots
    constexpr int U = 4;
    const int piece = threadIdx.x % P;
    const int slot = threadIdx.x / P;
    const int64_t s0 = (M - 1) * B;
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
    // This thread's query head row (loads overlap the reduction below).
    const int j = threadIdx.x & (kMaxH - 1);
    float qr[kD];
    load_head_row<DT>(q, (seq * H + (j < H ? j : 0)) * kD, qr);
#pragma unroll
    for (int e = 0; e < EPP; ++e) lastp[slot][piece * EPP + e] = acc[e];
    __syncthreads();
    if (threadIdx.x < kD) {
      float sum = 0.f;
#pragma unroll
      for (int sl = 0; sl < KPR; ++sl) sum += lastp[sl][threadIdx.x];
      const float m = sum / static_cast<float>(nl);
      ps[threadIdx.x] = m;
      pooled[(seq * M + M - 1) * kD + threadIdx.x] = m;
    }
    __syncthreads();
    if (threadIdx.x < kMaxH) out[threadIdx.x] = relu(dot_lds_row(qr, ps));
    return;
  }
  // Cached blocks [b0, b0 + nb) on 16x16x32 bf16 MFMA: wave w takes heads
  // [16w, 16w + 16) as A (q codes are exact in bf16: bf16 inputs, or e4m3
  // widened), 16 blocks per column tile as B, each pooled key split into a
  // bf16 hi part and the bf16 rounding of its remainder (two MFMAs), so the
  // products carry ~16 mantissa bits of the fp32 pooled keys.  The head-dim
  // pieces follow the key scorer's permutation (piece 4*ks + lane/16).
  const int64_t b0 = static_cast<int64_t>(c) * kChunk;
  const int nb = static_cast<int>(min<int64_t>(kChunk, (M - 1) - b0));
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int col = lane & 15;
  const int qq = lane >> 4;
  const int jh = 16 * wave + col;  // head of this lane's A row
  bf16x8 qa[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (jh < H) {
      if constexpr (DT == kBF16) {
        v = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(q) + (seq * H + jh) * kD)[4 * ks + qq];
      } else {
        const uint2 c8 = reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(q) + (seq * H + jh) * kD)[4 * ks + qq];
        uint32_t b16[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          b16[e] = __float_as_uint(fp8_to_f32(((e < 4 ? c8.x : c8.y) >> (8 * (e & 3))) & 0xFF)) >> 16;
        v = make_uint4(b16[0] | (b16[1] << 16), b16[2] | (b16[3] << 16), b16[4] | (b16[5] << 16),
                       b16[6] | (b16[7] << 16));
      }
    }
    qa[ks] = as_bf16x8(v);
  }
  f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int bl = 16 * ct + col;
    const bool ok = bl < nb;
    const float4* src = reinterpret_cast<const float4*>(pooled + (seq * M + b0 + (ok ? bl : 0)) * kD);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      // dims 8*(4ks+qq) .. +8: float4s 2*(4ks+qq) and 2*(4ks+qq)+1
      float4 x0 = make_float4(0.f, 0.f, 0.f, 0.f), x1 = x0;
      if (ok) {
        x0 = src[2 * (4 * ks + qq)];
        x1 = src[2 * (4 * ks + qq) + 1];
      }
      uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
      split_bf16(x0, h0, h1, l0, l1);
      split_bf16(x1, h2, h3, l2, l3);
      acc[ct] = mfma16_bf16(qa[ks], as_bf16x8(make_uint4(h0, h1, h2, h3)), acc[ct]);
      acc[ct] = mfma16_bf16(qa[ks], as_bf16x8(make_uint4(l0, l1, l2, l3)), acc[ct]);
    }
  }
  // C layout: lane holds heads 16w + 4qq + i (i < 4) for blocks col and 16 + col.
  float rs[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) rs[i] = relu(acc[0][i]) + relu(acc[1][i]);
#pragma unroll
  for (int o = 1; o < 16; o <<= 1)
#pragma unroll
    for (int i = 0; i < 4; ++i) rs[i] += __shfl_xor(rs[i], o, kWave);
  if (col == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[16 * wave + 4 * qq + i] = rs[i];
  }
}

// Single-kernel decode step (router + scoring) for batches that fill the
// chip: G = ceil(256 / batch) workgroups per sequence, all on one XCD (the
// workgroup id's residue mod 8 is the sequence's), so that the sequence's
// pooled keys are read from HBM once and then from that XCD's L2.  Every
// workgroup
//  1. stages the query's head rows (padded LDS rows) and weights;
//  2. recomputes the mean of the newest block M-1 from its keys (Eq. (4));
//     workgroup 0 writes it back to the pooled cache;
//  3. forms S_j = sum over the M blocks of ReLU(q_j . p_m) on 16x16x32 bf16
//     MFMA (16-block column tiles dealt round-robin to the waves; pooled keys
//     split into bf16 hi + lo, fp8 query codes widened exactly), then E_j and the top-h heads
//     (Eq. (7)-(8)); workgroup 0 writes them;
//  4. scores its key range with the routed heads (two 64-key groups in
//     flight per wave), writes the scores and its own digit histogram (no
//     atomics, so nothing needs clearing first) and, in workgroup 0, clears
//     the sequence's compaction counter for the select kernels.
constexpr int kStepThreads = 512;
constexpr int kSyncSpin = 1 << 16;  // bounded wait for the peers' router partials
constexpr int kStepMaxG = 32;       // workgroups per sequence (batch >= 8)


constexpr int kStepWaves = kStepThreads / kWave;

struct StepArgs {
  const void* q;
  const float* q_scale;
  const float* w;
  float* pooled;
  const void* k;
  const float* k_scale;
  int32_t* heads_out;
  float* E_out;
  float* rows;
  uint32_t* ghist;  // [batch, G, kHistWords]
  uint32_t* cnt;    // [batch]
  uint32_t* done;   // [batch]
  uint32_t* rpart;  // [batch, G, 64] published router partials (fp32 bits)
  uint64_t* rsync;  // [batch] (magic << 16) | arrivals; reset by the compact kernel
  int64_t M;
  int32_t L, H, B, h, G, batch, keys_per_wave;
};

template <int DT>
__global__ __launch_bounds__(kStepThreads) void decode_step_kernel(StepArgs a) {
  constexpr int EB = (DT == kBF16) ? 2 : 1;
  constexpr int QP = kD * 2 + 16;  // router staging pitch (bf16 rows + pad), bytes
  constexpr int SP = kD * EB + 16;  // scorer staging pitch, bytes
  __shared__ __attribute__((aligned(16))) uint32_t hist[kDigits];  // also the newest-block partial sums
  __shared__ __attribute__((aligned(16))) uint8_t qr_lds[kMaxH * QP];  // bf16 head rows (router)
  __shared__ __attribute__((aligned(16))) uint8_t qs_lds[DT == kBF16 ? 16 : kMaxH * SP];  // fp8 codes (scorer)
  __shared__ __attribute__((aligned(16))) float meanv[kD];
  __shared__ float w_lds[kMaxH];
  __shared__ float red[kStepWaves][kMaxH];
  __shared__ int32_t sh_heads[16];
  __shared__ int sh_flag;
  __shared__ float xpart[kStepMaxG * kMaxH];  // the sequence's published router partials
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t seq = blockIdx.x % a.batch;
  const int g = blockIdx.x / a.batch;
  const int64_t M = a.M;
  const int H = a.H;

  // The first pooled tile of this workgroup's router chunk (section 3) is
  // requested before the staging and newest-block loads below, so the three
  // round trips overlap.
  const int col = lane & 15;
  const int qq = lane >> 4;
  struct PTile {
    float4 x[8];
  };
  auto load_tile = [&](int64_t c0, PTile& t) {
    const int64_t b = c0 + col;
    const bool cached = b < M - 1;
    const float4* src = reinterpret_cast<const float4*>(a.pooled + (seq * M + (cached ? b : 0)) * kD);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      t.x[2 * ks] = src[(32 * ks + 8 * qq) / 4];
      t.x[2 * ks + 1] = src[(32 * ks + 8 * qq) / 4 + 1];
    }
  };
  const int G = a.G;
  const int64_t own_cb = static_cast<int64_t>(g) * M / G, own_ce = static_cast<int64_t>(g + 1) * M / G;
  PTile t_first;
  if (own_cb + 16 * wave < own_ce) load_tile(own_cb + 16 * wave, t_first);

  // 1-2. Loads of the head rows, weights and the newest block's first keys
  // are all issued before any of them is used: one round trip (overlapping
  // the pooled tile above) instead of one per loop iteration.
  constexpr int PPR = kD * EB / 16;  // 16-byte pieces per head row / key row
  constexpr int NPC = kMaxH * PPR / kStepThreads;  // staging pieces per thread
  static_assert(NPC * kStepThreads == kMaxH * PPR, "staging pieces split evenly");
  const uint4* qsrc = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.q) + seq * H * kD * EB);
  uint4 qv[NPC];
#pragma unroll
  for (int u = 0; u < NPC; ++u) {
    const int pc = threadIdx.x + u * kStepThreads;
    qv[u] = pc / PPR < H ? qsrc[pc] : make_uint4(0, 0, 0, 0);
  }
  const float wv = threadIdx.x < H ? a.w[seq * H + threadIdx.x] : 0.f;
  // Mean of keys [(M-1)B, L): thread t takes 16-byte piece t % PPR of key
  // slots t / PPR + NSL * u, four keys per round; the slots' sums meet in
  // LDS.
  constexpr int NSL = kStepThreads / PPR;
  constexpr int KR = 4;  // keys per slot per round
  static_assert(NSL * kD <= kDigits, "slot sums fit the histogram area");
  const int piece = threadIdx.x % PPR;
  const int slot = threadIdx.x / PPR;
  const int64_t s0 = (M - 1) * a.B;
  const int nl = static_cast<int>(a.L - s0);
  const uint8_t* kbm = static_cast<const uint8_t*>(a.k) + (seq * a.L + s0) * kD * EB;
  uint4 mv[KR];
  float msc[KR];
  auto mean_load = [&](int k0) {
#pragma unroll
    for (int u = 0; u < KR; ++u) {
      const int key = k0 + u * NSL;
      const bool ok = key < nl;
      mv[u] = ok ? reinterpret_cast<const uint4*>(kbm + static_cast<int64_t>(key) * kD * EB)[piece]
                 : make_uint4(0, 0, 0, 0);
      msc[u] = (DT == kFP8 && ok) ? a.k_scale[seq * a.L + s0 + key] : 0.f;
    }
  };
  mean_load(slot);

  // 1. Head rows -> LDS (router copy widened to bf16; fp8 codes kept for the
  // scorer), weights.
#pragma unroll
  for (int u = 0; u < NPC; ++u) {
    const int pc = threadIdx.x + u * kStepThreads;
    const int row = pc / PPR, c = pc % PPR;
    const uint4 v = qv[u];
    if constexpr (DT == kBF16) {
      *reinterpret_cast<uint4*>(qr_lds + row * QP + 16 * c) = v;
    } else {
      *reinterpret_cast<uint4*>(qs_lds + row * SP + 16 * c) = v;
      const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
      uint32_t o[8];
#pragma unroll
      for (int u2 = 0; u2 < 4; ++u2) {
        // e4m3 -> fp32 is exact and bf16 holds the 4-bit significand exactly.
        const float f0 = fp8_to_f32(wd[u2] & 0xFF), f1 = fp8_to_f32((wd[u2] >> 8) & 0xFF);
        const float f2 = fp8_to_f32((wd[u2] >> 16) & 0xFF), f3 = fp8_to_f32(wd[u2] >> 24);
        o[2 * u2] = (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xFFFF0000u);
        o[2 * u2 + 1] = (__float_as_uint(f2) >> 16) | (__float_as_uint(f3) & 0xFFFF0000u);
      }
      uint4* dst = reinterpret_cast<uint4*>(qr_lds + row * QP + 32 * c);
      dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
      dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
  }
  if (threadIdx.x < kMaxH) w_lds[threadIdx.x] = wv;

  // 2. The mean itself.
  {
    constexpr int EPP = 16 / EB;
    float* part = reinterpret_cast<float*>(hist);  // [NSL][kD]
    float acc[EPP];
#pragma unroll
    for (int e = 0; e < EPP; ++e) acc[e] = 0.f;
    for (int k0 = slot; k0 < nl; k0 += KR * NSL) {
#pragma unroll
      for (int u = 0; u < KR; ++u) {
        const uint32_t wd[4] = {mv[u].x, mv[u].y, mv[u].z, mv[u].w};
        if constexpr (DT == kBF16) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[2 * e] += __uint_as_float(wd[e] << 16);
            acc[2 * e + 1] += __uint_as_float(wd[e] & 0xFFFF0000u);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[e] += fp8_to_f32((wd[e / 4] >> (8 * (e % 4))) & 0xFF) * msc[u];
        }
      }
      if (k0 + KR * NSL < nl) mean_load(k0 + KR * NSL);
    }
#pragma unroll
    for (int e = 0; e < EPP; ++e) part[slot * kD + piece * EPP + e] = acc[e];
    __syncthreads();
    if (threadIdx.x < kD) {
      float sum = 0.f;
      for (int sl = 0; sl < NSL; ++sl) sum += part[sl * kD + threadIdx.x];
      const float m = sum / static_cast<float>(nl);
      meanv[threadIdx.x] = m;
      if (g == 0) a.pooled[(seq * M + M - 1) * kD + threadIdx.x] = m;
    }
    __syncthreads();
  }

  // 3. Router.  The M blocks are cut into G chunks; workgroup g computes
  // chunk g's partial P_g[j] = sum over its blocks of ReLU(q_j . p_m) and
  // publishes it, then S_j = P_0[j] + ... + P_{G-1}[j] in that order from
  // the published partials.  When the exchange cannot be trusted (first call
  // on a workspace, or a peer missing for too long) the workgroup computes
  // every chunk itself with the same code and summation order, so S is the
  // same bits either way.
  //
  // A chunk's 16-block column tiles are dealt to the waves (tile i to wave
  // i % 8); lane l supplies block c0 + l%16, head-dim elements
  // 32 ks + 8 (l/16) .. + 8 (A and B alike).
  float rs[4][4];
  auto mul_tile = [&](int64_t c0, int64_t ce, const PTile& t) {
    const int64_t b = c0 + col;
    f32x4 acc[4];
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) acc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int e0 = 32 * ks + 8 * qq;
      float4 x0 = t.x[2 * ks], x1 = t.x[2 * ks + 1];
      if (b == M - 1) {  // the newest block: its mean, just recomputed
        x0 = *reinterpret_cast<const float4*>(meanv + e0);
        x1 = *reinterpret_cast<const float4*>(meanv + e0 + 4);
      }
      uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
      split_bf16(x0, h0, h1, l0, l1);
      split_bf16(x1, h2, h3, l2, l3);
      const bf16x8 bh = as_bf16x8(make_uint4(h0, h1, h2, h3));
      const bf16x8 bl = as_bf16x8(make_uint4(l0, l1, l2, l3));
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) {
        const bf16x8 qa = as_bf16x8(*reinterpret_cast<const uint4*>(qr_lds + (16 * ht + col) * QP + 2 * e0));
        acc[ht] = mfma16_bf16(qa, bh, acc[ht]);
        acc[ht] = mfma16_bf16(qa, bl, acc[ht]);
      }
    }
    // C layout: lane holds heads 16 ht + 4 qq + i for block column col.
    const bool ok = b < ce;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
      for (int i = 0; i < 4; ++i) rs[ht][i] += ok ? relu(acc[ht][i]) : 0.f;
  };
  constexpr int64_t kTileStep = 16 * kStepWaves;
  // Chunk [cb, ce): every wave writes its per-head sums to red[wave][.];
  // callers synchronise, then add red[0..7][j] in wave order.  One tile is
  // multiplied while the next loads; the loop is not unrolled further
  // because this code runs once, from a cold instruction cache.
  auto chunk_sums = [&](int64_t cb, int64_t ce, const PTile* first) {
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
      for (int i = 0; i < 4; ++i) rs[ht][i] = 0.f;
    const int64_t c_first = cb + 16 * wave;
    // Two tiles in fixed roles (ping-pong; a copy tc = tn would wait for the
    // loads in flight).
    PTile ta, tb;
    if (c_first < ce) {
      if (first) ta = *first;
      else load_tile(c_first, ta);
    }
    if (c_first + kTileStep < ce) load_tile(c_first + kTileStep, tb);
#pragma unroll 1
    for (int64_t c0 = c_first; c0 < ce; c0 += 2 * kTileStep) {
      mul_tile(c0, ce, ta);
      if (c0 + 2 * kTileStep < ce) load_tile(c0 + 2 * kTileStep, ta);
      if (c0 + kTileStep < ce) {
        mul_tile(c0 + kTileStep, ce, tb);
        if (c0 + 3 * kTileStep < ce) load_tile(c0 + 3 * kTileStep, tb);
      }
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1)
#pragma unroll
      for (int ht = 0; ht < 4; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i) rs[ht][i] += __shfl_xor(rs[ht][i], o, kWave);
    if (col == 0) {
#pragma unroll
      for (int ht = 0; ht < 4; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][16 * ht + 4 * qq + i] = rs[ht][i];
    }
  };
  auto red_sum = [&]() {  // wave 0, lane j: the chunk partial of head j
    float p = 0.f;
#pragma unroll
    for (int w8 = 0; w8 < kStepWaves; ++w8) p += red[w8][lane];
    return p;
  };
  chunk_sums(own_cb, own_ce, &t_first);
  __syncthreads();
  float S = 0.f;  // wave 0, lane j: S_j
  if (wave == 0) {
    const float mine = red_sum();
    uint32_t* pub = a.rpart + (seq * G + g) * kMaxH;
    __hip_atomic_store(pub + lane, __float_as_uint(mine), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    vmcnt_zero_wait();  // the partial is globally visible before it is counted
    int ok = 0;
    if (lane == 0) {
      const uint64_t old = __hip_atomic_fetch_add(a.rsync + seq, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ok = ((old >> 16) == kSyncMagic && (old & 0xFFFF) < static_cast<uint64_t>(G)) ? 1 : 0;
      for (int it = 0; ok && it < kSyncSpin; ++it) {
        const uint64_t v = __hip_atomic_load(a.rsync + seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((v & 0xFFFF) >= static_cast<uint64_t>(G)) break;
        if (it + 1 == kSyncSpin) ok = 0;
        __builtin_amdgcn_s_sleep(2);
      }
    }
    ok = __shfl(ok, 0, kWave);
    if (lane == 0) sh_flag = ok;
  }
  __syncthreads();
  if (sh_flag) {
    // All G partials of the sequence, fetched by the whole workgroup at once
    // (coherent loads), then added by wave 0 in chunk order.
    constexpr int NXP = kStepMaxG * kMaxH / kStepThreads;
    uint32_t xv[NXP];
#pragma unroll
    for (int u = 0; u < NXP; ++u) {
      const int i = threadIdx.x + u * kStepThreads;
      xv[u] = i < G * kMaxH ? __hip_atomic_load(a.rpart + seq * G * kMaxH + i, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT)
                            : 0u;
    }
#pragma unroll
    for (int u = 0; u < NXP; ++u) {
      const int i = threadIdx.x + u * kStepThreads;
      if (i < G * kMaxH) xpart[i] = __uint_as_float(xv[u]);
    }
    __syncthreads();
    if (wave == 0)
      for (int c = 0; c < G; ++c) S += xpart[c * kMaxH + lane];
  }
  if (!sh_flag) {
    S = 0.f;
    for (int c = 0; c < G; ++c) {
      chunk_sums(static_cast<int64_t>(c) * M / G, static_cast<int64_t>(c + 1) * M / G, nullptr);
      __syncthreads();
      if (wave == 0) S += red_sum();
      __syncthreads();
    }
  }

  // Key range of this wave; its first group loads while the heads are
  // chosen.  (Requested earlier, the key stream would delay the router's own
  // round trips more than it gains.)
  const void* krows = static_cast<const void*>(static_cast<const uint8_t*>(a.k) + seq * a.L * kD * EB);
  const int64_t s_begin = (static_cast<int64_t>(g) * kStepWaves + wave) * a.keys_per_wave;
  const int64_t s_end = min<int64_t>(s_begin + a.keys_per_wave, a.L);
  typename RowScorer<DT, 1>::Keys kb0;
  if (s_begin < s_end) RowScorer<DT, 1>::load64(krows, s_begin, s_end, s_begin, kb0);

  const float sq = (DT == kFP8) ? a.q_scale[seq] : 1.f;
  if (wave == 0) {
    float e = -2.f;
    if (lane < H) {
      e = fabsf(w_lds[lane]) * sq * S / static_cast<float>(M);
      if (g == 0 && a.E_out) a.E_out[seq * H + lane] = e;
    }
    wave_top_heads_rank(e, H, a.h, sh_heads);
  }
  for (int b = threadIdx.x; b < kDigits; b += kStepThreads) hist[b] = 0;
  __syncthreads();
  if (g == 0 && threadIdx.x < a.h) a.heads_out[seq * a.h + threadIdx.x] = sh_heads[threadIdx.x];
  if (g == 0 && threadIdx.x == 0) {
    a.cnt[seq] = 0;
    a.done[seq] = 0;
  }
  RowScorer<DT, 1> sc;
  if constexpr (DT == kBF16) sc.init_rows(qr_lds, w_lds, sq, sh_heads, a.h, H, QP / 2);
  else sc.init_rows(qs_lds, w_lds, sq, sh_heads, a.h, H, SP);

  // 4. Scores, two groups in flight per wave.
  float* row = a.rows + seq * a.L;
  auto emit = [&](float res, int64_t s0) {
    const int64_t s = s0 + lane;
    if (s < s_end) {
      float v = res;
      if constexpr (DT == kFP8) v *= a.k_scale[seq * a.L + s];
      row[s] = v;
      atomicAdd(&hist[key_digit(v)], 1u);
    }
  };
  {
    typename RowScorer<DT, 1>::Keys kb1;
    if (s_begin + 64 < s_end) RowScorer<DT, 1>::load64(krows, s_begin + 64, s_end, s_begin, kb1);
    for (int64_t s0 = s_begin; s0 < s_end; s0 += 128) {
      const float r0 = sc.compute64(kb0);
      if (s0 + 128 < s_end) RowScorer<DT, 1>::load64(krows, s0 + 128, s_end, s_begin, kb0);
      emit(r0, s0);
      if (s0 + 64 < s_end) {
        const float r1 = sc.compute64(kb1);
        if (s0 + 192 < s_end) RowScorer<DT, 1>::load64(krows, s0 + 192, s_end, s_begin, kb1);
        emit(r1, s0 + 64);
      }
    }
  }
  __syncthreads();
  // This workgroup's histogram record (fine bins, then coarse sums).
  uint32_t* gh = a.ghist + (seq * a.G + g) * kHistWords;
  for (int b = threadIdx.x; b < kDigits; b += kStepThreads) gh[b] = hist[b];
  for (int cb = threadIdx.x; cb < kCoarse; cb += kStepThreads) {
    uint32_t c = 0;
#pragma unroll
    for (int u = 0; u < kFinePerCoarse; ++u) c += hist[cb * kFinePerCoarse + (u + cb) % kFinePerCoarse];
    gh[kDigits + cb] = c;
  }
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
  uint32_t* cnt;    // [batch] packed compaction counters, then
  uint32_t* done;   // [batch] select-kernel arrivals, followed by
  uint32_t* ghist;  // [batch, kHistWords] (single-kernel step: [batch, G, kHistWords])
  int64_t zero_words;  // counters + one record per sequence
  float* cand_s;
  int32_t* cand_i;
  float* part;
  uint32_t* rpart;  // single-kernel step: [batch, G, 64] router partials
  uint64_t* rsync;  // single-kernel step: [batch] arrival words
  size_t total;
};

// Router chunks of the cached blocks 0 .. M-2 (the newest block has its own
// workgroup).
int32_t step_main_chunks(const Shape& s) {
  return static_cast<int32_t>((s.M() - 1 + kChunk - 1) / kChunk);
}

// Workgroups per sequence of the single-kernel step, or 0 when the batch is
// too small to fill the chip that way and the step runs as router + score
// kernels.
int32_t step_groups(const Shape& s) {
  if (s.batch < 8) return 0;
  const int32_t G = (256 + s.batch - 1) / s.batch;
  return G <= kStepMaxG ? G : 0;
}

DecodeWs decode_layout(const Shape& s, void* ws) {
  const uintptr_t base = reinterpret_cast<uintptr_t>(ws);
  const size_t nb = static_cast<size_t>(s.batch);
  DecodeWs d{};
  size_t off = 0;
  d.rows = reinterpret_cast<float*>(base + off);
  off += align_up(nb * s.L * sizeof(float));
  // Counters first, then the histogram records: the kernels that need both
  // zeroed clear one range [cnt, cnt + zero_words).
  const size_t nrec = nb * static_cast<size_t>(s.T == 1 && step_groups(s) > 0 ? step_groups(s) : 1);
  const size_t cnt_words = (2 * nb + 63) / 64 * 64;
  d.cnt = reinterpret_cast<uint32_t*>(base + off);
  d.done = d.cnt + nb;
  d.ghist = d.cnt + cnt_words;
  d.zero_words = static_cast<int64_t>(cnt_words + nb * kHistWords);
  off += align_up((cnt_words + nrec * kHistWords) * sizeof(uint32_t));
  d.cand_s = reinterpret_cast<float*>(base + off);
  off += align_up(nb * kCandCap * sizeof(float));
  d.cand_i = reinterpret_cast<int32_t*>(base + off);
  off += align_up(nb * kCandCap * sizeof(int32_t));
  d.part = reinterpret_cast<float*>(base + off);
  off += align_up(nb * (step_main_chunks(s) + 1) * kMaxH * sizeof(float));
  d.rpart = reinterpret_cast<uint32_t*>(base + off);
  off += align_up(nrec * kMaxH * sizeof(uint32_t));
  d.rsync = reinterpret_cast<uint64_t*>(base + off);
  off += align_up(nb * sizeof(uint64_t));
  d.total = off;
  return d;
}

// Rows: s.batch of them, s.L scores apart; T consecutive rows per sequence
// (row r's prefix holds s.L - T + 1 + r % T keys).
void launch_select(const Shape& s, const DecodeWs& d, int32_t k, int32_t* idx, float* scores_out,
                   hipStream_t st, int32_t G = 1, int32_t T = 1) {
  dim3 g((s.L + kCompactChunk - 1) / kCompactChunk, s.batch);
  decode_select_kernel<<<g, kCompactThreads, 0, st>>>(d.rows, d.ghist, d.cnt, d.done, d.cand_s, d.cand_i,
                                                      idx, scores_out, s.L, k, G, d.rsync, T);
}

// ---------------------------------------------------------------------------
// Multi-query decode: T (2 .. kMaxMQ) queries per sequence at the end of its
// context (query t at position L - T + t, for instance draft tokens being
// verified), scored in one pass over the keys.  The A operand of the 16x16
// MFMA tiles holds every query's routed head rows: row rr of tile rt is head
// slot rr % HP of query (16 rt + rr) / HP (HP = the head count rounded up to
// 4, 8 or 16), so a query's rows share a 4-, 8- or 16-row band and its
// ReLU * w head sum needs at most two cross-lane adds.  Each key is read once
// for all T queries; the scores of query t go to row seq * T + t (keys past
// its position are not written).  A row histogram kernel then records every
// row's digit histogram, and the select kernel takes each row's top-k.
constexpr int kMaxMQ = 8;

struct MQArgs {
  const void* q;
  const float* q_scale;
  const float* w;
  const void* k;
  const float* k_scale;
  const int32_t* heads;  // [batch, T, nh] (nullptr: heads 0 .. nh-1)
  int32_t nh;
  float* rows;  // [batch * T, L]
  int32_t L, T, H, keys_per_wave;
};

template <int DT, int HP, int NRT>
__global__ __launch_bounds__(kDecThreads) void mq_score_kernel(MQArgs a) {
  static_assert(HP == 4 || HP == 8 || HP == 16, "head band of 4, 8 or 16 rows");
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int col = lane & 15;
  const int qq = lane >> 4;
  const int64_t seq = blockIdx.y;
  const int64_t L = a.L;
  const void* krows = (DT == kBF16) ? static_cast<const void*>(static_cast<const uint16_t*>(a.k) + seq * L * kD)
                                    : static_cast<const void*>(static_cast<const uint8_t*>(a.k) + seq * L * kD);
  const int64_t s_begin = (static_cast<int64_t>(blockIdx.x) * kDecWaves + wave) * a.keys_per_wave;
  const int64_t s_end = min<int64_t>(s_begin + a.keys_per_wave, L);
  using Keys = typename RowScorer<DT, 1>::Keys;
  Keys kb0, kb1;
  if (s_begin < s_end) RowScorer<DT, 1>::load64(krows, s_begin, s_end, s_begin, kb0);
  if (s_begin + 64 < s_end) RowScorer<DT, 1>::load64(krows, s_begin + 64, s_end, s_begin, kb1);

  // A operands and per-row weights (times the query's fp8 scale).
  auto head_of = [&](int rr) -> int {  // head of tile row rr, or -1
    const int t = rr / HP, slot = rr % HP;
    if (t >= a.T || slot >= a.nh) return -1;
    const int j = a.heads ? a.heads[(seq * a.T + t) * a.nh + slot] : slot;
    return (j >= 0 && j < a.H) ? j : -1;
  };
  bf16x8 a16[NRT][4];
  i32x8 a8[NRT];
  float wl[NRT][4];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = rt * 16 + 4 * qq + i;
      const int j = head_of(rr);
      const int64_t qr = seq * a.T + rr / HP;
      wl[rt][i] = j >= 0 ? a.w[qr * a.H + j] * ((DT == kFP8) ? a.q_scale[qr] : 1.f) : 0.f;
    }
    const int rr = rt * 16 + col;
    const int j = head_of(rr);
    const int64_t qoff = ((seq * a.T + rr / HP) * a.H + (j < 0 ? 0 : j)) * kD;
    if constexpr (DT == kBF16) {
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) + (j < 0 ? 0 : qoff));
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) a16[rt][ks] = as_bf16x8(j < 0 ? make_uint4(0, 0, 0, 0) : src[4 * ks + qq]);
    } else {
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.q) + (j < 0 ? 0 : qoff));
      const uint4 lo = j < 0 ? make_uint4(0, 0, 0, 0) : src[qq];
      const uint4 hi = j < 0 ? make_uint4(0, 0, 0, 0) : src[4 + qq];
      a8[rt] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
  }
  // Lanes that write: the first lane group of each query's band.
  const bool writer = HP == 4 || (HP == 8 && (qq & 1) == 0) || (HP == 16 && qq == 0);

  auto score = [&](const Keys& kb, int64_t s0) __attribute__((always_inline)) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int64_t s = s0 + 16 * g + col;
      const float sk = (DT == kFP8 && s < s_end) ? a.k_scale[seq * L + s] : 1.f;
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
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) part += wl[rt][i] * relu(acc[i]);
        if constexpr (HP >= 8) part += __shfl_xor(part, 16, kWave);
        if constexpr (HP == 16) part += __shfl_xor(part, 32, kWave);
        const int t = (rt * 16 + 4 * qq) / HP;
        if (writer && t < a.T && s < s_end && s <= L - a.T + t) a.rows[(seq * a.T + t) * L + s] = part * sk;
      }
    }
  };
  // Two 64-key groups in flight per wave (fixed roles).
  for (int64_t s0 = s_begin; s0 < s_end; s0 += 128) {
    score(kb0, s0);
    if (s0 + 128 < s_end) RowScorer<DT, 1>::load64(krows, s0 + 128, s_end, s_begin, kb0);
    if (s0 + 64 < s_end) {
      score(kb1, s0 + 64);
      if (s0 + 192 < s_end) RowScorer<DT, 1>::load64(krows, s0 + 192, s_end, s_begin, kb1);
    }
  }
}

// Digit histogram record of each row (one 1024-thread workgroup per row,
// the row's prefix n = L - T + 1 + r % T read in rounds of 16 scores per
// thread, all of a round's loads in flight): fine bins, then coarse sums.
constexpr int kRowHistThreads = 1024;

__global__ __launch_bounds__(kRowHistThreads) void row_hist_kernel(const float* __restrict__ rows,
                                                                   uint32_t* __restrict__ ghist, int32_t L,
                                                                   int32_t T) {
  __shared__ uint32_t hist[kDigits];
  const int64_t r = blockIdx.x;
  const int32_t n = L - T + 1 + static_cast<int32_t>(r % T);
  const float* row = rows + r * L;
  for (int b = threadIdx.x; b < kDigits; b += kRowHistThreads) hist[b] = 0;
  __syncthreads();
  constexpr int U = 16;
  for (int c0 = 0; c0 < n; c0 += U * kRowHistThreads) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = c0 + u * kRowHistThreads + static_cast<int>(threadIdx.x);
      v[u] = row[i < n ? i : n - 1];
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (c0 + u * kRowHistThreads + static_cast<int>(threadIdx.x) < n) atomicAdd(&hist[key_digit(v[u])], 1u);
  }
  __syncthreads();
  uint32_t* gh = ghist + r * kHistWords;
  for (int b = threadIdx.x; b < kDigits; b += kRowHistThreads) gh[b] = hist[b];
  for (int cb = threadIdx.x; cb < kCoarse; cb += kRowHistThreads) {
    uint32_t c = 0;
#pragma unroll
    for (int u = 0; u < kFinePerCoarse; ++u) c += hist[cb * kFinePerCoarse + (u + cb) % kFinePerCoarse];
    gh[kDigits + cb] = c;
  }
}

int mq_band(int32_t nh) { return nh <= 4 ? 4 : (nh <= 8 ? 8 : 16); }

// One row per (sequence, query): the layout of a T = 1 problem over
// batch * T sequences.
Shape mq_rows_shape(const Shape& s) {
  Shape r = s;
  r.batch = s.batch * s.T;
  r.T = 1;
  return r;
}

template <int DT, int HP>
void launch_mq_dt(const Shape& s, const MQArgs& a, hipStream_t st) {
  dim3 grid((s.L + kDecWaves * a.keys_per_wave - 1) / (kDecWaves * a.keys_per_wave), s.batch);
  const int nrt = (s.T * HP + 15) / 16;
  if (nrt <= 1) mq_score_kernel<DT, HP, 1><<<grid, kDecThreads, 0, st>>>(a);
  else if (nrt == 2) mq_score_kernel<DT, HP, 2><<<grid, kDecThreads, 0, st>>>(a);
  else if (nrt == 3) mq_score_kernel<DT, HP, 3><<<grid, kDecThreads, 0, st>>>(a);
  else mq_score_kernel<DT, HP, 4><<<grid, kDecThreads, 0, st>>>(a);
}

}  // namespace

size_t decode_ws_bytes(const Shape& s) { return decode_layout(s, nullptr).total; }

bool decode_mq_supported(const Shape& s, int32_t nh) {
  return s.T >= 2 && s.T <= kMaxMQ && s.dtype != kF32 && nh >= 1 && nh <= 16 && s.T * mq_band(nh) <= 64 &&
         static_cast<int64_t>(s.batch) * s.T <= 65535;
}

size_t decode_mq_ws_bytes(const Shape& s) { return decode_layout(mq_rows_shape(s), nullptr).total; }

hipError_t launch_decode_mq_score_topk(const Shape& s, int32_t nh, const int32_t* heads, int32_t k,
                                       const void* q, const float* q_scale, const float* w,
                                       const void* kk, const float* k_scale, int32_t* idx,
                                       float* scores_out, void* ws, hipStream_t st) {
  const Shape sr = mq_rows_shape(s);
  const DecodeWs d = decode_layout(sr, ws);
  const int64_t ncnt = 2 * static_cast<int64_t>(sr.batch);  // compaction counters and arrivals
  clear_kernel<<<static_cast<unsigned>((ncnt + 1023) / 1024), 256, 0, st>>>(d.cnt, ncnt);
  MQArgs a{q, q_scale, w, kk, k_scale, heads, nh, d.rows, s.L, s.T, s.H, MISA_DECODE_KEYS_PER_WAVE};
  const int hp = mq_band(nh);
#define MQ(DT) \
  if (hp == 4) launch_mq_dt<DT, 4>(s, a, st); \
  else if (hp == 8) launch_mq_dt<DT, 8>(s, a, st); \
  else launch_mq_dt<DT, 16>(s, a, st);
  if (s.dtype == kBF16) { MQ(kBF16) } else { MQ(kFP8) }
#undef MQ
  row_hist_kernel<<<static_cast<unsigned>(sr.batch), kRowHistThreads, 0, st>>>(d.rows, d.ghist, s.L, s.T);
  dim3 g((s.L + kCompactChunk - 1) / kCompactChunk, sr.batch);
  decode_select_kernel<<<g, kCompactThreads, 0, st>>>(d.rows, d.ghist, d.cnt, d.done, d.cand_s, d.cand_i,
                                                      idx, scores_out, s.L, k, 1, nullptr, s.T);
  return hipGetLastError();
}

// Keys per wave of decode_score_kernel: 512 while the grid keeps at least
// 512 workgroups, else 256.  Each workgroup clears and flushes a histogram of
// kDigits bins, so larger chunks take that fixed cost over more keys (C2
// dense 70 -> 64 us, C4 62 -> 59 us); small batches keep more workgroups.
int32_t decode_keys_per_wave(const Shape& s) {
  constexpr int64_t kLarge = 512;
  const int64_t wgs = static_cast<int64_t>(s.batch) * ((s.L + kDecWaves * kLarge - 1) / (kDecWaves * kLarge));
  return wgs >= 512 ? static_cast<int32_t>(kLarge) : MISA_DECODE_KEYS_PER_WAVE;
}

hipError_t launch_decode_score_topk(const Shape& s, int32_t nh, const int32_t* heads, int32_t k,
                                    const void* q, const float* q_scale, const float* w,
                                    const void* kk, const float* k_scale, int32_t* idx,
                                    float* scores_out, void* ws, hipStream_t st) {
  const DecodeWs d = decode_layout(s, ws);
  const int64_t nz = d.zero_words;
  clear_kernel<<<static_cast<unsigned>((nz + 1023) / 1024), 256, 0, st>>>(d.cnt, nz);
  DecodeArgs a{q, q_scale, w, kk, k_scale, heads, nh, nullptr, 0, 0, nullptr, nullptr, 0,
               d.rows, d.ghist, s.L, s.H, decode_keys_per_wave(s)};
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
  if (const int32_t G = step_groups(s)) {
    const int32_t kpw = static_cast<int32_t>(
        (((s.L + static_cast<int64_t>(G) * kStepWaves - 1) / (static_cast<int64_t>(G) * kStepWaves)) + 63) / 64 * 64);
    StepArgs sa{q, q_scale, w, pooled, kk, k_scale, heads, E_out, d.rows, d.ghist, d.cnt, d.done,
                d.rpart, d.rsync, M, s.L, s.H, s.B, h, G, s.batch, kpw};
    const unsigned grid = static_cast<unsigned>(G) * static_cast<unsigned>(s.batch);
    if (s.dtype == kBF16) decode_step_kernel<kBF16><<<grid, kStepThreads, 0, st>>>(sa);
    else decode_step_kernel<kFP8><<<grid, kStepThreads, 0, st>>>(sa);
    launch_select(s, d, k, idx, scores_out, st, G);
    return hipGetLastError();
  }
  const int32_t nmain = step_main_chunks(s);
  const int32_t nch = nmain + 1;
  const int64_t nz = d.zero_words;
  dim3 g1(nch, s.batch);
  if (s.dtype == kBF16)
    step_route_kernel<kBF16><<<g1, 256, 0, st>>>(q, pooled, kk, k_scale, d.part, d.cnt, nz, s.L,
                                                 s.H, s.B, M, nmain);
  else
    step_route_kernel<kFP8><<<g1, 256, 0, st>>>(q, pooled, kk, k_scale, d.part, d.cnt, nz, s.L,
                                                s.H, s.B, M, nmain);
  DecodeArgs a{q, q_scale, w, kk, k_scale, nullptr, h, d.part, nch, h, heads, E_out, M,
               d.rows, d.ghist, s.L, s.H, decode_keys_per_wave(s)};
  if (s.dtype == kBF16) launch_score<kBF16, true>(s, a, st);
  else launch_score<kFP8, true>(s, a, st);
  launch_select(s, d, k, idx, scores_out, st);
  return hipGetLastError();
}

}  // namespace misa
