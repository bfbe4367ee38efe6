// Block-wide exact top-k by radix select (Eq. (2), (8), (10)-(12) of the MISA
// summary page: TopK over a score row or a candidate list).
//
// Keys are the order-preserving u32 images of fp32 scores.  Three histogram
// passes over 11/11/10-bit digits (2048-bin LDS histogram) find the k-th
// largest key K*; if more tokens tie at K* than slots remain, three more
// passes over the complemented token index pick the lowest indices among the
// ties.  A last pass writes the k winners with an ordered block compaction, so
// the output order is deterministic (source order).
#pragma once

#include "common.hpp"

namespace misa {

constexpr int kRadixBins = 2048;

struct TopkSmem {
  uint32_t hist[kRadixBins];
  int scan_tmp[32];
  uint32_t sel_digit;
  int sel_above;
  int sel_count;
};

// Among elements i in [0, n) with pred(i), find the `want`-th largest value of
// val(i) (1-based).  Returns that value; `above` = how many elements have a
// strictly larger value, `equal` = how many equal it.  Requires the number of
// elements with pred(i) >= want >= 1.
template <int NT, class Pred, class Val>
__device__ __forceinline__ uint32_t block_select_kth(int64_t n, int want, Pred pred, Val val, TopkSmem& sm,
                                     int& above, int& equal) {
  uint32_t prefix = 0, prefix_mask = 0;
  int remaining = want;
  int above_total = 0;
  int eq = 0;
  for (int pass = 0; pass < 3; ++pass) {
    // Digits: bits 31..21, 20..10, 9..0.
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t m = pass == 2 ? 0x3FFu : 0x7FFu;
    for (int b = threadIdx.x; b < kRadixBins; b += NT) sm.hist[b] = 0;
    __syncthreads();
    for (int64_t i = threadIdx.x; i < n; i += NT) {
      if (!pred(i)) continue;
      const uint32_t v = val(i);
      if ((v & prefix_mask) == prefix) atomicAdd(&sm.hist[(v >> shift) & m], 1u);
    }
    __syncthreads();
    // Suffix sums over bins: bins handled per thread in descending order.
    constexpr int BPT = kRadixBins / NT;  // bins per thread
    const int nb = static_cast<int>(m) + 1;
    // Thread r owns bins [nb-1-r*BPT-(BPT-1), nb-1-r*BPT] walking downward.
    int local[BPT > 0 ? BPT : 1];
    int lsum = 0;
#pragma unroll
    for (int c = 0; c < BPT; ++c) {
      const int bin = nb - 1 - (threadIdx.x * BPT + c);
      local[c] = (bin >= 0) ? static_cast<int>(sm.hist[bin]) : 0;
      lsum += local[c];
    }
    int total;
    int run = block_exclusive_sum<NT>(lsum, sm.scan_tmp, total);  // count in higher bins
#pragma unroll
    for (int c = 0; c < BPT; ++c) {
      const int bin = nb - 1 - (threadIdx.x * BPT + c);
      if (bin >= 0 && run < remaining && run + local[c] >= remaining) {
        sm.sel_digit = static_cast<uint32_t>(bin);
        sm.sel_above = run;
        sm.sel_count = local[c];
      }
      run += local[c];
    }
    __syncthreads();
    const uint32_t digit = sm.sel_digit;
    remaining -= sm.sel_above;
    above_total += sm.sel_above;
    eq = sm.sel_count;
    prefix |= digit << shift;
    prefix_mask |= m << shift;
    __syncthreads();
  }
  above = above_total;
  equal = eq;
  return prefix;
}

// Select the k best elements (key(i) larger is better; equal keys: smaller
// idx(i) first) among i in [0, n) with valid(i), and write their idx/score to
// out_idx/out_score[0..k) in source order.  Unused slots (fewer than k valid
// elements) get idx -1 and score -inf.  All threads of the block must call.
template <int NT, class Valid, class Key, class Idx, class Score>
__device__ __forceinline__ void block_topk(int64_t n, int k, Valid valid, Key key, Idx idx, Score score,
                           int32_t* out_idx, float* out_score, TopkSmem& sm) {
  // Count valid elements.
  int cnt = 0;
  for (int64_t i = threadIdx.x; i < n; i += NT) cnt += valid(i) ? 1 : 0;
  int nvalid;
  (void)block_exclusive_sum<NT>(cnt, sm.scan_tmp, nvalid);

  bool take_all = nvalid <= k;
  uint32_t kth = 0, ith = 0;
  bool tiebreak = false;
  if (!take_all) {
    int above, equal;
    kth = block_select_kth<NT>(n, k, valid, key, sm, above, equal);
    const int need = k - above;  // how many of the ties at kth to keep
    if (equal > need) {
      tiebreak = true;
      int a2, e2;
      auto tie = [=](int64_t i) { return valid(i) && key(i) == kth; };
      auto inv_idx = [=](int64_t i) { return ~static_cast<uint32_t>(idx(i)); };
      ith = block_select_kth<NT>(n, need, tie, inv_idx, sm, a2, e2);
    }
  }
  // Ordered compaction of the winners.
  int base = 0;
  for (int64_t r0 = 0; r0 < n; r0 += NT) {
    const int64_t i = r0 + threadIdx.x;
    bool sel = false;
    if (i < n && valid(i)) {
      if (take_all) {
        sel = true;
      } else {
        const uint32_t kv = key(i);
        sel = kv > kth || (kv == kth && (!tiebreak || ~static_cast<uint32_t>(idx(i)) >= ith));
      }
    }
    int tot;
    const int pos = base + block_exclusive_sum<NT>(sel ? 1 : 0, sm.scan_tmp, tot);
    if (sel && pos < k) {  // pos >= k only with duplicate candidate ids
      out_idx[pos] = idx(i);
      if (out_score) out_score[pos] = score(i);
    }
    base += tot;
  }
  for (int p = min(base, k) + threadIdx.x; p < k; p += NT) {
    out_idx[p] = -1;
    if (out_score) out_score[p] = -__builtin_inff();
  }
}

// ---------------------------------------------------------------- score digits

constexpr int kDigits = 8192;  // histogram bins of key_digit

// Histogram digit of a score: a monotone (non-decreasing) map of the
// order-preserving key to [0, kDigits) that spends its bins where top-k
// thresholds live.  Bin 0 holds every negative value, bin 1 zero (either
// sign) and positive subnormals; positive values with binary exponent in a
// 63-binade window get 128 bins per binade (7 mantissa bits: bins 0.8%
// wide), values below or above the window share the window's first or last
// bin.  A 13-bit prefix of the order-preserving key
// would spend 7/8 of its bins on exponents that scores never reach and leave
// bins 6% wide.
constexpr int kExpLo = 127 - 31;  // window: values in [2^-31, 2^32)
constexpr int kExpBins = 63;
// Straight-line selects (no branches: it runs per entry in the top-k
// kernels).  Inside the window the digit is 2 + (e - kExpLo) * 128 + the top
// 7 mantissa bits, i.e. (u >> 16) - kExpLo * 128 + 2.
__host__ __device__ __forceinline__ uint32_t key_digit(float v) {
  const uint32_t key = float_key(v);  // -0 has the key of +0
  const uint32_t u = key & 0x7FFFFFFFu;
  const uint32_t e = u >> 23;
  uint32_t d = (u >> 16) - (static_cast<uint32_t>(kExpLo) << 7) + 2u;
  d = e >= static_cast<uint32_t>(kExpLo + kExpBins) ? 2u + ((kExpBins - 1) << 7) + 127u : d;
  d = e < static_cast<uint32_t>(kExpLo) ? 2u : d;
  d = e == 0u ? 1u : d;
  return key < 0x80000000u ? 0u : d;
}
static_assert(2 + (kExpBins << 7) <= kDigits, "digit range");
constexpr uint32_t kTopDigit = 2u + ((kExpBins - 1) << 7) + 127u;

// The smallest order-preserving key (float_key) whose score has digit d, for
// 0 <= d <= kTopDigit: key_digit(v) >= d  <=>  float_key(v) >= digit_lo_key(d).
__host__ __device__ __forceinline__ uint32_t digit_lo_key(uint32_t d) {
  if (d == 0) return 0u;
  if (d == 1) return 0x80000000u;  // +0
  if (d == 2) return 0x80800000u;  // smallest positive normal
  const uint32_t b = d - 2;
  return 0x80000000u | ((kExpLo + (b >> 7)) << 23) | ((b & 127u) << 16);
}
// The largest key with digit d.
__host__ __device__ __forceinline__ uint32_t digit_hi_key(uint32_t d) {
  return d >= kTopDigit ? 0xFFFFFFFFu : digit_lo_key(d + 1) - 1u;
}

// ---------------------------------------------------------------- relative bins
//
// Candidate lists (the prefill candidates, the re-ranked lists) are binned
// relative to their own range.  A score's coarse key g = float_key >> 16
// keeps the sign, the exponent and the top 7 mantissa bits: monotone in the
// score, 128 bins per binade, four instructions cheaper per entry than the
// digit above.  bin = min((max(g, gb) - gb) >> shift, kRelBinCount - 1):
// every key below gb shares bin 0, every key far above shares the last bin.
constexpr int kRelBinCount = 2048;
constexpr int kRelBinBits = 11;
// Coarse key of 2^-31: in a list's own range, values below it (zeros,
// negatives, subnormals) share the lowest bin, as they share the lowest
// digits above.
constexpr uint32_t kCoarseFloor = (0x80000000u | (static_cast<uint32_t>(127 - 31) << 23)) >> 16;

struct RelBins {
  uint32_t gb;     // coarse key of bin 0's upper part
  uint32_t shift;  // coarse keys per bin: 2^shift

  // A list whose every entry scores >= tau (the candidate threshold).
  __host__ __device__ static RelBins above(float tau) { return RelBins{float_key(tau) >> 16, 0u}; }
  // A list whose valid entries have coarse keys in [gmin, gmax] (gmin <=
  // gmax): bins of 2^shift coarse keys from max(gmin, kCoarseFloor), the
  // shift fitting the range in kRelBinCount bins.
  __host__ __device__ static RelBins range(uint32_t gmin, uint32_t gmax) {
    const uint32_t lo = gmin > kCoarseFloor ? gmin : kCoarseFloor;
    const uint32_t hi = gmax > kCoarseFloor ? gmax : kCoarseFloor;
    const uint32_t span = hi - lo;
    const uint32_t sh = span < static_cast<uint32_t>(kRelBinCount)
                            ? 0u
                            : static_cast<uint32_t>(32 - __builtin_clz(span) - kRelBinBits);
    return RelBins{lo, sh};
  }
  __host__ __device__ uint32_t bin_of_coarse(uint32_t g) const {
    const uint32_t x = ((g > gb ? g : gb) - gb) >> shift;
    return x < static_cast<uint32_t>(kRelBinCount) ? x : static_cast<uint32_t>(kRelBinCount - 1);
  }
  __host__ __device__ uint32_t bin(float v) const { return bin_of_coarse(float_key(v) >> 16); }
  // Keys [lo, hi] of bin b: every key with bin_of_coarse(key >> 16) == b
  // lies in it (bin 0 reaches down to key 0, the last bin up to the largest
  // key).  A bin past every key gets the empty interval lo > hi.
  __host__ __device__ void interval(uint32_t b, uint32_t& lo, uint32_t& hi) const {
    const uint64_t g0 = static_cast<uint64_t>(gb) + (static_cast<uint64_t>(b) << shift);
    const uint64_t g1 = static_cast<uint64_t>(gb) + (static_cast<uint64_t>(b + 1) << shift);
    if (b != 0 && g0 > 0xFFFFu) {
      lo = 0xFFFFFFFFu;
      hi = 0xFFFFFFFEu;
      return;
    }
    lo = b == 0 ? 0u : static_cast<uint32_t>(g0 << 16);
    hi = (b + 1 >= static_cast<uint32_t>(kRelBinCount) || g1 > 0xFFFFu) ? 0xFFFFFFFFu
                                                                      : static_cast<uint32_t>((g1 << 16) - 1u);
  }
};

// ---------------------------------------------------------------- candidate certificate
//
// A threshold-filtered candidate list (every key of split s scoring >= tau_s
// was kept; no segment overflowed unless `overflow`) holds the true top-k
// when at least k candidates score >= tau_max = max_s tau_s: any filtered key
// scores below its own tau_s <= tau_max, so it cannot beat those k.  What a
// select does with a list before it has counted the candidates >= tau_max:
//   kRepair  - cannot be certified (an overflow, or fewer than k candidates
//              while some key was filtered out);
//   kTakeAll - nothing was filtered (tau_max = -inf) and at most k
//              candidates: the list is the whole prefix, take every entry;
//   kCount   - count the candidates >= tau_max; select if there are >= k,
//              else repair.  This includes a list of exactly k candidates
//              with a finite tau_max: a candidate of a low-tau split may lie
//              below a filtered key of the tau_max split.
enum class CandVerdict : int { kRepair = 0, kTakeAll = 1, kCount = 2 };

__host__ __device__ __forceinline__ CandVerdict cand_verdict(bool overflow, int total, int k,
                                                             float tau_max) {
  const bool filtered = !(tau_max == -__builtin_inff());
  if (overflow || (total < k && filtered)) return CandVerdict::kRepair;
  if (total <= k && !filtered) return CandVerdict::kTakeAll;
  return CandVerdict::kCount;
}

// ---------------------------------------------------------------- list resolve
//
// The `need` best of a short LDS list (score, token), written to out[0..need)
// in any order (ties: lower token first).  Up to kDirectRank entries are ranked
// pairwise; a longer list is cut once more by a 2048-bin histogram over its
// own key range (the bin is monotone in the score): entries of bins above the
// threshold bin are written directly, the threshold bin is ranked pairwise.
// Returns false (nothing written) when even that bin exceeds kRankMax; the
// caller then falls back to block_topk.  All threads must call.

constexpr int kRankMax = 256;
constexpr int kDirectRank = 128;  // longer lists take the histogram cut first
constexpr int kResolveBins = 2048;

struct ResolveSmem {
  uint32_t hist[kResolveBins];
  alignas(16) float s2[kRankMax];
  alignas(16) int32_t i2[kRankMax];
  int scan_tmp[32];
  int bin, above, count, n_hi, n_at;
  uint32_t kmin, kmax;
};

// Entry t of the list is ranked by how many entries beat it: larger key, or
// equal key and lower token (one 64-bit compare of key:~token).  The list is
// read four entries at a time (cs and ci 16-byte aligned, with capacity a
// multiple of 4; entries past n are masked).
__device__ __forceinline__ uint64_t rank_key(float s, int32_t id) {
  return (static_cast<uint64_t>(float_key(s)) << 32) | static_cast<uint32_t>(~id);
}

// The comparisons of each entry are split over P = NT / n threads (at most
// 16): thread q n + e counts the entries of part q that beat entry e, and the
// part counts meet in racc (LDS, at least n words).  A list of n <= NT / 4
// then takes n / 4 rounds of compares instead of n on one thread.  All NT
// threads call; racc is free again when it returns.
template <int NT>
__device__ __forceinline__ void rank_write(const float* cs, const int32_t* ci, int n, int need,
                                           int32_t* out_idx, float* out_score, uint32_t* racc) {
  if (n <= 0) return;  // (uniform)
  const int P = min(max(NT / n, 1), 16);
  const int per = ((n + P - 1) / P + 3) & ~3;  // entries per part, a multiple of 4
  const float4* cs4 = reinterpret_cast<const float4*>(cs);
  const int4* ci4 = reinterpret_cast<const int4*>(ci);
  for (int t = threadIdx.x; t < n; t += NT) racc[t] = 0;
  __syncthreads();
  for (int t = threadIdx.x; t < n * P; t += NT) {
    const int e = t % n, q = t / n;
    const uint64_t me = rank_key(cs[e], ci[e]);
    const int j0 = q * per, j1 = min(n, j0 + per);
    int rank = 0;
    for (int j = j0; j < j1; j += 4) {
      const float4 c = cs4[j / 4];
      const int4 d = ci4[j / 4];
      rank += (j + 0 < j1 && rank_key(c.x, d.x) > me) ? 1 : 0;
      rank += (j + 1 < j1 && rank_key(c.y, d.y) > me) ? 1 : 0;
      rank += (j + 2 < j1 && rank_key(c.z, d.z) > me) ? 1 : 0;
      rank += (j + 3 < j1 && rank_key(c.w, d.w) > me) ? 1 : 0;
    }
    if (rank) atomicAdd(&racc[e], static_cast<uint32_t>(rank));
  }
  __syncthreads();
  for (int t = threadIdx.x; t < n; t += NT) {
    const int rank = static_cast<int>(racc[t]);
    if (rank < need) {
      out_idx[rank] = ci[t] < 0 ? -1 : ci[t];  // negative ids: distinct padding, printed as -1
      if (out_score) out_score[rank] = cs[t];
    }
  }
}

template <int NT>
__device__ __forceinline__ bool resolve_list(const float* cs, const int32_t* ci, int n, int need,
                                             int32_t* out_idx, float* out_score, ResolveSmem& rs) {
  // Every slot gets one rank when the tokens are distinct; -1 guards the rest.
  for (int p = threadIdx.x; p < need; p += NT) out_idx[p] = -1;
  if (n <= kDirectRank) {
    rank_write<NT>(cs, ci, n, need, out_idx, out_score, rs.hist);  // (its first barrier)
    return true;
  }
  if (threadIdx.x == 0) {
    rs.kmin = 0xFFFFFFFFu;
    rs.kmax = 0;
    rs.n_hi = 0;
    rs.n_at = 0;
  }
  for (int b = threadIdx.x; b < kResolveBins; b += NT) rs.hist[b] = 0;
  __syncthreads();
  uint32_t lo = 0xFFFFFFFFu, hi = 0;
  for (int t = threadIdx.x; t < n; t += NT) {
    const uint32_t key = float_key(cs[t]);
    lo = min(lo, key);
    hi = max(hi, key);
  }
  // One LDS atomic per wave: same-address atomics from every thread serialize.
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) {
    lo = min(lo, static_cast<uint32_t>(__shfl_xor(static_cast<int>(lo), o, kWave)));
    hi = max(hi, static_cast<uint32_t>(__shfl_xor(static_cast<int>(hi), o, kWave)));
  }
  if ((threadIdx.x & (kWave - 1)) == 0 && lo <= hi) {
    atomicMin(&rs.kmin, lo);
    atomicMax(&rs.kmax, hi);
  }
  __syncthreads();
  const uint32_t kmin = rs.kmin, span = rs.kmax - rs.kmin;
  const int shift = span < static_cast<uint32_t>(kResolveBins) ? 0 : 32 - __clz(span) - 11;
  for (int t = threadIdx.x; t < n; t += NT)
    atomicAdd(&rs.hist[(float_key(cs[t]) - kmin) >> shift], 1u);
  __syncthreads();
  {
    constexpr int BPT = (kResolveBins + NT - 1) / NT;
    int local[BPT];
    int lsum = 0;
#pragma unroll
    for (int c = 0; c < BPT; ++c) {
      const int bin = kResolveBins - 1 - (threadIdx.x * BPT + c);
      local[c] = bin >= 0 ? static_cast<int>(rs.hist[bin]) : 0;
      lsum += local[c];
    }
    int total;
    int run = block_exclusive_sum<NT>(lsum, rs.scan_tmp, total);
#pragma unroll
    for (int c = 0; c < BPT; ++c) {
      const int bin = kResolveBins - 1 - (threadIdx.x * BPT + c);
      if (bin >= 0 && run < need && run + local[c] >= need) {
        rs.bin = bin;
        rs.above = run;
        rs.count = local[c];
      }
      run += local[c];
    }
    __syncthreads();
  }
  const uint32_t b2 = static_cast<uint32_t>(rs.bin);
  const int above = rs.above, cnt2 = rs.count;
  if (cnt2 > kRankMax) return false;
  // Positions from wave ballots and one LDS atomic per wave and list (the
  // loop bound is wave-uniform).
  const int lane = threadIdx.x & (kWave - 1);
  for (int t0 = threadIdx.x - lane; t0 < n; t0 += NT) {
    const int t = t0 + lane;
    const bool ok = t < n;
    const uint32_t bin = ok ? (float_key(cs[t]) - kmin) >> shift : 0u;
    const bool h = ok && bin > b2;
    const bool at = ok && bin == b2;
    const uint64_t mh = __ballot(h);
    const uint64_t ma = __ballot(at);
    if (mh) {
      int p = 0;
      if (lane == 0) p = atomicAdd(&rs.n_hi, __popcll(mh));
      p = __shfl(p, 0, kWave) + lanes_below(mh);
      if (h && p < above) {
        out_idx[p] = ci[t] < 0 ? -1 : ci[t];
        if (out_score) out_score[p] = cs[t];
      }
    }
    if (ma) {
      int p = 0;
      if (lane == 0) p = atomicAdd(&rs.n_at, __popcll(ma));
      p = __shfl(p, 0, kWave) + lanes_below(ma);
      if (at && p < kRankMax) {
        rs.s2[p] = cs[t];
        rs.i2[p] = ci[t];
      }
    }
  }
  __syncthreads();
  rank_write<NT>(rs.s2, rs.i2, cnt2, need - above, out_idx + above,
                 out_score ? out_score + above : nullptr, rs.hist);
  return true;
}

// ---------------------------------------------------------------- fast path
//
// Same contract as block_topk, for scores held as fp32.  Wave w owns the
// contiguous range [w*CW, (w+1)*CW) (CW a multiple of 64); at step j lane l
// handles element w*CW + 64j + l, so every load is coalesced and (step, lane)
// order is index order.  Ranges of at most kRegCache steps stay in registers
// across the passes:
//   1. count + min/max of the valid scores (block reductions);
//   2. a histogram over kLinBins bins of the order-preserving key range
//      [key(min), key(max)] (bin = (key - key(min)) >> shift, shift chosen so
//      the range fits): the bin is a monotone function of the score, so every
//      element of a higher bin has a strictly larger score, and the bins are
//      log-spaced in value, so a few large outliers cannot crowd all scores
//      into a few bins.  A suffix scan gives the bin b* holding the k-th best
//      and `above`, the count in higher bins;
//   3. one compaction pass (wave ballots + LDS counters; set semantics):
//      elements of bins above b* go straight to the output, those of b* to an
//      LDS list;
//   4. the b* list is resolved exactly: by pairwise rank when it is short,
//      else by block_topk.
// When the range is degenerate or b* holds more than kLinCap elements the
// whole input goes through block_topk instead.

constexpr int kLinBins = 4096;
constexpr int kLinCap = 4096;
constexpr int kRegCache = 32;

struct TopkFastSmem {
  TopkSmem base;
  ResolveSmem rs;
  uint32_t hist[kLinBins];
  alignas(16) float cand_score[kLinCap];
  alignas(16) int32_t cand_idx[kLinCap];
  float red[2][32];
  int wtot[2][32];
  int sel_bin, sel_above, sel_count;
  int cnt_hi, cnt_at;
};

__device__ __forceinline__ int lin_bin(float s, uint32_t kmin, int shift) {
  const uint32_t d = float_key(s) - kmin;  // < 2^(shift+12) for s in [min, max]
  const uint32_t b = d >> shift;
  return b < static_cast<uint32_t>(kLinBins) ? static_cast<int>(b) : kLinBins - 1;
}

template <int NT, class Valid, class Score, class Idx>
__device__ __forceinline__ bool block_topk_fast(int64_t n, int k, Valid valid, Score score, Idx idx,
                                                int32_t* out_idx, float* out_score,
                                                TopkFastSmem& sm,
                                                float gate = -__builtin_inff()) {
  constexpr int NW = NT / kWave;
  const int lane = lane_id();
  const int wid = threadIdx.x / kWave;
  const int64_t CW = ((n + NW - 1) / NW + kWave - 1) / kWave * kWave;
  const int J = static_cast<int>(CW / kWave);
  const int64_t wbase = static_cast<int64_t>(wid) * CW + lane;
  const bool cached = J <= kRegCache;
  // Register cache of this lane's elements (score, token); ok bit j marks a
  // valid element.  Steps j >= J are skipped with wave-uniform branches.
  float rc[kRegCache];
  int32_t ri[kRegCache];
  uint32_t okm = 0;
  // 1. count, min, max, and the count of scores >= gate.
  int cnt = 0, cge = 0;
  float mn = __builtin_inff(), mx = -__builtin_inff();
  if (cached) {
#pragma unroll
    for (int j = 0; j < kRegCache; ++j) {
      rc[j] = 0.f;
      ri[j] = -1;
      if (j < J) {
        const int64_t i = wbase + 64 * j;
        const bool ok = i < n && valid(i);
        const float v = ok ? score(i) : 0.f;
        rc[j] = v;
        ri[j] = ok ? idx(i) : -1;
        okm |= ok ? (1u << j) : 0u;
        cnt += ok ? 1 : 0;
        cge += (ok && v >= gate) ? 1 : 0;
        mn = ok ? fminf(mn, v) : mn;
        mx = ok ? fmaxf(mx, v) : mx;
      }
    }
  } else {
    for (int j = 0; j < J; ++j) {
      const int64_t i = wbase + 64 * j;
      if (i >= n || !valid(i)) continue;
      const float v = score(i);
      ++cnt;
      cge += v >= gate ? 1 : 0;
      mn = fminf(mn, v);
      mx = fmaxf(mx, v);
    }
  }
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) {
    cnt += __shfl_xor(cnt, o, kWave);
    cge += __shfl_xor(cge, o, kWave);
    mn = fminf(mn, __shfl_xor(mn, o, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
  }
  if (lane == 0) {
    sm.base.scan_tmp[wid] = cnt;
    sm.wtot[0][wid] = cge;
    sm.red[0][wid] = mn;
    sm.red[1][wid] = mx;
  }
  for (int b = threadIdx.x; b < kLinBins; b += NT) sm.hist[b] = 0;
  __syncthreads();
  int nvalid = 0, nge = 0;
  mn = __builtin_inff();
  mx = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    nvalid += sm.base.scan_tmp[i];
    nge += sm.wtot[0][i];
    mn = fminf(mn, sm.red[0][i]);
    mx = fmaxf(mx, sm.red[1][i]);
  }
  __syncthreads();
  // Gate: the caller needs at least k valid scores >= gate (else nothing is
  // written and false is returned).
  if (gate != -__builtin_inff() && nge < k) return false;
  const uint32_t kmin = float_key(mn);
  const uint32_t kspan = float_key(mx) - kmin;
  // Smallest shift with (kspan >> shift) < kLinBins.
  const int shift = kspan < static_cast<uint32_t>(kLinBins) ? 0 : 32 - __clz(kspan) - 12;
  const bool degenerate = !(mx > mn);  // all equal (or NaN): one bin
  if (nvalid <= k || degenerate) {
    block_topk<NT>(n, k, valid, [=](int64_t i) { return float_key(score(i)); }, idx, score,
                   out_idx, out_score, sm.base);
    return true;
  }
  // 2. histogram of the key bins, then the bin holding the k-th best.
  if (cached) {
#pragma unroll
    for (int j = 0; j < kRegCache; ++j)
      if (j < J && (okm & (1u << j))) atomicAdd(&sm.hist[lin_bin(rc[j], kmin, shift)], 1u);
  } else {
    for (int j = 0; j < J; ++j) {
      const int64_t i = wbase + 64 * j;
      if (i < n && valid(i)) atomicAdd(&sm.hist[lin_bin(score(i), kmin, shift)], 1u);
    }
  }
  __syncthreads();
  {
    constexpr int BPT = kLinBins / NT;
    int local[BPT];
    int lsum = 0;
#pragma unroll
    for (int c = 0; c < BPT; ++c) {
      local[c] = static_cast<int>(sm.hist[kLinBins - 1 - (threadIdx.x * BPT + c)]);
      lsum += local[c];
    }
    int total;
    int run = block_exclusive_sum<NT>(lsum, sm.base.scan_tmp, total);
#pragma unroll
    for (int c = 0; c < BPT; ++c) {
      if (run < k && run + local[c] >= k) {
        sm.sel_bin = kLinBins - 1 - (threadIdx.x * BPT + c);
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
  const int bstar = sm.sel_bin;
  const int above = sm.sel_above;
  const int bcount = sm.sel_count;
  if (bcount > kLinCap) {
    __syncthreads();
    block_topk<NT>(n, k, valid, [=](int64_t i) { return float_key(score(i)); }, idx, score,
                   out_idx, out_score, sm.base);
    return true;
  }
  // 3. compaction: bins above b* -> output, bin b* -> LDS list.  Positions
  //    come from wave ballots and two LDS counters (set semantics).
  auto emit = [&](bool ok, float v, int32_t id) {
    const int b = ok ? lin_bin(v, kmin, shift) : -1;
    const bool hi = b > bstar, at = b == bstar;
    const uint64_t mh = __ballot(hi);
    const uint64_t ma = __ballot(at);
    if (mh) {
      int base = 0;
      if (lane == 0) base = atomicAdd(&sm.cnt_hi, __popcll(mh));
      base = __shfl(base, 0, kWave);
      if (hi) {
        const int p = base + lanes_below(mh);
        if (p < k) {
          out_idx[p] = id;
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
        if (p < kLinCap) {
          sm.cand_score[p] = v;
          sm.cand_idx[p] = id;
        }
      }
    }
  };
  if (cached) {
#pragma unroll
    for (int j = 0; j < kRegCache; ++j)
      if (j < J) emit((okm >> j) & 1u, rc[j], ri[j]);
  } else {
    for (int j = 0; j < J; ++j) {
      const int64_t i = wbase + 64 * j;
      const bool ok = i < n && valid(i);
      emit(ok, ok ? score(i) : 0.f, ok ? idx(i) : -1);
    }
  }
  __syncthreads();
  // 4. the (k - above) best of the b* list, written after the `above` slots.
  const int need = k - above;
  const float* cs = sm.cand_score;
  const int32_t* ci = sm.cand_idx;
  if (resolve_list<NT>(cs, ci, bcount, need, out_idx + above,
                       out_score ? out_score + above : nullptr, sm.rs))
    return true;
  __syncthreads();
  block_topk<NT>(
      bcount, need, [](int64_t) { return true; }, [=](int64_t j) { return float_key(cs[j]); },
      [=](int64_t j) { return ci[j]; }, [=](int64_t j) { return cs[j]; }, out_idx + above,
      out_score ? out_score + above : nullptr, sm.base);
  return true;
}

}  // namespace misa
