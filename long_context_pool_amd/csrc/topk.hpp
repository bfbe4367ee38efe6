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
__device__ uint32_t block_select_kth(int64_t n, int want, Pred pred, Val val, TopkSmem& sm,
                                     int& above, int& equal) {
  constexpr int shifts[3] = {21, 10, 0};
  constexpr uint32_t masks[3] = {0x7FFu, 0x7FFu, 0x3FFu};
  uint32_t prefix = 0, prefix_mask = 0;
  int remaining = want;
  int above_total = 0;
  int eq = 0;
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = shifts[pass];
    const uint32_t m = masks[pass];
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
__device__ void block_topk(int64_t n, int k, Valid valid, Key key, Idx idx, Score score,
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
      auto tie = [&](int64_t i) { return valid(i) && key(i) == kth; };
      auto inv_idx = [&](int64_t i) { return ~static_cast<uint32_t>(idx(i)); };
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

}  // namespace misa
