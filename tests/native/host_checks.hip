// Host-side checks of top-k helpers shipped in the library's csrc/topk.hpp.
// This file is compiled for the host only (no device code, no GPU needed) and
// includes the library header itself, so what is checked is the code the
// kernels run, not a copy of it.
//
//   digits      every 32-bit order-preserving key: the score digit is
//               monotone, lies in [0, kTopDigit], and every key of digit d
//               lies in [digit_lo_key(d), digit_hi_key(d)]; the intervals of
//               consecutive digits tile the key space.
//   certificate the candidate-list verdicts of cand_verdict() on the cases
//               that decide between repair, take-all and counting.
//   relbins     the relative bins of candidate lists (RelBins), for bins set
//               from thresholds and from coarse-key ranges: over every coarse
//               key (a key's bin depends on its top 16 bits only, and interval
//               ends are multiples of 2^16) the bin is monotone, both end keys
//               of each coarse key lie in its bin's interval, and the
//               intervals of the bins that keys reach tile the key space.
//
// Prints "ok <what>" per passed check; exits non-zero on the first failure.
#include "topk.hpp"

#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

using misa::CandVerdict;

namespace {

float float_of_key(uint32_t key) {
  const uint32_t u = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
  float f;
  std::memcpy(&f, &u, sizeof f);
  return f;
}

int check_digits() {
  // Interval endpoints: lo strictly increasing, hi(d) = lo(d+1) - 1.
  for (uint32_t d = 0; d < misa::kTopDigit; ++d) {
    if (!(misa::digit_lo_key(d + 1) > misa::digit_lo_key(d))) {
      std::printf("FAIL lo(%u) >= lo(%u)\n", d, d + 1);
      return 1;
    }
    if (misa::digit_hi_key(d) != misa::digit_lo_key(d + 1) - 1u) {
      std::printf("FAIL hi(%u) != lo(%u) - 1\n", d, d + 1);
      return 1;
    }
  }
  if (misa::digit_hi_key(misa::kTopDigit) != 0xFFFFFFFFu || misa::digit_lo_key(0) != 0u) {
    std::printf("FAIL outer interval ends\n");
    return 1;
  }
  // Every key that is the image of a non-NaN float.
  const unsigned nt = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
  std::atomic<int> bad{0};
  std::atomic<uint64_t> checked{0};
  std::vector<std::thread> th;
  for (unsigned t = 0; t < nt; ++t) {
    th.emplace_back([&, t] {
      const uint64_t lo = (uint64_t{1} << 32) * t / nt, hi = (uint64_t{1} << 32) * (t + 1) / nt;
      uint32_t prev_d = 0;
      bool have_prev = false;
      uint64_t n = 0;
      for (uint64_t kk = lo; kk < hi; ++kk) {
        const uint32_t key = static_cast<uint32_t>(kk);
        const float v = float_of_key(key);
        if (std::isnan(v) || misa::float_key(v) != key) continue;
        const uint32_t d = misa::key_digit(v);
        ++n;
        if (d > misa::kTopDigit || key < misa::digit_lo_key(d) || key > misa::digit_hi_key(d) ||
            (have_prev && d < prev_d)) {
          if (bad.fetch_add(1) == 0)
            std::printf("FAIL key %08x (value %a): digit %u, interval [%08x, %08x]\n", key,
                        static_cast<double>(v), d, misa::digit_lo_key(d), misa::digit_hi_key(d));
          return;
        }
        prev_d = d;
        have_prev = true;
      }
      checked += n;
    });
  }
  for (auto& x : th) x.join();
  if (bad.load()) return 1;
  std::printf("ok digits (%llu keys)\n", static_cast<unsigned long long>(checked.load()));
  return 0;
}

int check_relbins_one(const misa::RelBins& rb, const char* what) {
  uint32_t prev_b = 0;
  uint32_t next_lo = 0;  // the first key the next reached bin must start at
  for (uint32_t g = 0; g <= 0xFFFFu; ++g) {
    const uint32_t b = rb.bin_of_coarse(g);
    if (b >= static_cast<uint32_t>(misa::kRelBinCount) || (g > 0 && b < prev_b)) {
      std::printf("FAIL relbins %s (gb %u shift %u): coarse %04x bin %u after %u\n", what, rb.gb, rb.shift, g, b,
                  prev_b);
      return 1;
    }
    uint32_t lo, hi;
    rb.interval(b, lo, hi);
    const uint32_t k0 = g << 16, k1 = k0 | 0xFFFFu;
    if (k0 < lo || k1 > hi) {
      std::printf("FAIL relbins %s (gb %u shift %u): keys %08x-%08x outside bin %u [%08x, %08x]\n", what, rb.gb,
                  rb.shift, k0, k1, b, lo, hi);
      return 1;
    }
    if (g == 0 || b != prev_b) {  // a new reached bin: it starts where the last one ended
      if (lo != next_lo) {
        std::printf("FAIL relbins %s (gb %u shift %u): bin %u starts at %08x, want %08x\n", what, rb.gb, rb.shift, b,
                    lo, next_lo);
        return 1;
      }
      next_lo = hi + 1u;
      if (float_of_key(k0) == float_of_key(k0) && rb.bin(float_of_key(k0)) != b && misa::float_key(float_of_key(k0)) == k0) {
        std::printf("FAIL relbins %s: bin(v) != bin_of_coarse\n", what);
        return 1;
      }
    }
    prev_b = b;
  }
  if (next_lo != 0u) {  // the last reached bin ends at the largest key (hi + 1 wraps to 0)
    std::printf("FAIL relbins %s (gb %u shift %u): the bins stop short of the largest key\n", what, rb.gb, rb.shift);
    return 1;
  }
  return 0;
}

int check_relbins() {
  int n = 0;
  const float taus[] = {1e-30f, 1e-9f, 0.001f, 0.37f, 1.0f, 3.5f, 1000.0f, 3e9f, 1e30f, 0.0f, -0.0f, -1.0f, -1e20f};
  for (float t : taus) {
    if (check_relbins_one(misa::RelBins::above(t), "above")) return 1;
    ++n;
  }
  const uint32_t gs[] = {0u, 0x007Fu, 0x3F80u, 0x8000u, 0xA000u, misa::kCoarseFloor - 1, misa::kCoarseFloor,
                         misa::kCoarseFloor + 1, 0xBF00u, 0xBF80u, 0xC000u, 0xC120u, 0xF000u, 0xFF7Fu, 0xFFFFu};
  for (uint32_t a : gs)
    for (uint32_t b : gs) {
      if (a > b) continue;
      if (check_relbins_one(misa::RelBins::range(a, b), "range")) return 1;
      ++n;
    }
  for (uint32_t w = 1; w <= 0xFFFFu; w = w * 3 + 1) {  // spans around every shift
    const uint32_t a = misa::kCoarseFloor, b = a + w > 0xFFFFu ? 0xFFFFu : a + w;
    if (check_relbins_one(misa::RelBins::range(a, b), "span")) return 1;
    ++n;
  }
  std::printf("ok relbins (%d bin sets)\n", n);
  return 0;
}

int check_certificate() {
  const float inf = INFINITY;
  struct Case {
    bool overflow;
    int total, k;
    float tau_max;
    CandVerdict want;
  } cases[] = {
      {false, 100, 100, 0.5f, CandVerdict::kCount},     // exactly k, finite tau: must count
      {false, 100, 100, -inf, CandVerdict::kTakeAll},   // exactly k, nothing filtered
      {false, 60, 100, -inf, CandVerdict::kTakeAll},    // short prefix, nothing filtered
      {false, 99, 100, 0.5f, CandVerdict::kRepair},     // fewer than k after filtering
      {false, 99, 100, -1e30f, CandVerdict::kRepair},   // a finite (very low) tau still filters
      {false, 150, 100, 0.5f, CandVerdict::kCount},
      {false, 150, 100, -inf, CandVerdict::kCount},     // more than k, all kept: select
      {true, 150, 100, 0.5f, CandVerdict::kRepair},     // a segment overflowed
      {true, 50, 100, -inf, CandVerdict::kRepair},
  };
  for (const Case& c : cases) {
    const CandVerdict got = misa::cand_verdict(c.overflow, c.total, c.k, c.tau_max);
    if (got != c.want) {
      std::printf("FAIL cand_verdict(overflow=%d, total=%d, k=%d, tau_max=%g) = %d, want %d\n",
                  c.overflow, c.total, c.k, static_cast<double>(c.tau_max), static_cast<int>(got),
                  static_cast<int>(c.want));
      return 1;
    }
  }
  std::printf("ok certificate\n");
  return 0;
}

}  // namespace

int main(int argc, char** argv) {
  const char* what = argc > 1 ? argv[1] : "all";
  int rc = 0;
  if (!std::strcmp(what, "all") || !std::strcmp(what, "certificate")) rc |= check_certificate();
  if (!std::strcmp(what, "all") || !std::strcmp(what, "digits")) rc |= check_digits();
  if (!std::strcmp(what, "all") || !std::strcmp(what, "relbins")) rc |= check_relbins();
  return rc;
}
