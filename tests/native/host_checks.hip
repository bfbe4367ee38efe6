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
  return rc;
}
