// CPU oracle for the MISA indexer -- TEST INFRASTRUCTURE ONLY.
//
// Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
// load this library.  The GPU library never links it and it never links the GPU
// library; the two share no code, headers or tables.
//
// Source: "MISA: Mixture of Indexer Sparse Attention for Long-Context LLM
// Inference" (summary page, picx.dev), sections "Introduction and Theoretical
// Foundation" (Eq. 1, Eq. 2) and "Methodology" 1 (Eq. 4, 7, 8, 9, 10) and
// 2 (MISA-dagger, Eq. 11, 12).
//
// Everything is the plain definition, written out: inputs are decoded exactly
// into double, every sum runs in double in index order, every top-k is a full
// sort.  No blocking, fusion or reordering.  Readings taken where the page is
// silent (causal prefix, partial last block, tie order, -1 padding) are listed
// next to the function that takes them.
//
// Build: g++ -O2 -ffp-contract=off -fno-fast-math -shared -fPIC.
// (-ffp-contract=off keeps a*b+c as two rounded double operations.)

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <numeric>
#include <vector>

namespace {

// bfloat16: the upper 16 bits of an IEEE binary32.
double bf16_to_double(uint16_t v) {
  uint32_t u = static_cast<uint32_t>(v) << 16;
  float f;
  std::memcpy(&f, &u, sizeof f);
  return static_cast<double>(f);
}

// OCP FP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent (bias 7), 3 mantissa bits,
// no infinities, S.1111.111 is NaN, exponent field 0 is subnormal (m/8 * 2^-6).
double e4m3fn_to_double(uint8_t v) {
  const int sign = (v >> 7) & 1;
  const int ex = (v >> 3) & 0xF;
  const int man = v & 0x7;
  double mag;
  if (ex == 0xF && man == 0x7) {
    mag = NAN;
  } else if (ex == 0) {
    mag = std::ldexp(static_cast<double>(man) / 8.0, -6);
  } else {
    mag = std::ldexp(1.0 + static_cast<double>(man) / 8.0, ex - 7);
  }
  return sign ? -mag : mag;
}

// Dot product of two length-d double vectors, summed in index order.
double dot(const double* a, const double* b, int32_t d) {
  double acc = 0.0;
  for (int32_t i = 0; i < d; ++i) acc += a[i] * b[i];
  return acc;
}

double relu(double x) { return x > 0.0 ? x : 0.0; }

// Sort order of every TopK on the page, with the tie rule this oracle fixes:
// larger value first; among equal values, the smaller index first.
struct ByValueThenIndex {
  const double* v;
  bool operator()(int64_t a, int64_t b) const {
    if (v[a] != v[b]) return v[a] > v[b];
    return a < b;
  }
};

}  // namespace

extern "C" {

// Element types of the raw input buffers.
enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_FP8_E4M3 = 2 };

// Decode a row-major [rows, cols] buffer of `dtype` into double.  When
// `row_scale` is non-null, row r is multiplied by row_scale[r] (the per-token
// fp32 scale of the fp8 inputs: value = code * scale).  The product of a 4-bit
// and a 24-bit significand is exact in double.
void orc_decode(int32_t dtype, const void* src, const float* row_scale, int64_t rows,
                int64_t cols, double* dst) {
  for (int64_t r = 0; r < rows; ++r) {
    const double s = row_scale ? static_cast<double>(row_scale[r]) : 1.0;
    for (int64_t c = 0; c < cols; ++c) {
      const int64_t i = r * cols + c;
      double v;
      if (dtype == ORC_F32) {
        v = static_cast<double>(static_cast<const float*>(src)[i]);
      } else if (dtype == ORC_BF16) {
        v = bf16_to_double(static_cast<const uint16_t*>(src)[i]);
      } else {
        v = e4m3fn_to_double(static_cast<const uint8_t*>(src)[i]);
      }
      dst[i] = row_scale ? v * s : v;
    }
  }
}

// Eq. (4): the prefix of L keys is cut into M = ceil(L/B) blocks
// [bB, min((b+1)B, L)); each block is summarised by one pooled key.
// Reading: Pool is the arithmetic mean over the block's actual members, so a
// partial last block is the mean of the keys it holds.
void orc_pool(const double* K, int64_t L, int32_t d, int32_t B, double* pooled) {
  const int64_t M = (L + B - 1) / B;
  for (int64_t b = 0; b < M; ++b) {
    const int64_t s0 = b * B;
    const int64_t s1 = std::min<int64_t>(s0 + B, L);
    for (int32_t i = 0; i < d; ++i) {
      double acc = 0.0;
      for (int64_t s = s0; s < s1; ++s) acc += K[s * d + i];
      pooled[b * d + i] = acc / static_cast<double>(s1 - s0);
    }
  }
}

// Eq. (7) for one query at absolute position `pos` (its causal prefix is the
// n = pos+1 keys 0..pos):
//   A_{j,b} = w_j * ReLU(q_j . k~_b),   E_j = (1/M_t) * sum_b |A_{j,b}|.
// Reading of the causal router: the query sees the M_t = ceil(n/B) blocks of
// its own prefix.  Blocks lying wholly inside the prefix use the pooled keys
// of Eq. (4) (`pooled`, from orc_pool over the full sequence); when n is not a
// multiple of B the last block is the partial block [floor(n/B)*B, pos] and its
// pooled key is the mean of just those keys.
// q is [H, d] (row j is head j), w is [H].
void orc_expert_scores(const double* K, const double* pooled, int64_t pos, int32_t d, int32_t B,
                       int32_t H, const double* q, const double* w, double* E) {
  const int64_t n = pos + 1;
  const int64_t full = n / B;
  const int64_t Mt = (n + B - 1) / B;
  std::vector<double> partial;
  if (Mt > full) {
    partial.assign(d, 0.0);
    const int64_t s0 = full * B;
    for (int32_t i = 0; i < d; ++i) {
      double acc = 0.0;
      for (int64_t s = s0; s <= pos; ++s) acc += K[s * d + i];
      partial[i] = acc / static_cast<double>(n - s0);
    }
  }
  for (int32_t j = 0; j < H; ++j) {
    double sum = 0.0;
    for (int64_t b = 0; b < Mt; ++b) {
      const double* kb = (b < full) ? pooled + b * d : partial.data();
      const double a = w[j] * relu(dot(q + static_cast<int64_t>(j) * d, kb, d));
      sum += std::fabs(a);
    }
    E[j] = sum / static_cast<double>(Mt);
  }
}

// Block scores of the MISA x HISA combination ("Methodology" 1, "Key
// distinction from HISA"; "Theoretical and Practical Implications",
// "Scalability"): the same affinities A_{j,b} = w_j * ReLU(q_j . k~_b) as in
// Eq. (7), reduced across the heads instead of across the blocks:
//   G_b = sum_{j < H, ascending} A_{j,b},   b < M_t,
// over the same causal blocks as orc_expert_scores (complete blocks pooled by
// Eq. (4), the partial last block pooled over [floor(n/B)*B, pos]).
// Reading: the head reduction is the plain sum of the signed A (the page's
// HISA aggregates the heads' block affinities; |A| belongs to the head
// ranking of Eq. (7)).  G has M_t = ceil((pos+1)/B) entries.
void orc_block_scores(const double* K, const double* pooled, int64_t pos, int32_t d, int32_t B,
                      int32_t H, const double* q, const double* w, double* G) {
  const int64_t n = pos + 1;
  const int64_t full = n / B;
  const int64_t Mt = (n + B - 1) / B;
  std::vector<double> partial;
  if (Mt > full) {
    partial.assign(d, 0.0);
    const int64_t s0 = full * B;
    for (int32_t i = 0; i < d; ++i) {
      double acc = 0.0;
      for (int64_t s = s0; s <= pos; ++s) acc += K[s * d + i];
      partial[i] = acc / static_cast<double>(n - s0);
    }
  }
  for (int64_t b = 0; b < Mt; ++b) {
    const double* kb = (b < full) ? pooled + b * d : partial.data();
    double sum = 0.0;
    for (int32_t j = 0; j < H; ++j) sum += w[j] * relu(dot(q + static_cast<int64_t>(j) * d, kb, d));
    G[b] = sum;
  }
}

// Eq. (8): the h heads with the largest E (ties: the lower head index first),
// written out in ascending head order.
void orc_top_heads(const double* E, int32_t H, int32_t h, int32_t* heads) {
  std::vector<int64_t> order(H);
  std::iota(order.begin(), order.end(), 0);
  std::sort(order.begin(), order.end(), ByValueThenIndex{E});
  std::vector<int32_t> pick(order.begin(), order.begin() + h);
  std::sort(pick.begin(), pick.end());
  std::copy(pick.begin(), pick.end(), heads);
}

// Eq. (9) (and Eq. (1) when `heads` lists every head): for s = 0..pos,
//   I_s = sum_{j in heads, ascending} w_j * ReLU(q_j . k_s).
// Reading: the query's own position is inside its prefix (s <= pos).
void orc_token_scores(const double* K, int64_t pos, int32_t d, const double* q, const double* w,
                      const int32_t* heads, int32_t nh, double* I) {
  for (int64_t s = 0; s <= pos; ++s) {
    double acc = 0.0;
    for (int32_t a = 0; a < nh; ++a) {
      const int32_t j = heads[a];
      acc += w[j] * relu(dot(q + static_cast<int64_t>(j) * d, K + s * d, d));
    }
    I[s] = acc;
  }
}

// Eq. (2) / (10) / (11): the k largest of n scores.  Indices are written in
// rank order (largest first, ties by lower index); when n < k the remaining
// slots are -1.
void orc_topk(const double* I, int64_t n, int32_t k, int32_t* idx) {
  std::vector<int64_t> order(n);
  std::iota(order.begin(), order.end(), 0);
  std::sort(order.begin(), order.end(), ByValueThenIndex{I});
  for (int32_t r = 0; r < k; ++r) idx[r] = (r < n) ? static_cast<int32_t>(order[r]) : -1;
}

// Eq. (12), the fine stage of MISA-dagger: over the candidate tokens
// Omega = cand[0..kp) (entries < 0 are padding and skipped), score each with
// all H heads as in Eq. (1) and keep the k best (same order and padding rule as
// orc_topk).  `scores` receives the Eq. (1) score of each kept token (0 for
// padding).  Ties between equal scores go to the lower token index.
void orc_rerank(const double* K, int32_t d, const double* q, const double* w, int32_t H,
                const int32_t* cand, int32_t kp, int32_t k, int32_t* idx, double* scores) {
  std::vector<int64_t> tok;
  for (int32_t c = 0; c < kp; ++c)
    if (cand[c] >= 0) tok.push_back(cand[c]);
  std::vector<double> val(tok.size());
  for (size_t c = 0; c < tok.size(); ++c) {
    double acc = 0.0;
    for (int32_t j = 0; j < H; ++j)
      acc += w[j] * relu(dot(q + static_cast<int64_t>(j) * d, K + tok[c] * d, d));
    val[c] = acc;
  }
  std::vector<int64_t> order(tok.size());
  std::iota(order.begin(), order.end(), 0);
  std::sort(order.begin(), order.end(), [&](int64_t a, int64_t b) {
    if (val[a] != val[b]) return val[a] > val[b];
    return tok[a] < tok[b];
  });
  for (int32_t r = 0; r < k; ++r) {
    if (static_cast<size_t>(r) < order.size()) {
      idx[r] = static_cast<int32_t>(tok[order[r]]);
      scores[r] = val[order[r]];
    } else {
      idx[r] = -1;
      scores[r] = 0.0;
    }
  }
}

}  // extern "C"
