// Eq. (12) of the MISA summary page ("Methodology" 2, MISA-dagger fine
// stage): every candidate token kept by the routed pass is re-scored with all
// H heads (the Eq. (1) score) and the k best candidates are kept.
//
// bf16 / fp8: the query's H head rows are the A operand of 32x32 MFMA tiles
// (held in registers); 32-candidate column tiles are the B operand.  The key
// rows of a tile are gathered whole-row-coalesced into LDS (buffer-to-LDS
// loads, rerank_lds_kernel); the ReLU * w head sum is taken on the
// accumulators, and the scores go to the workspace.  A sequence whose keys
// exceed a buffer descriptor's 32-bit reach is gathered with flat loads
// straight into B registers instead (rerank_gather_kernel).
// fp32: one thread per candidate (query rows staged in LDS).
// Then one workgroup per query selects the k best of its k' scores in
// registers: a histogram of relative bins in LDS, the threshold bin from a
// block scan, a block-scan compaction, and an exact resolve of that bin.
#include "common.hpp"
#include "launch.hpp"
#include "mfma.hpp"
#include "topk.hpp"

namespace misa {

namespace {

constexpr int kRerankThreads = 256;
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

#ifndef MISA_RERANK_NTW
#define MISA_RERANK_NTW 2
#endif
constexpr int kRRThreads = 256;
constexpr int kRRWaves = kRRThreads / kWave;
constexpr int kMaxKprime = 8192;

// Candidate ids of a query's list: entry i of an explicit list, or of the
// list that m blocks of B tokens spell out (entry i < m B is token
// blocks[i / B] * B + i % B, -1 for a padding block; entries past m B are
// -1).  Out-of-prefix ids are masked by the callers.
struct ListIds {
  static constexpr bool kBlocks = false;
  const int32_t* p;
  __device__ __forceinline__ int32_t operator()(int64_t i) const { return p[i]; }
};
struct BlockIds {
  static constexpr bool kBlocks = true;
  const int32_t* blk;  // the query's m blocks
  int32_t B, nb;       // block size, m B
  float invB;          // 1 / B (the quotient is corrected below)
  int32_t lgB;         // log2 B when B is a power of two, else -1
  __device__ __forceinline__ BlockIds(const int32_t* blk_, int32_t B_, int32_t m)
      : blk(blk_), B(B_), nb(m * B_), invB(1.f / static_cast<float>(B_)),
        lgB((B_ & (B_ - 1)) == 0 ? 31 - __clz(B_) : -1) {}
  // Entry i as (block slot, offset in the block); slot -1 past m B.
  __device__ __forceinline__ void split(int32_t i, int32_t& qb, int32_t& rem) const {
    if (i >= nb) {
      qb = -1;
      rem = 0;
    } else if (lgB >= 0) {
      qb = i >> lgB;
      rem = i & (B - 1);
    } else {
      qb = static_cast<int32_t>(static_cast<float>(i) * invB);
      rem = i - qb * B;
      if (rem < 0) {
        --qb;
        rem += B;
      } else if (rem >= B) {
        ++qb;
        rem -= B;
      }
    }
  }
  // The loaded block of a slot (-1 for slot -1) and an offset -> token id.
  __device__ __forceinline__ int32_t block_of(int32_t qb) const { return qb < 0 ? -1 : blk[qb]; }
  __device__ __forceinline__ int32_t token(int32_t b, int32_t rem) const { return b < 0 ? -1 : b * B + rem; }
  __device__ __forceinline__ int32_t operator()(int64_t i) const {
    int32_t qb, rem;
    split(static_cast<int32_t>(i), qb, rem);
    return token(block_of(qb), rem);
  }
};

// Per-wave state: the query's head rows (A) and per-lane row weights.  NI:
// accumulator values per lane and row tile that can hold a listed head (16;
// 8 or 4 when at most 16 or 8 heads are scored: the lane's rows
// 8 (i / 4) + 4 hf + i % 4 past them are zero).
template <int DT, int RT, int NI = 16>
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

  // This lane's half of a key row (krow always a valid row; the caller
  // masks invalid candidates).
  struct KeyB {
    uint4 b[DT == kBF16 ? 8 : 4];
  };
  __device__ __forceinline__ static KeyB load(const void* krow) {
    const int hf = lane_id() >> 5;
    KeyB kb;
    if constexpr (DT == kBF16) {
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(krow) + 64 * hf);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) kb.b[ks] = src[ks];
    } else {
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(krow) + 64 * hf);
#pragma unroll
      for (int u = 0; u < 4; ++u) kb.b[u] = src[u];
    }
    return kb;
  }

  // Score of this lane's column candidate from its loaded key half.
  __device__ __forceinline__ float compute(const KeyB& kb) const {
    f32x16 acc[RT];
    if constexpr (DT == kBF16) {
      const uint4* b = kb.b;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          acc[rt] = mfma32_bf16(a16[rt][ks], as_bf16x8(b[ks]), ks == 0 ? f32x16{} : acc[rt]);
    } else {
      const uint4* b = kb.b;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const i32x8 bb{(int)b[2 * ks].x, (int)b[2 * ks].y, (int)b[2 * ks].z, (int)b[2 * ks].w,
                       (int)b[2 * ks + 1].x, (int)b[2 * ks + 1].y, (int)b[2 * ks + 1].z, (int)b[2 * ks + 1].w};
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[rt] = mfma32_fp8(a8[rt][ks], bb, ks == 0 ? f32x16{} : acc[rt]);
      }
    }
    static_assert(NI == 16 || (RT == 1 && (NI == 8 || NI == 4)), "narrow head sums: one row tile");
    float part = 0.f;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < NI; ++i) part += wl[rt][i] * relu(acc[rt][i]);
    return part + __shfl_xor(part, 32, kWave);  // rows 4hf..: the other half-wave
  }

  __device__ __forceinline__ float score(const void* krow) const { return compute(load(krow)); }
};

template <int DT>
__device__ __forceinline__ const void* key_row(const void* k, int64_t row) {
  if constexpr (DT == kBF16) return static_cast<const uint16_t*>(k) + row * kD;
  else return static_cast<const uint8_t*>(k) + row * kD;
}

// Workgroup (chunk, row): wave w scores NTW tiles of 32 candidates, issuing
// every tile's key gathers (and fp8 key scales) before the first MFMA.
template <int DT, int RT, int NTW>
__global__ __launch_bounds__(kRRThreads) void rerank_gather_kernel(
    const void* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    const void* __restrict__ k, const float* __restrict__ k_scale,
    const int32_t* __restrict__ cand, int32_t kprime, int32_t L, int32_t T, int32_t H,
    float* __restrict__ out) {
  const int64_t seq = blockIdx.z;
  const int64_t r = seq * T + blockIdx.y;
  const int64_t pos = static_cast<int64_t>(L) - T + blockIdx.y;
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int cbase = (blockIdx.x * kRRWaves + wave) * 32 * NTW + (lane & 31);
  typename CandScorer<DT, RT>::KeyB kb[NTW];
  bool okv[NTW];
  float skv[NTW];
#pragma unroll
  for (int u = 0; u < NTW; ++u) {
    const int c = cbase + 32 * u;
    const int32_t s = c < kprime ? cand[r * kprime + c] : -1;
    okv[u] = s >= 0 && s <= pos;
    const int64_t row = seq * L + (okv[u] ? s : 0);
    kb[u] = CandScorer<DT, RT>::load(key_row<DT>(k, row));
    skv[u] = (DT == kFP8) ? k_scale[row] : 1.f;
  }
  CandScorer<DT, RT> cs;
  cs.init(q, q_scale, w, r, H);
#pragma unroll
  for (int u = 0; u < NTW; ++u) {
    const int c = cbase + 32 * u;
    const float v = cs.compute(kb[u]) * skv[u];
    if (lane < 32 && c < kprime) out[r * kprime + c] = okv[u] ? v : -__builtin_inff();
  }
}

// Top-k of one query's k' (score, candidate) list, in one workgroup: the
// list is read once into registers, a histogram of relative bins (LDS) gives
// the threshold bin b*; each wave's entries above b* take one run of the
// output after those of the lower waves (slot by slot, wave ballots, so
// the stores coalesce) and those at b* go to an LDS list, which is resolved
// exactly.  Invalid candidates carry score -inf and a distinct negative id
// (so ties among them resolve), written out as -1.
// 1024 threads per query when there are few queries (each workgroup's
// latency is the time), 256 when there are many: 32 entries per thread in at
// most 128 registers, so four workgroups share a CU and overlap one
// another's load and barrier latency (C5: 277 -> 242 us against 512
// threads, three per CU).
constexpr int kLSCap = 2048;
constexpr int kLSBins = 2048;  // relative bins
constexpr int kLSBlk = 512;    // block candidates: blocks staged in LDS (m B <= 8192, B >= 16)

template <int kLSThreads>
struct LSelSmem {
  uint32_t hist[kLSBins];
  alignas(16) float cand_score[kLSCap];
  alignas(16) int32_t cand_idx[kLSCap];
  union {
    ResolveSmem rs;
    TopkSmem base;
  };
  int scan_tmp[32];
  int32_t blk[kLSBlk];
  int wtot[kLSThreads / kWave];
  int digit, above, count;
  uint32_t dmin, dmax;
};

// The k best of one query's list: srow/crow its k' scores and candidates,
// pos the query's position (candidates outside [0, pos] are invalid), out /
// out_s its k output slots.  All kLSThreads threads of the workgroup call.
template <int kLSThreads, bool CACHE, class Ids>
__device__ __forceinline__ void list_select_row(const float* __restrict__ srow, const Ids crow,
                                                int32_t kprime, int64_t pos, int32_t k,
                                                int32_t* __restrict__ out, float* __restrict__ out_s,
                                                LSelSmem<kLSThreads>& sm) {
  constexpr int kLSPer = kMaxKprime / kLSThreads;  // list entries per thread (bits of a 32-bit mask)
  static_assert(kLSPer <= 32, "entry slots are bits of a 32-bit mask");
  for (int b = threadIdx.x; b < kLSBins; b += kLSThreads) sm.hist[b] = 0;
  if (threadIdx.x == 0) {
    sm.dmin = 0xFFFFFFFFu;
    sm.dmax = 0u;
  }
  // Block candidates: the ids are formed only for the entries written out,
  // from the query's blocks staged in LDS (held ids would cost 32 registers
  // per thread).  Their invalid entries (padding, outside the prefix) carry
  // score -inf from the scoring pass, and a valid one never does (a finite
  // sum), so the score tells them apart.
  constexpr bool kBlk = Ids::kBlocks;
  float v[kLSPer];
  int32_t id[kBlk ? 1 : kLSPer];
  bool blk_lds = false;
  if constexpr (kBlk) {
    const int32_t m = crow.nb / crow.B;
    blk_lds = m <= kLSBlk;
    if (blk_lds)
      for (int i = threadIdx.x; i < m; i += kLSThreads) sm.blk[i] = crow.blk[i];
    // (published by the barrier after the coarse-key range below)
  }
#pragma unroll
  for (int j = 0; j < kLSPer; ++j) {
    const int i = j * kLSThreads + threadIdx.x;
    const int ic = min(i, kprime - 1);
    const float x = srow[ic];
    if constexpr (kBlk) {
      v[j] = x;
    } else {
      const int32_t c = crow(ic);
      const bool ok = c >= 0 && c <= pos;
      v[j] = ok ? x : -__builtin_inff();
      id[j] = ok ? c : -1 - i;
    }
  }
  auto id_of = [&](int j) -> int32_t {
    if constexpr (kBlk) {
      const int i = j * kLSThreads + threadIdx.x;
      if (v[j] == -__builtin_inff()) return -1 - i;
      int32_t qb, rem;
      crow.split(i, qb, rem);
      return crow.token(blk_lds ? sm.blk[qb] : crow.blk[qb], rem);
    } else {
      return id[j];
    }
  };
  // Relative bins (RelBins) over the list's coarse-key range [gmin, gmax].
  // CACHE: each entry's coarse key is computed once and kept, two 16-bit
  // keys per register (where the registers allow); the histogram and the
  // classification below then work on it (an entry lies above / in the
  // threshold bin exactly when its coarse key does).
  uint32_t dgp[CACHE ? (kLSPer + 1) / 2 : 1];
  if constexpr (CACHE) {
#pragma unroll
    for (int j = 0; j < kLSPer; j += 2) {
      const uint32_t g0j = float_key(v[j]) >> 16;
      const uint32_t g1j = j + 1 < kLSPer ? float_key(v[j + 1]) >> 16 : 0u;
      dgp[j / 2] = g0j | (g1j << 16);
    }
  }
  auto coarse_of = [&](int j) -> uint32_t {
    if constexpr (CACHE) return (dgp[j / 2] >> (16 * (j & 1))) & 0xFFFFu;
    else return float_key(v[j]) >> 16;
  };
  {
    uint32_t dmin = 0xFFFFFFFFu, dmax = 0u;
#pragma unroll
    for (int j = 0; j < kLSPer; ++j)
      if (j * kLSThreads + static_cast<int>(threadIdx.x) < kprime) {
        const uint32_t g = coarse_of(j);
        dmin = min(dmin, g);
        dmax = max(dmax, g);
      }
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) {
      dmin = min(dmin, static_cast<uint32_t>(__shfl_xor(static_cast<int>(dmin), o, kWave)));
      dmax = max(dmax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(dmax), o, kWave)));
    }
    if ((threadIdx.x & (kWave - 1)) == 0) {
      atomicMin(&sm.dmin, dmin);
      atomicMax(&sm.dmax, dmax);
    }
  }
  __syncthreads();
  const RelBins rb = RelBins::range(sm.dmin, sm.dmax);  // kprime >= 1 entries
  static_assert(kLSBins == kRelBinCount, "list bins are relative bins");
  auto rel_of = [&](int j) -> uint32_t { return rb.bin_of_coarse(coarse_of(j)); };
#pragma unroll
  for (int j = 0; j < kLSPer; ++j)
    if (j * kLSThreads + static_cast<int>(threadIdx.x) < kprime) atomicAdd(&sm.hist[rel_of(j)], 1u);
  __syncthreads();
  {
    constexpr int BPT = kLSBins / kLSThreads;
    int local[BPT];
    int lsum = 0;
#pragma unroll
    for (int u = 0; u < BPT; ++u) {
      local[u] = static_cast<int>(sm.hist[kLSBins - 1 - (threadIdx.x * BPT + u)]);
      lsum += local[u];
    }
    int tot;
    int run = block_exclusive_sum<kLSThreads>(lsum, sm.scan_tmp, tot);
#pragma unroll
    for (int u = 0; u < BPT; ++u) {
      if (run < k && run + local[u] >= k) {
        sm.digit = kLSBins - 1 - (threadIdx.x * BPT + u);
        sm.above = run;
        sm.count = local[u];
      }
      run += local[u];
    }
    __syncthreads();
  }
  const uint32_t bstar = static_cast<uint32_t>(sm.digit);
  const int above = sm.above;
  const int bcount = sm.count;
  if (bcount > kLSCap) {
    // Exact fallback over the whole list (e.g. fewer than k valid candidates
    // with thousands of -inf ties).
    block_topk<kLSThreads>(
        kprime, k, [](int64_t) { return true; },
        [=](int64_t i) { const int32_t c = crow(i); return float_key(c >= 0 && c <= pos ? srow[i] : -__builtin_inff()); },
        [=](int64_t i) { const int32_t c = crow(i); return c >= 0 && c <= pos ? c : static_cast<int32_t>(-1 - i); },
        [=](int64_t i) { const int32_t c = crow(i); return c >= 0 && c <= pos ? srow[i] : -__builtin_inff(); },
        out, out_s, sm.base);
    __syncthreads();
    for (int p = threadIdx.x; p < k; p += kLSThreads)
      if (out[p] < 0) out[p] = -1;
  } else {
    // Above / in the relative bin b*: by the cached coarse keys, or by the
    // key interval of b*.
    uint32_t mh = 0, ma = 0;
    if constexpr (CACHE) {
#pragma unroll
      for (int j = 0; j < kLSPer; ++j) {
        const bool in = j * kLSThreads + static_cast<int>(threadIdx.x) < kprime;
        const uint32_t rb = rel_of(j);
        mh |= (in && rb > bstar) ? (1u << j) : 0u;
        ma |= (in && rb == bstar) ? (1u << j) : 0u;
      }
    } else {
      uint32_t lo, hi;
      rb.interval(bstar, lo, hi);
#pragma unroll
      for (int j = 0; j < kLSPer; ++j) {
        const bool in = j * kLSThreads + static_cast<int>(threadIdx.x) < kprime;
        const uint32_t key = float_key(v[j]);
        mh |= (in && key > hi) ? (1u << j) : 0u;
        ma |= (in && key >= lo && key <= hi) ? (1u << j) : 0u;
      }
    }
    // Per-wave packed counts (above-b* low 16 bits: < k <= 8192; at-b*
    // high), then each wave's runs.
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    int wt = __popc(mh) | (__popc(ma) << 16);
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) wt += __shfl_xor(wt, o, kWave);
    if (lane == 0) sm.wtot[wave] = wt;
    __syncthreads();
    int wb = 0;
#pragma unroll
    for (int w = 0; w < kLSThreads / kWave; ++w) wb += w < wave ? sm.wtot[w] : 0;
    int ph = wb & 0xFFFF;
    int pa = wb >> 16;
#pragma unroll
    for (int j = 0; j < kLSPer; ++j) {
      const bool h = (mh >> j) & 1u;
      const bool at = (ma >> j) & 1u;
      const uint64_t bh = __ballot(h);
      const uint64_t ba = __ballot(at);
      if (h) {
        const int pos = ph + lanes_below(bh);
        if (pos < k) {
          out[pos] = id_of(j);  // above b*: a valid candidate
          if (out_s) out_s[pos] = v[j];
        }
      } else if (at) {
        const int pos = pa + lanes_below(ba);
        if (pos < kLSCap) {
          sm.cand_score[pos] = v[j];
          sm.cand_idx[pos] = id_of(j);
        }
      }
      ph += __popcll(bh);
      pa += __popcll(ba);
    }
    __syncthreads();
    if (!resolve_list<kLSThreads>(sm.cand_score, sm.cand_idx, bcount, k - above, out + above,
                                  out_s ? out_s + above : nullptr, sm.rs)) {
      __syncthreads();
      const float* cs = sm.cand_score;
      const int32_t* ci = sm.cand_idx;
      block_topk<kLSThreads>(
          bcount, k - above, [](int64_t) { return true; }, [=](int64_t j) { return float_key(cs[j]); },
          [=](int64_t j) { return ci[j]; }, [=](int64_t j) { return cs[j]; }, out + above,
          out_s ? out_s + above : nullptr, sm.base);
      __syncthreads();
      for (int p = above + threadIdx.x; p < k; p += kLSThreads)
        if (out[p] < 0) out[p] = -1;
    }
  }
}

// BLK: `cand` holds each query's m blocks of B tokens (BlockIds), else its
// explicit list.
template <int kLSThreads, bool BLK>
__global__ __launch_bounds__(kLSThreads, kLSThreads == 256 ? 4 : 1) void list_select_kernel(
    const float* __restrict__ sc, const int32_t* __restrict__ cand, int32_t kprime, int32_t L,
    int32_t T, int32_t k, int32_t* __restrict__ idx, float* __restrict__ scores_out, int32_t m,
    int32_t B) {
  __shared__ LSelSmem<kLSThreads> sm;
  const int64_t r = static_cast<int64_t>(blockIdx.y) * T + blockIdx.x;
  const int64_t pos = static_cast<int64_t>(L) - T + blockIdx.x;
  float* so = scores_out ? scores_out + r * k : nullptr;
  // 256 threads (32 entries each, four workgroups per CU): no room to keep
  // the coarse keys.
  constexpr bool kCache = kLSThreads != 256;
  if constexpr (BLK)
    list_select_row<kLSThreads, kCache>(sc + r * kprime, BlockIds(cand + r * m, B, m), kprime, pos,
                                        k, idx + r * k, so, sm);
  else
    list_select_row<kLSThreads, kCache>(sc + r * kprime, ListIds{cand + r * kprime}, kprime, pos, k,
                                        idx + r * k, so, sm);
}

// Gathers through LDS: a lane-per-candidate gather (lane l reads 16 bytes of
// candidate l%32's row per instruction) touches 32 rows per instruction and
// is limited by the address unit, not by memory.  Here each load instruction
// instead covers whole rows -- 64 lanes = RPI rows of CPR 16-byte chunks --
// and lands directly in LDS (buffer-to-LDS loads); the MFMA B operands are
// then read from LDS.  Chunk c of tile row j sits at chunk position
// c ^ (j % CPR), so the B reads (32 rows, one chunk each) hit distinct banks.
// Workgroup (chunk, row): the query's head rows are staged once in LDS; wave
// w scores NTW tiles of 32 candidates per round, all of a round's loads in
// flight before its first MFMA, and its tiles are private (no barrier).

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rr_rsrc(const void* base, int32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ void rr_load16_lds(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void rr_vmcnt0() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <int DT, int NTW>
struct RerankScoreSmem {
  static constexpr int ROWB = kD * (DT == kBF16 ? 2 : 1);
  alignas(16) uint8_t keys[kRRWaves][NTW][32 * ROWB];
  alignas(16) uint8_t qst[kMaxHeads * ROWB];
  float wst[kMaxHeads];
};

// FUSED (one workgroup per query, per_wg >= kprime): after scoring, the same
// workgroup selects the query's k best from its scores (re-read from L2; the
// score phase's LDS is reused) and writes idx / scores_out, so no list-select
// launch follows and the scores never make the round trip to HBM.
// BLK: the candidates are the tokens of m blocks per query (`cand` holds the
// blocks, [rows, m], of B tokens; entries past m B are padding), else an
// explicit list.  NI as for CandScorer.
template <int DT, int RT, int NTW, bool FUSED, bool BLK, int NI>
__global__ __launch_bounds__(kRRThreads) void rerank_lds_kernel(
    const void* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    const void* __restrict__ k, const float* __restrict__ k_scale,
    const int32_t* __restrict__ cand, int32_t kprime, int32_t L, int32_t T, int32_t H,
    int32_t per_wg, float* __restrict__ out, int32_t k_top, int32_t* __restrict__ idx,
    float* __restrict__ scores_out, const int32_t* __restrict__ heads, int32_t nh, int32_t m,
    int32_t B) {
  constexpr int ROWB = kD * (DT == kBF16 ? 2 : 1);  // key row bytes
  constexpr int CPR = ROWB / 16;                     // 16-byte chunks per row
  constexpr int RPI = kWave / CPR;                   // rows per load instruction
  __shared__ union Smem {
    RerankScoreSmem<DT, NTW> score;
    LSelSmem<kRRThreads> sel;
  } smem;
  auto& keys = smem.score.keys;
  uint8_t* qst = smem.score.qst;
  float* wst = smem.score.wst;
  const int64_t seq = blockIdx.z;
  const int64_t r = seq * T + blockIdx.y;
  const int64_t pos = static_cast<int64_t>(L) - T + blockIdx.y;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = lane_id();
  const int hf = lane >> 5;
  const int col = lane & 31;

  // Query head rows and weights -> LDS: row a is head a (every head), or
  // the a-th listed head (heads != nullptr: nh of them; ids outside [0, H)
  // contribute nothing).
  const uint8_t* qrow = static_cast<const uint8_t*>(q) + r * H * ROWB;
  auto head_of = [&](int a) -> int {
    const int j = heads ? (a < nh ? heads[r * nh + a] : -1) : (a < H ? a : -1);
    return (j >= 0 && j < H) ? j : -1;
  };
  for (int i = threadIdx.x; i < kMaxHeads * CPR; i += kRRThreads) {
    const int j = head_of(i / CPR);
    reinterpret_cast<uint4*>(qst)[i] =
        j >= 0 ? reinterpret_cast<const uint4*>(qrow + j * ROWB)[i % CPR] : make_uint4(0, 0, 0, 0);
  }
  const float sq = (DT == kFP8) ? q_scale[r] : 1.f;
  if (threadIdx.x < kMaxHeads) {
    const int j = head_of(threadIdx.x);
    wst[threadIdx.x] = j >= 0 ? w[r * H + j] * sq : 0.f;
  }
  __syncthreads();
  CandScorer<DT, RT, NI> cs;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int j = rt * 32 + col;
    const uint8_t* src = qst + j * ROWB;
    if constexpr (DT == kBF16) {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) cs.a16[rt][ks] = as_bf16x8(reinterpret_cast<const uint4*>(src + 128 * hf)[ks]);
    } else {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const uint4 lo = reinterpret_cast<const uint4*>(src + 64 * hf)[2 * ks];
        const uint4 hi = reinterpret_cast<const uint4*>(src + 64 * hf)[2 * ks + 1];
        cs.a8[rt][ks] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) cs.wl[rt][i] = wst[rt * 32 + 8 * (i / 4) + 4 * hf + (i % 4)];
  }

  const __amdgpu_buffer_rsrc_t rk =
      rr_rsrc(static_cast<const uint8_t*>(k) + seq * static_cast<int64_t>(L) * ROWB, L * ROWB);
  const auto crow = [&]() {
    if constexpr (BLK) return BlockIds(cand + r * m, B, m);
    else return ListIds{cand + r * kprime};
  }();
  float* orow = out + r * kprime;
  const int c_wg = blockIdx.x * per_wg;
  const int c_end = min(c_wg + per_wg, kprime);
  constexpr int kRoundStep = kRRWaves * NTW * 32;
  // This lane's candidate of each tile of a round (lanes l and l+32 share
  // one).  The next round's are loaded while this round's rows are gathered
  // (block candidates: the block is loaded then, and the token id formed
  // when the round starts, so nothing waits for the load before that).
  int32_t svn[NTW], svr[NTW];
  auto load_ids = [&](int c_round) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NTW; ++u) {
      const int c = c_round + 32 * u + col;
      if constexpr (BLK) {
        int32_t qb;
        crow.split(c < c_end ? c : crow.nb, qb, svr[u]);
        svn[u] = crow.block_of(qb);
      } else {
        svn[u] = c < c_end ? crow(c) : -1;
      }
    }
  };
  if (c_wg + wave * NTW * 32 < c_end) load_ids(c_wg + wave * NTW * 32);
  for (int c_round = c_wg + wave * NTW * 32; c_round < c_end; c_round += kRoundStep) {
    int32_t sid[NTW];
    float skv[NTW];
#pragma unroll
    for (int u = 0; u < NTW; ++u) {
      int32_t id = svn[u];
      if constexpr (BLK) id = crow.token(id, svr[u]);
      sid[u] = (id >= 0 && id <= pos) ? id : -1;
    }
    if (c_round + kRoundStep < c_end) load_ids(c_round + kRoundStep);
    // The tiles' key scales, and their rows into this wave's LDS slots.
#pragma unroll
    for (int u = 0; u < NTW; ++u) skv[u] = (DT == kFP8 && sid[u] >= 0) ? k_scale[seq * L + sid[u]] : 1.f;
#pragma unroll
    for (int u = 0; u < NTW; ++u) {
#pragma unroll
      for (int i = 0; i < 32 / RPI; ++i) {
        const int j = i * RPI + lane / CPR;        // tile row of this lane's chunk
        const int pc = lane % CPR;                 // its chunk position in LDS
        const int lc = pc ^ (j % CPR);             // the row chunk stored there
        const int32_t sj = __shfl(sid[u], j, kWave);
        const uint32_t voff = static_cast<uint32_t>(sj < 0 ? 0 : sj) * ROWB + 16u * lc;
        rr_load16_lds(rk, &keys[wave][u][i * 1024], voff);
      }
    }
    rr_vmcnt0();  // this wave's rows have landed (its LDS slots are private)
#pragma unroll
    for (int u = 0; u < NTW; ++u) {
      typename CandScorer<DT, RT, NI>::KeyB kb;
      const uint8_t* trow = &keys[wave][u][col * ROWB];
      if constexpr (DT == kBF16) {
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) kb.b[ks] = reinterpret_cast<const uint4*>(trow)[(8 * hf + ks) ^ (col % CPR)];
      } else {
#pragma unroll
        for (int uu = 0; uu < 4; ++uu) kb.b[uu] = reinterpret_cast<const uint4*>(trow)[(4 * hf + uu) ^ (col % CPR)];
      }
      const float v = cs.compute(kb) * skv[u];
      const int c = c_round + 32 * u + col;
      if (lane < 32 && c < c_end) orow[c] = sid[u] >= 0 ? v : -__builtin_inff();
    }
    // The next round's loads overwrite these slots: reads must be done.
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  }
  if constexpr (FUSED) {
    __syncthreads();  // every score is written; the score phase's LDS is free
    list_select_row<kRRThreads, true>(orow, crow, kprime, pos, k_top, idx + r * k_top,
                                scores_out ? scores_out + r * k_top : nullptr, smem.sel);
  }
}

}  // namespace

size_t rerank_ws_bytes(const Shape& s, int32_t kprime) {
  return align_up(static_cast<size_t>(s.batch) * s.T * kprime * sizeof(float));
}

hipError_t launch_rerank(const Shape& s, int32_t kprime, int32_t k, const void* q,
                         const float* q_scale, const float* w, const void* kk, const float* k_scale,
                         const int32_t* cand, int32_t* idx, float* scores_out, void* ws,
                         hipStream_t st) {
  return launch_rerank_heads(s, kprime, k, q, q_scale, w, kk, k_scale, cand, 0, nullptr, s.H, idx,
                             scores_out, ws, st);
}

hipError_t launch_rerank_heads(const Shape& s, int32_t kprime, int32_t k, const void* q,
                               const float* q_scale, const float* w, const void* kk,
                               const float* k_scale, const int32_t* cand, int32_t m,
                               const int32_t* heads, int32_t nh, int32_t* idx, float* scores_out,
                               void* ws, hipStream_t st) {
  const int64_t rows = static_cast<int64_t>(s.batch) * s.T;
  float* sc = static_cast<float*>(ws);
  bool fused = false;  // the score kernel also took each query's top-k
  const int64_t seq_bytes_all = static_cast<int64_t>(s.L) * kD * (s.dtype == kBF16 ? 2 : 1);
  if ((heads || m > 0) && (s.dtype == kF32 || seq_bytes_all >= (int64_t{1} << 31)))
    return hipErrorInvalidValue;  // head lists and block candidates: the LDS-gather kernel only
  if (m > 0 && (!heads || nh > 16)) return hipErrorInvalidValue;
  if (s.dtype != kF32) {
    const bool two = (heads ? nh : s.H) > 32;
    // Two tiles of 32 candidates in flight per wave (fp8: 64 B per lane
    // each, bf16: 128 B).  Rounds per wave: as many as keep at least eight
    // workgroups per CU, up to 32, so the query rows staged into LDS once
    // per workgroup are reused over many candidate tiles on long prefill
    // lists, while a short decode batch still spreads over the chip.
    constexpr int kNtw = MISA_RERANK_NTW;
    // bf16 block candidates (MISA x HISA): one tile per round, so two
    // workgroups fit a CU's LDS (their few heads leave the gathers exposed).
    const int ntw = (m > 0 && s.dtype == kBF16) ? 1 : kNtw;
    int rounds = 32 * kNtw / ntw;
    while (rounds > 1) {
      const int64_t per = static_cast<int64_t>(kRRWaves) * 32 * ntw * rounds;
      if (rows * ((kprime + per - 1) / per) >= 2048) break;
      rounds >>= 1;
    }
    const int per_wg = kRRWaves * 32 * ntw * rounds;
    const int64_t seq_bytes = static_cast<int64_t>(s.L) * kD * (s.dtype == kBF16 ? 2 : 1);
    if (seq_bytes < (int64_t{1} << 31)) {
      dim3 g((kprime + per_wg - 1) / per_wg, s.T, s.batch);
      fused = per_wg >= kprime;
#define RG(DT, RT, NTW, F, BLK, NI) rerank_lds_kernel<DT, RT, NTW, F, BLK, NI><<<g, kRRThreads, 0, st>>>(q, q_scale, w, kk, k_scale, cand, kprime, s.L, s.T, s.H, per_wg, sc, k, idx, scores_out, heads, nh, m, s.B)
#define RGF(DT, RT) if (fused) RG(DT, RT, kNtw, true, false, 16); else RG(DT, RT, kNtw, false, false, 16);
#define RGB(DT, NI) if (fused) RG(DT, 1, kNtw, true, true, NI); else RG(DT, 1, kNtw, false, true, NI);
#define RGB1(DT, NI) if (fused) RG(DT, 1, 1, true, true, NI); else RG(DT, 1, 1, false, true, NI);
      if (m > 0) {
        // Block candidates with at most 16 routed heads: one row tile.
        if (s.dtype == kBF16) { if (nh <= 8) { RGB1(kBF16, 4) } else { RGB1(kBF16, 8) } }
        else { if (nh <= 8) { RGB(kFP8, 4) } else { RGB(kFP8, 8) } }
      } else if (s.dtype == kBF16) { if (two) { RGF(kBF16, 2) } else { RGF(kBF16, 1) } }
      else { if (two) { RGF(kFP8, 2) } else { RGF(kFP8, 1) } }
#undef RGB1
#undef RGB
#undef RGF
#undef RG
    } else {
      // A sequence's keys beyond the 32-bit reach of a buffer descriptor:
      // gather with flat addresses instead.
      constexpr int kNtwF8 = 4, kNtwB16 = 2;
      const int per = kRRWaves * 32 * (s.dtype == kBF16 ? kNtwB16 : kNtwF8);
      dim3 g((kprime + per - 1) / per, s.T, s.batch);
#define RG(DT, RT, NTW) rerank_gather_kernel<DT, RT, NTW><<<g, kRRThreads, 0, st>>>(q, q_scale, w, kk, k_scale, cand, kprime, s.L, s.T, s.H, sc)
      if (s.dtype == kBF16) { if (two) RG(kBF16, 2, kNtwB16); else RG(kBF16, 1, kNtwB16); }
      else { if (two) RG(kFP8, 2, kNtwF8); else RG(kFP8, 1, kNtwF8); }
#undef RG
    }
  } else {
    dim3 g1((kprime + kRerankThreads - 1) / kRerankThreads, s.T, s.batch);
    rerank_score_kernel<kF32><<<g1, kRerankThreads, 0, st>>>(q, q_scale, w, kk, k_scale, cand,
                                                             kprime, sc, s.L, s.T, s.H);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || fused) return e;
  dim3 g2(s.T, s.batch);
#define LS(NT, BLK) list_select_kernel<NT, BLK><<<g2, NT, 0, st>>>(sc, cand, kprime, s.L, s.T, k, idx, scores_out, m, s.B)
  if (rows >= 1024) { if (m > 0) LS(256, true); else LS(256, false); }
  else { if (m > 0) LS(1024, true); else LS(1024, false); }
#undef LS
  return hipGetLastError();
}

}  // namespace misa
