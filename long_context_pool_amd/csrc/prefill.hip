// Prefill token scoring + top-k, Eq. (9)-(10) (routed heads) and Eq. (1)-(2)
// (all heads) of the MISA summary page, on the gfx950 matrix cores.
//
// Every indexer head scores the same key, so for a tile of queries the scores
// are one dense contraction: the gathered head rows of the tile (A operand,
// held in registers for the whole pass) times K^T (B operand, 64-key tiles
// loaded straight into LDS by buffer-to-LDS loads, three tile buffers so two
// tiles are in flight while one is multiplied, shared by the workgroup's four
// waves), 32x32x16 bf16 or 32x32x64 fp8 MFMA, fp32 accumulation.  The
// epilogue of one tile (head sums, candidate selection and appends) is
// interleaved with the next tile's MFMAs.  The ReLU * w head
// sum runs on the accumulators: the row order inside a 32-row tile is chosen
// so that each lane holds all heads of its query for its key column.
//
// Exact selection without writing the score rows (1-4 GiB at long context):
//  * a workgroup owns 32 consecutive queries (h = 8; fewer for more heads)
//    and one of S key splits; blocks are numbered so that all workgroups of
//    one split land on the same XCD and share its L2;
//  * it first scores a strided 512-key sample of its split and sets, per
//    query, a threshold tau at the sample's (m k/n)-quantile, margin m =
//    2.5, or 2 when that still puts the quantile at sample rank >= 64;
//  * the full pass appends every score >= tau of a key inside the query's
//    prefix to the (query, split) candidate segment (wave ballots give the
//    positions, so each store writes consecutive entries; each segment has a
//    single writer wave);
//  * the select kernel takes the top-k of a query's candidates.  That is the
//    true top-k iff at least k candidates score >= max over splits of tau
//    (every non-candidate is below its split's tau); otherwise, or when a
//    segment overflowed, the query is queued and the repair kernel scores its
//    whole prefix into a scratch row and selects from that.
#include "common.hpp"
#include "launch.hpp"
#include "mfma.hpp"
#include "row_scorer.hpp"
#include "topk.hpp"

namespace misa {

namespace {

constexpr int kPThreads = 256;
constexpr int kPWaves = 4;
constexpr int kRT = 2;             // 32-row tiles per wave
constexpr int kTileKeys = 64;      // keys per LDS tile (two 32-key column tiles)
constexpr int kSamplesLog2 = 9;
constexpr int kSamples = 1 << kSamplesLog2;  // sample keys per (workgroup, split) and chunk
constexpr int kMaxSampleChunks = 4;
constexpr int kKeep = 128;         // sample values kept per query between chunks
// Sampling plan.  The threshold of a (query, split) is the sample's j-th
// largest, j = m k (samples) / n: about m k n_s / n keys of the split pass
// it, and the query's candidates hold its true top-k when at least k of them
// pass the largest split threshold.  The fraction of the split above the
// sample's j-th largest is Beta-distributed; it falls below 1/m of its mean
// -- too few candidates, so the query goes to the slow repair -- with
// probability P(Poisson(j / m) >= j).  One repaired query costs a whole
// prefix scored and selected by one workgroup, a latency tail of hundreds of
// microseconds, so the plan keeps the expected repairs per call (T S P)
// below kMaxRepairs.
constexpr double kMaxRepairs = 0.01;
constexpr float kMargins[] = {1.75f, 2.0f, 2.5f, 3.0f, 4.0f};

// P(X >= j) for X ~ Poisson(lambda), j >= 1 (host).
double poisson_tail(double lambda, int j) {
  double logp = -lambda + j * __builtin_log(lambda) - __builtin_lgamma(j + 1.0);
  double term = __builtin_exp(logp), sum = 0.0;
  for (int x = j; x < j + 4096 && term > sum * 1e-12; ++x) {
    sum += term;
    term *= lambda / (x + 1);
  }
  return sum;
}
constexpr int kRepairSlots = 64;   // repair workgroups (one scratch row each)
constexpr int kRepThreads = 512;
constexpr int kTopkThreadsSel = 1024;

template <int DT>
constexpr int lds_row_bytes() { return DT == kBF16 ? kD * 2 + 16 : kD + 16; }

// Queries per wave for HPQ padded heads per query (rows of a 32-row tile).
template <int HPQ>
constexpr int qpw() { return HPQ == 8 ? 8 : (HPQ == 16 ? 4 : (HPQ == 32 ? 2 : 1)); }

// Row r of row tile rt (A operand) -> (query within wave, head slot).
template <int HPQ>
__device__ __forceinline__ void row_map(int rt, int r, int& qw, int& hs) {
  if constexpr (HPQ == 8) {
    qw = rt * 4 + (r >> 4) + 2 * ((r >> 2) & 1);
    hs = ((r >> 3) & 1) * 4 + (r & 3);
  } else if constexpr (HPQ == 16) {
    qw = rt * 2 + ((r >> 2) & 1);
    hs = 4 * (r >> 3) + (r & 3);
  } else if constexpr (HPQ == 32) {
    qw = rt;
    hs = r;
  } else {
    qw = 0;
    hs = 32 * rt + r;
  }
}

// Score slots per lane: how many (query) sums a lane forms per column tile.
template <int HPQ>
constexpr int nslots() { return HPQ == 8 ? 4 : (HPQ == 16 ? 2 : (HPQ == 32 ? 2 : 1)); }

// Slot -> query within wave for a lane in half hf.
template <int HPQ>
__device__ __forceinline__ int slot_query(int slot, int hf) {
  if constexpr (HPQ == 8) return (slot >> 1) * 4 + 2 * hf + (slot & 1);
  else if constexpr (HPQ == 16) return slot * 2 + hf;
  else if constexpr (HPQ == 32) return slot;
  else return 0;
}

// Slots past a segment's capacity.  One append adds at most 32 entries to a
// segment (one half-wave's passing lanes) at a position clamped to the
// capacity, so it always lands inside the segment.
constexpr int kSegPad = 32;

struct PrefillArgs {
  const void* q;
  const float* q_scale;
  const float* w;
  const void* k;
  const float* k_scale;
  const int32_t* heads;  // [batch*T, nh] or nullptr (all heads)
  int32_t nh;            // heads scored per query
  int32_t L, T, H, k_top;
  int32_t S;             // key splits
  int64_t chunk;         // keys per split
  int32_t cap;           // candidate capacity per (query, split)
  int32_t seg;           // segment stride: cap + kSegPad slots
  int32_t nqt;           // query tiles per sequence
  int32_t batch;
  uint2* cand;           // [rows, S, seg] (score bits, token)
  int32_t* cnt;          // [rows, S]
  float* tau;            // [rows*S]
  float margin;          // threshold sample rank = margin * k * samples / n_q
  int32_t nch;           // sample chunks (1 .. kMaxSampleChunks)
};

// Buffer resource over [base, base + bytes): loads past the end read zero,
// stores past it are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
// Direct buffer-to-LDS loads: lane l's 16 (4) bytes at voff land at
// lds + 16 l (4 l); lds is wave-uniform.
__device__ __forceinline__ void load16_to_lds(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void load4_to_lds(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, voff, 0, 0, 0);
}
__device__ __forceinline__ uint2 buffer_load_u32x2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ void buffer_store_u32x2(uint32_t lo, uint32_t hi, __amdgpu_buffer_rsrc_t r, uint32_t off,
                                                   uint32_t soff = 0) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{lo, hi}, r, off, soff, 0);
}
// Wait until at most N vector-memory operations of this wave are
// outstanding, then a workgroup barrier; the signal fences keep the
// compiler from moving memory operations across.
template <int N>
__device__ __forceinline__ void vmcnt_barrier() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate in the low field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
__device__ __forceinline__ void vmcnt_zero() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ void compiler_fence() { __atomic_signal_fence(__ATOMIC_SEQ_CST); }

// A pointer the compiler cannot prove wave-uniform but that is: pinned to
// scalar registers (a buffer resource built from it then needs no per-lane
// loop).
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
  return reinterpret_cast<T*>((static_cast<uint64_t>(hi) << 32) | lo);
}

template <int DT, int HPQ>
__global__ __launch_bounds__(kPThreads, 2) void prefill_score_kernel(PrefillArgs a) {
  constexpr int QPW = qpw<HPQ>();
  constexpr int QWG = QPW * kPWaves;
  constexpr int NS = nslots<HPQ>();
  constexpr int RB = lds_row_bytes<DT>();
  constexpr int TILE_BYTES = kTileKeys * RB;
  constexpr int SAMPLE_BYTES = kPWaves * QPW * kSamples * 2;  // top 16 bits of each sample's key
  constexpr int STAGE_BYTES = 32 * RB;                        // one 32-key sample tile
  constexpr int NDMA = (TILE_BYTES + 4 * 1024 - 1) / (4 * 1024);  // 1 KiB direct loads per thread per tile
  // Three main-pass tile buffers, separate objects so that the compiler can
  // tell a buffer being filled by direct loads from the one being read.  The
  // sample pass borrows them first: the samples of waves 0-1 in buffer 0,
  // of waves 2-3 in buffer 1, its key stage in buffer 2.
  constexpr int BUF_DMA = kPWaves * NDMA * 1024;
  constexpr int BUF_BYTES = BUF_DMA > SAMPLE_BYTES / 2 ? BUF_DMA : SAMPLE_BYTES / 2;
  static_assert(STAGE_BYTES <= BUF_BYTES, "sample stage fits a tile buffer");
  __shared__ __attribute__((aligned(16))) uint8_t tb0[BUF_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t tb1[BUF_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t tb2[BUF_BYTES];
  __shared__ float sk_tile[2][32];  // fp8 key scales of the two sample stage slots
  __shared__ __attribute__((aligned(16))) uint16_t kept[kPWaves][QPW][kKeep];  // between sample chunks
  // fp8 key scales of the tile in buffer 0, 1, 2 (one copy per wave).
  __shared__ float sk0[DT == kFP8 ? kPWaves : 1][kTileKeys];
  __shared__ float sk1[DT == kFP8 ? kPWaves : 1][kTileKeys];
  __shared__ float sk2[DT == kFP8 ? kPWaves : 1][kTileKeys];

  // XCD-aware numbering: workgroups of one split share an XCD (id % 8).
  const int id = blockIdx.x;
  const int xcd = id & 7;
  const int split = xcd % a.S;
  const int64_t qt_global = static_cast<int64_t>(id >> 3) * (8 / a.S) + xcd / a.S;
  if (qt_global >= static_cast<int64_t>(a.nqt) * a.batch) return;
  const int64_t seq = qt_global / a.nqt;
  const int t0 = static_cast<int>(qt_global % a.nqt) * QWG;

  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
  const int hf = lane >> 5;
  const int colr = lane & 31;
  const int tw0 = t0 + wave * QPW;  // first query of this wave

  // Key range of this workgroup: its split of [0, pos_last].
  const int t_last = min(t0 + QWG - 1, a.T - 1);
  const int64_t pos_last = static_cast<int64_t>(a.L) - a.T + t_last;
  const int64_t s_begin = split * a.chunk;
  const int64_t s_end = min<int64_t>(s_begin + a.chunk, pos_last + 1);

  // ---- A operand: this wave's gathered head rows, and per-lane weights.
  bf16x8 a16[kRT][8];
  i32x8 a8[kRT][2];
  float wl[kRT][16];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    int qw, hs;
    row_map<HPQ>(rt, colr, qw, hs);
    const int t = tw0 + qw;
    int j = -1;
    if (t < a.T && hs < a.nh) {
      const int64_t r = seq * a.T + t;
      j = a.heads ? a.heads[r * a.nh + hs] : hs;
      if (j < 0 || j >= a.H) j = -1;
    }
    const int64_t qrow = (seq * a.T + (t < a.T ? t : 0)) * a.H + (j < 0 ? 0 : j);
    if constexpr (DT == kBF16) {
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) + qrow * kD + 64 * hf);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) a16[rt][ks] = as_bf16x8(j < 0 ? make_uint4(0, 0, 0, 0) : src[ks]);
    } else {
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.q) + qrow * kD + 64 * hf);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const uint4 lo = j < 0 ? make_uint4(0, 0, 0, 0) : src[2 * ks];
        const uint4 hi = j < 0 ? make_uint4(0, 0, 0, 0) : src[2 * ks + 1];
        a8[rt][ks] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
    }
    // Weights of the accumulator rows this lane holds (rows 8*(i/4)+4hf+i%4).
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      int qw2, hs2;
      row_map<HPQ>(rt, 8 * (i / 4) + 4 * hf + (i % 4), qw2, hs2);
      const int t2 = tw0 + qw2;
      float wv = 0.f;
      if (t2 < a.T && hs2 < a.nh) {
        const int64_t r2 = seq * a.T + t2;
        const int j2 = a.heads ? a.heads[r2 * a.nh + hs2] : hs2;
        if (j2 >= 0 && j2 < a.H) {
          wv = a.w[r2 * a.H + j2];
          if constexpr (DT == kFP8) wv *= a.q_scale[r2];
        }
      }
      wl[rt][i] = wv;
    }
  }

  // Scores of one staged 32-key column tile: out[slot] for this lane's column.
  auto score_tile = [&](const uint8_t* tile, int c, float (&out)[NS]) {
    f32x16 acc[kRT];
    const uint8_t* brow = tile + (32 * c + colr) * RB;
    if constexpr (DT == kBF16) {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 b = as_bf16x8(*reinterpret_cast<const uint4*>(brow + 128 * hf + 16 * ks));
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt)
          acc[rt] = mfma32_bf16(a16[rt][ks], b, ks == 0 ? f32x16{} : acc[rt]);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const uint4 lo = *reinterpret_cast<const uint4*>(brow + 64 * hf + 32 * ks);
        const uint4 hi = *reinterpret_cast<const uint4*>(brow + 64 * hf + 32 * ks + 16);
        const i32x8 b{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt)
          acc[rt] = mfma32_fp8(a8[rt][ks], b, ks == 0 ? f32x16{} : acc[rt]);
      }
    }
#pragma unroll
    for (int sl = 0; sl < NS; ++sl) out[sl] = 0.f;
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float v = wl[rt][i] * relu(acc[rt][i]);
        if constexpr (HPQ == 8) out[rt * 2 + (i >> 3)] += v;
        else if constexpr (HPQ == 16) out[rt] += v;
        else if constexpr (HPQ == 32) out[rt] += v;
        else out[0] += v;
      }
    if constexpr (HPQ >= 32) {
#pragma unroll
      for (int sl = 0; sl < NS; ++sl) out[sl] += __shfl_xor(out[sl], 32, kWave);
    }
  };

  // Query positions of this lane's slots (and of the wave's queries).
  int pos_slot[NS];  // L < 2^31
#pragma unroll
  for (int sl = 0; sl < NS; ++sl) {
    const int t = tw0 + slot_query<HPQ>(sl, hf);
    pos_slot[sl] = t < a.T ? a.L - a.T + t : -1;
  }

  // ---- 1. sample pass: thresholds per (query, split).
  //
  // The split's sample is a.nch (1, 2 or 4) chunks of kSamples strided keys
  // (sample i of chunk c is key s_begin + ((i nch + c) len) / (kSamples nch),
  // so every chunk spreads over the whole split).  Between chunks each query keeps
  // the kKeep largest sample values seen so far (16-bit key prefixes) in
  // LDS; the threshold is the j-th largest over all chunks, j <= kKeep
  // (with one chunk, j <= kSamples).
  const int64_t len = s_end - s_begin;
  const int nch = a.nch;
  const int nch_log2 = nch == 4 ? 2 : (nch == 2 ? 1 : 0);   // nch is 1, 2 or 4
  const int msamp_log2 = kSamplesLog2 + nch_log2;            // sample keys per split: 2^msamp_log2
  uint16_t* smp = reinterpret_cast<uint16_t*>(wave < 2 ? tb0 : tb1) + (wave & 1) * QPW * kSamples;  // [QPW][kSamples]
  float tau_slot[NS];
  int nvs_acc = 0;  // valid samples of this lane's query group so far
  for (int ch = 0; ch < nch; ++ch) {
  // Sample tiles (32 keys) are staged in buffer 2 (two stage slots); each
  // tile's scores go straight to the sample area (sample m of query qw at
  // smp[qw][m]).  The strided sample rows are loaded four tiles ahead into
  // registers, so their latency overlaps the scoring of earlier tiles.
  {
    static_assert(2 * 32 * RB <= BUF_BYTES, "two sample stage slots fit buffer 2");
    const int kr = threadIdx.x >> 3;  // 8 threads per key row
    const int part = threadIdx.x & 7;
    struct SReg {
      uint4 v0, v1;
      float sk;
    };
    auto sample_key = [&](int m) -> int64_t {
      return len > 0 ? s_begin + (((static_cast<int64_t>(m) << nch_log2) + ch) * len >> msamp_log2) : -1;
    };
    auto sload = [&](int st) -> SReg {
      SReg r;
      const int m_ld = st * 32 + kr;
      const int64_t key_ld = st < kSamples / 32 ? sample_key(m_ld) : -1;
      const int64_t row = seq * a.L + (key_ld < 0 ? 0 : key_ld);
      if constexpr (DT == kBF16) {
        const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.k) + row * kD + 16 * part);
        r.v0 = key_ld < 0 ? make_uint4(0, 0, 0, 0) : src[0];
        r.v1 = key_ld < 0 ? make_uint4(0, 0, 0, 0) : src[1];
        r.sk = 1.f;
      } else {
        const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.k) + row * kD + 16 * part);
        r.v0 = key_ld < 0 ? make_uint4(0, 0, 0, 0) : src[0];
        r.v1 = make_uint4(0, 0, 0, 0);
        r.sk = (key_ld >= 0 && part == 0) ? a.k_scale[row] : 1.f;
      }
      return r;
    };
    // One tile from the registers r: stage it, score it, store its keys.
    auto sample_tile = [&](int st, const SReg& r) {
      uint8_t* stage = tb2 + (st & 1) * 32 * RB;
      if constexpr (DT == kBF16) {
        uint4* dst = reinterpret_cast<uint4*>(stage + kr * RB + 32 * part);
        dst[0] = r.v0;
        dst[1] = r.v1;
      } else {
        *reinterpret_cast<uint4*>(stage + kr * RB + 16 * part) = r.v0;
        if (part == 0) sk_tile[st & 1][kr] = r.sk;
      }
      __syncthreads();
      float out[NS];
      score_tile(stage, 0, out);
      const int m = st * 32 + colr;
      const int64_t key = sample_key(m);
      float skv = 1.f;
      if constexpr (DT == kFP8) skv = sk_tile[st & 1][colr];
#pragma unroll
      for (int sl = 0; sl < NS; ++sl) {
        const bool ok = key >= 0 && key <= pos_slot[sl];
        const int qw = slot_query<HPQ>(sl, hf);
        // 0 marks a missing sample (no score has a key below 2^16).
        if (HPQ < 32 || hf == 0)
          smp[qw * kSamples + m] = ok ? static_cast<uint16_t>(float_key(out[sl] * skv) >> 16) : 0;
      }
    };
    // Four register sets in fixed roles (a rotation by copies would wait
    // for the loads being copied).
    SReg r0 = sload(0), r1 = sload(1), r2 = sload(2), r3 = sload(3);
    static_assert((kSamples / 32) % 4 == 0, "sample tiles come in fours");
    for (int st = 0; st < kSamples / 32; st += 4) {
      sample_tile(st, r0);
      r0 = sload(st + 4);
      sample_tile(st + 1, r1);
      r1 = sload(st + 5);
      sample_tile(st + 2, r2);
      r2 = sload(st + 6);
      sample_tile(st + 3, r3);
      r3 = sload(st + 7);
    }
    __syncthreads();
  }
  {
    // Lanes [g*LPQ, (g+1)*LPQ) serve query g: VPL of this chunk's samples
    // and KPL of the kept values per lane, as 16-bit keys two per register.
    constexpr int LPQ = kWave / QPW;
    constexpr int VPL = kSamples / LPQ;
    constexpr int KPL = kKeep / LPQ;
    const int g = lane / LPQ;
    const int lg = lane % LPQ;
    static_assert(VPL % 8 == 0 && KPL % 2 == 0, "samples are read 8, kept values 2 at a time");
    uint32_t kv[VPL / 2], kk[KPL / 2];
    int nvs = 0;
#pragma unroll
    for (int e = 0; e < VPL / 8; ++e) {
      const uint4 w4 = reinterpret_cast<const uint4*>(smp + g * kSamples + lg * VPL)[e];
      kv[4 * e] = w4.x;
      kv[4 * e + 1] = w4.y;
      kv[4 * e + 2] = w4.z;
      kv[4 * e + 3] = w4.w;
    }
    uint16_t* kq = &kept[wave][g][0];
#pragma unroll
    for (int e = 0; e < KPL / 2; ++e) kk[e] = ch > 0 ? reinterpret_cast<const uint32_t*>(kq + lg * KPL)[e] : 0u;
#pragma unroll
    for (int e = 0; e < VPL / 2; ++e)
      nvs += ((kv[e] & 0xFFFFu) != 0 ? 1 : 0) + ((kv[e] >> 16) != 0 ? 1 : 0);
#pragma unroll
    for (int o = LPQ / 2; o >= 1; o >>= 1) nvs += __shfl_xor(nvs, o, kWave);
    nvs_acc += nvs;
    const int t = tw0 + g;
    const bool last = ch + 1 == nch;
    // Rank searched: kKeep between chunks; after the last, j = ceil(margin
    // k nvs / n_q) (at most kKeep over several chunks).  Padding queries (t
    // >= T) never pass; a query whose split holds fewer sampled keys than j
    // keeps every key of the split (tau = -inf).
    int rank = kKeep;
    bool search = true;
    if (last) {
      const int64_t nq = static_cast<int64_t>(a.L) - a.T + t + 1;
      const double jd = static_cast<double>(a.margin) * a.k_top * nvs_acc / static_cast<double>(nq > 0 ? nq : 1);
      rank = static_cast<int>(jd) + 1;
      if (nch > 1 && rank > kKeep) rank = kKeep;
      search = t < a.T && nvs_acc > 0 && rank < nvs_acc;
    }
    // The largest 16-bit value v with #{values >= v} >= rank (0 when fewer
    // than rank values are valid): a bitwise search from the top bit.
    uint32_t v = 0;
    for (int bit = 15; bit >= 0; --bit) {
      const uint32_t c = v | (1u << bit);
      int n = 0;
#pragma unroll
      for (int e = 0; e < VPL / 2; ++e) n += ((kv[e] & 0xFFFFu) >= c ? 1 : 0) + ((kv[e] >> 16) >= c ? 1 : 0);
#pragma unroll
      for (int e = 0; e < KPL / 2; ++e) n += ((kk[e] & 0xFFFFu) >= c ? 1 : 0) + ((kk[e] >> 16) >= c ? 1 : 0);
#pragma unroll
      for (int o = LPQ / 2; o >= 1; o >>= 1) n += __shfl_xor(n, o, kWave);
      if (n >= rank && search) v = c;
    }
    if (!last) {
      // Keep the kKeep largest: every value above v, then copies of v.
      int gt = 0;
#pragma unroll
      for (int e = 0; e < VPL / 2; ++e) gt += ((kv[e] & 0xFFFFu) > v ? 1 : 0) + ((kv[e] >> 16) > v ? 1 : 0);
#pragma unroll
      for (int e = 0; e < KPL / 2; ++e) gt += ((kk[e] & 0xFFFFu) > v ? 1 : 0) + ((kk[e] >> 16) > v ? 1 : 0);
      int off = gt;  // inclusive scan over the group's lanes
#pragma unroll
      for (int o = 1; o < LPQ; o <<= 1) {
        const int y = __shfl_up(off, o, kWave);
        if (lg >= o) off += y;
      }
      const int total_gt = __shfl(off, g * LPQ + LPQ - 1, kWave);
      off -= gt;
      __builtin_amdgcn_wave_barrier();  // every lane has read the kept values
#pragma unroll
      for (int e = 0; e < VPL / 2; ++e) {
        const uint32_t x0 = kv[e] & 0xFFFFu, x1 = kv[e] >> 16;
        if (x0 > v) kq[off++] = static_cast<uint16_t>(x0);
        if (x1 > v) kq[off++] = static_cast<uint16_t>(x1);
      }
#pragma unroll
      for (int e = 0; e < KPL / 2; ++e) {
        const uint32_t x0 = kk[e] & 0xFFFFu, x1 = kk[e] >> 16;
        if (x0 > v) kq[off++] = static_cast<uint16_t>(x0);
        if (x1 > v) kq[off++] = static_cast<uint16_t>(x1);
      }
      for (int i = total_gt + lg; i < kKeep; i += LPQ) kq[i] = static_cast<uint16_t>(v);
      __builtin_amdgcn_wave_barrier();
    } else {
      float tq = t < a.T ? -__builtin_inff() : __builtin_inff();
      if (search) {
        // The smallest float whose key has top bits v: every sample counted
        // above scores at least this.
        const uint32_t key = v << 16;
        const uint32_t u = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
        tq = __uint_as_float(u);
      }
      // Broadcast: every lane needs the tau of its slots' queries.
      float tau_q[QPW];
#pragma unroll
      for (int qq = 0; qq < QPW; ++qq) tau_q[qq] = __shfl(tq, qq * LPQ, kWave);
#pragma unroll
      for (int sl = 0; sl < NS; ++sl) {
        const int qw0 = slot_query<HPQ>(sl, 0), qw1 = slot_query<HPQ>(sl, 1);
        tau_slot[sl] = hf ? tau_q[qw1] : tau_q[qw0];
      }
      if (lg == 0 && t < a.T) a.tau[(seq * a.T + t) * a.S + split] = tq;
    }
  }
  }  // chunks
  __syncthreads();  // sample area is reused as tile buffers below

  // ---- 2. full pass over [s_begin, s_end): append scores >= tau.
  //
  // Key tiles (64 keys) reach LDS by direct buffer-to-LDS loads (no VGPR
  // staging, no LDS store instructions) into three buffers: tile ti+2 is in
  // flight while tile ti is multiplied.  Every thread issues the same number
  // of vector-memory operations per tile (NL loads, NS candidate stores per
  // column tile), so a fixed vmcnt wait before each barrier proves that the
  // next tile has landed.  The column tiles are software-pipelined: the
  // MFMAs of column tile j are issued among the epilogue (ReLU * w head sum,
  // threshold test, candidate append) of column tile j-1, with no branch in
  // either.
  //
  // Candidate append: per slot, the wave ballot of passing lanes gives each
  // lane its position in its half's (query's) segment, so the entries of a
  // slot land next to each other; the entry is written by a buffer store
  // whose offset is pushed out of range for lanes that do not pass.  A batch
  // that starts past a segment's capacity is written at the capacity, into
  // the segment's padding (overwriting entries there; the count still grows
  // past the capacity, which sends the query to repair).
  constexpr int ROWB = kD * (DT == kBF16 ? 2 : 1);  // key row bytes in HBM
  constexpr int NL = NDMA + (DT == kFP8 ? 1 : 0);
  // This thread's byte offset inside a tile's key rows for each of its DMA
  // slots (LDS row pitch RB keeps the MFMA operand reads conflict-free; the
  // 16-byte pads and the spare tail load row 0, never read).
  uint32_t dma_off[NDMA];
#pragma unroll
  for (int j = 0; j < NDMA; ++j) {
    const int o = 1024 * (NDMA * wave + j) + 16 * lane;
    const int r = o / RB, c = (o % RB) / 16;
    dma_off[j] = (r < kTileKeys && c < ROWB / 16) ? static_cast<uint32_t>(r * ROWB + 16 * c) : 0u;
  }
  const uint8_t* kseq = static_cast<const uint8_t*>(a.k) + seq * a.L * static_cast<int64_t>(ROWB);
  const float* kscale_seq = (DT == kFP8) ? a.k_scale + seq * a.L : nullptr;
  // Tile ti -> LDS buffer tb (key scales: sk); rows at or past s_end read as
  // zero.
  auto issue = [&](int64_t ti, uint8_t* tb, float (*sk)[kTileKeys]) __attribute__((always_inline)) {
    const int64_t key0 = s_begin + ti * kTileKeys;
    const int64_t nrows = s_end - key0;
    const int32_t nb = nrows <= 0 ? 0 : static_cast<int32_t>(nrows < kTileKeys ? nrows : kTileKeys);
    const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(kseq + (nrows <= 0 ? 0 : key0 * ROWB), nb * ROWB);
#pragma unroll
    for (int j = 0; j < NDMA; ++j) load16_to_lds(rk, tb + 1024 * (NDMA * wave + j), dma_off[j]);
    if constexpr (DT == kFP8) {
      const __amdgpu_buffer_rsrc_t rsk = buffer_rsrc(kscale_seq + (nrows <= 0 ? 0 : key0), nb * 4);
      load4_to_lds(rsk, &sk[wave][0], 4u * lane);
    }
  };
  // Per-slot constants: the last key a slot may take (split end and causal
  // bound), and the byte offset of the slot's segment from the wave's first.
  const bool owner = HPQ < 32 || hf == 0;
  int lim_slot[NS];
  uint32_t seg_off[NS];
#pragma unroll
  for (int sl = 0; sl < NS; ++sl) {
    const int64_t lim = min<int64_t>(s_end - 1, pos_slot[sl]);
    lim_slot[sl] = owner ? static_cast<int>(lim) : -1;
    seg_off[sl] = static_cast<uint32_t>(slot_query<HPQ>(sl, hf)) * static_cast<uint32_t>(a.S) *
                  static_cast<uint32_t>(a.seg) * 8u;
  }
  const __amdgpu_buffer_rsrc_t rcand =
      buffer_rsrc(uniform_ptr(a.cand + ((seq * a.T + tw0) * a.S + split) * static_cast<int64_t>(a.seg)),
                  __builtin_amdgcn_readfirstlane(QPW * a.S * a.seg * 8));
  // Candidate counts per (slot, half): scalar; (sl, h) is query
  // slot_query(sl, h).  They go to cnt at the end and may exceed the
  // capacity (the select kernel then queues the query for repair).
  int ctr2[NS][2];
#pragma unroll
  for (int sl = 0; sl < NS; ++sl) ctr2[sl][0] = ctr2[sl][1] = 0;
  // All ones in the upper half of the wave, zero in the lower; opaque to the
  // compiler, so that (x & upper) stays one AND with a scalar operand instead
  // of becoming a select that needs the scalar copied to a vector register.
  uint32_t upper = 0u - static_cast<uint32_t>(hf);
  asm volatile("" : "+v"(upper));

  // Epilogue, in parts: part 2*sl sums slot sl's heads (ReLU * w), part
  // 2*sl+1 tests and appends it.  live = false marks a placeholder column
  // tile that stores nothing but issues the same instructions.  chk = false
  // (a compile-time constant at every call) drops the per-key limit test, for
  // column tiles that lie wholly at or below every query's limit.
  auto epi_part = [&](int p, const f32x16 (&acc)[kRT], int key0, bool live, bool chk, float sk,
                      float (&out)[NS]) __attribute__((always_inline)) {
    const int sl = p >> 1;
    if ((p & 1) == 0) {
      float sum = 0.f;
      if constexpr (HPQ == 8) {
#pragma unroll
        for (int i = 0; i < 8; ++i) sum += wl[sl >> 1][8 * (sl & 1) + i] * relu(acc[sl >> 1][8 * (sl & 1) + i]);
      } else if constexpr (HPQ == 16 || HPQ == 32) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sum += wl[sl][i] * relu(acc[sl][i]);
      } else {
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
          for (int i = 0; i < 16; ++i) sum += wl[rt][i] * relu(acc[rt][i]);
      }
      if constexpr (HPQ >= 32) sum += __shfl_xor(sum, 32, kWave);
      out[sl] = (DT == kFP8) ? sum * sk : sum;
      return;
    }
    const int key = key0 + colr;
    const float v = out[sl];
    uint64_t m = __builtin_amdgcn_ballot_w64(v >= tau_slot[sl]) & (live ? ~0ull : 0ull);
    if (chk) m &= __builtin_amdgcn_ballot_w64(key <= lim_slot[sl]);
    const uint32_t mlo = static_cast<uint32_t>(m), mhi = static_cast<uint32_t>(m >> 32);
    const int plo = __builtin_popcount(mlo), phi = __builtin_popcount(mhi);
    // Write bases of the two halves, scalar: the half's count, at most the
    // capacity, so that the batch (at most 32 entries) stays inside the
    // padded segment; a count past the capacity sends the query to repair.
    const int blo = min(ctr2[sl][0], a.cap);
    const int bhi = min(ctr2[sl][1], a.cap);
    // Entry position minus blo: lower half, the passing lanes below; upper
    // half, (bhi - blo) + the passing upper lanes below, which is the 64-lane
    // count plus (bhi - plo - blo).  blo itself goes in the store's scalar
    // offset.  The upper half's segment starts at least seg > cap entries
    // after the lower half's, so the vector offset never goes below zero.
    const uint32_t dhalf = static_cast<uint32_t>(bhi - plo - blo);
    const uint32_t rel = __builtin_amdgcn_mbcnt_hi(mhi, __builtin_amdgcn_mbcnt_lo(mlo, dhalf & upper));
    const uint32_t voff = seg_off[sl] + 8u * rel;
    // Lanes that do not pass store at offset 0xC0800000 (the bits of -4.0,
    // an inline operand), past the end of any candidate buffer: dropped.
    uint32_t off;
    asm("v_cndmask_b32_e64 %0, -4.0, %1, %2" : "=v"(off) : "v"(voff), "s"(m));
    buffer_store_u32x2(__float_as_uint(v), static_cast<uint32_t>(key), rcand, off,
                       8u * static_cast<uint32_t>(blo));
    ctr2[sl][0] += plo;
    ctr2[sl][1] += phi;
  };

  // One step: acc = this wave's rows x column tile c of buffer tb (skv = the
  // fp8 scale of this lane's key column), with the epilogue of the previous
  // column tile (pacc, its first key pkey0) spread between the k-steps.  The
  // B operands are read two k-steps ahead; scheduling barriers keep the
  // order, so the VALU work runs while the MFMAs execute.
  constexpr int NKS = DT == kBF16 ? 8 : 2;
  constexpr int NP = 2 * NS;
  auto step = [&](const uint8_t* tb, const float (*sk)[kTileKeys], int c, f32x16 (&acc)[kRT], float& skv,
                  const f32x16 (&pacc)[kRT], int pkey0, bool plive, bool pchk, float pskv)
      __attribute__((always_inline)) {
    const uint8_t* brow = tb + (32 * c + colr) * RB;
    float out[NS];
    if constexpr (DT == kBF16) {
      uint4 bv[3];
      bv[0] = *reinterpret_cast<const uint4*>(brow + 128 * hf);
      bv[1] = *reinterpret_cast<const uint4*>(brow + 128 * hf + 16);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        if (ks + 2 < NKS) bv[(ks + 2) % 3] = *reinterpret_cast<const uint4*>(brow + 128 * hf + 16 * (ks + 2));
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt)
          acc[rt] = mfma32_bf16(a16[rt][ks], as_bf16x8(bv[ks % 3]), ks == 0 ? f32x16{} : acc[rt]);
#pragma unroll
        for (int p = ks * NP / NKS; p < (ks + 1) * NP / NKS; ++p) epi_part(p, pacc, pkey0, plive, pchk, pskv, out);
        __builtin_amdgcn_sched_barrier(0);
      }
      skv = 1.f;
    } else {
      i32x8 bv[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const uint4 lo = *reinterpret_cast<const uint4*>(brow + 64 * hf + 32 * ks);
        const uint4 hi = *reinterpret_cast<const uint4*>(brow + 64 * hf + 32 * ks + 16);
        bv[ks] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
      skv = sk[wave][32 * c + colr];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
          acc[rt] = mfma32_fp8(a8[rt][ks], bv[ks], ks == 0 ? f32x16{} : acc[rt]);
          constexpr int PPM = NP / (NKS * kRT) > 0 ? NP / (NKS * kRT) : 1;  // parts per MFMA
          const int m = ks * kRT + rt;
#pragma unroll
          for (int p = m * PPM; p < (m + 1) * PPM && p < NP; ++p)
            epi_part(p, pacc, pkey0, plive, pchk, pskv, out);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  };
  // Epilogue only (the last column tile).
  auto epi_all = [&](const f32x16 (&pacc)[kRT], int pkey0, bool pchk, float pskv) __attribute__((always_inline)) {
    float out[NS];
#pragma unroll
    for (int p = 0; p < NP; ++p) epi_part(p, pacc, pkey0, true, pchk, pskv, out);
  };

  const int64_t ntiles = len > 0 ? (len + kTileKeys - 1) / kTileKeys : 0;
  // vmcnt(N) with N = the operations issued after the tile that must have
  // landed: the next tile's loads and one step's stores.
  constexpr int kWaitCnt = NL + NS;
  if (ntiles > 0) {
    issue(0, tb0, sk0);
    issue(1, tb1, sk1);
    vmcnt_barrier<NL>();  // tile 0 landed (tile 1 may be in flight)
    f32x16 acc_a[kRT], acc_b[kRT];
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) acc_b[rt] = f32x16{};
    float sk_a = 1.f, sk_b = 1.f;
    // Column tile 0 beside a placeholder epilogue.
    step(tb0, sk0, 0, acc_a, sk_a, acc_b, 0, false, false, 1.f);
    // Tile ti sits in buffer ti % 3: the loops are unrolled by three so that
    // every buffer reference is static.  chk: the epilogues of tile ti test
    // each key against the query limits.
    auto tile_iter = [&](int64_t ti, uint8_t* tcur, float (*scur)[kTileKeys], uint8_t* tnext,
                         float (*snext)[kTileKeys], uint8_t* tfill, float (*sfill)[kTileKeys], bool chk)
        __attribute__((always_inline)) {
      const int key0 = static_cast<int>(s_begin + ti * kTileKeys);
      issue(ti + 2, tfill, sfill);
      compiler_fence();
      step(tcur, scur, 1, acc_b, sk_b, acc_a, key0, true, chk, sk_a);
      vmcnt_barrier<kWaitCnt>();
      if (ti + 1 < ntiles) step(tnext, snext, 0, acc_a, sk_a, acc_b, key0 + 32, true, chk, sk_b);
      else epi_all(acc_b, key0 + 32, chk, sk_b);
    };
    // The first nfull tiles lie wholly at or below the limit of every query
    // of the workgroup (the split end and the causal bound of its first
    // query), so their epilogues skip the limit test.  Workgroups with
    // padding queries (never passing, limit -1) or with half-wave owners
    // (32 or more heads per query) test every tile.
    const int64_t lim_min = min<int64_t>(s_end - 1, static_cast<int64_t>(a.L) - a.T + t0);
    const int64_t nlim = (HPQ < 32 && t0 + QWG <= a.T) ? (lim_min - s_begin + 1) / kTileKeys : 0;
    const int64_t nfull = nlim < 0 ? 0 : (nlim < ntiles ? nlim : ntiles);
    int64_t ti = 0;
    for (; ti + 3 <= nfull; ti += 3) {
      tile_iter(ti, tb0, sk0, tb1, sk1, tb2, sk2, false);
      tile_iter(ti + 1, tb1, sk1, tb2, sk2, tb0, sk0, false);
      tile_iter(ti + 2, tb2, sk2, tb0, sk0, tb1, sk1, false);
    }
    for (; ti < ntiles; ti += 3) {
      tile_iter(ti, tb0, sk0, tb1, sk1, tb2, sk2, true);
      if (ti + 1 >= ntiles) break;
      tile_iter(ti + 1, tb1, sk1, tb2, sk2, tb0, sk0, true);
      if (ti + 2 >= ntiles) break;
      tile_iter(ti + 2, tb2, sk2, tb0, sk0, tb1, sk1, true);
    }
  }
  // No load may still be writing LDS when the wave ends.
  vmcnt_zero();
  if (lane == 0) {
#pragma unroll
    for (int sl = 0; sl < NS; ++sl)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (HPQ >= 32 && h == 1) continue;
        const int t = tw0 + slot_query<HPQ>(sl, h);
        if (t < a.T) a.cnt[(seq * a.T + t) * a.S + split] = ctr2[sl][h];
      }
  }
}

__global__ void prefill_clear_kernel(int32_t* fail_count) {
  if (threadIdx.x == 0) *fail_count = 0;
}

// Top-k of query r's candidates, or a place in the repair queue when the
// candidates cannot be shown to hold the true top-k.  Certificate: no
// segment overflowed and at least k candidates score >= tau_max = max over
// splits of tau (every non-candidate of split s scores below tau_s).  Then:
//  1. one pass over the candidates (the S segments viewed as one list: entry
//     c lies in segment s with pre[s] <= c < pre[s+1]; wave w holds the
//     R 64-entry chunks from chunk R w in registers, R <= NR as few as hold
//     the list, lane l entry 64 (R w + u) + l in slot u, all of its loads in
//     flight at once)
//     builds an LDS histogram of their relative bins (RelBins: from tau_min,
//     which every candidate reaches) and counts the candidates >= tau_max;
//  2. the bin b* holding the k-th best comes from a block scan of the
//     histogram;
//  3. per-wave counts (one barrier) and wave ballots place the entries
//     above b* in the output and those at b* in an LDS list;
//  4. the list is resolved exactly (ties: lower token).
// Entries beyond the registers' NR * NT are read again from global memory,
// 8 NT at a time (wave w: 8 consecutive 64-entry chunks).  Each wave holding
// a consecutive run of the list makes the output come out in list order:
// sorted by split and token.
constexpr int kPCandCap = 1024;
// Workgroup size and candidates held in registers per thread: 256 threads x
// kSelRegsSmall while the expected count (about margin k) fits
// comfortably (120 registers: four workgroups per CU), else 512 threads x
// kSelRegsLarge (two per CU; 34 keeps it within 128 registers without
// spills, and holds about 1.2 times the expected count of k = 8192 at the
// lowest margin, so that few queries need a round from memory).  Queries
// are independent, so more workgroups per CU overlap more of each one's load
// and barrier latency: 256 x 32 took the C3 select from 133 to 111 us
// against 512 x 16 (three per CU).
constexpr int kSelThreadsSmall = 256;
constexpr int kSelRegsSmall = 32;
constexpr int kSelThreadsLarge = 512;
constexpr int kSelRegsLarge = 34;
constexpr int kRelBins = 2048;
// 64-entry chunks of the register-held entries (at most 512 x 34 of them);
// a chunk that straddles a segment boundary is marked mixed.
constexpr int kSelChunks = (kSelThreadsLarge * kSelRegsLarge + 63) / 64;
constexpr int kChunkMixed = -0x7FFFFFFF;

struct PSelSmem {
  uint32_t hist[kRelBins];
  alignas(16) float cand_score[kPCandCap];
  alignas(16) int32_t cand_idx[kPCandCap];
  union {
    ResolveSmem rs;
    TopkSmem ts;
  };
  int pre[9];
  int ctab[kSelChunks];  // per 64-entry chunk: the slot offset of its one segment, or kChunkMixed
  int scan_tmp[32];
  int digit, above, count, nge, bad;
  int wtot[kTopkThreadsSel / kWave];  // per-wave packed counts above / at b* (up to 16 waves)
  uint32_t dmin, dmax;                 // candidate coarse-key range (tau_min = -inf)
  float tau_max, tau_min;
};

template <int NT, int NR>
__global__ __launch_bounds__(NT, 4) void prefill_select_kernel(
    const uint2* __restrict__ cand, const int32_t* __restrict__ cnt, const float* __restrict__ tau,
    int32_t S, int32_t cap, int32_t seg, int32_t k, int32_t* __restrict__ idx,
    float* __restrict__ scores_out, int32_t* __restrict__ fail_count, int32_t* __restrict__ fail_list) {
  static_assert(NT <= kTopkThreadsSel && NR >= 1 && NR <= 64, "entry slots are bits of a 64-bit mask");
  constexpr int NO = 8;  // entries per thread per round beyond the registers
  __shared__ PSelSmem sm;
  const int64_t r = blockIdx.x;
  const int lane = lane_id();
  int32_t* out = idx + r * k;
  float* out_s = scores_out ? scores_out + r * k : nullptr;
  const uint2* base = cand + r * S * static_cast<int64_t>(seg);
  for (int b = threadIdx.x; b < kRelBins; b += NT) sm.hist[b] = 0;
  if (threadIdx.x == 0) {
    int total = 0, bad = 0;
    float tmax = -__builtin_inff(), tmin = __builtin_inff();
    for (int sp = 0; sp < 8; ++sp) {
      sm.pre[sp] = total;
      if (sp < S) {
        const int c = cnt[r * S + sp];
        bad |= c > cap;
        total += c < cap ? c : cap;
        const float t = tau[r * S + sp];
        tmax = fmaxf(tmax, t);
        tmin = fminf(tmin, t);
      }
    }
    sm.pre[8] = total;
    sm.tau_max = tmax;
    sm.tau_min = tmin;
    sm.bad = bad;
    sm.nge = 0;
    sm.dmin = 0xFFFFFFFFu;
    sm.dmax = 0u;
  }
  __syncthreads();
  int pre[9];
#pragma unroll
  for (int u = 0; u < 9; ++u) pre[u] = sm.pre[u];
  const int total = pre[8];
  const float tm = sm.tau_max;
  // The query's S segments through one buffer resource (32-bit offsets:
  // S * seg * 8 bytes < 2^31 for L <= 2^24); entry c at byte offset
  // 8 (s seg + c - pre[s]).
  const __amdgpu_buffer_rsrc_t crs = buffer_rsrc(uniform_ptr(base), S * seg * 8);
  auto entry = [=](int c) -> uint2 {
    int sg = 0, b = 0;
#pragma unroll
    for (int u = 1; u < 8; ++u) {
      const bool ge = c >= pre[u] && u < S;
      sg = ge ? u : sg;
      b = ge ? pre[u] : b;
    }
    return buffer_load_u32x2(crs, static_cast<uint32_t>(sg * seg + (c - b)) * 8u);
  };
  const CandVerdict verdict = cand_verdict(sm.bad != 0, total, k, tm);
  if (verdict == CandVerdict::kRepair) {
    if (threadIdx.x == 0) fail_list[atomicAdd(fail_count, 1)] = static_cast<int32_t>(r);
    return;
  }
  if (verdict == CandVerdict::kTakeAll) {
    // Every key of the prefix is a candidate: take them all, pad with -1.
    for (int c = threadIdx.x; c < total; c += NT) {
      const uint2 e = entry(c);
      out[c] = static_cast<int32_t>(e.y);
      if (out_s) out_s[c] = __uint_as_float(e.x);
    }
    for (int p = total + threadIdx.x; p < k; p += NT) {
      out[p] = -1;
      if (out_s) out_s[p] = -__builtin_inff();
    }
    return;
  }
  // 1. entries 64 (R w + u) + l (u < R) into registers.  Entry c of
  // segment s sits at slot c + s seg - pre[s]; the 64 entries a wave loads
  // per step form one chunk, and for a chunk within one segment that offset
  // is taken from a table built here (one entry per thread), so only the few
  // chunks that straddle a boundary search the segments lane by lane.
  static_assert(NT % kWave == 0 && NT * NR <= kSelChunks * 64, "chunk table covers the registers");
  const int nchunk = (min(total, NR * NT) + 63) / 64;
  for (int j = threadIdx.x; j < nchunk; j += NT) {
    auto seg_of = [&](int c) {
      int sg = 0;
#pragma unroll
      for (int u = 1; u < 8; ++u) sg = (c >= pre[u] && u < S) ? u : sg;
      return sg;
    };
    const int s_lo = seg_of(64 * j), s_hi = seg_of(min(64 * j + 63, total - 1));
    sm.ctab[j] = s_lo == s_hi ? s_lo * seg - pre[s_lo] : kChunkMixed;
  }
  __syncthreads();
  const int wave_e = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  // Round entries: slot u of this wave in a round of n slots per wave
  // starting at list entry c0 is entry c0 + 64 (n w + u) + lane; its first
  // entry (uniform) is c0 + 64 (n w + u), and it holds entries when u < n
  // and that first entry is below total.  The register round takes R slots
  // per wave, as few as hold the list (so the waves share it evenly).
  constexpr int NW = NT / kWave;
  const int R = min(NR, (nchunk + NW - 1) / NW);
  struct Round {
    int base, nu, nf, lane;  // this wave's first entry; slots holding entries; full slots
    __device__ bool used(int u) const { return u < nu; }
    __device__ bool full(int u) const { return u < nf; }
    __device__ int entry(int u) const { return base + 64 * u + lane; }
  };
  auto make_round = [=](int c0, int n) {
    const int base = c0 + 64 * n * wave_e;
    const int rem = total - base;
    const int nu = min(max((rem + 63) >> 6, 0), n), nf = min(max(rem >> 6, 0), n);
    return Round{__builtin_amdgcn_readfirstlane(base), __builtin_amdgcn_readfirstlane(nu),
                 __builtin_amdgcn_readfirstlane(nf), lane};
  };
  // Lane u reads the table entry of this wave's chunk of register slot u
  // (one LDS read per wave; slot u then takes it with a lane read).
  static_assert(NR <= kWave, "one table entry per lane");
  int ctv = kChunkMixed;
  {
    const int j = wave_e * R + lane;
    if (lane < R && j < nchunk) ctv = sm.ctab[j];
  }
  const Round r0 = make_round(0, R);
  uint2 e[NR];
#pragma unroll
  for (int u = 0; u < NR; ++u) {
    const int c = r0.entry(u);
    if (r0.used(u)) {
      const int o = __builtin_amdgcn_readlane(ctv, u);  // this wave's chunk (uniform)
      if (c >= total) e[u] = make_uint2(0u, 0u);
      else if (o != kChunkMixed) e[u] = buffer_load_u32x2(crs, static_cast<uint32_t>(c + o) * 8u);
      else e[u] = entry(c);
    } else {
      e[u] = make_uint2(0u, 0u);
    }
  }
  // Relative bins (RelBins).  Every candidate is >= tau_min, so with a
  // finite tau_min the bins start at its coarse key.  When some split kept
  // every key, the candidates' own coarse-key range sets the base and the
  // shift.
  const float tmin = sm.tau_min;
  RelBins rb;
  if (tmin != -__builtin_inff()) {
    rb = RelBins::above(tmin);
  } else {
    uint32_t gmin = 0xFFFFFFFFu, gmax = 0u;
    auto range_entry = [&](int c, uint2 x) __attribute__((always_inline)) {
      if (c < total) {
        const uint32_t g = float_key(__uint_as_float(x.x)) >> 16;
        gmin = min(gmin, g);
        gmax = max(gmax, g);
      }
    };
#pragma unroll
    for (int u = 0; u < NR; ++u)
      if (r0.used(u)) range_entry(r0.entry(u), e[u]);
    for (int c0 = NR * NT; c0 < total; c0 += NT)  // beyond the registers
      range_entry(c0 + static_cast<int>(threadIdx.x),
                  c0 + static_cast<int>(threadIdx.x) < total ? entry(c0 + threadIdx.x) : make_uint2(0u, 0u));
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) {
      gmin = min(gmin, static_cast<uint32_t>(__shfl_xor(static_cast<int>(gmin), o, kWave)));
      gmax = max(gmax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(gmax), o, kWave)));
    }
    if (lane == 0) {
      atomicMin(&sm.dmin, gmin);
      atomicMax(&sm.dmax, gmax);
    }
    __syncthreads();
    rb = RelBins::range(sm.dmin, sm.dmax);  // total > 0 here, so gmin <= gmax
  }
  static_assert(kRelBins == kRelBinCount, "select bins are relative bins");
  // Histogram and certificate count (register slots that every lane fills
  // skip the per-entry test).
  int nge = 0;
  auto count_entry = [&](int c, uint2 x) __attribute__((always_inline)) {
    if (c < total) {
      const float v = __uint_as_float(x.x);
      atomicAdd(&sm.hist[rb.bin(v)], 1u);
      nge += v >= tm ? 1 : 0;
    }
  };
#pragma unroll
  for (int u = 0; u < NR; ++u) {
    if (r0.full(u)) {  // every lane's slot u holds an entry (uniform)
      const float v = __uint_as_float(e[u].x);
      atomicAdd(&sm.hist[rb.bin(v)], 1u);
      nge += v >= tm ? 1 : 0;
    } else if (r0.used(u)) {
      count_entry(r0.entry(u), e[u]);
    }
  }
  for (int c0 = NR * NT; c0 < total; c0 += NO * NT) {  // beyond the registers
    const Round rr = make_round(c0, NO);
    uint2 f[NO];
#pragma unroll
    for (int u = 0; u < NO; ++u) {
      const int c = rr.entry(u);
      f[u] = c < total ? entry(c) : make_uint2(0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < NO; ++u) count_entry(rr.entry(u), f[u]);
  }
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) nge += __shfl_xor(nge, o, kWave);
  if (lane == 0) atomicAdd(&sm.nge, nge);
  __syncthreads();
  if (sm.nge < k) {
    if (threadIdx.x == 0) fail_list[atomicAdd(fail_count, 1)] = static_cast<int32_t>(r);
    return;
  }
  // 2. b*: thread t owns relative bins kRelBins-1-t*BPT downwards.
  {
    constexpr int BPT = kRelBins / NT;
    int local[BPT];
    int lsum = 0;
#pragma unroll
    for (int u = 0; u < BPT; ++u) {
      local[u] = static_cast<int>(sm.hist[kRelBins - 1 - (threadIdx.x * BPT + u)]);
      lsum += local[u];
    }
    int tot;
    int run = block_exclusive_sum<NT>(lsum, sm.scan_tmp, tot);
#pragma unroll
    for (int u = 0; u < BPT; ++u) {
      if (run < k && run + local[u] >= k) {
        sm.digit = kRelBins - 1 - (threadIdx.x * BPT + u);
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
  if (bcount > kPCandCap) {
    if (threadIdx.x == 0) fail_list[atomicAdd(fail_count, 1)] = static_cast<int32_t>(r);
    return;
  }
  // 3. compaction by relative bin: per-thread counts above and at b*
  // (packed: above in the low 16 bits, total < k <= 8192; at-b* high, total
  // <= kPCandCap), one block scan for the positions.
  // Positions: each wave's entries above b* (at b*) take one run of the
  // output (list), after those of the lower waves; inside the run, entry
  // slot by slot (ballots), so the stores of a slot coalesce.
  // Relative bin b* as a key interval [blo, bhi].
  uint32_t blo, bhi;
  rb.interval(bstar, blo, bhi);
  auto classify = [&](const uint2* ev, int n, const Round& rnd, uint64_t& mh, uint64_t& ma) __attribute__((always_inline)) {
    mh = 0;
    ma = 0;
#pragma unroll
    for (int u = 0; u < n; ++u) {
      if (rnd.used(u)) {  // (uniform)
        const int c = rnd.entry(u);
        const uint32_t key = float_key(__uint_as_float(ev[u].x));
        mh |= (c < total && key > bhi) ? (uint64_t{1} << u) : uint64_t{0};
        ma |= (c < total && key >= blo && key <= bhi) ? (uint64_t{1} << u) : uint64_t{0};
      }
    }
  };
  const int wave = threadIdx.x / kWave;
  int run_h = 0, run_a = 0;  // entries placed by earlier rounds (block totals)
  // The output goes through buffer resources of k entries (the scores': of
  // none when out_s is null).  A lane that places nothing stores past the
  // end, where the range check drops it, so placing takes no branch.
  const __amdgpu_buffer_rsrc_t rout = buffer_rsrc(uniform_ptr(out), k * 4);
  const __amdgpu_buffer_rsrc_t routs =
      buffer_rsrc(uniform_ptr(out_s ? reinterpret_cast<int32_t*>(out_s) : out), out_s ? k * 4 : 0);
  auto place = [&](const uint2* ev, int n, const Round& rnd, uint64_t mh, uint64_t ma) __attribute__((always_inline)) {
    int wt = __popcll(mh) | (__popcll(ma) << 16);
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) wt += __shfl_xor(wt, o, kWave);
    if (lane == 0) sm.wtot[wave] = wt;
    __syncthreads();
    int base = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NT / kWave; ++w) {
      const int v = sm.wtot[w];
      base += w < wave ? v : 0;
      all += v;
    }
    // The wave's output and list positions (uniform).
    int ph = __builtin_amdgcn_readfirstlane(run_h + (base & 0xFFFF));
    int pa = __builtin_amdgcn_readfirstlane(run_a + (base >> 16));
#pragma unroll
    for (int u = 0; u < n; ++u) {
      if (!rnd.used(u)) continue;  // (uniform)
      const bool h = (mh >> u) & 1u;
      const bool at = (ma >> u) & 1u;
      const uint64_t bh = __ballot(h);
      const uint32_t off = h ? static_cast<uint32_t>(ph + lanes_below(bh)) * 4u : 0x80000000u;
      __builtin_amdgcn_raw_buffer_store_b32(ev[u].y, rout, off, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(ev[u].x, routs, off, 0, 0);
      ph += __popcll(bh);
      const uint64_t ba = __ballot(at);
      if (ba != 0) {  // entries of the threshold bin (few)
        if (at) {
          const int pos = pa + lanes_below(ba);
          if (pos < kPCandCap) {
            sm.cand_score[pos] = __uint_as_float(ev[u].x);
            sm.cand_idx[pos] = static_cast<int32_t>(ev[u].y);
          }
        }
        pa += __popcll(ba);
      }
    }
    run_h += all & 0xFFFF;
    run_a += all >> 16;
    __syncthreads();  // wtot is reused
  };
  {
    uint64_t mh, ma;
    classify(e, NR, r0, mh, ma);
    place(e, NR, r0, mh, ma);
  }
  for (int c0 = NR * NT; c0 < total; c0 += NO * NT) {  // beyond the registers
    const Round rr = make_round(c0, NO);
    uint2 f[NO];
#pragma unroll
    for (int u = 0; u < NO; ++u) {
      const int c = rr.entry(u);
      f[u] = c < total ? entry(c) : make_uint2(0u, 0u);
    }
    uint64_t mh, ma;
    classify(f, NO, rr, mh, ma);
    place(f, NO, rr, mh, ma);
  }
  __syncthreads();
  // 4. the (k - above) best of the b* list.
  if (resolve_list<NT>(sm.cand_score, sm.cand_idx, bcount, k - above, out + above,
                       out_s ? out_s + above : nullptr, sm.rs))
    return;
  // A b* bin of more than kRankMax entries: exact fallback, reusing
  // the resolve area (no longer needed) for the radix select.
  __syncthreads();
  TopkSmem& tsm = sm.ts;
  const float* cs = sm.cand_score;
  const int32_t* ci = sm.cand_idx;
  block_topk<NT>(
      bcount, k - above, [](int64_t) { return true; }, [=](int64_t j) { return float_key(cs[j]); },
      [=](int64_t j) { return ci[j]; }, [=](int64_t j) { return cs[j]; }, out + above,
      out_s ? out_s + above : nullptr, tsm);
}

// Repair: queries whose candidates could not be certified are scored over
// their whole prefix (16x16 MFMA key streaming) into this workgroup's scratch
// row and selected from it.  The grid is fixed; each workgroup walks the
// queue with stride gridDim.x and exits when it is exhausted.
template <int DT, int NRT>
__global__ __launch_bounds__(kRepThreads) void prefill_repair_kernel(
    const void* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    const void* __restrict__ k, const float* __restrict__ k_scale,
    const int32_t* __restrict__ heads, int32_t nh, int32_t L, int32_t T, int32_t H, int32_t k_top,
    const int32_t* __restrict__ fail_count, const int32_t* __restrict__ fail_list,
    float* __restrict__ scratch, int32_t* __restrict__ idx, float* __restrict__ scores_out) {
  __shared__ TopkFastSmem sm;
  constexpr int NW = kRepThreads / kWave;
  const int nfail = *fail_count;
  float* row = scratch + static_cast<int64_t>(blockIdx.x) * L;
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  for (int f = blockIdx.x; f < nfail; f += gridDim.x) {
    const int64_t r = fail_list[f];
    const int64_t seq = r / T;
    const int64_t n = static_cast<int64_t>(L) - T + (r % T) + 1;
    RowScorer<DT, NRT> sc;
    sc.init(q, q_scale, w, heads, nh, r, H);
    const void* krows = (DT == kBF16) ? static_cast<const void*>(static_cast<const uint16_t*>(k) + seq * L * kD)
                                      : static_cast<const void*>(static_cast<const uint8_t*>(k) + seq * L * kD);
    for (int64_t s0 = static_cast<int64_t>(wave) * 64; s0 < n; s0 += NW * 64) {
      const float res = sc.score64(krows, s0, n, 0);
      const int64_t s = s0 + lane;
      if (s < n) {
        float v = res;
        if constexpr (DT == kFP8) v *= k_scale[seq * L + s];
        row[s] = v;
      }
    }
    __syncthreads();
    block_topk_fast<kRepThreads>(
        n, k_top, [](int64_t) { return true; }, [=](int64_t i) { return row[i]; },
        [](int64_t i) { return static_cast<int32_t>(i); }, idx + r * k_top,
        scores_out ? scores_out + r * k_top : nullptr, sm);
    __syncthreads();
  }
}

struct PrefillPlan {
  int32_t S, cap, seg, nqt, qwg, nch;
  float margin;
  int64_t chunk;
  size_t off_cnt, off_tau, off_fail, off_list, off_scratch, total;
};

int32_t qwg_for(int32_t nh) {
  const int hpq = nh <= 8 ? 8 : (nh <= 16 ? 16 : (nh <= 32 ? 32 : 64));
  return (hpq == 8 ? 8 : hpq == 16 ? 4 : hpq == 32 ? 2 : 1) * kPWaves;
}

PrefillPlan plan_prefill(const Shape& s, int32_t nh, int32_t k) {
  PrefillPlan p{};
  p.qwg = qwg_for(nh);
  p.nqt = (s.T + p.qwg - 1) / p.qwg;
  const int64_t tiles = static_cast<int64_t>(p.nqt) * s.batch;
  int S = 1;
  while (S < 8 && tiles * S < 512 && s.L / (2 * S) >= 2048) S *= 2;
  p.S = S;
  p.chunk = ((static_cast<int64_t>(s.L) + S - 1) / S + kTileKeys - 1) / kTileKeys * kTileKeys;
  // Candidates per (query, split): about margin * k * (split keys in the
  // prefix) / n_q, at most margin * k * chunk / (L - T + 1).  The threshold
  // comes from a sample quantile with relative spread ~1/sqrt(j) (j >= ~20);
  // at j ~ 20 the count can run ~2x its mean in a few of thousands of
  // queries: 2.5x + 16 sigma + 512 leaves overflow (then repair) very rare.
  const double nmin = static_cast<double>(s.L - s.T + 1);
  const double share = static_cast<double>(p.chunk) / nmin < 1.0 ? static_cast<double>(p.chunk) / nmin : 1.0;
  // Margin and sample chunks: the cheapest (candidates appended and
  // selected, 2 m k / L per key, against sample keys scored, c kSamples per
  // split key) whose expected repairs stay below kMaxRepairs; if none does,
  // the one with the fewest.  The sample rank is taken for the worst split:
  // the last one, of which the first query's prefix covers the least.
  {
    const double cover = static_cast<double>(s.L - s.T + 1 - (p.S - 1) * p.chunk) / static_cast<double>(p.chunk);
    const double f = cover < 0.25 ? 0.25 : (cover > 1.0 ? 1.0 : cover);
    const double nrows = static_cast<double>(s.batch) * s.T * p.S;
    double best_cost = 1e300, best_rep = 1e300;
    bool found = false;
    p.margin = kMargins[0];
    p.nch = 1;
    for (int c = 1; c <= kMaxSampleChunks; c *= 2) {  // 1, 2 or 4: a power-of-two sample count
      if (c > 1 && static_cast<int64_t>(c) * kSamples > p.chunk) break;
      for (const float m : kMargins) {
        const double j = static_cast<double>(m) * k * c * kSamples / static_cast<double>(s.L);
        if (c > 1 && j > kKeep) continue;
        const int jw = static_cast<int>(f * j) + 1;
        const double rep = nrows * poisson_tail(jw / static_cast<double>(m), jw);
        const double cost = 2.0 * m * k / s.L + static_cast<double>(c) * kSamples / static_cast<double>(p.chunk);
        if (rep <= kMaxRepairs) {
          if (!found || cost < best_cost) {
            best_cost = cost;
            p.margin = m;
            p.nch = c;
          }
          found = true;
        } else if (!found && rep < best_rep) {
          best_rep = rep;
          p.margin = m;
          p.nch = c;
        }
      }
    }
  }
  const double mean = p.margin * k * share;
  int64_t cap = static_cast<int64_t>(2.5 * mean + 16.0 * __builtin_sqrt(mean) + 512.0);
  cap = cap < p.chunk ? cap : p.chunk;
  cap = (cap + 63) / 64 * 64;
  p.cap = static_cast<int32_t>(cap);
  p.seg = p.cap + kSegPad;
  const int64_t rows = static_cast<int64_t>(s.batch) * s.T;
  const size_t segs = static_cast<size_t>(rows) * S;
  size_t off = align_up(segs * p.seg * sizeof(uint2));
  p.off_cnt = off;
  off += align_up(segs * sizeof(int32_t));
  p.off_tau = off;
  off += align_up(static_cast<size_t>(rows) * S * sizeof(float));
  p.off_fail = off;
  off += 256;
  p.off_list = off;
  off += align_up(static_cast<size_t>(rows) * sizeof(int32_t));
  p.off_scratch = off;
  off += align_up(static_cast<size_t>(kRepairSlots) * s.L * sizeof(float));
  p.total = off;
  return p;
}

template <int DT, int HPQ>
void launch_prefill_dt(const Shape& s, const PrefillPlan& pl, PrefillArgs args, hipStream_t st) {
  const int64_t tiles = static_cast<int64_t>(pl.nqt) * s.batch;
  const int per8 = 8 / pl.S;
  const int64_t nblocks = (tiles + per8 - 1) / per8 * 8;
  prefill_score_kernel<DT, HPQ><<<static_cast<unsigned>(nblocks), kPThreads, 0, st>>>(args);
}

}  // namespace

// The candidate stores address a wave's segments through a buffer resource
// with 32-bit offsets (at most ~64 L bytes): L up to 2^24 keeps them below 2^31.
bool prefill_supported(const Shape& s) { return s.T > 1 && s.dtype != kF32 && s.L <= (1 << 24); }

size_t prefill_ws_bytes(const Shape& s, int32_t nh, int32_t k) {
  return plan_prefill(s, nh, k).total;
}

hipError_t launch_prefill_score_topk(const Shape& s, int32_t nh, const int32_t* heads, int32_t k,
                                     const void* q, const float* q_scale, const float* w,
                                     const void* kk, const float* k_scale, int32_t* idx,
                                     float* scores_out, void* ws, hipStream_t st) {
  const PrefillPlan pl = plan_prefill(s, nh, k);
  char* base = static_cast<char*>(ws);
  PrefillArgs args{q, q_scale, w, kk, k_scale, heads, nh, s.L, s.T, s.H, k, pl.S, pl.chunk,
                   pl.cap, pl.seg, pl.nqt, s.batch, reinterpret_cast<uint2*>(base),
                   reinterpret_cast<int32_t*>(base + pl.off_cnt),
                   reinterpret_cast<float*>(base + pl.off_tau), pl.margin, pl.nch};
  int32_t* fail_count = reinterpret_cast<int32_t*>(base + pl.off_fail);
  int32_t* fail_list = reinterpret_cast<int32_t*>(base + pl.off_list);
  float* scratch = reinterpret_cast<float*>(base + pl.off_scratch);
  prefill_clear_kernel<<<1, 64, 0, st>>>(fail_count);
  const int hpq = nh <= 8 ? 8 : (nh <= 16 ? 16 : (nh <= 32 ? 32 : 64));
#define PF(DT) \
  if (hpq == 8) launch_prefill_dt<DT, 8>(s, pl, args, st); \
  else if (hpq == 16) launch_prefill_dt<DT, 16>(s, pl, args, st); \
  else if (hpq == 32) launch_prefill_dt<DT, 32>(s, pl, args, st); \
  else launch_prefill_dt<DT, 64>(s, pl, args, st);
  if (s.dtype == kBF16) { PF(kBF16) } else { PF(kFP8) }
#undef PF
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = static_cast<int64_t>(s.batch) * s.T;
  if (pl.margin * 1.25f * k <= static_cast<float>(kSelRegsSmall * kSelThreadsSmall))
    prefill_select_kernel<kSelThreadsSmall, kSelRegsSmall><<<static_cast<unsigned>(rows), kSelThreadsSmall, 0, st>>>(
        args.cand, args.cnt, args.tau, pl.S, pl.cap, pl.seg, k, idx, scores_out, fail_count, fail_list);
  else
    prefill_select_kernel<kSelThreadsLarge, kSelRegsLarge><<<static_cast<unsigned>(rows), kSelThreadsLarge, 0, st>>>(
        args.cand, args.cnt, args.tau, pl.S, pl.cap, pl.seg, k, idx, scores_out, fail_count, fail_list);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nrt = nh <= 16 ? 1 : (nh <= 32 ? 2 : 4);
#define RP(DT, NRT) prefill_repair_kernel<DT, NRT><<<kRepairSlots, kRepThreads, 0, st>>>(q, q_scale, w, kk, k_scale, heads, nh, s.L, s.T, s.H, k, fail_count, fail_list, scratch, idx, scores_out)
  if (s.dtype == kBF16) {
    if (nrt == 1) RP(kBF16, 1); else if (nrt == 2) RP(kBF16, 2); else RP(kBF16, 4);
  } else {
    if (nrt == 1) RP(kFP8, 1); else if (nrt == 2) RP(kFP8, 2); else RP(kFP8, 4);
  }
#undef RP
  return hipGetLastError();
}

}  // namespace misa
