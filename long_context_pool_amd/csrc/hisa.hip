// MISA x HISA: the combination the MISA summary page describes in
// "Methodology" 1 ("Key distinction from HISA") and "Theoretical and Practical
// Implications" ("Scalability").  MISA reduces the router affinities
// A_{t,j,b} = w_{t,j} * ReLU(q_{t,j} . p_b) of Eq. (7) across the blocks to
// pick heads; HISA reduces the same affinities across the heads to pick
// blocks.  Here both run: the query's top-m blocks by
//   G_{t,b} = sum_{j < H} A_{t,j,b}
// (the same causal blocks as the router: complete blocks from the pooled
// cache of Eq. (4), the partial last block pooled over the query's own keys)
// bound the Eq. (9) routed-head scoring, and the top-k of those tokens is
// the selection.
//
// Kernels:
//  1. hisa_block_kernel: one query per wave, its H head rows as the A operand
//     of 32x32x16 MFMA tiles (held in registers; fp8 codes widen to bf16
//     exactly), 32-block pooled tiles as B (bf16 hi and lo planes of the
//     pooled keys, staged in LDS by buffer-to-LDS loads and shared by the
//     workgroup's four waves).  A lane then holds 16 heads of one block, so
//     w * ReLU and the head sum stay in the lane (one cross-half add).  The
//     partial block's G comes from per-key MFMA dots on the raw keys.  G goes
//     to the workspace; the wave then finds the m-th largest G by a bitwise
//     search on the order-preserving keys (ballot counts) and writes its m
//     blocks in ascending order (ties: lower block).  With few queries
//     (decode) each query's blocks are split over up to 64 workgroups and
//     hisa_topm_kernel picks the blocks afterwards.
//  2. the re-rank kernels with the routed heads and the blocks as candidates
//     (launch_rerank_heads with m > 0): entry i of a query's list is token
//     blocks[i / B] * B + i % B, so no list is written; Eq. (9) over them and
//     their top-k (tokens past the query's position, padding blocks and the
//     entries past m B that pad the list to k are invalid).
#include "common.hpp"
#include "launch.hpp"
#include "mfma.hpp"
#include "topk.hpp"

namespace misa {

namespace {

constexpr int kHThreads = 256;
constexpr int kHWaves = 4;
constexpr int kHTileBytes = 32 * kD * 2;  // one bf16 plane of a 32-block pooled tile
constexpr int kHMaxCache = 64;            // G values per lane kept in registers for the top-m

__device__ __forceinline__ __amdgpu_buffer_rsrc_t hs_rsrc(const void* base, int32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ void hs_load16_lds(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}
template <int N>
__device__ __forceinline__ void hs_vmcnt_barrier() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate in the low field");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
__device__ __forceinline__ void hs_vmcnt_zero() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
template <class T>
__device__ __forceinline__ T* hs_uniform(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<T*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// The inverse of float_key.
__device__ __forceinline__ float key_float(uint32_t key) {
  return __builtin_bit_cast(float, (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// 32x32x16 fragments (8 k-steps) of one head or key row `row` (< 0: zeros):
// this lane's elements [64*(l/32), 64*(l/32)+64); fp8 codes widen to bf16.
template <int DT>
__device__ __forceinline__ void row_frags(const void* base, int64_t row, bf16x8 (&a)[8]) {
  const int hf = lane_id() >> 5;
  if (row < 0) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) a[ks] = as_bf16x8(make_uint4(0, 0, 0, 0));
    return;
  }
  if constexpr (DT == kBF16) {
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + row * kD + 64 * hf);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) a[ks] = as_bf16x8(src[ks]);
  } else {
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(base) + row * kD + 64 * hf);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 v = src[c];
      const uint32_t wds[4] = {v.x, v.y, v.z, v.w};
      uint32_t o[8];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float f0 = fp8_to_f32(wds[u] & 0xFF), f1 = fp8_to_f32((wds[u] >> 8) & 0xFF);
        const float f2 = fp8_to_f32((wds[u] >> 16) & 0xFF), f3 = fp8_to_f32(wds[u] >> 24);
        o[2 * u] = (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xFFFF0000u);
        o[2 * u + 1] = (__float_as_uint(f2) >> 16) | (__float_as_uint(f3) & 0xFFFF0000u);
      }
      a[2 * c] = as_bf16x8(make_uint4(o[0], o[1], o[2], o[3]));
      a[2 * c + 1] = as_bf16x8(make_uint4(o[4], o[5], o[6], o[7]));
    }
  }
}

// Top-m blocks of one query's block scores Gq[0 .. Mt), written ascending
// to bq (and their scores to bs when non-null); one wave; ties go to the
// lower block.  The m-th largest order-preserving key v is found bit by bit
// (ballot counts of keys >= a candidate value), starting below the leading
// bits that every key shares; keys above v are taken, then the lowest blocks
// of those equal to v.  CN > 0: the query's ceil(Mt / 64) <= CN keys per
// lane are held in registers (CN a compile-time size, so the loops carry no
// per-entry branch); CN = 0: they are re-read from memory.
template <int CN>
__device__ __forceinline__ void hisa_topm_n(const float* __restrict__ Gq, int64_t Mt, int32_t m,
                                            int32_t* __restrict__ bq, float* __restrict__ bs) {
  const int lane = lane_id();
  const int nch = static_cast<int>((Mt + kWave - 1) / kWave);
  constexpr int NC = CN > 0 ? CN : 1;
  uint32_t kc[NC];
  if constexpr (CN > 0) {
    // Every load first (lanes past Mt re-read the last score, so no lane
    // branches around a load), then the keys; padding keys are 0.
    float gv[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int64_t b = static_cast<int64_t>(j) * kWave + lane;
      gv[j] = Gq[b < Mt ? b : Mt - 1];
    }
#pragma unroll
    for (int j = 0; j < NC; ++j) kc[j] = static_cast<int64_t>(j) * kWave + lane < Mt ? float_key(gv[j]) : 0u;
  }
  auto key_of = [&](int j) -> uint32_t {
    const int64_t b = static_cast<int64_t>(j) * kWave + lane;
    return b < Mt ? float_key(Gq[b]) : 0u;
  };
  // Count of keys >= c (every valid key is >= 0x00800000: float_key of any
  // finite float is at least that, so the padding key 0 never counts).
  auto count_ge = [&](uint32_t c) -> int {
    int cnt = 0;
    if constexpr (CN > 0) {
#pragma unroll
      for (int j = 0; j < NC; ++j) cnt += __popcll(__ballot(kc[j] >= c));
    } else {
      for (int j = 0; j < nch; ++j) cnt += __popcll(__ballot(key_of(j) >= c));
    }
    return cnt;
  };
  uint32_t kand = 0xFFFFFFFFu, kor = 0u;
  if constexpr (CN > 0) {
#pragma unroll
    for (int j = 0; j < NC; ++j)
      if (static_cast<int64_t>(j) * kWave + lane < Mt) {
        kand &= kc[j];
        kor |= kc[j];
      }
  } else {
    for (int j = 0; j < nch; ++j)
      if (static_cast<int64_t>(j) * kWave + lane < Mt) {
        const uint32_t key = key_of(j);
        kand &= key;
        kor |= key;
      }
  }
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) {
    kand &= static_cast<uint32_t>(__shfl_xor(static_cast<int>(kand), o, kWave));
    kor |= static_cast<uint32_t>(__shfl_xor(static_cast<int>(kor), o, kWave));
  }
  const uint32_t diff = kand ^ kor;  // zero: every key is the same
  const int top = diff ? 31 - __clz(static_cast<int>(diff)) : -1;
  uint32_t v = top < 0 ? kand : (top == 31 ? 0u : kand & ~((2u << top) - 1u));
  for (int bit = top; bit >= 0; --bit) {
    const uint32_t c = v | (1u << bit);
    if (count_ge(c) >= m) v = c;
  }
  const int need_eq = m - count_ge(v + 1u);
  int base = 0, eq_seen = 0;
  auto emit = [&](int j, uint32_t key) __attribute__((always_inline)) {
    const int64_t b = static_cast<int64_t>(j) * kWave + lane;
    const bool valid = b < Mt;
    const uint64_t eqm = __ballot(valid && key == v);
    const bool sel = valid && (key > v || (key == v && eq_seen + lanes_below(eqm) < need_eq));
    const uint64_t sm = __ballot(sel);
    if (sel) {
      const int p = base + lanes_below(sm);
      bq[p] = static_cast<int32_t>(b);
      if (bs) bs[p] = key_float(key);  // the score itself (-0 comes back as +0)
    }
    base += __popcll(sm);
    eq_seen += __popcll(eqm);
  };
  if constexpr (CN > 0) {
#pragma unroll
    for (int j = 0; j < NC; ++j) emit(j, kc[j]);
  } else {
    for (int j = 0; j < nch; ++j) emit(j, key_of(j));
  }
}

__device__ __forceinline__ void hisa_topm(const float* __restrict__ Gq, int64_t Mt, int32_t m,
                                          int32_t* __restrict__ bq, float* __restrict__ bs) {
  if (Mt <= m) {  // every block, then padding
    for (int i = lane_id(); i < m; i += kWave) {
      bq[i] = i < Mt ? i : -1;
      if (bs) bs[i] = i < Mt ? Gq[i] : -__builtin_inff();
    }
    return;
  }
  const int64_t nch = (Mt + kWave - 1) / kWave;
  if (nch <= 4) hisa_topm_n<4>(Gq, Mt, m, bq, bs);
  else if (nch <= 8) hisa_topm_n<8>(Gq, Mt, m, bq, bs);
  else if (nch <= 16) hisa_topm_n<16>(Gq, Mt, m, bq, bs);
  else if (nch <= 32) hisa_topm_n<32>(Gq, Mt, m, bq, bs);
  else if (nch <= kHMaxCache) hisa_topm_n<kHMaxCache>(Gq, Mt, m, bq, bs);
  else hisa_topm_n<0>(Gq, Mt, m, bq, bs);
}

// Block scores and the top-m blocks.  Workgroup = four queries (one per
// wave) of one sequence; RT = 32-head row tiles (1 for H <= 32, else 2).
template <int DT, int RT>
__global__ __launch_bounds__(kHThreads, 2) void hisa_block_kernel(
    const void* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    const uint16_t* __restrict__ phi, const uint16_t* __restrict__ plo, const void* __restrict__ k,
    const float* __restrict__ k_scale, int32_t L, int32_t T, int32_t H, int32_t B, int64_t M,
    int32_t m, int32_t nsplit, float* __restrict__ G, int32_t* __restrict__ blocks,
    float* __restrict__ bscores) {
  // Hi and lo bf16 planes of the pooled-key tiles.
  __shared__ __attribute__((aligned(16))) uint8_t h0[kHTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t h1[kHTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t h2[kHTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t l0[kHTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t l1[kHTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t l2[kHTileBytes];
  __shared__ float pdot[kHWaves][64];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = lane_id();
  const int hf = lane >> 5;
  const int64_t seq = blockIdx.y;
  const int t0 = blockIdx.x * kHWaves;
  const int t = t0 + wave;
  const bool active = t < T;
  const int64_t r = seq * T + (active ? t : t0);
  const int64_t pos = static_cast<int64_t>(L) - T + (active ? t : t0);
  const int64_t n = pos + 1;
  const int64_t full = n / B;
  const int64_t Mt = (n + B - 1) / B;
  const int tl = min(t0 + kHWaves - 1, T - 1);
  const int64_t full_max = (static_cast<int64_t>(L) - T + tl + 1) / B;
  float* Gq = G + r * M;

  // A operand: head rows rt*32 + l%32; row weights w * s_q (fp8 q scale, > 0,
  // so it commutes with ReLU) of the lane's accumulator rows.
  bf16x8 a[RT][8];
  float wl[RT][16];
  const float sq = (DT == kFP8) ? q_scale[r] : 1.f;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int j = rt * 32 + (lane & 31);
    row_frags<DT>(q, j < H ? r * H + j : -1, a[rt]);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = rt * 32 + 8 * (i / 4) + 4 * hf + (i % 4);
      wl[rt][i] = row < H ? w[r * H + row] * sq : 0.f;
    }
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) asm volatile("" : "+v"(a[rt][ks]));
  hs_vmcnt_zero();

  // Pooled tiles: three LDS buffers, two tiles in flight (the router's
  // pattern); 16-byte chunk c of tile row rr at chunk position c ^ (rr % 16).
  constexpr int NL = 4;
  // Split z of nsplit takes tiles [tile0, tile1) (nsplit > 1: few queries,
  // so each query's blocks are spread over more workgroups; the last split
  // also takes the partial block, and hisa_topm_kernel picks the blocks).
  const int z = blockIdx.z;
  const int64_t ntiles_all = (full_max + 31) / 32;
  const int64_t tps = (ntiles_all + nsplit - 1) / nsplit;
  const int64_t tile0 = min<int64_t>(static_cast<int64_t>(z) * tps, ntiles_all);
  const int64_t tile1 = min<int64_t>(tile0 + tps, ntiles_all);
  const int64_t ntiles = tile1 - tile0;
  const int64_t last = ntiles > 0 ? tile1 - 1 : 0;
  const __amdgpu_buffer_rsrc_t rh = hs_rsrc(hs_uniform(phi + seq * M * kD), static_cast<int32_t>(M * kD * 2));
  const __amdgpu_buffer_rsrc_t rl = hs_rsrc(hs_uniform(plo + seq * M * kD), static_cast<int32_t>(M * kD * 2));
  int rowi[2];
  uint32_t chk[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    rowi[i] = 8 * wave + 4 * i + lane / 16;
    chk[i] = 16u * static_cast<uint32_t>((lane % 16) ^ (rowi[i] & 15));
  }
  auto issue = [&](int64_t bt, uint8_t* hb, uint8_t* lb) __attribute__((always_inline)) {
    const int64_t tb = bt < last ? bt : last;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t blk = tb * 32 + rowi[i];
      const uint32_t voff = static_cast<uint32_t>((blk < full_max ? blk : 0) * (kD * 2)) + chk[i];
      hs_load16_lds(rh, hb + 1024 * (2 * wave + i), voff);
      hs_load16_lds(rl, lb + 1024 * (2 * wave + i), voff);
    }
  };
  // G of the tile's 32 blocks: lane (l % 32) holds its block's 16 heads per
  // half-wave; the two halves add.
  auto tile = [&](int64_t bt, const uint8_t* hb, const uint8_t* lb) __attribute__((always_inline)) {
    const int rr = lane & 31;
    const uint8_t* rowh = hb + rr * (kD * 2);
    const uint8_t* rowl = lb + rr * (kD * 2);
    f32x16 acc[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) acc[rt] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int pc = (8 * hf + ks) ^ (rr & 15);
      const bf16x8 bh = as_bf16x8(*reinterpret_cast<const uint4*>(rowh + 16 * pc));
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) acc[rt] = mfma32_bf16(a[rt][ks], bh, acc[rt]);
      const bf16x8 bl = as_bf16x8(*reinterpret_cast<const uint4*>(rowl + 16 * pc));
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) acc[rt] = mfma32_bf16(a[rt][ks], bl, acc[rt]);
    }
    float g = 0.f;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 16; ++i) g += wl[rt][i] * relu(acc[rt][i]);
    g += __shfl_xor(g, 32, kWave);
    const int64_t blk = bt * 32 + rr;
    if (active && lane < 32 && blk < full) Gq[blk] = g;
  };
  if (ntiles > 0) {
    issue(tile0, h0, l0);
    issue(tile0 + 1, h1, l1);
  }
  auto step = [&](int64_t bt, const uint8_t* hb, const uint8_t* lb, uint8_t* nh, uint8_t* nl)
      __attribute__((always_inline)) {
    hs_vmcnt_barrier<NL>();  // tile bt has landed; every wave is done with tile bt-1
    issue(bt + 2, nh, nl);
    tile(bt, hb, lb);
  };
  for (int64_t bt = tile0; bt < tile1; bt += 3) {
    step(bt, h0, l0, h2, l2);
    if (bt + 1 < tile1) step(bt + 1, h1, l1, h0, l0);
    if (bt + 2 < tile1) step(bt + 2, h2, l2, h1, l1);
  }
  hs_vmcnt_zero();

  // The partial last block [full B, pos]: G = sum_j w_j ReLU(mean_s q_j . k_s)
  // with the per-key dots from MFMA tiles (32 raw keys as B, the fp8 key
  // scale per column), summed over the keys.
  if (active && Mt > full && z == nsplit - 1) {
    f32x16 ps[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) ps[rt] = f32x16{};
    const int64_t s_lo = full * B;
    for (int64_t s0 = s_lo; s0 <= pos; s0 += 32) {
      const int64_t sk_i = s0 + (lane & 31);
      const bool ok = sk_i <= pos;
      const int64_t row = seq * L + (ok ? sk_i : s_lo);
      bf16x8 kb[8];
      row_frags<DT>(k, row, kb);
      const float skv = ok ? ((DT == kFP8) ? k_scale[row] : 1.f) : 0.f;
      f32x16 acc[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) acc[rt] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[rt] = mfma32_bf16(a[rt][ks], kb[ks], acc[rt]);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 16; ++i) ps[rt][i] += acc[rt][i] * skv;
    }
    // Sum over the key columns: head row rt*32 + 8(i/4) + 4hf + i%4.
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float v = ps[rt][i];
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
        if ((lane & 31) == 0) pdot[wave][rt * 32 + 8 * (i / 4) + 4 * hf + (i % 4)] = v;
      }
    __builtin_amdgcn_wave_barrier();
    const float cnt = static_cast<float>(pos - s_lo + 1);
    float g = lane < H ? w[r * H + lane] * sq * relu(pdot[wave][lane] / cnt) : 0.f;
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) g += __shfl_xor(g, o, kWave);
    if (lane == 0) Gq[full] = g;
  }
  if (!active || nsplit > 1) return;
  // The lanes read back G values other lanes of this wave stored: once the
  // stores have completed they are visible to loads from the same compute
  // unit (its vector L1 is write-through and shared by the unit's waves).
  hs_vmcnt_zero();
  __builtin_amdgcn_wave_barrier();
  hisa_topm(Gq, Mt, m, blocks + r * m, bscores ? bscores + r * m : nullptr);
}

// The top-m blocks of each query from the block scores of the split kernel
// (one wave per query row).
__global__ __launch_bounds__(kHThreads) void hisa_topm_kernel(const float* __restrict__ G, int32_t L,
                                                               int32_t T, int32_t B, int64_t M,
                                                               int64_t rows, int32_t m,
                                                               int32_t* __restrict__ blocks,
                                                               float* __restrict__ bscores) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * kHWaves + threadIdx.x / kWave;
  if (r >= rows) return;
  const int64_t n = static_cast<int64_t>(L) - T + r % T + 1;
  hisa_topm(G + r * M, (n + B - 1) / B, m, blocks + r * m, bscores ? bscores + r * m : nullptr);
}

struct HisaLayout {
  size_t planes, G, blocks, rerank, total;
};

// Candidate list length: the m blocks' tokens, at least k entries.
int32_t hisa_cands(const Shape& s, int32_t m, int32_t k) { return max(m * s.B, k); }

HisaLayout hisa_layout(const Shape& s, int32_t m, int32_t k) {
  HisaLayout lo{};
  const size_t rows = static_cast<size_t>(s.batch) * s.T;
  const size_t plane = align_up(static_cast<size_t>(s.batch) * s.M() * kD * sizeof(uint16_t));
  size_t off = 0;
  lo.planes = off;
  off += 2 * plane;
  lo.G = off;
  off += align_up(rows * s.M() * sizeof(float));
  lo.blocks = off;
  off += align_up(rows * m * sizeof(int32_t));
  lo.rerank = off;
  off += rerank_ws_bytes(s, hisa_cands(s, m, k));
  lo.total = off;
  return lo;
}

}  // namespace

bool hisa_supported(const Shape& s, int32_t m) {
  return s.dtype != kF32 && static_cast<int64_t>(m) * s.B <= 8192 &&
         static_cast<int64_t>(s.L) * kD * (s.dtype == kBF16 ? 2 : 1) < (int64_t{1} << 31) &&
         s.M() * kD * 2 < (int64_t{1} << 31);
}

size_t hisa_ws_bytes(const Shape& s, int32_t m, int32_t k) { return hisa_layout(s, m, k).total; }

// Block splits per query group: enough workgroups (about 512) to spread
// the block scoring over the chip when the queries alone do not (decode).
int32_t hisa_splits(const Shape& s) {
  const int64_t wgs = static_cast<int64_t>((s.T + kHWaves - 1) / kHWaves) * s.batch;
  if (wgs >= 512) return 1;
  const int64_t tiles = (s.M() + 31) / 32;
  int64_t n = (512 + wgs - 1) / wgs;
  n = n < tiles ? n : tiles;
  return static_cast<int32_t>(n < 1 ? 1 : (n > 64 ? 64 : n));
}

hipError_t launch_hisa_score_topk(const Shape& s, int32_t nh, const int32_t* heads, int32_t m,
                                  int32_t k, const void* q, const float* q_scale, const float* w,
                                  const float* pooled, const void* kk, const float* k_scale,
                                  int32_t* blocks_out, float* block_scores_out, int32_t* idx,
                                  float* scores_out, void* ws, hipStream_t st) {
  const HisaLayout lo = hisa_layout(s, m, k);
  char* base = static_cast<char*>(ws);
  const size_t plane = align_up(static_cast<size_t>(s.batch) * s.M() * kD * sizeof(uint16_t));
  uint16_t* phi = reinterpret_cast<uint16_t*>(base + lo.planes);
  uint16_t* plo = reinterpret_cast<uint16_t*>(base + lo.planes + plane);
  hipError_t e = launch_pooled_split(s, pooled, phi, plo, st);
  if (e != hipSuccess) return e;
  float* G = reinterpret_cast<float*>(base + lo.G);
  int32_t* blocks = blocks_out ? blocks_out : reinterpret_cast<int32_t*>(base + lo.blocks);
  const int32_t nsplit = hisa_splits(s);
  dim3 g1((s.T + kHWaves - 1) / kHWaves, s.batch, nsplit);
  const bool two = s.H > 32;
#define HB(DT, RT) hisa_block_kernel<DT, RT><<<g1, kHThreads, 0, st>>>(q, q_scale, w, phi, plo, kk, k_scale, s.L, s.T, s.H, s.B, s.M(), m, nsplit, G, blocks, block_scores_out)
  if (s.dtype == kBF16) { if (two) HB(kBF16, 2); else HB(kBF16, 1); }
  else { if (two) HB(kFP8, 2); else HB(kFP8, 1); }
#undef HB
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (nsplit > 1) {
    const int64_t rows = static_cast<int64_t>(s.batch) * s.T;
    hisa_topm_kernel<<<static_cast<unsigned>((rows + kHWaves - 1) / kHWaves), kHThreads, 0, st>>>(
        G, s.L, s.T, s.B, s.M(), rows, m, blocks, block_scores_out);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_rerank_heads(s, hisa_cands(s, m, k), k, q, q_scale, w, kk, k_scale, blocks, m, heads,
                             nh, idx, scores_out, base + lo.rerank, st);
}

}  // namespace misa
