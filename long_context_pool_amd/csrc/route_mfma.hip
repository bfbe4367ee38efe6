// Eq. (7)-(8) of the MISA summary page ("Methodology" 1) on the matrix cores,
// for bf16 and fp8 inputs.
//
// For query t the router needs S_{t,j} = sum over the floor(n_t/B) complete
// blocks of ReLU(q_{t,j} . p_b): a dense contraction of the pooled keys (A
// operand, 32 blocks per row tile: fp32 rounded to bf16, plus the bf16
// rounding of the remainder, so q.p = q.p_hi + q.p_lo holds to ~2^-16; a
// single bf16 rounding of p alone put E 2.2% off on a two-block prefix, past
// even the fp8 tolerance) with the query head rows (B operand, 32 heads per column tile,
// bf16; fp8 codes widen to bf16 exactly) on 32x32x16 MFMA tiles.  Each lane
// then holds 16 blocks of one head, so ReLU and the block sum stay in the
// lane; one cross-half add per head finishes the sum.
// The partial last block (B not dividing n_t) uses ReLU(mean_s q . k_s): the
// per-key dots come from the same MFMA tiles on the raw keys (the 32x32x16
// fragments are laid out alike for A and B, so the query fragments serve as
// A there).  Then E_{t,j} = |w_{t,j}| * s_t * (S + partial) / M_t (s_t = the
// fp8 query scale, else 1) and the h best heads are picked by h rounds of a
// wave arg-max (ties to the lower head) and written ascending.
//
// Prefill: each wave holds four column tiles of query head rows in registers
// (two queries of 64 heads, or four of 32), so every A fragment read from LDS
// feeds four MFMAs (eight with the lo plane); the 32-block pooled tiles are
// staged in LDS once per workgroup and shared by its four waves.  (Decode
// has a single query per sequence and is routed on the vector ALU,
// route_decode.hip.)
#include "common.hpp"
#include "launch.hpp"
#include "mfma.hpp"
#include "route_common.hpp"

namespace misa {

namespace {

constexpr int kRThreads = 256;
constexpr int kRWaves = 4;
constexpr int kTileBytes = 32 * kD * 2;  // one bf16 plane of a 32-block pooled tile

// Buffer resource over [base, base + bytes); direct buffer-to-LDS load of
// lane l's 16 bytes at voff to lds + 16 l (lds wave-uniform); wait until at
// most N of this wave's vector-memory operations are outstanding, then a
// workgroup barrier.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rt_rsrc(const void* base, int32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ void rt_load16_lds(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}
template <int N>
__device__ __forceinline__ void rt_vmcnt_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits: [3:0] and [15:14]");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
__device__ __forceinline__ void rt_vmcnt_zero() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// The wave-uniform value of a pointer, pinned to scalar registers.
template <class T>
__device__ __forceinline__ T* rt_uniform(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<T*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Column tiles (32 query heads each) per wave.  Two (one query of 64 heads)
// measured the same at 3% more time, and running one tile's block sums
// among the next tile's MFMAs (two accumulator sets) gained nothing: the
// kernel is not limited by the epilogue's issue slots.
constexpr int kRCols = 4;

// One 32x32x16 fragment set of a head row (either operand): this lane's head
// row `row` (< 0: zeros), head-dim elements [64*(l/32), 64*(l/32)+64) over 8
// k-steps; fp8 codes widen to bf16 exactly.
template <int DT>
__device__ __forceinline__ void load_head_frags(const void* q, int64_t row, bf16x8 (&a)[8]) {
  const int hf = lane_id() >> 5;
  if (row < 0) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) a[ks] = as_bf16x8(make_uint4(0, 0, 0, 0));
    return;
  }
  if constexpr (DT == kBF16) {
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(q) + row * kD + 64 * hf);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) a[ks] = as_bf16x8(src[ks]);
  } else {
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(q) + row * kD + 64 * hf);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 v = src[c];  // 16 fp8 codes = k-steps 2c, 2c+1
      const uint32_t wds[4] = {v.x, v.y, v.z, v.w};
      uint32_t o[8];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        // e4m3 -> fp32 is exact and bf16 holds the 4-bit significand exactly.
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

// One 32-block pooled tile against the wave's kRCols column tiles:
// acc[c] (blocks x heads) = P_hi . Q_c + P_lo . Q_c, then rs[c] += the
// lane's 16 blocks of ReLU(acc[c]) -- all of them (MASK false), or those of
// tile row < lim[c] (the column's complete-block count minus the tile's first
// block).  P comes from an LDS tile of unpadded 256-byte rows whose 16-byte
// chunk c of row r sits at chunk position c ^ (r % 16), so the 32 rows of a
// read hit distinct banks; each fragment read feeds kRCols MFMAs.
template <bool MASK>
__device__ __forceinline__ void accumulate_tile(const bf16x8 (&bq)[kRCols][8], const uint8_t* hb,
                                                const uint8_t* lb, const int (&lim)[kRCols],
                                                float (&rs)[kRCols]) {
  const int lane = lane_id();
  const int r = lane & 31;
  const int hf = lane >> 5;
  const uint8_t* rowh = hb + r * (kD * 2);
  const uint8_t* rowl = lb + r * (kD * 2);
  f32x16 acc[kRCols];
#pragma unroll
  for (int c = 0; c < kRCols; ++c) acc[c] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const int pos = (8 * hf + ks) ^ (r & 15);
    const bf16x8 ph = as_bf16x8(*reinterpret_cast<const uint4*>(rowh + 16 * pos));
#pragma unroll
    for (int c = 0; c < kRCols; ++c) acc[c] = mfma32_bf16(ph, bq[c][ks], acc[c]);
    const bf16x8 pl = as_bf16x8(*reinterpret_cast<const uint4*>(rowl + 16 * pos));
#pragma unroll
    for (int c = 0; c < kRCols; ++c) acc[c] = mfma32_bf16(pl, bq[c][ks], acc[c]);
  }
#pragma unroll
  for (int c = 0; c < kRCols; ++c) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float v = relu(acc[c][i]);
      if constexpr (MASK) s += (8 * (i / 4) + 4 * hf + (i % 4) < lim[c]) ? v : 0.f;
      else s += v;
    }
    rs[c] += s;
  }
}

// Pooled keys -> bf16 hi and lo (bf16 rounding of the remainder) planes,
// [batch*M, 128] each; one thread per 4 elements.
__global__ void pooled_split_kernel(const float* __restrict__ pooled, uint32_t* __restrict__ hi,
                                    uint32_t* __restrict__ lo, int64_t n4) {
  const int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  if (i >= n4) return;
  const float4 x = reinterpret_cast<const float4*>(pooled)[i];
  uint32_t h0, h1, l0, l1;
  split_bf16(x, h0, h1, l0, l1);
  hi[2 * i] = h0;
  hi[2 * i + 1] = h1;
  lo[2 * i] = l0;
  lo[2 * i + 1] = l1;
}

// HG: 32-head groups per query (1 for H <= 32, 2 for H <= 64); the wave's
// kRCols column tiles are its kRCols / HG queries' head groups.
// Pooled-tile buffers per workgroup (16 KiB per tile: the hi and lo bf16
// planes); NBUF - 1 tiles are in flight.  Deeper rings (up to eight tiles of
// one plane) measured the same: the tiles come from L2.  The budget is two
// workgroups per CU with the partial-block staging.
constexpr int kRNBuf = 3;

template <int DT, int HG>
__global__ __launch_bounds__(kRThreads, 2) void route_prefill_kernel(
    const void* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    const uint16_t* __restrict__ phi, const uint16_t* __restrict__ plo, const void* __restrict__ k,
    const float* __restrict__ k_scale, int32_t* __restrict__ heads, float* __restrict__ E_out,
    int32_t L, int32_t T, int32_t H, int32_t B, int64_t M, int32_t h, int32_t nsplit,
    float* __restrict__ part) {
  constexpr int QW = kRCols / HG;         // queries per wave
  constexpr int QWG = QW * kRWaves;       // queries per workgroup
  constexpr int NBUF = kRNBuf;            // tile buffers: NBUF - 1 tiles in flight
  __shared__ __attribute__((aligned(16))) uint8_t hbuf[NBUF][kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t lbuf[NBUF][kTileBytes];
  __shared__ float rowsum[kRWaves][QW][64];
  __shared__ float partial[kRWaves][QW][64];
  // Raw keys of the workgroup's partial blocks, [full_min B, last position]:
  // at most B + QWG - 1 rows, staged once for all its queries when they fit
  // (16-byte chunk c of row r at chunk position c ^ (r % chunks per row)).
  constexpr int ROWB = DT == kBF16 ? kD * 2 : kD;
  constexpr int CPR = ROWB / 16;
  constexpr int kPartRows = DT == kBF16 ? 80 : 160;  // B = 64 (bf16) or 128 (fp8) + QWG - 1 rows
  constexpr int kPartLoads = kPartRows * ROWB / 1024 / kRWaves;  // 1 KiB loads per wave
  static_assert(kPartLoads * kRWaves * 1024 == kPartRows * ROWB, "whole loads per wave");
  __shared__ __attribute__((aligned(16))) uint8_t pkeys[kPartRows * ROWB];
  __shared__ float pscale[DT == kFP8 ? kRWaves * 64 : 1];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = lane_id();
  const int hf = lane >> 5;
  const int64_t seq = blockIdx.y;
  const int t0 = blockIdx.x * QWG;
  const int tw = t0 + wave * QW;  // first query of this wave
  // Complete-block counts: the workgroup's smallest and largest.
  const int tl = min(t0 + QWG - 1, T - 1);
  const int64_t full_min = (static_cast<int64_t>(L) - T + t0 + 1) / B;
  const int64_t full_max = (static_cast<int64_t>(L) - T + tl + 1) / B;

  int64_t full_c[kRCols];
#pragma unroll
  for (int c = 0; c < kRCols; ++c) {
    const int t = tw + c / HG;
    full_c[c] = t < T ? (static_cast<int64_t>(L) - T + t + 1) / B : 0;
  }
  float rs[kRCols];
#pragma unroll
  for (int c = 0; c < kRCols; ++c) rs[c] = 0.f;

  // Pooled tiles of 32 blocks reach LDS by direct buffer-to-LDS loads into
  // NBUF buffers: while tile bt is multiplied, tiles bt+1 .. bt+NBUF-1 are in
  // flight.  Each thread issues NL loads per tile (instruction i of wave w
  // fills rows 8w + 4i .. +3 of a plane; lane l loads chunk
  // (l % 16) ^ (row % 16) of its row into chunk position l % 16), so a fixed
  // vmcnt wait before each barrier proves that a tile has landed.  Rows past
  // the last complete block load block 0 and are masked in the sums; tiles
  // past the last repeat it, so every iteration issues the same loads.
  constexpr int NL = 4;
  // Split z of nsplit takes tiles [tile0, tile1) (nsplit > 1: few query
  // groups, so the blocks are spread over more workgroups; the partial sums
  // then go to `part` and a finalize kernel adds them in split order).
  const int z = blockIdx.z;
  const int64_t ntiles_all = (full_max + 31) / 32;
  const int64_t tps = (ntiles_all + nsplit - 1) / nsplit;
  const int64_t tile0 = min<int64_t>(static_cast<int64_t>(z) * tps, ntiles_all);
  const int64_t tile1 = min<int64_t>(tile0 + tps, ntiles_all);
  const int64_t last = tile1 > tile0 ? tile1 - 1 : tile0;
  const __amdgpu_buffer_rsrc_t rh = rt_rsrc(rt_uniform(phi + seq * M * kD), static_cast<int32_t>(M * kD * 2));
  const __amdgpu_buffer_rsrc_t rl = rt_rsrc(rt_uniform(plo + seq * M * kD), static_cast<int32_t>(M * kD * 2));
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
      rt_load16_lds(rh, hb + 1024 * (2 * wave + i), voff);
      rt_load16_lds(rl, lb + 1024 * (2 * wave + i), voff);
    }
  };
  // Issue order: the partial-block keys (last split), the first NBUF - 1
  // tiles, then the query rows, so that the three latencies overlap; all of
  // it has landed at the wait below, after which each step issues one tile.
  const int64_t p_base = full_min * B;
  const int64_t p_cnt = static_cast<int64_t>(L) - T + tl - p_base + 1;
  const bool staged = z == nsplit - 1 && p_cnt <= kPartRows;  // workgroup-uniform
  if (staged) {
    const uint8_t* kb0 = static_cast<const uint8_t*>(k) + (seq * L + p_base) * static_cast<int64_t>(ROWB);
    const __amdgpu_buffer_rsrc_t rk = rt_rsrc(rt_uniform(kb0), static_cast<int32_t>(p_cnt * ROWB));
#pragma unroll
    for (int i = 0; i < kPartLoads; ++i) {
      const int o = 1024 * (wave * kPartLoads + i) + 16 * lane;  // LDS byte of this lane's chunk
      const int row = o / ROWB, pc = (o % ROWB) / 16;
      rt_load16_lds(rk, pkeys + 1024 * (wave * kPartLoads + i),
                    static_cast<uint32_t>(row * ROWB + 16 * (pc ^ (row % CPR))));
    }
    if constexpr (DT == kFP8) {
      const __amdgpu_buffer_rsrc_t rs_k =
          rt_rsrc(rt_uniform(k_scale + seq * L + p_base), static_cast<int32_t>(p_cnt * 4));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_k, (__attribute__((address_space(3))) void*)(pscale + 64 * wave),
                                               4, static_cast<uint32_t>(4 * (64 * wave + lane)), 0, 0, 0);
    }
  }
  const bool any = tile1 > tile0;
  if (any) {
#pragma unroll
    for (int u = 0; u + 1 < NBUF; ++u) issue(tile0 + u, hbuf[u], lbuf[u]);
  }
  // B operand: column tile c = query tw + c / HG, heads 32 (c % HG) + l % 32.
  bf16x8 bq[kRCols][8];
#pragma unroll
  for (int c = 0; c < kRCols; ++c) {
    const int t = tw + c / HG;
    const int j = 32 * (c % HG) + (lane & 31);
    load_head_frags<DT>(q, (t < T && j < H) ? (seq * T + t) * H + j : -1, bq[c]);
  }
  rt_vmcnt_zero();
  auto tile_lim = [&](int64_t bt, int (&lim)[kRCols]) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < kRCols; ++c) lim[c] = static_cast<int>(full_c[c] - bt * 32);
  };
  // Tile bt sits in buffer (bt - tile0) % NBUF; the loop is unrolled by
  // NBUF so that every buffer reference is static.
  for (int64_t base = tile0; base < tile1; base += NBUF) {
#pragma unroll
    for (int u = 0; u < NBUF; ++u) {
      const int64_t bt = base + u;
      if (bt >= tile1) break;
      // Tile bt has landed (the NBUF - 2 tiles after it may be in flight);
      // every wave is done with tile bt-1, whose buffer takes tile
      // bt + NBUF - 1.
      rt_vmcnt_barrier<NL * (NBUF - 2)>();
      issue(bt + NBUF - 1, hbuf[(u + NBUF - 1) % NBUF], lbuf[(u + NBUF - 1) % NBUF]);
      int lim[kRCols];
      tile_lim(bt, lim);
      if ((bt + 1) * 32 <= full_min) accumulate_tile<false>(bq, hbuf[u], lbuf[u], lim, rs);
      else accumulate_tile<true>(bq, hbuf[u], lbuf[u], lim, rs);
    }
  }
  rt_vmcnt_zero();  // the last tiles' loads (repeats) before the buffers are left
  // Head sums: the two half-waves held different blocks of the same head.
#pragma unroll
  for (int c = 0; c < kRCols; ++c) {
    const float v = rs[c] + __shfl_xor(rs[c], 32, kWave);
    if (lane < 32) rowsum[wave][c / HG][32 * (c % HG) + lane] = v;
  }
  // Partial block [full*B, pos] of each query (last split only): ReLU(q .
  // mean of its keys) = ReLU(mean of q . k_s).  The per-key dots come from
  // MFMA tiles with the query fragments as A (rows = heads) and 32 raw keys
  // as B (fp8 codes widened to bf16 exactly, the key scale applied per
  // column), summed over the block's keys and divided by their count.  The
  // keys come from the staged LDS rows, or from global memory when the
  // workgroup's partial blocks did not fit (B large against the staging).
  __syncthreads();  // every wave's staged rows have landed (each waited above)
  // B fragments of staged key row `row` (relative to p_base).
  auto staged_frags = [&](int row, bf16x8 (&kb)[8]) __attribute__((always_inline)) {
    const uint8_t* kr = pkeys + row * ROWB;
    if constexpr (DT == kBF16) {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        kb[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(kr + 16 * ((8 * hf + ks) ^ (row % CPR))));
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 v = *reinterpret_cast<const uint4*>(kr + 16 * ((4 * hf + c) ^ (row % CPR)));
        const uint32_t wds[4] = {v.x, v.y, v.z, v.w};
        uint32_t o[8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float f0 = fp8_to_f32(wds[u] & 0xFF), f1 = fp8_to_f32((wds[u] >> 8) & 0xFF);
          const float f2 = fp8_to_f32((wds[u] >> 16) & 0xFF), f3 = fp8_to_f32(wds[u] >> 24);
          o[2 * u] = (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xFFFF0000u);
          o[2 * u + 1] = (__float_as_uint(f2) >> 16) | (__float_as_uint(f3) & 0xFFFF0000u);
        }
        kb[2 * c] = as_bf16x8(make_uint4(o[0], o[1], o[2], o[3]));
        kb[2 * c + 1] = as_bf16x8(make_uint4(o[4], o[5], o[6], o[7]));
      }
    }
  };
  bool has_partial[QW];
#pragma unroll
  for (int qw = 0; qw < QW; ++qw) {
    const int t = tw + qw;
    const int64_t n = static_cast<int64_t>(L) - T + t + 1;
    has_partial[qw] = t < T && n % B != 0 && z == nsplit - 1;
    if (!has_partial[qw]) continue;
    const int64_t pos = n - 1;
    const int64_t s_lo = (n / B) * B;
    f32x16 ps[HG];
#pragma unroll
    for (int g = 0; g < HG; ++g) ps[g] = f32x16{};
    for (int64_t s0 = s_lo; s0 <= pos; s0 += 32) {
      const int64_t sk_i = s0 + (lane & 31);
      const bool ok = sk_i <= pos;
      const int64_t row = seq * L + (ok ? sk_i : s_lo);
      bf16x8 kb[8];
      float skv;
      if (staged) {
        const int sr = static_cast<int>((ok ? sk_i : s_lo) - p_base);
        staged_frags(sr, kb);
        skv = ok ? ((DT == kFP8) ? pscale[sr] : 1.f) : 0.f;
      } else {
        load_head_frags<DT>(k, row, kb);
        skv = ok ? ((DT == kFP8) ? k_scale[row] : 1.f) : 0.f;
      }
      f32x16 acc[HG];
#pragma unroll
      for (int g = 0; g < HG; ++g) acc[g] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int g = 0; g < HG; ++g) acc[g] = mfma32_bf16(bq[qw * HG + g][ks], kb[ks], acc[g]);
#pragma unroll
      for (int g = 0; g < HG; ++g)
#pragma unroll
        for (int i = 0; i < 16; ++i) ps[g][i] += acc[g][i] * skv;
    }
    // Sum over the 32 key columns of each half-wave; rows are heads.
#pragma unroll
    for (int g = 0; g < HG; ++g)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float v = ps[g][i];
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
        if ((lane & 31) == 0) partial[wave][qw][32 * g + 8 * (i / 4) + 4 * hf + (i % 4)] = v;
      }
    __builtin_amdgcn_wave_barrier();
    const float cnt = static_cast<float>(pos - s_lo + 1);
    partial[wave][qw][lane] = fmaxf(partial[wave][qw][lane] / cnt, 0.f);
  }
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int qw = 0; qw < QW; ++qw) {
    const int t = tw + qw;
    if (t >= T) break;
    const int64_t r = seq * T + t;
    const int64_t n = static_cast<int64_t>(L) - T + t + 1;
    const int64_t Mt = (n + B - 1) / B;
    if (nsplit == 1) {
      const float sq = (DT == kFP8) ? q_scale[r] : 1.f;
      finalize_query(&rowsum[wave][qw], 1, has_partial[qw] ? partial[wave][qw] : nullptr, H, h, w,
                     sq, r, Mt, heads, E_out);
    } else {
      // Slot z: this split's block sums; slot nsplit: the partial-block term.
      float* pr = part + r * (nsplit + 1) * 64;
      pr[z * 64 + lane] = rowsum[wave][qw][lane];
      if (z == nsplit - 1) pr[nsplit * 64 + lane] = has_partial[qw] ? partial[wave][qw][lane] : 0.f;
    }
  }
}

// Split router, second step: query row r's split sums added in split order,
// plus its partial-block term, then E and the top-h heads.
__global__ __launch_bounds__(kWave) void route_split_finalize_kernel(
    const float* __restrict__ part, const float* __restrict__ q_scale, const float* __restrict__ w,
    int32_t* __restrict__ heads, float* __restrict__ E_out, int32_t L, int32_t T, int32_t H, int32_t B,
    int32_t h, int32_t nsplit, int32_t fp8) {
  __shared__ float rowsum[1][64];
  __shared__ float ptail[64];
  const int lane = lane_id();
  const int64_t r = blockIdx.x;
  const int64_t n = static_cast<int64_t>(L) - T + 1 + r % T;
  const int64_t full = n / B;
  const int64_t Mt = (n + B - 1) / B;
  const float* pr = part + r * (nsplit + 1) * 64;
  // Every load in flight at once (nsplit <= 64), then the adds in order.
  float v[65];
#pragma unroll
  for (int z = 0; z < 65; ++z) v[z] = z <= nsplit ? pr[z * 64 + lane] : 0.f;
  float sum = 0.f;
#pragma unroll
  for (int z = 0; z < 64; ++z) sum += z < nsplit ? v[z] : 0.f;
  float tail = 0.f;
#pragma unroll
  for (int z = 0; z < 65; ++z) tail = z == nsplit ? v[z] : tail;
  rowsum[0][lane] = sum;
  ptail[lane] = tail;
  __builtin_amdgcn_wave_barrier();
  const float sq = fp8 ? q_scale[r] : 1.f;
  finalize_query(rowsum, 1, Mt > full ? ptail : nullptr, H, h, w, sq, r, Mt, heads, E_out);
}

}  // namespace

bool route_mfma_supported(const Shape& s) { return s.dtype != kF32 && s.H <= 64 && s.T > 1; }

// Block splits per query group: enough workgroups (about 512) to spread the
// pooled keys over the chip when the queries alone do not.
int32_t route_qwg(const Shape& s) { return kRCols / (s.H > 32 ? 2 : 1) * kRWaves; }

int32_t route_splits(const Shape& s) {
  const int64_t wgs = static_cast<int64_t>((s.T + route_qwg(s) - 1) / route_qwg(s)) * s.batch;
  if (wgs >= 512) return 1;
  const int64_t tiles = (s.M() + 31) / 32;
  int64_t n = (512 + wgs - 1) / wgs;
  n = n < tiles ? n : tiles;
  return static_cast<int32_t>(n < 1 ? 1 : (n > 64 ? 64 : n));
}

size_t route_mfma_ws_bytes(const Shape& s) {
  const int32_t ns = route_splits(s);
  const size_t part = ns > 1 ? align_up(static_cast<size_t>(s.batch) * s.T * (ns + 1) * 64 * sizeof(float)) : 0;
  return 2 * align_up(static_cast<size_t>(s.batch) * s.M() * kD * sizeof(uint16_t)) + part;
}

hipError_t launch_pooled_split(const Shape& s, const float* pooled, uint16_t* hi, uint16_t* lo,
                               hipStream_t st) {
  const int64_t n4 = static_cast<int64_t>(s.batch) * s.M() * kD / 4;
  pooled_split_kernel<<<static_cast<unsigned>((n4 + 255) / 256), 256, 0, st>>>(
      pooled, reinterpret_cast<uint32_t*>(hi), reinterpret_cast<uint32_t*>(lo), n4);
  return hipGetLastError();
}

hipError_t launch_route_mfma(const Shape& s, int32_t h, const void* q, const float* q_scale,
                             const float* w, const float* pooled, const void* k,
                             const float* k_scale, int32_t* heads, float* E_out, void* ws,
                             hipStream_t st) {
  const size_t plane = align_up(static_cast<size_t>(s.batch) * s.M() * kD * sizeof(uint16_t));
  uint16_t* phi = static_cast<uint16_t*>(ws);
  uint16_t* plo = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + plane);
  const int64_t n4 = static_cast<int64_t>(s.batch) * s.M() * kD / 4;
  pooled_split_kernel<<<static_cast<unsigned>((n4 + 255) / 256), 256, 0, st>>>(
      pooled, reinterpret_cast<uint32_t*>(phi), reinterpret_cast<uint32_t*>(plo), n4);
  const bool two = s.H > 32;
  const int32_t ns = route_splits(s);
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + 2 * plane);
  dim3 grid((s.T + route_qwg(s) - 1) / route_qwg(s), s.batch, ns);
#define RP(DT, HG) route_prefill_kernel<DT, HG><<<grid, kRThreads, 0, st>>>(q, q_scale, w, phi, plo, k, k_scale, heads, E_out, s.L, s.T, s.H, s.B, s.M(), h, ns, part)
  if (s.dtype == kBF16) { if (two) RP(kBF16, 2); else RP(kBF16, 1); }
  else { if (two) RP(kFP8, 2); else RP(kFP8, 1); }
#undef RP
  if (ns > 1) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    route_split_finalize_kernel<<<static_cast<unsigned>(s.batch) * s.T, kWave, 0, st>>>(
        part, q_scale, w, heads, E_out, s.L, s.T, s.H, s.B, h, ns, s.dtype == kFP8 ? 1 : 0);
  }
  return hipGetLastError();
}

}  // namespace misa
