// Eq. (7)-(8) of the MISA summary page ("Methodology" 1) on the matrix cores,
// for bf16 and fp8 inputs.
//
// For query t the router needs S_{t,j} = sum over the floor(n_t/B) complete
// blocks of ReLU(q_{t,j} . p_b): a dense contraction of the query's H head rows
// (A operand, bf16; fp8 codes widen to bf16 exactly) with the pooled keys (B
// operand: fp32 rounded to bf16, and for bf16 inputs also the bf16 rounding of
// the remainder, so q.p = q.p_hi + q.p_lo holds to ~2^-16 -- a single bf16
// rounding of p costs ~1e-3 relative in E on short prefixes), 32x32x16 MFMA
// tiles, ReLU and a masked
// running sum on the accumulators, then one cross-lane reduction per row.
// The partial last block (B not dividing n_t) uses ReLU(mean_s q . k_s): the
// per-key dots come from the same MFMA tiles on the raw keys.  Then E_{t,j} = |w_{t,j}| * s_t * (S + partial) / M_t
// (s_t = the fp8 query scale, else 1) and the h best heads are picked by h
// rounds of a wave arg-max (ties to the lower head) and written ascending.
//
// Prefill: one wave per query (4 per workgroup); the pooled tile is converted
// to bf16 once into LDS and shared by the four waves.  (Decode has a single
// query per sequence and is routed on the vector ALU, route_decode.hip.)
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
  static_assert(N >= 0 && N < 16, "vmcnt immediate in the low field");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
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

// Load the A operand: head rows rt*32 + l%32 of query r, head-dim elements
// [64*(l/32), 64*(l/32)+64) split over 8 k-steps.  Rows >= H are zero.
template <int DT, int RT>
__device__ __forceinline__ void load_q_rows(const void* q, int64_t r, int H, bf16x8 (&a)[RT][8]) {
  const int lane = lane_id();
  const int hf = lane >> 5;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int j = rt * 32 + (lane & 31);
    if (j >= H) {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) a[rt][ks] = as_bf16x8(make_uint4(0, 0, 0, 0));
      continue;
    }
    if constexpr (DT == kBF16) {
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(q) +
                                                        (r * H + j) * kD + 64 * hf);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) a[rt][ks] = as_bf16x8(src[ks]);
    } else {
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(q) +
                                                        (r * H + j) * kD + 64 * hf);
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
        a[rt][2 * c] = as_bf16x8(make_uint4(o[0], o[1], o[2], o[3]));
        a[rt][2 * c + 1] = as_bf16x8(make_uint4(o[4], o[5], o[6], o[7]));
      }
    }
  }
}

// acc (rows x 32 blocks) = A . B_hi [+ A . B_lo]; rs += ReLU(acc) when
// col_ok.  B comes from an LDS tile of unpadded 256-byte rows (this lane's
// block row, its 64-element half) whose 16-byte chunk c of row r sits at
// chunk position c ^ (r % 16), so the 32 rows of a read hit distinct banks.
// The hi and lo products share one accumulator per row tile, the RT row
// tiles giving independent chains.
template <int RT, bool SPLIT>
__device__ __forceinline__ void accumulate_tile_sw(const bf16x8 (&a)[RT][8], const uint8_t* hb,
                                                   const uint8_t* lb, bool col_ok, f32x16 (&rs)[RT]) {
  const int lane = lane_id();
  const int r = lane & 31;
  const int hf = lane >> 5;
  const uint8_t* rowh = hb + r * (kD * 2);
  const uint8_t* rowl = lb + r * (kD * 2);
  f32x16 acc[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) acc[rt] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const int pos = (8 * hf + ks) ^ (r & 15);
    const bf16x8 bh = as_bf16x8(*reinterpret_cast<const uint4*>(rowh + 16 * pos));
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) acc[rt] = mfma32_bf16(a[rt][ks], bh, acc[rt]);
    if constexpr (SPLIT) {
      const bf16x8 bl = as_bf16x8(*reinterpret_cast<const uint4*>(rowl + 16 * pos));
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) acc[rt] = mfma32_bf16(a[rt][ks], bl, acc[rt]);
    }
  }
  if (col_ok) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 16; ++i) rs[rt][i] += relu(acc[rt][i]);
  }
}

// Sum rs over the 32 columns held by each half-wave; returns through LDS
// rowsum[row] for rows of this wave (row = rt*32 + 8*(i/4) + 4*hf + i%4).
template <int RT>
__device__ __forceinline__ void reduce_rows(f32x16 (&rs)[RT], float* rowsum) {
  const int lane = lane_id();
  const int hf = lane >> 5;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float v = rs[rt][i];
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
      if ((lane & 31) == 0) {
        const int row = rt * 32 + 8 * (i / 4) + 4 * hf + (i % 4);
        rowsum[row] = v;
      }
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

template <int DT, int RT>
__global__ __launch_bounds__(kRThreads) void route_prefill_kernel(
    const void* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    const uint16_t* __restrict__ phi, const uint16_t* __restrict__ plo, const void* __restrict__ k,
    const float* __restrict__ k_scale, int32_t* __restrict__ heads, float* __restrict__ E_out,
    int32_t L, int32_t T, int32_t H, int32_t B, int64_t M, int32_t h, int32_t nsplit,
    float* __restrict__ part) {
  constexpr bool SPLIT = DT == kBF16;
  constexpr int LB = SPLIT ? kTileBytes : 16;
  __shared__ __attribute__((aligned(16))) uint8_t h0[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t h1[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t h2[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t l0[LB];
  __shared__ __attribute__((aligned(16))) uint8_t l1[LB];
  __shared__ __attribute__((aligned(16))) uint8_t l2[LB];
  __shared__ float rowsum[kRWaves][64];
  __shared__ float partial[kRWaves][64];
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int64_t seq = blockIdx.y;
  const int t0 = blockIdx.x * kRWaves;
  const int t = t0 + wave;
  const bool active = t < T;
  const int64_t r = seq * T + (active ? t : t0);
  const int64_t pos = static_cast<int64_t>(L) - T + (active ? t : t0);
  const int64_t n = pos + 1;
  const int64_t full = n / B;
  const int64_t Mt = (n + B - 1) / B;
  // Largest complete-block count among the workgroup's queries.
  const int tl = min(t0 + kRWaves - 1, T - 1);
  const int64_t full_max = (static_cast<int64_t>(L) - T + tl + 1) / B;

  bf16x8 a[RT][8];
  load_q_rows<DT, RT>(q, r, H, a);
  f32x16 rs[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) rs[rt] = f32x16{};

  // Pooled tiles of 32 blocks reach LDS by direct buffer-to-LDS loads into
  // three buffers: while tile bt is multiplied, tiles bt+1 and bt+2 are in
  // flight.  Each thread issues NL loads per tile (instruction i of wave w
  // fills rows 8w + 4i .. +3 of a plane; lane l loads chunk
  // (l % 16) ^ (row % 16) of its row into chunk position l % 16), so a fixed
  // vmcnt wait before each barrier proves that a tile has landed.  Rows past
  // the last complete block load block 0 and are masked in the product;
  // tiles past the last repeat it, so every iteration issues the same loads.
  constexpr int NL = SPLIT ? 4 : 2;
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
      if constexpr (SPLIT) rt_load16_lds(rl, lb + 1024 * (2 * wave + i), voff);
    }
  };
  // The A-operand loads complete here (the empty asm redefines the
  // registers, so no later use waits on those loads): the counts below are
  // the tiles' alone.
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) asm volatile("" : "+v"(a[rt][ks]));
  rt_vmcnt_zero();
  const bool any = tile1 > tile0;
  if (any) {
    issue(tile0, h0, l0);
    issue(tile0 + 1, h1, l1);
  }
  auto step = [&](int64_t bt, const uint8_t* hb, const uint8_t* lb, uint8_t* nh, uint8_t* nl)
      __attribute__((always_inline)) {
    rt_vmcnt_barrier<NL>();  // tile bt has landed; every wave is done with tile bt-1
    issue(bt + 2, nh, nl);   // into tile bt-1's buffer
    accumulate_tile_sw<RT, SPLIT>(a, hb, lb, bt * 32 + (lane & 31) < full, rs);
  };
  for (int64_t bt = tile0; bt < tile1; bt += 3) {
    step(bt, h0, l0, h2, l2);
    if (bt + 1 < tile1) step(bt + 1, h1, l1, h0, l0);
    if (bt + 2 < tile1) step(bt + 2, h2, l2, h1, l1);
  }
  rt_vmcnt_zero();  // the last two tiles' loads (repeats) before the buffers are left
  reduce_rows<RT>(rs, rowsum[wave]);
  const bool has_partial = Mt > full && z == nsplit - 1;
  if (has_partial) {
    // Partial block [full*B, pos]: ReLU(q . mean of its keys) = ReLU(mean of
    // q . k_s), so the per-key dots come from the same MFMA tiles (raw keys
    // as B, 32 per column tile, fp8 codes widened to bf16 exactly and the
    // key scale applied per column), summed over the block and divided.
    f32x16 ps[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) ps[rt] = f32x16{};
    const int64_t s_lo = full * B;
    const int hf = lane >> 5;
    for (int64_t s0 = s_lo; s0 <= pos; s0 += 32) {
      const int64_t sk_i = s0 + (lane & 31);
      const bool ok = sk_i <= pos;
      const int64_t row = seq * L + (ok ? sk_i : s_lo);
      bf16x8 b[8];
      if constexpr (DT == kBF16) {
        const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(k) + row * kD + 64 * hf);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) b[ks] = as_bf16x8(src[ks]);
      } else {
        const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(k) + row * kD + 64 * hf);
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
          b[2 * c] = as_bf16x8(make_uint4(o[0], o[1], o[2], o[3]));
          b[2 * c + 1] = as_bf16x8(make_uint4(o[4], o[5], o[6], o[7]));
        }
      }
      const float skv = ok ? ((DT == kFP8) ? k_scale[row] : 1.f) : 0.f;
      f32x16 acc[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) acc[rt] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[rt] = mfma32_bf16(a[rt][ks], b[ks], acc[rt]);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 16; ++i) ps[rt][i] += acc[rt][i] * skv;
    }
    reduce_rows<RT>(ps, partial[wave]);
    __builtin_amdgcn_wave_barrier();
    if (lane < 64) {
      const float cnt = static_cast<float>(pos - s_lo + 1);
      partial[wave][lane] = fmaxf(partial[wave][lane] / cnt, 0.f);
    }
  }
  __syncthreads();
  if (!active) return;
  if (nsplit == 1) {
    const float sq = (DT == kFP8) ? q_scale[r] : 1.f;
    finalize_query(&rowsum[wave], 1, has_partial ? partial[wave] : nullptr, H, h, w, sq, r, Mt,
                   heads, E_out);
  } else {
    // Slot z: this split's block sums; slot nsplit: the partial block's term.
    float* pr = part + r * (nsplit + 1) * 64;
    pr[z * 64 + lane] = rowsum[wave][lane];
    if (z == nsplit - 1) pr[nsplit * 64 + lane] = has_partial ? partial[wave][lane] : 0.f;
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
int32_t route_splits(const Shape& s) {
  const int64_t wgs = static_cast<int64_t>((s.T + kRWaves - 1) / kRWaves) * s.batch;
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
  dim3 grid((s.T + kRWaves - 1) / kRWaves, s.batch, ns);
#define RP(DT, RT) route_prefill_kernel<DT, RT><<<grid, kRThreads, 0, st>>>(q, q_scale, w, phi, plo, k, k_scale, heads, E_out, s.L, s.T, s.H, s.B, s.M(), h, ns, part)
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
