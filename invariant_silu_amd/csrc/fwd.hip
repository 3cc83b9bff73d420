// Forward of the AdaLN final modulation (RL-Kernel pull request 538, "What";
// rounding points of miles_diffusion pull request 108):
//
//   emb  = bf16(fl32(SiLU(temb) W^T) + b)          (scale | shift), 3072 -> 6144
//   mu   = fl32(sum_d x_d) / D,  var = fl32(sum_d (x_d - mu)^2) / D
//   rstd = 1 / sqrt(var + eps),  n = (x - mu) * rstd
//   out  = bf16((n * m) + shift),  m = bf16(1 + scale)
//
// The projection's sum for one (sample, row of W) has one fixed shape: a tree
// of 64 leaves of 48 products each (described with the kernels below).
//
// proj_block<NB> (B = NB <= 4): 8 rows of W per block (4 waves x 2 rows) in
//   registers, lane l holding leaf l of each row.  The temb loads are issued
//   first; their SiLU (silu8_fast, with the rare near-tie elements redone by
//   silu_bf16_exact: identical bits to the float64 definition) goes to LDS
//   while W is in flight.  Leaves accumulate in fp64 fused multiply-adds,
//   then wave_sum_f64; one rounding to fp32, the bias added in fp32, one
//   rounding to bf16.
// proj_mfma_kernel (B > 4): the same leaves and tree on the fp64 matrix
//   cores, from a = bf16(SiLU(temb)) computed once by silu_kernel.  emb of a
//   sample has the same bits whatever B and whichever kernel produced it.
// row_stats: one wave per row, the lane's 48 values summed in fp64 in order,
//   then wave_sum_f64; (x - mu) and its square in fp32; correctly rounded
//   sqrt and divide.
// modulate: two fp32 operations per element, one bf16 rounding.
//
// Kernels: proj_fwd_kernel / proj_mfma_kernel (adaln_proj_fwd),
// norm_mod_fwd_kernel (statistics and modulation, adaln_norm_mod_fwd), and
// for the one-call forward adaln_fwd with B <= 4 and x of at most 32 MiB:
// fwd_stage1_kernel (projection blocks and statistics blocks in one grid: two
// independent HBM streams, W and x) then norm_modulate_kernel, which re-reads
// x from the caches; with B <= 4 and a larger x, proj_fwd_kernel then
// norm_mod_fwd_kernel (x read once); with B > 4, silu_kernel and
// proj_mfma_kernel, then norm_mod_fwd_kernel.
#include "common.hpp"
#include "launch.hpp"
#include "mfma.hpp"

namespace adaln {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kLaneChunks = kChunks / 64;                  // 6
constexpr int kRows = 2;                                   // rows of W per wave
constexpr int kProjRowsPerBlock = kWaves * kRows;          // 8
constexpr int kProjBlocks = kN / kProjRowsPerBlock;        // 768
constexpr int kMaxNarrowBatch = 4;                         // proj_block up to here
// x up to this size (bytes) is read twice by the B <= 4 forward, the second
// read served by the caches right after the first; beyond it one
// statistics-and-modulation pass after the projection reads it once (the
// faster of the two there, measured)
constexpr int64_t kStage1MaxXBytes = int64_t(32) << 20;
static_assert(kN % kProjRowsPerBlock == 0 && kN6 % kProjRowsPerBlock == 0, "rows per block must divide N");

// ----------------------------------------------------------- projection ----
// The sum for one (sample, row of W) is a tree of 64 leaves.  Leaf l covers
// k in [48 l, 48 l + 48), taken as 12 steps of 4: step s adds the elements
// 48 l + 12 g + s for g = 0, 1, 2, 3 in that order, each an fp64 fused
// multiply-add of bf16-valued operands (the product is exact, the add rounds
// once), starting from +0.  The 64 leaves are then added pairwise in index
// order (0+1, 2+3, ..., then pairs of pairs).  The VALU blocks below hold
// leaf l in lane l and take the tree with wave_sum_f64; the matrix-core
// kernel feeds the same four terms of a step to one v_mfma_f64_16x16x4f64
// (a chain of four fused multiply-adds in k order) and builds the same tree
// in registers.  Every path therefore produces the same bits.
constexpr int kLeafK = kD / 64;                            // 48
constexpr int kLeafSteps = kLeafK / 4;                     // 12

template <int NB>
struct ProjShared {
  // a of each sample, per leaf (lane) 24 dwords in step-pair order: position
  // 4 t + g holds dword 6 g + t of the leaf (elements 12 g + 2t, 12 g + 2t + 1);
  // 28 dwords per lane so 16 lanes' 16-byte reads hit distinct banks
  uint32_t a[NB * 64 * 28];
};
constexpr int kLdsLane = 28;

// byte offset in ProjShared::a of dword d (0..23, natural order) of leaf l
__device__ __forceinline__ int a_lds_dword(int bb, int l, int d) {
  return (bb * 64 + l) * kLdsLane + 4 * (d % 6) + d / 6;
}

// Projection blocks for B = NB <= 4 (one pass over the samples); N rows of W.
template <int NB, int N = kN>
__device__ __forceinline__ void proj_block(const uint16_t* __restrict__ temb,
                                           const uint16_t* __restrict__ W,
                                           const uint16_t* __restrict__ bias,
                                           uint16_t* __restrict__ emb, int blk, uint32_t* a_lds) {
  constexpr int kStage = (NB * kChunks + kThreads - 1) / kThreads;
  static_assert(kStage <= 8, "redo mask holds 8 chunks of 8 elements");
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int row0 = (blk * kWaves + wave) * kRows;

  // small loads first: the memory counter drains in issue order, so the
  // SiLU below waits only for these while the W rows stay in flight
  uint4 tz[kStage];
#pragma unroll
  for (int k = 0; k < kStage; ++k) {
    const int c = threadIdx.x + kThreads * k;
    if (c < NB * kChunks) tz[k] = ld16(temb + (c / kChunks) * kD + (c % kChunks) * 8);
  }
  float bias_f[kRows];
#pragma unroll
  for (int r = 0; r < kRows; ++r) bias_f[r] = bf16_to_f32(bias[row0 + r]);
  // lane l: the 48 elements of leaf l of each row (6 x 16 bytes)
  uint4 w[kLaneChunks][kRows];
#pragma unroll
  for (int q = 0; q < kLaneChunks; ++q)
#pragma unroll
    for (int r = 0; r < kRows; ++r)
      w[q][r] = ld16(W + static_cast<int64_t>(row0 + r) * kD + lane * kLeafK + 8 * q);

  // SiLU of the NB samples into LDS (chunk c of a sample is dwords 4 (c % 6)
  // .. + 3 of leaf c / 6); elements the fast path flags are redone from
  // memory in a separate, rarely taken loop
  uint64_t redo = 0;
#pragma unroll
  for (int k = 0; k < kStage; ++k) {
    const int c = threadIdx.x + kThreads * k;
    if (c < NB * kChunks) {
      uint32_t m;
      const uint4 v = silu8_fast(tz[k], m);
      const int bb = c / kChunks, cc = c % kChunks;
      const int l = cc / 6, d0 = 4 * (cc % 6);
      a_lds[a_lds_dword(bb, l, d0 + 0)] = v.x;
      a_lds[a_lds_dword(bb, l, d0 + 1)] = v.y;
      a_lds[a_lds_dword(bb, l, d0 + 2)] = v.z;
      a_lds[a_lds_dword(bb, l, d0 + 3)] = v.w;
      redo |= static_cast<uint64_t>(m) << (8 * k);
    }
  }
  while (redo != 0) {
    const int bit = __builtin_ctzll(redo);
    redo &= redo - 1;
    const int c = threadIdx.x + kThreads * (bit / 8);
    const int e = bit % 8;
    const int bb = c / kChunks, cc = c % kChunks;
    const uint16_t h =
        silu_bf16_exact(bf16_to_f32(temb[bb * kD + cc * 8 + e]));
    reinterpret_cast<uint16_t*>(a_lds)[2 * a_lds_dword(bb, cc / 6, 4 * (cc % 6) + e / 2) + (e & 1)] = h;
  }
  __syncthreads();

  double acc[kRows][NB];
#pragma unroll
  for (int r = 0; r < kRows; ++r)
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) acc[r][bb] = 0.0;
  const uint32_t(&wd)[kLaneChunks][kRows][4] = reinterpret_cast<const uint32_t(&)[kLaneChunks][kRows][4]>(w);
#pragma unroll
  for (int t = 0; t < kLeafSteps / 2; ++t) {
    // steps 2t and 2t + 1: dwords 6 g + t of the leaf, low then high halves
    uint4 av[NB];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb)
      av[bb] = *reinterpret_cast<const uint4*>(a_lds + (bb * 64 + lane) * kLdsLane + 4 * t);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 6 * g + t;
#pragma unroll
        for (int r = 0; r < kRows; ++r) {
          const double wv = bf_half64(wd[d / 4][r][d % 4], h);
#pragma unroll
          for (int bb = 0; bb < NB; ++bb) {
            const uint32_t ad = g == 0 ? av[bb].x : g == 1 ? av[bb].y : g == 2 ? av[bb].z : av[bb].w;
            acc[r][bb] = __builtin_fma(bf_half64(ad, h), wv, acc[r][bb]);
          }
        }
      }
    }
    // the accumulators are materialised here: each step pair's fp64
    // conversions stay next to their uses instead of being kept for later
#pragma unroll
    for (int r = 0; r < kRows; ++r)
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) asm volatile("" : "+v"(acc[r][bb]));
  }
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      const double tot = wave_sum_f64(acc[r][bb]);
      if (lane == r * NB + bb) {
        const float v = static_cast<float>(tot) + bias_f[r];
        emb[bb * N + row0 + r] = f32_to_bf16(v);
      }
    }
  }
}

// ------------------------------------------------ projection, matrix cores --
// B > 4.  Block: 16 rows of W (j0 ..) x 16 kTiles samples (b0 ..); its
// kSplit waves split the 64 leaves: wave w takes leaves (64 / kSplit) w ..
// for every (sample, row) of the block, one accumulator chain per sample
// tile (the W operand is shared between them).  A lane (r = lane % 16,
// g = lane / 16) feeds v_mfma_f64_16x16x4f64 with a[b0 + 16 t + r][48 l + 12 g
// + s] and W[j0 + r][48 l + 12 g + s] at step s of leaf l: 24 contiguous bytes
// of each per leaf, loaded two leaves ahead.  A wave adds its leaf results in
// the leaf tree as they complete (in registers); the waves' subtrees meet in
// LDS, pairwise in leaf order.  Rows past B load sample B - 1 and are never
// stored.
constexpr int kMfmaRows = 16;                               // rows of W per block
constexpr int kLeafAhead = 2;                               // leaves in flight

template <int kTiles, typename T>
struct LeafRaw {
  RowRun<12, T> a[kTiles], w;   // 12 elements per operand (steps 0..11)
};

// T: storage type of a, W, bias and emb (bf16 bit patterns or fp32); N rows of W
template <int kTiles, int kSplit, typename T, int N = kN>
__global__ __launch_bounds__(64 * kSplit) void proj_mfma_kernel(const T* __restrict__ a,
                                                                const T* __restrict__ W,
                                                                const T* __restrict__ bias,
                                                                T* __restrict__ emb, int64_t B) {
  constexpr int kWaveLeaves = 64 / kSplit;
  constexpr int kSamples = 16 * kTiles;
  constexpr uint32_t kEl = sizeof(T);
  static_assert(kSplit == 1 || kSplit == 2 || kSplit == 4 || kSplit == 8, "leaf split");
  __shared__ f64x4_t sub[kSplit > 1 ? kSplit - 1 : 1][kTiles][64];
  // wave index through readfirstlane: the leaf offsets below stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int j0 = static_cast<int>(blockIdx.x) * kMfmaRows;
  const int64_t bblk = static_cast<int64_t>(blockIdx.y) * kSamples;
  const int rows_here = static_cast<int>((B - bblk) < kSamples ? (B - bblk) : kSamples);

  const Buffer abuf(a + bblk * kD, static_cast<uint32_t>(rows_here) * kD * kEl);
  const Buffer wbuf(W + static_cast<int64_t>(j0) * kD, kMfmaRows * kD * kEl);
  uint32_t a_off[kTiles];
#pragma unroll
  for (int t = 0; t < kTiles; ++t) {
    const int ra = (16 * t + r) < rows_here ? (16 * t + r) : rows_here - 1;
    a_off[t] = static_cast<uint32_t>(ra) * kD * kEl + 12 * g * kEl;
  }
  const uint32_t w_off = static_cast<uint32_t>(r) * kD * kEl + 12 * g * kEl;
  const uint32_t leaf_base = static_cast<uint32_t>(wave * kWaveLeaves) * kLeafK * kEl;

  LeafRaw<kTiles, T> raw[kLeafAhead + 1];
  auto load_leaf = [&](LeafRaw<kTiles, T>& d, int n) {
    const uint32_t off = leaf_base + static_cast<uint32_t>(n) * kLeafK * kEl;
    d.w.load(wbuf, w_off, off);
#pragma unroll
    for (int t = 0; t < kTiles; ++t) d.a[t].load(abuf, a_off[t], off);
  };
#pragma unroll
  for (int n = 0; n < kLeafAhead; ++n) load_leaf(raw[n], n);

  PairTree<ilog2(kWaveLeaves), f64x4_t> tree[kTiles];
  static_for<0, kWaveLeaves>([&](auto nc) {
    constexpr int n = decltype(nc)::value;
    if constexpr (n + kLeafAhead < kWaveLeaves) load_leaf(raw[(n + kLeafAhead) % (kLeafAhead + 1)], n + kLeafAhead);
    const LeafRaw<kTiles, T>& cur = raw[n % (kLeafAhead + 1)];
    f64x4_t acc[kTiles];
#pragma unroll
    for (int t = 0; t < kTiles; ++t) acc[t] = f64x4_t{0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int s = 0; s < kLeafSteps; ++s) {
      const double wv = cur.w.at(s);
#pragma unroll
      for (int t = 0; t < kTiles; ++t) acc[t] = mfma_f64(cur.a[t].at(s), wv, acc[t]);
    }
#pragma unroll
    for (int t = 0; t < kTiles; ++t) tree[t].template push<n>(acc[t]);
  });
  constexpr int kTop = ilog2(kWaveLeaves);

  // subtrees of the waves, pairwise in leaf order: ((w0 + w1) + (w2 + w3)) ...
  f64x4_t tot[kTiles];
#pragma unroll
  for (int t = 0; t < kTiles; ++t) tot[t] = tree[t].node[kTop];
  if constexpr (kSplit > 1) {
    if (wave > 0)
#pragma unroll
      for (int t = 0; t < kTiles; ++t) sub[wave - 1][t][lane] = tot[t];
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      f64x4_t v[kSplit];
      v[0] = tot[t];
#pragma unroll
      for (int w = 1; w < kSplit; ++w) v[w] = sub[w - 1][t][lane];
      tot[t] = pair_reduce(v);
    }
  }
  // lane holds rows g + 4 v of each sample tile, column r (row j0 + r of W)
  const float bias_f = Storage<T>::load1(bias[j0 + r]);
#pragma unroll
  for (int t = 0; t < kTiles; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int sr = 16 * t + g + 4 * v;
      if (sr < rows_here)
        emb[(bblk + sr) * N + j0 + r] = Storage<T>::store1(static_cast<float>(tot[t][v]) + bias_f);
    }
}

// ------------------------------------------------------------ LayerNorm ----
__device__ __forceinline__ void load_row(const uint16_t* __restrict__ x, int64_t row, int lane,
                                         uint4 (&xv)[kLaneChunks]) {
#pragma unroll
  for (int i = 0; i < kLaneChunks; ++i) xv[i] = ld16(x + row * kD + (lane + 64 * i) * 8);
}

__device__ __forceinline__ void row_stats(const uint4 (&xv)[kLaneChunks], float eps, float& mu,
                                          float& rs) {
  double acc = 0.0;
#pragma unroll
  for (int i = 0; i < kLaneChunks; ++i) {
    float v[8];
    unpack8(xv[i], v);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += static_cast<double>(v[e]);
  }
  mu = static_cast<float>(wave_sum_f64(acc)) / static_cast<float>(kD);
  double acc2 = 0.0;
#pragma unroll
  for (int i = 0; i < kLaneChunks; ++i) {
    float v[8];
    unpack8(xv[i], v);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float d = v[e] - mu;
      acc2 += static_cast<double>(d * d);
    }
  }
  const float var = static_cast<float>(wave_sum_f64(acc2)) / static_cast<float>(kD);
  rs = 1.0f / __builtin_sqrtf(var + eps);
}

// (1 + scale) and shift of sample b: loads (issue early), then LDS stores
struct ModRegs {
  uint2 sc[3], sh[3];
};
__device__ __forceinline__ void load_mod(const uint16_t* __restrict__ emb, int64_t b, ModRegs& r) {
  const uint2* scale = reinterpret_cast<const uint2*>(emb + b * kN);
  const uint2* shift = reinterpret_cast<const uint2*>(emb + b * kN + kD);
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    r.sc[k] = scale[threadIdx.x + kThreads * k];
    r.sh[k] = shift[threadIdx.x + kThreads * k];
  }
}
__device__ __forceinline__ void store_mod(const ModRegs& r, float4* m_lds, float4* sh_lds) {
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int c = threadIdx.x + kThreads * k;
    m_lds[c] = make_float4(round_bf16(1.0f + bf_lo(r.sc[k].x)), round_bf16(1.0f + bf_hi(r.sc[k].x)),
                           round_bf16(1.0f + bf_lo(r.sc[k].y)), round_bf16(1.0f + bf_hi(r.sc[k].y)));
    sh_lds[c] = make_float4(bf_lo(r.sh[k].x), bf_hi(r.sh[k].x), bf_lo(r.sh[k].y), bf_hi(r.sh[k].y));
  }
}

__device__ __forceinline__ void modulate(const uint4 (&xv)[kLaneChunks], float mu, float rs,
                                         const float4* m_lds, const float4* sh_lds,
                                         uint16_t* __restrict__ orow, int lane) {
#pragma unroll
  for (int i = 0; i < kLaneChunks; ++i) {
    const int c = lane + 64 * i;
    float v[8];
    unpack8(xv[i], v);
    const float4 m0 = m_lds[2 * c], m1 = m_lds[2 * c + 1];
    const float4 h0 = sh_lds[2 * c], h1 = sh_lds[2 * c + 1];
    const float mm[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
    const float hh[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float n = (v[e] - mu) * rs;
      o[e] = n * mm[e] + hh[e];
    }
    st16_nt(orow + c * 8, pack8(o));
  }
}

// ------------------------------------------------------------- kernels ----
template <int NB, int N>
__global__ __launch_bounds__(kThreads) void proj_fwd_kernel(const uint16_t* __restrict__ temb,
                                                            const uint16_t* __restrict__ W,
                                                            const uint16_t* __restrict__ bias,
                                                            uint16_t* __restrict__ emb) {
  __shared__ ProjShared<NB> sh;
  proj_block<NB, N>(temb, W, bias, emb, blockIdx.x, sh.a);
}

// 4 rows of one sample per block (one per wave): statistics and modulation
__global__ __launch_bounds__(kThreads) void norm_mod_fwd_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ emb, uint16_t* __restrict__ out,
    float* __restrict__ mean, float* __restrict__ rstd, int64_t S, float eps) {
  __shared__ float4 m_lds[kD / 4];
  __shared__ float4 sh_lds[kD / 4];
  const int64_t b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int64_t s = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  // a wave past the end redoes row S - 1 (same bytes as its owner): no branch
  // after the barrier, so the row loads stay ahead of it
  const int64_t row = b * S + (s < S ? s : S - 1);
  ModRegs mr;
  load_mod(emb, b, mr);
  uint4 xv[kLaneChunks];
  load_row(x, row, lane, xv);
  store_mod(mr, m_lds, sh_lds);
  __syncthreads();
  float mu, rs;
  row_stats(xv, eps, mu, rs);
  modulate(xv, mu, rs, m_lds, sh_lds, out + row * kD, lane);
  if (lane == 0) {
    mean[row] = mu;
    rstd[row] = rs;
  }
}

// B = NB <= 4: projection blocks [0, 768), then statistics blocks (4 rows
// each, rows of all samples in order).  The statistics run last on purpose: the block for
// rows 4i..4i+3 runs on XCD i % 8, and (S a multiple of 4) so does the
// modulation block for the same rows right after, so the second read of x
// follows the first closely (the byte counters show it served beyond L2, by
// the memory-side cache).
template <int NB>
__global__ __launch_bounds__(kThreads) void fwd_stage1_kernel(
    const uint16_t* __restrict__ temb, const uint16_t* __restrict__ W,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ emb, const uint16_t* __restrict__ x,
    float* __restrict__ mean, float* __restrict__ rstd, int64_t S, float eps) {
  constexpr int64_t B = NB;
  __shared__ ProjShared<NB> sh;
  const int blk = blockIdx.x;
  if (blk < kProjBlocks) {
    proj_block<NB>(temb, W, bias, emb, blk, sh.a);
    return;
  }
  const int64_t idx = blk - kProjBlocks;
  const int lane = threadIdx.x & 63;
  const int64_t r = idx * kWaves + (threadIdx.x >> 6);
  if (r >= B * S) return;
  uint4 xv[kLaneChunks];
  load_row(x, r, lane, xv);
  float mu, rs;
  row_stats(xv, eps, mu, rs);
  if (lane == 0) {
    mean[r] = mu;
    rstd[r] = rs;
  }
}

__global__ __launch_bounds__(kThreads) void norm_modulate_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ emb, const float* __restrict__ mean,
    const float* __restrict__ rstd, uint16_t* __restrict__ out, int64_t S) {
  __shared__ float4 m_lds[kD / 4];
  __shared__ float4 sh_lds[kD / 4];
  const int64_t b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int64_t s = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  const int64_t row = b * S + (s < S ? s : S - 1);   // as in norm_mod_fwd_kernel
  ModRegs mr;
  load_mod(emb, b, mr);
  const float mu = mean[row];
  const float rs = rstd[row];
  uint4 xv[kLaneChunks];
  load_row(x, row, lane, xv);
  store_mod(mr, m_lds, sh_lds);
  __syncthreads();
  modulate(xv, mu, rs, m_lds, sh_lds, out + row * kD, lane);
}

// ----------------------------------------------------- a block's norm site ----
// The norm sites of a block (reading of miles_diffusion pull request 108,
// "Fused-norm rounding points"), kRes selects the form:
//   ScaleResidualLayerNormScaleShift (kRes):
//     h   = bf16(residual + bf16(gate * x))      eager bf16 multiply and add
//     out = bf16((LayerNorm(h) * bf16(1 + scale)) + shift)
//   LayerNormScaleShift: out = bf16((LayerNorm(x) * bf16(1 + scale)) + shift)
// shift, scale, gate: rows of sample b at view + b * ld.  One wave per row: the
// row's h is formed in registers, stored, and goes through row_stats and
// modulate as the final modulation's x does.
template <bool kRes>
__device__ __forceinline__ void load_view(const ModView& mv, int64_t b, ModRegs& r, uint2 (&gt)[3]) {
  const uint2* shift = reinterpret_cast<const uint2*>(mv.shift + b * mv.ld);
  const uint2* scale = reinterpret_cast<const uint2*>(mv.scale + b * mv.ld);
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    r.sc[k] = scale[threadIdx.x + kThreads * k];
    r.sh[k] = shift[threadIdx.x + kThreads * k];
  }
  if (kRes) {
    const uint2* gate = reinterpret_cast<const uint2*>(mv.gate + b * mv.ld);
#pragma unroll
    for (int k = 0; k < 3; ++k) gt[k] = gate[threadIdx.x + kThreads * k];
  }
}

template <bool kRes>
__global__ __launch_bounds__(kThreads) void site_fwd_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ residual, const ModView mv,
    uint16_t* __restrict__ h, uint16_t* __restrict__ out, float* __restrict__ mean, float* __restrict__ rstd,
    int64_t S, float eps) {
  __shared__ float4 m_lds[kD / 4];
  __shared__ float4 sh_lds[kD / 4];
  __shared__ float4 gate_lds[kD / 4];
  const int64_t b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int64_t s = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  // a wave past the end redoes row S - 1 (same bytes as its owner)
  const int64_t row = b * S + (s < S ? s : S - 1);
  ModRegs mr;
  uint2 gt[3];
  load_view<kRes>(mv, b, mr, gt);
  uint4 xv[kLaneChunks], rv[kLaneChunks];
  load_row(x, row, lane, xv);
  if (kRes) load_row(residual, row, lane, rv);
  store_mod(mr, m_lds, sh_lds);
  if (kRes)
#pragma unroll
    for (int k = 0; k < 3; ++k)
      gate_lds[threadIdx.x + kThreads * k] =
          make_float4(bf_lo(gt[k].x), bf_hi(gt[k].x), bf_lo(gt[k].y), bf_hi(gt[k].y));
  __syncthreads();
  uint4 hv[kLaneChunks];
#pragma unroll
  for (int i = 0; i < kLaneChunks; ++i) {
    if (!kRes) {
      hv[i] = xv[i];
      continue;
    }
    const int c = lane + 64 * i;
    float xf[8], rf[8], hf[8];
    unpack8(xv[i], xf);
    unpack8(rv[i], rf);
    const float4 g0 = gate_lds[2 * c], g1 = gate_lds[2 * c + 1];
    const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) hf[e] = rf[e] + round_bf16(gg[e] * xf[e]);
    hv[i] = pack8(hf);
    st16_nt(h + row * kD + c * 8, hv[i]);
  }
  float mu, rs;
  row_stats(hv, eps, mu, rs);
  modulate(hv, mu, rs, m_lds, sh_lds, out + row * kD, lane);
  if (lane == 0) {
    mean[row] = mu;
    rstd[row] = rs;
  }
}

// LayerNorm statistics only (mean, rstd), one wave per row: the statistics
// blocks of fwd_stage1_kernel as a kernel of their own
__global__ __launch_bounds__(kThreads) void row_stats_kernel(const uint16_t* __restrict__ x,
                                                             float* __restrict__ mean, float* __restrict__ rstd,
                                                             int64_t rows, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  if (r >= rows) return;
  uint4 xv[kLaneChunks];
  load_row(x, r, lane, xv);
  float mu, rs;
  row_stats(xv, eps, mu, rs);
  if (lane == 0) {
    mean[r] = mu;
    rstd[r] = rs;
  }
}

// B <= 4: proj_block with NB = B; larger batches: proj_mfma_kernel
template <typename F>
hipError_t by_batch(int64_t B, F&& f) {
  switch (B) {
    case 1: return f(std::integral_constant<int, 1>{});
    case 2: return f(std::integral_constant<int, 2>{});
    case 3: return f(std::integral_constant<int, 3>{});
    case 4: return f(std::integral_constant<int, 4>{});
    default: return hipErrorInvalidValue;
  }
}

// a = SiLU(temb) computed once into `a`, then the matrix-core projection.
// Sample tiles per wave and waves per block by batch (cold timings of the
// bf16 projection): one tile and 4 waves up to 16 samples; two tiles below
// 128 (fewer blocks would idle CUs); four tiles from 128 (a converted W
// operand feeds four chains: B = 256 221 -> 202 us, B = 2048 1572 -> 1475),
// with 2 waves per block from 1024 samples (B = 2048: 1435 us).  fp32 storage
// keeps two tiles (its operands take twice the registers).
template <int kTiles, int kSplit, typename T, int N>
hipError_t launch_mfma_tiles(const T* a, const T* W, const T* bias, T* emb, int64_t B, hipStream_t s) {
  const int64_t by = (B + 16 * kTiles - 1) / (16 * kTiles);
  hipLaunchKernelGGL((proj_mfma_kernel<kTiles, kSplit, T, N>), dim3(N / kMfmaRows, static_cast<unsigned>(by)),
                     dim3(64 * kSplit), 0, s, a, W, bias, emb, B);
  return hipGetLastError();
}
template <typename T, int N = kN>
hipError_t launch_mfma_from_a(const T* a, const T* W, const T* bias, T* emb, int64_t B, hipStream_t s) {
  if (B <= 16) return launch_mfma_tiles<1, 4, T, N>(a, W, bias, emb, B, s);
  if constexpr (sizeof(T) == 2) {
    if (B >= 1024) return launch_mfma_tiles<4, 2, T, N>(a, W, bias, emb, B, s);
    if (B >= 128) return launch_mfma_tiles<4, 4, T, N>(a, W, bias, emb, B, s);
  }
  return launch_mfma_tiles<2, 4, T, N>(a, W, bias, emb, B, s);
}
template <int N = kN>
hipError_t launch_mfma(const uint16_t* temb, uint16_t* a, const uint16_t* W, const uint16_t* bias,
                       uint16_t* emb, int64_t B, hipStream_t s) {
  if (hipError_t e = launch_silu(temb, a, B * kD, s); e != hipSuccess) return e;
  return launch_mfma_from_a<uint16_t, N>(a, W, bias, emb, B, s);
}

template <int N>
hipError_t proj_fwd_rows(const uint16_t* temb, const uint16_t* W, const uint16_t* bias, uint16_t* emb,
                         uint16_t* a, int64_t B, hipStream_t s) {
  if (B > kMaxNarrowBatch) return launch_mfma<N>(temb, a, W, bias, emb, B, s);
  return by_batch(B, [&](auto nb) {
    hipLaunchKernelGGL((proj_fwd_kernel<decltype(nb)::value, N>), dim3(N / kProjRowsPerBlock), dim3(kThreads), 0,
                       s, temb, W, bias, emb);
    return hipGetLastError();
  });
}

}  // namespace

hipError_t launch_proj_fwd(const uint16_t* temb, const uint16_t* W, const uint16_t* bias,
                           uint16_t* emb, uint16_t* a, int64_t B, int64_t N, hipStream_t s) {
  if (N == kN) return proj_fwd_rows<kN>(temb, W, bias, emb, a, B, s);
  if (N == kN6) return proj_fwd_rows<kN6>(temb, W, bias, emb, a, B, s);
  return hipErrorInvalidValue;
}

hipError_t launch_norm_mod_fwd(const uint16_t* x, const uint16_t* emb, uint16_t* out, float* mean,
                               float* rstd, int64_t B, int64_t S, float eps, hipStream_t s) {
  const int64_t gx = (S + kWaves - 1) / kWaves;
  hipLaunchKernelGGL(norm_mod_fwd_kernel, dim3(static_cast<unsigned>(gx), static_cast<unsigned>(B)),
                     dim3(kThreads), 0, s, x, emb, out, mean, rstd, S, eps);
  return hipGetLastError();
}

hipError_t launch_fwd(const uint16_t* temb, const uint16_t* W, const uint16_t* bias,
                      const uint16_t* x, uint16_t* emb, uint16_t* out, float* mean, float* rstd,
                      int64_t B, int64_t S, float eps, hipStream_t s) {
  if (B > kMaxNarrowBatch) {
    // SiLU once (into the first B * 3072 elements of `out`, which the
    // modulation overwrites later), the matrix-core projection, then
    // statistics and modulation in one pass over x
    if (hipError_t e = launch_mfma(temb, out, W, bias, emb, B, s); e != hipSuccess) return e;
    return launch_norm_mod_fwd(x, emb, out, mean, rstd, B, S, eps, s);
  }
  if (B * S * kD * 2 > kStage1MaxXBytes) {
    if (hipError_t e = proj_fwd_rows<kN>(temb, W, bias, emb, nullptr, B, s); e != hipSuccess) return e;
    return launch_norm_mod_fwd(x, emb, out, mean, rstd, B, S, eps, s);
  }
  const int64_t stat_blocks = (B * S + kWaves - 1) / kWaves;
  hipError_t e = by_batch(B, [&](auto nb) {
    hipLaunchKernelGGL(fwd_stage1_kernel<decltype(nb)::value>,
                       dim3(static_cast<unsigned>(kProjBlocks + stat_blocks)), dim3(kThreads), 0, s,
                       temb, W, bias, emb, x, mean, rstd, S, eps);
    return hipGetLastError();
  });
  if (e != hipSuccess) return e;
  const int64_t gx = (S + kWaves - 1) / kWaves;
  hipLaunchKernelGGL(norm_modulate_kernel, dim3(static_cast<unsigned>(gx), static_cast<unsigned>(B)),
                     dim3(kThreads), 0, s, x, emb, mean, rstd, out, S);
  return hipGetLastError();
}

// emb, mean and rstd of the one-call forward without the modulation: B <= 4
// fwd_stage1_kernel (the same launch as adaln_fwd's first); B > 4 the SiLU into
// a, the matrix-core projection and row_stats_kernel
hipError_t launch_fwd_stats(const uint16_t* temb, const uint16_t* W, const uint16_t* bias, const uint16_t* x,
                            uint16_t* emb, float* mean, float* rstd, uint16_t* a, int64_t B, int64_t S, float eps,
                            hipStream_t s) {
  if (B > kMaxNarrowBatch) {
    if (hipError_t e = launch_mfma(temb, a, W, bias, emb, B, s); e != hipSuccess) return e;
    hipLaunchKernelGGL(row_stats_kernel, dim3(static_cast<unsigned>((B * S + kWaves - 1) / kWaves)), dim3(kThreads),
                       0, s, x, mean, rstd, B * S, eps);
    return hipGetLastError();
  }
  const int64_t stat_blocks = (B * S + kWaves - 1) / kWaves;
  return by_batch(B, [&](auto nb) {
    hipLaunchKernelGGL(fwd_stage1_kernel<decltype(nb)::value>,
                       dim3(static_cast<unsigned>(kProjBlocks + stat_blocks)), dim3(kThreads), 0, s,
                       temb, W, bias, emb, x, mean, rstd, S, eps);
    return hipGetLastError();
  });
}

hipError_t launch_proj_fwd_f32(const float* temb, float* a, const float* W, const float* bias, float* emb,
                               int64_t B, hipStream_t s) {
  if (hipError_t e = launch_silu_f32(temb, a, B * kD, s); e != hipSuccess) return e;
  if (B <= kMaxNarrowBatch) return launch_proj_f32_small(a, W, bias, emb, B, s);   // the same sums, vector units
  return launch_mfma_from_a(a, W, bias, emb, B, s);
}

hipError_t launch_site_fwd(const uint16_t* x, const uint16_t* residual, ModView mv, uint16_t* h, uint16_t* out,
                           float* mean, float* rstd, int64_t B, int64_t S, float eps, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((S + kWaves - 1) / kWaves), static_cast<unsigned>(B));
  if (residual)
    hipLaunchKernelGGL(site_fwd_kernel<true>, grid, dim3(kThreads), 0, s, x, residual, mv, h, out, mean, rstd, S,
                       eps);
  else
    hipLaunchKernelGGL(site_fwd_kernel<false>, grid, dim3(kThreads), 0, s, x, residual, mv, h, out, mean, rstd, S,
                       eps);
  return hipGetLastError();
}

}  // namespace adaln
