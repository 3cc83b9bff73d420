// Backward of the AdaLN final modulation (RL-Kernel pull request 538, "What";
// token sums per the review-thread fix of token_sum.cu; SiLU VJP per the
// review thread).
//
// LayerNorm + modulation, per row r = (b, s), with m = bf16(1 + scale) and n
// recomputed exactly as in the forward from the saved mean / rstd:
//   gy    = g * m                            (exact: bf16 x bf16)
//   alpha = fl32(sum_d gy) / D,  beta = fl32(sum_d gy * n) / D
//   dx    = bf16(rstd * ((gy - alpha) - n * beta))
//   (fp64 lane partials, chunks and columns in order, then wave_sum_f64)
// and the level-0 pairs of the token tree, per (b, 32-token tile, column):
// Neumaier (s, c) of g (-> d_shift) and of g * n (-> d_scale), tokens in
// ascending order.  Levels >= 1 are folded by tree_fold_kernel.
//
// Projection, from the fp32 d_emb = (d_scale | d_shift):
//   dW[j,k]  = bf16(fl32(sum_b d_emb[b,j] * a[b,k]))      (fp32 products)
//   db[j]    = bf16(fl32(sum_b d_emb[b,j]))
//   da[b,k]  = fl32(sum_j d_emb[b,j] * W[j,k])             (fp32 products)
//   dtemb    = bf16(da * silu'(temb))
// Sums accumulate fp32 products in fp64 in fixed orders: samples ascending
// for dW and db; for da, 32 parts of 192 rows, in a part 8 row slots walking
// every 8th row in order, slots as a pairwise tree, parts added in order.
//
// Device pieces are shared by every kernel, so the standalone entry points
// and the overlapped stage kernel compute identical bits, and no order
// depends on the batch size or the grid.
//
// Kernels:
//   norm_mod_bwd_kernel<role>  dx rows and/or level-0 tiles of a 32-token
//                              tile, the 14 blocks of a tile on one XCD
//   proj_bwd_small_kernel<NB>  B <= 4: dW-writing and W-reading blocks in one grid
//   silu/dW/da kernels         B > 4
//   proj_bwd_final_kernel      dtemb from the partials, and db
//   bwd_stage2_kernel<NB>      one-call backward, B <= 4: da-partial blocks,
//                              dW blocks and dx row blocks side by side
#include <hip/hip_ext.h>

#include "common.hpp"
#include "launch.hpp"

namespace adaln {

namespace {

constexpr int kThreads = 256;
constexpr int kLaneChunks = kChunks / 64;          // 6
constexpr int kRowBlocks = kTile / 4;              // 8 row blocks of 4 rows per tile
constexpr int kColPairs = kThreads;                // 256 column pairs per column block
constexpr int kColBlockCols = 2 * kColPairs;       // 512 columns
constexpr int kColBlocks = kD / kColBlockCols;     // 6
constexpr int kBlocksPerTile = kRowBlocks + kColBlocks;   // 14

enum Role { kBoth = 0, kRowsOnly = 1, kColsOnly = 2 };

__device__ __forceinline__ void row_pass(const uint16_t* __restrict__ g, const uint16_t* __restrict__ x,
                                         const float* __restrict__ mean, const float* __restrict__ rstd,
                                         const uint16_t* __restrict__ emb, uint16_t* __restrict__ dx,
                                         int64_t b, int64_t s, int64_t S, float4* m_lds) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const bool valid = s < S;
  const int64_t row = b * S + (valid ? s : 0);

  // small loads first: the memory counter drains in issue order, so staging
  // m needs only these, while the row loads below stay in flight
  const uint2* scale = reinterpret_cast<const uint2*>(emb + b * kN);
  uint2 sc[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) sc[k] = scale[threadIdx.x + kThreads * k];
  uint4 gv[kLaneChunks], xv[kLaneChunks];
#pragma unroll
  for (int i = 0; i < kLaneChunks; ++i) {
    gv[i] = ld16(g + row * kD + (lane + 64 * i) * 8);
    xv[i] = ld16(x + row * kD + (lane + 64 * i) * 8);
  }
  const float mu = mean[row];
  const float rs = rstd[row];
#pragma unroll
  for (int k = 0; k < 3; ++k)
    m_lds[threadIdx.x + kThreads * k] =
        make_float4(round_bf16(1.0f + bf_lo(sc[k].x)), round_bf16(1.0f + bf_hi(sc[k].x)),
                    round_bf16(1.0f + bf_lo(sc[k].y)), round_bf16(1.0f + bf_hi(sc[k].y)));
  __syncthreads();
  (void)wave;
  if (!valid) return;   // whole wave

  double q1 = 0.0, q2 = 0.0;
#pragma unroll
  for (int i = 0; i < kLaneChunks; ++i) {
    const int c = lane + 64 * i;
    float gf[8], xf[8];
    unpack8(gv[i], gf);
    unpack8(xv[i], xf);
    const float4 m0 = m_lds[2 * c], m1 = m_lds[2 * c + 1];
    const float mm[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float n = (xf[e] - mu) * rs;
      const float gy = gf[e] * mm[e];
      q1 += static_cast<double>(gy);
      q2 += static_cast<double>(gy * n);
    }
  }
  const float alpha = static_cast<float>(wave_sum_f64(q1)) / static_cast<float>(kD);
  const float beta = static_cast<float>(wave_sum_f64(q2)) / static_cast<float>(kD);
  // keep the packed rows packed across the reduction (recompute below rather
  // than hold 96 unpacked values in registers)
#pragma unroll
  for (int i = 0; i < kLaneChunks; ++i) {
    asm volatile("" : "+v"(gv[i].x), "+v"(gv[i].y), "+v"(gv[i].z), "+v"(gv[i].w));
    asm volatile("" : "+v"(xv[i].x), "+v"(xv[i].y), "+v"(xv[i].z), "+v"(xv[i].w));
  }

  uint16_t* drow = dx + row * kD;
#pragma unroll
  for (int i = 0; i < kLaneChunks; ++i) {
    const int c = lane + 64 * i;
    float gf[8], xf[8], d[8];
    unpack8(gv[i], gf);
    unpack8(xv[i], xf);
    const float4 m0 = m_lds[2 * c], m1 = m_lds[2 * c + 1];
    const float mm[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float n = (xf[e] - mu) * rs;
      const float gy = gf[e] * mm[e];
      d[e] = rs * ((gy - alpha) - n * beta);
    }
    st16_nt(drow + c * 8, pack8(d));
  }
}

__device__ __forceinline__ void col_pass(const uint16_t* __restrict__ g, const uint16_t* __restrict__ x,
                                         const float* __restrict__ mean, const float* __restrict__ rstd,
                                         float* __restrict__ part_s, float* __restrict__ part_c,
                                         int64_t b, int64_t tile, int cb, int64_t S, int64_t T0,
                                         float* mu_s, float* rs_s) {
  const int col = cb * kColBlockCols + 2 * threadIdx.x;
  const int rows = static_cast<int>((S - tile * kTile) < kTile ? (S - tile * kTile) : kTile);
  const int64_t row0 = b * S + tile * kTile;

  float mu_l = 0.0f, rs_l = 0.0f;
  if (threadIdx.x < rows) {
    mu_l = mean[row0 + threadIdx.x];
    rs_l = rstd[row0 + threadIdx.x];
  }
  uint32_t gw[kTile], xw[kTile];
#pragma unroll
  for (int r = 0; r < kTile; ++r) {
    if (r < rows) {
      const int64_t off = (row0 + r) * kD + col;
      gw[r] = *reinterpret_cast<const uint32_t*>(g + off);
      xw[r] = *reinterpret_cast<const uint32_t*>(x + off);
    }
  }
  if (threadIdx.x < rows) {
    mu_s[threadIdx.x] = mu_l;
    rs_s[threadIdx.x] = rs_l;
  }
  __syncthreads();

  float sg0 = 0.0f, cg0 = 0.0f, sg1 = 0.0f, cg1 = 0.0f;
  float sn0 = 0.0f, cn0 = 0.0f, sn1 = 0.0f, cn1 = 0.0f;
#pragma unroll
  for (int r = 0; r < kTile; ++r) {
    if (r < rows) {
      const float mu = mu_s[r], rs = rs_s[r];
      const float g0 = bf_lo(gw[r]), g1 = bf_hi(gw[r]);
      const float n0 = (bf_lo(xw[r]) - mu) * rs;
      const float n1 = (bf_hi(xw[r]) - mu) * rs;
      neumaier_add(sg0, cg0, g0);
      neumaier_add(sg1, cg1, g1);
      neumaier_add(sn0, cn0, g0 * n0);
      neumaier_add(sn1, cn1, g1 * n1);
    }
  }
  // columns [0, D) of d_emb: d_scale (g * n); [D, 2D): d_shift (g)
  const int64_t base = (b * T0 + tile) * kN + col;
  *reinterpret_cast<float2*>(part_s + base) = make_float2(sn0, sn1);
  *reinterpret_cast<float2*>(part_c + base) = make_float2(cn0, cn1);
  *reinterpret_cast<float2*>(part_s + base + kD) = make_float2(sg0, sg1);
  *reinterpret_cast<float2*>(part_c + base + kD) = make_float2(cg0, cg1);
}

// grid: 1-D, ceil(B*T0 / 8) * 8 * blocks_per_tile blocks (blocks_per_tile = 14,
// 8 or 6 for kBoth / kRowsOnly / kColsOnly).  Block L runs on XCD L % 8; on
// that XCD its index j = L / 8 selects tile (j / bpt) * 8 + L % 8 and role j % bpt.
template <int kRole>
__global__ __launch_bounds__(kThreads) void norm_mod_bwd_kernel(
    const uint16_t* __restrict__ g, const uint16_t* __restrict__ x,
    const float* __restrict__ mean, const float* __restrict__ rstd,
    const uint16_t* __restrict__ emb, uint16_t* __restrict__ dx,
    float* __restrict__ part_s, float* __restrict__ part_c, int64_t B, int64_t S, int64_t T0) {
  constexpr int bpt = kRole == kBoth ? kBlocksPerTile : (kRole == kRowsOnly ? kRowBlocks : kColBlocks);
  __shared__ float4 m_lds[kD / 4];   // row blocks: m = bf16(1 + scale); column blocks: mean/rstd
  const int64_t L = blockIdx.x;
  const int64_t j = L >> 3;
  const int64_t G = (j / bpt) * 8 + (L & 7);
  const int role = static_cast<int>(j % bpt);
  if (G >= B * T0) return;
  const int64_t b = G / T0;
  const int64_t tile = G % T0;
  if (kRole != kColsOnly && role < kRowBlocks) {
    const int64_t s = tile * kTile + role * 4 + (threadIdx.x >> 6);
    row_pass(g, x, mean, rstd, emb, dx, b, s, S, m_lds);
  } else {
    const int cb = kRole == kColsOnly ? role : role - kRowBlocks;
    float* f = reinterpret_cast<float*>(m_lds);
    col_pass(g, x, mean, rstd, part_s, part_c, b, tile, cb, S, T0, f, f + kTile);
  }
}

constexpr int kTileCols = 256;                       // columns per block (32 threads x 8)
constexpr int kColThreads = kTileCols / 8;           // 32
constexpr int kSlots = 8;                            // row slots per block
constexpr int kBlockThreads = kColThreads * kSlots;  // 256
constexpr int kRowsPerPart = kN / kProjBwdParts;     // 192
constexpr int kSteps = kRowsPerPart / kSlots;        // 24 rows per thread
constexpr int kBatchChunk = 4;

static_assert(kN % kProjBwdParts == 0 && kRowsPerPart % kSlots == 0, "part layout");
static_assert(kD % kTileCols == 0, "column blocks");

// slots combined as ((s0+s1)+(s2+s3)) + ((s4+s5)+(s6+s7)) (the same tree in
// every kernel that forms da partials)
__device__ __forceinline__ double slot_tree(const double (*red)[kBatchChunk][kTileCols], int b, int c) {
  return ((red[0][b][c] + red[1][b][c]) + (red[2][b][c] + red[3][b][c])) +
         ((red[4][b][c] + red[5][b][c]) + (red[6][b][c] + red[7][b][c]));
}

// dW tile (192 rows x 256 columns of part p, column block kb): a write
// stream; a = bf16(SiLU(temb)) per thread for its 8 columns.
template <int NB>
__device__ __forceinline__ void dw_tile(const float* __restrict__ d_emb,
                                        const uint16_t* __restrict__ temb, uint16_t* __restrict__ dW,
                                        int p, int kb, float (*de_lds)[kRowsPerPart]) {
  const int ct = threadIdx.x % kColThreads;
  const int slot = threadIdx.x / kColThreads;
  const int col = kb * kTileCols + ct * 8;
  const int jbase = p * kRowsPerPart;
  constexpr int kDeLoads = (NB * kRowsPerPart + kBlockThreads - 1) / kBlockThreads;
  float de_r[kDeLoads];
#pragma unroll
  for (int k = 0; k < kDeLoads; ++k) {
    const int idx = threadIdx.x + kBlockThreads * k;
    if (idx < NB * kRowsPerPart)
      de_r[k] = d_emb[static_cast<int64_t>(idx / kRowsPerPart) * kN + jbase + idx % kRowsPerPart];
  }
  uint4 tz[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) tz[b] = ld16(temb + static_cast<int64_t>(b) * kD + col);
#pragma unroll
  for (int k = 0; k < kDeLoads; ++k) {
    const int idx = threadIdx.x + kBlockThreads * k;
    if (idx < NB * kRowsPerPart) de_lds[idx / kRowsPerPart][idx % kRowsPerPart] = de_r[k];
  }
  float av[NB][8];
  uint32_t redo = 0;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    uint32_t m;
    unpack8(silu8_fast(tz[b], m), av[b]);
    redo |= m << (8 * b);
  }
  while (redo != 0) {   // rarely taken: elements the fast SiLU cannot decide
    const int bit = __builtin_ctz(redo);
    redo &= redo - 1;
    const int b = bit / 8, e = bit % 8;
    const float v = bf16_to_f32(silu_bf16_exact(bf16_to_f32(temb[static_cast<int64_t>(b) * kD + col + e])));
#pragma unroll
    for (int bb = 0; bb < NB; ++bb)
#pragma unroll
      for (int ee = 0; ee < 8; ++ee)
        if (bb == b && ee == e) av[bb][ee] = v;
  }
  __syncthreads();
#pragma unroll 4
  for (int i = 0; i < kSteps; ++i) {
    const int jl = slot + kSlots * i;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      double s = 0.0;
#pragma unroll
      for (int b = 0; b < NB; ++b) s += static_cast<double>(de_lds[b][jl] * av[b][e]);
      o[e] = static_cast<float>(s);
    }
    st16_nt(dW + static_cast<int64_t>(jbase + jl) * kD + col, pack8(o));
  }
}

// da partial tile (same tiling): a read stream over W.
template <int NB>
__device__ __forceinline__ void da_tile(const float* __restrict__ d_emb, const uint16_t* __restrict__ W,
                                        double* __restrict__ part, int p, int kb,
                                        float (*de_lds)[kRowsPerPart], double (*red)[NB][kTileCols]) {
  const int ct = threadIdx.x % kColThreads;
  const int slot = threadIdx.x / kColThreads;
  const int col = kb * kTileCols + ct * 8;
  const int jbase = p * kRowsPerPart;
  constexpr int kDeLoads = (NB * kRowsPerPart + kBlockThreads - 1) / kBlockThreads;
  float de_r[kDeLoads];
#pragma unroll
  for (int k = 0; k < kDeLoads; ++k) {
    const int idx = threadIdx.x + kBlockThreads * k;
    if (idx < NB * kRowsPerPart)
      de_r[k] = d_emb[static_cast<int64_t>(idx / kRowsPerPart) * kN + jbase + idx % kRowsPerPart];
  }
  uint4 wv[kSteps];
#pragma unroll
  for (int i = 0; i < kSteps; ++i)
    wv[i] = ld16(W + static_cast<int64_t>(jbase + slot + kSlots * i) * kD + col);
#pragma unroll
  for (int k = 0; k < kDeLoads; ++k) {
    const int idx = threadIdx.x + kBlockThreads * k;
    if (idx < NB * kRowsPerPart) de_lds[idx / kRowsPerPart][idx % kRowsPerPart] = de_r[k];
  }
  __syncthreads();
  double acc[NB][8];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[b][e] = 0.0;
#pragma unroll
  for (int i = 0; i < kSteps; ++i) {
    const int jl = slot + kSlots * i;
    float w[8];
    unpack8(wv[i], w);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float d = de_lds[b][jl];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[b][e] += static_cast<double>(d * w[e]);
    }
  }
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int e = 0; e < 8; ++e) red[slot][b][ct * 8 + e] = acc[b][e];
  __syncthreads();
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int c = threadIdx.x;
    const double v = ((red[0][b][c] + red[1][b][c]) + (red[2][b][c] + red[3][b][c])) +
                     ((red[4][b][c] + red[5][b][c]) + (red[6][b][c] + red[7][b][c]));
    part[(static_cast<int64_t>(p) * NB + b) * kD + kb * kTileCols + c] = v;
  }
}

// Small batches (B <= 4, a template parameter): one grid, blockIdx.z = 0
// writes dW, blockIdx.z = 1 reads W for the da partials; the two streams run
// side by side.
template <int NB>
__global__ __launch_bounds__(kBlockThreads) void proj_bwd_small_kernel(
    const float* __restrict__ d_emb, const uint16_t* __restrict__ temb,
    const uint16_t* __restrict__ W, uint16_t* __restrict__ dW, double* __restrict__ part) {
  __shared__ double red[kSlots][NB][kTileCols];
  __shared__ float de_lds[NB][kRowsPerPart];
  if (blockIdx.z == 0) dw_tile<NB>(d_emb, temb, dW, blockIdx.x, blockIdx.y, de_lds);
  else da_tile<NB>(d_emb, W, part, blockIdx.x, blockIdx.y, de_lds, red);
}

// One-call backward, second stage (B <= 4).  Blocks [0, 384): da partial
// tiles; [384, 768): dW tiles; then dx row blocks (4 rows of one sample each,
// samples in order).  W in, dW out and the dx stream (g and x again, just
// read by the level-0 kernel, dx out) run side by side.
constexpr int kProjTiles = kProjBwdParts * (kD / kTileCols);   // 384

template <int NB>
__global__ __launch_bounds__(kThreads) void bwd_stage2_kernel(
    const float* __restrict__ d_emb, const uint16_t* __restrict__ temb,
    const uint16_t* __restrict__ W, uint16_t* __restrict__ dW, double* __restrict__ part,
    const uint16_t* __restrict__ g, const uint16_t* __restrict__ x, const float* __restrict__ mean,
    const float* __restrict__ rstd, const uint16_t* __restrict__ emb, uint16_t* __restrict__ dx,
    int64_t S) {
  static_assert(kBlockThreads == kThreads, "one block size for every role");
  // one LDS buffer, laid out per role
  constexpr size_t kRed = sizeof(double) * kSlots * NB * kTileCols;
  constexpr size_t kDe = sizeof(float) * NB * kRowsPerPart;
  constexpr size_t kMod = sizeof(float4) * (kD / 4);
  __shared__ __align__(16) unsigned char smem[(kRed + kDe) > kMod ? (kRed + kDe) : kMod];
  auto* red = reinterpret_cast<double (*)[NB][kTileCols]>(smem);
  auto* de_lds = reinterpret_cast<float (*)[kRowsPerPart]>(smem + kRed);
  auto* m_lds = reinterpret_cast<float4*>(smem);
  const int blk = blockIdx.x;
  if (blk < kProjTiles) {
    da_tile<NB>(d_emb, W, part, blk % kProjBwdParts, blk / kProjBwdParts, de_lds, red);
  } else if (blk < 2 * kProjTiles) {
    const int t = blk - kProjTiles;
    dw_tile<NB>(d_emb, temb, dW, t % kProjBwdParts, t / kProjBwdParts, de_lds);
  } else {
    const int64_t groups = (S + 3) / 4;
    const int64_t i = blk - 2 * kProjTiles;
    const int64_t b = i / groups;
    const int64_t s = (i % groups) * 4 + (threadIdx.x >> 6);
    row_pass(g, x, mean, rstd, emb, dx, b, s, S, m_lds);
  }
}

__global__ __launch_bounds__(256) void silu_kernel(const uint16_t* __restrict__ temb,
                                                   uint16_t* __restrict__ a, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) {
    const float z = bf16_to_f32(temb[i]);
    bool redo;
    const uint32_t v = silu_bf16_fast(z, redo);
    a[i] = redo ? silu_bf16_exact(z) : static_cast<uint16_t>(v);
  }
}

// ---- B > 4 ------------------------------------------------------------------
constexpr int kDwRows = 4;
constexpr int kDwThreads = kChunks;     // 384: one 16-byte chunk of a row each
constexpr int kDwBatch = 8;

__global__ __launch_bounds__(kDwThreads) void proj_bwd_dw_kernel(const float* __restrict__ d_emb,
                                                                 const uint16_t* __restrict__ a,
                                                                 uint16_t* __restrict__ dW,
                                                                 int64_t B) {
  const int t = threadIdx.x;
  const int j0 = blockIdx.x * kDwRows;
  double acc[kDwRows][8];
#pragma unroll
  for (int r = 0; r < kDwRows; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = 0.0;

  for (int64_t b0 = 0; b0 < B; b0 += kDwBatch) {
    const int nb = static_cast<int>((B - b0) < kDwBatch ? (B - b0) : kDwBatch);
    float av[kDwBatch][8];
#pragma unroll
    for (int bb = 0; bb < kDwBatch; ++bb)
      if (bb < nb) unpack8(ld16(a + (b0 + bb) * kD + t * 8), av[bb]);
#pragma unroll
    for (int bb = 0; bb < kDwBatch; ++bb) {
      if (bb < nb) {
#pragma unroll
        for (int r = 0; r < kDwRows; ++r) {
          const float d = d_emb[(b0 + bb) * kN + j0 + r];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[r][e] += static_cast<double>(d * av[bb][e]);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kDwRows; ++r) {
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = static_cast<float>(acc[r][e]);
    st16(dW + static_cast<int64_t>(j0 + r) * kD + t * 8, pack8(o));
  }
}

__global__ __launch_bounds__(kBlockThreads) void proj_bwd_da_kernel(const float* __restrict__ d_emb,
                                                                    const uint16_t* __restrict__ W,
                                                                    double* __restrict__ part,
                                                                    int64_t B) {
  __shared__ double red[kSlots][kBatchChunk][kTileCols];   // 64 KB
  const int p = blockIdx.x;
  const int kb = blockIdx.y;
  const int64_t b0 = static_cast<int64_t>(blockIdx.z) * kBatchChunk;
  const int nb = static_cast<int>((B - b0) < kBatchChunk ? (B - b0) : kBatchChunk);
  const int ct = threadIdx.x % kColThreads;
  const int slot = threadIdx.x / kColThreads;
  const int col = kb * kTileCols + ct * 8;
  const int jbase = p * kRowsPerPart;

  uint4 wv[kSteps];
#pragma unroll
  for (int i = 0; i < kSteps; ++i)
    wv[i] = ld16(W + static_cast<int64_t>(jbase + slot + kSlots * i) * kD + col);
  double acc[kBatchChunk][8];
#pragma unroll
  for (int bb = 0; bb < kBatchChunk; ++bb)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[bb][e] = 0.0;
#pragma unroll
  for (int i = 0; i < kSteps; ++i) {
    const int j = jbase + slot + kSlots * i;
    float w[8];
    unpack8(wv[i], w);
#pragma unroll
    for (int bb = 0; bb < kBatchChunk; ++bb) {
      if (bb < nb) {
        const float d = d_emb[(b0 + bb) * kN + j];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[bb][e] += static_cast<double>(d * w[e]);
      }
    }
  }
#pragma unroll
  for (int bb = 0; bb < kBatchChunk; ++bb)
#pragma unroll
    for (int e = 0; e < 8; ++e) red[slot][bb][ct * 8 + e] = acc[bb][e];
  __syncthreads();
  for (int o = threadIdx.x; o < kBatchChunk * kTileCols; o += kBlockThreads) {
    const int bb = o / kTileCols, c = o % kTileCols;
    if (bb < nb)
      part[(static_cast<int64_t>(p) * B + b0 + bb) * kD + kb * kTileCols + c] = slot_tree(red, bb, c);
  }
}

// ---- dtemb and db -------------------------------------------------------------
__global__ __launch_bounds__(256) void proj_bwd_final_kernel(const double* __restrict__ part,
                                                             const float* __restrict__ d_emb,
                                                             const uint16_t* __restrict__ temb,
                                                             uint16_t* __restrict__ dtemb,
                                                             uint16_t* __restrict__ db, int64_t B) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < B * kD) {
    double v[kProjBwdParts];
#pragma unroll
    for (int p = 0; p < kProjBwdParts; ++p) v[p] = part[static_cast<int64_t>(p) * B * kD + i];
    double s = 0.0;
#pragma unroll
    for (int p = 0; p < kProjBwdParts; ++p) s += v[p];
    dtemb[i] = f32_to_bf16(static_cast<float>(s) * dsilu_f32(bf16_to_f32(temb[i])));
  }
  if (i < kN) {
    double s = 0.0;
    for (int64_t b = 0; b < B; ++b) s += static_cast<double>(d_emb[b * kN + i]);
    db[i] = f32_to_bf16(static_cast<float>(s));
  }
}

template <int kRole>
hipError_t launch_role(const uint16_t* g, const uint16_t* x, const float* mean, const float* rstd,
                       const uint16_t* emb, uint16_t* dx, float* part_s, float* part_c, int64_t B,
                       int64_t S, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  constexpr int bpt = kRole == kBoth ? kBlocksPerTile : (kRole == kRowsOnly ? kRowBlocks : kColBlocks);
  const int64_t T0 = (S + kTile - 1) / kTile;
  const int64_t groups = (B * T0 + 7) / 8;
  const dim3 grid(static_cast<unsigned>(groups * 8 * bpt));
  if (e0 != nullptr && e1 != nullptr) {
    // events carried by the dispatch itself: no extra barrier in the stream
    hipExtLaunchKernelGGL(norm_mod_bwd_kernel<kRole>, grid, dim3(kThreads), 0, s, e0, e1, 0, g, x, mean,
                          rstd, emb, dx, part_s, part_c, B, S, T0);
  } else {
    hipLaunchKernelGGL(norm_mod_bwd_kernel<kRole>, grid, dim3(kThreads), 0, s, g, x, mean, rstd, emb, dx,
                       part_s, part_c, B, S, T0);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_norm_mod_bwd(const uint16_t* g, const uint16_t* x, const float* mean,
                               const float* rstd, const uint16_t* emb, uint16_t* dx, float* part_s,
                               float* part_c, int64_t B, int64_t S, hipStream_t s, hipEvent_t e0,
                               hipEvent_t e1) {
  static_assert(kD % kColBlockCols == 0, "column blocks must tile D");
  return launch_role<kBoth>(g, x, mean, rstd, emb, dx, part_s, part_c, B, S, s, e0, e1);
}

hipError_t launch_norm_mod_bwd_dx(const uint16_t* g, const uint16_t* x, const float* mean,
                                  const float* rstd, const uint16_t* emb, uint16_t* dx, int64_t B,
                                  int64_t S, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  return launch_role<kRowsOnly>(g, x, mean, rstd, emb, dx, nullptr, nullptr, B, S, s, e0, e1);
}

hipError_t launch_norm_mod_bwd_tiles(const uint16_t* g, const uint16_t* x, const float* mean,
                                     const float* rstd, float* part_s, float* part_c, int64_t B,
                                     int64_t S, hipStream_t s) {
  return launch_role<kColsOnly>(g, x, mean, rstd, nullptr, nullptr, part_s, part_c, B, S, s, nullptr,
                                nullptr);
}

int proj_bwd_fused_max_batch() { return kBatchChunk; }

hipError_t launch_proj_bwd_fused(const float* d_emb, const uint16_t* temb, const uint16_t* W,
                                 uint16_t* dW, double* part, int64_t B, hipStream_t s) {
  const dim3 grid(kProjBwdParts, kD / kTileCols, 2), block(kBlockThreads);
  switch (B) {
    case 1: hipLaunchKernelGGL(proj_bwd_small_kernel<1>, grid, block, 0, s, d_emb, temb, W, dW, part); break;
    case 2: hipLaunchKernelGGL(proj_bwd_small_kernel<2>, grid, block, 0, s, d_emb, temb, W, dW, part); break;
    case 3: hipLaunchKernelGGL(proj_bwd_small_kernel<3>, grid, block, 0, s, d_emb, temb, W, dW, part); break;
    case 4: hipLaunchKernelGGL(proj_bwd_small_kernel<4>, grid, block, 0, s, d_emb, temb, W, dW, part); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_proj_bwd_dw(const float* d_emb, const uint16_t* a, uint16_t* dW, int64_t B,
                              hipStream_t s) {
  hipLaunchKernelGGL(proj_bwd_dw_kernel, dim3(kN / kDwRows), dim3(kDwThreads), 0, s, d_emb, a, dW, B);
  return hipGetLastError();
}

hipError_t launch_proj_bwd_da(const float* d_emb, const uint16_t* W, double* part, int64_t B,
                              hipStream_t s) {
  const int64_t bz = (B + kBatchChunk - 1) / kBatchChunk;
  hipLaunchKernelGGL(proj_bwd_da_kernel, dim3(kProjBwdParts, kD / kTileCols, static_cast<unsigned>(bz)),
                     dim3(kBlockThreads), 0, s, d_emb, W, part, B);
  return hipGetLastError();
}

hipError_t launch_proj_bwd_final(const double* part, const float* d_emb, const uint16_t* temb,
                                 uint16_t* dtemb, uint16_t* db, int64_t B, hipStream_t s) {
  const int64_t n = B * kD > kN ? B * kD : kN;
  hipLaunchKernelGGL(proj_bwd_final_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                     s, part, d_emb, temb, dtemb, db, B);
  return hipGetLastError();
}

hipError_t launch_silu(const uint16_t* temb, uint16_t* a, int64_t n, hipStream_t s) {
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(silu_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, temb, a, n);
  return hipGetLastError();
}

hipError_t launch_bwd_stage2(const float* d_emb, const uint16_t* temb, const uint16_t* W, uint16_t* dW,
                             double* part, const uint16_t* g, const uint16_t* x, const float* mean,
                             const float* rstd, const uint16_t* emb, uint16_t* dx, int64_t B, int64_t S,
                             hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const int64_t blocks = 2 * kProjTiles + B * ((S + 3) / 4);
  const dim3 grid(static_cast<unsigned>(blocks)), block(kThreads);
  auto go = [&](auto kern) {
    if (e0 != nullptr && e1 != nullptr) {
      hipExtLaunchKernelGGL(kern, grid, block, 0, s, e0, e1, 0, d_emb, temb, W, dW, part, g, x, mean, rstd,
                            emb, dx, S);
    } else {
      hipLaunchKernelGGL(kern, grid, block, 0, s, d_emb, temb, W, dW, part, g, x, mean, rstd, emb, dx, S);
    }
    return hipGetLastError();
  };
  switch (B) {
    case 1: return go(bwd_stage2_kernel<1>);
    case 2: return go(bwd_stage2_kernel<2>);
    case 3: return go(bwd_stage2_kernel<3>);
    case 4: return go(bwd_stage2_kernel<4>);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace adaln
