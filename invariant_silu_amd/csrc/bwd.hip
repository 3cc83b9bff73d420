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
// for dW and db; for da, 128 row slots (slot t: rows t, t + 128, ... in
// order) added as a pairwise tree.
//
// Device pieces are shared by every kernel, so every entry point computes
// identical bits, and no order depends on the batch size or the grid.
//
// Kernels:
//   norm_mod_bwd_kernel<role>  dx rows and/or level-0 tiles of a 32-token
//                              tile, the 14 blocks of a tile on one XCD
//   proj_bwd_small_kernel<NB>  B <= 4: da column blocks (-> dtemb) and dW
//                              tiles (-> dW, db) in one grid
//   silu/dW/da kernels         B > 4
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
  const int lane = threadIdx.x & 63;
  // A wave past the end of the sample redoes row S - 1 and stores the same
  // bytes as the wave that owns it: no branch follows the barrier, so the
  // compiler keeps the row loads ahead of it.
  const int64_t row = b * S + (s < S ? s : S - 1);

  // small loads first: the memory counter drains in issue order, so staging
  // m needs only these, while the row loads below stay in flight
  const uint2* scale = reinterpret_cast<const uint2*>(emb + b * kN);
  uint2 sc[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) sc[k] = scale[threadIdx.x + kThreads * k];
  const float mu = mean[row];
  const float rs = rstd[row];
  uint4 gv[kLaneChunks], xv[kLaneChunks];
#pragma unroll
  for (int i = 0; i < kLaneChunks; ++i) {
    gv[i] = ld16(g + row * kD + (lane + 64 * i) * 8);
    xv[i] = ld16(x + row * kD + (lane + 64 * i) * 8);
  }
#pragma unroll
  for (int k = 0; k < 3; ++k)
    m_lds[threadIdx.x + kThreads * k] =
        make_float4(round_bf16(1.0f + bf_lo(sc[k].x)), round_bf16(1.0f + bf_hi(sc[k].x)),
                    round_bf16(1.0f + bf_lo(sc[k].y)), round_bf16(1.0f + bf_hi(sc[k].y)));
  __syncthreads();

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

// Level-0 pairs of one 32-token tile for 512 columns (2 per thread).  The
// tile's statistics are the same for the whole block (scalar loads, no LDS,
// no barrier).  A full tile takes the branch-free form: buffer loads (the
// lane's column offset in a VGPR, the row's in an SGPR, no per-load address
// arithmetic), and the memory counter lets the chains start on row 0 while
// later rows are in flight.  Only the last, ragged tile of a sample takes the
// guarded form.
template <bool kFull>
__device__ __forceinline__ void col_tile(const uint16_t* __restrict__ g, const uint16_t* __restrict__ x,
                                         const float* __restrict__ mean, const float* __restrict__ rstd,
                                         float* __restrict__ part, int64_t b, int64_t tile, int cb,
                                         int64_t S, int64_t T0, int rows) {
  const int col = cb * kColBlockCols + 2 * threadIdx.x;
  const int64_t row0 = b * S + tile * kTile;
  uint32_t gw[kTile], xw[kTile];
  if (kFull) {
    constexpr uint32_t kBytes = kTile * kD * 2;
    const Buffer gt(g + row0 * kD, kBytes), xt(x + row0 * kD, kBytes);
#pragma unroll
    for (int r = 0; r < kTile; ++r) {
      gw[r] = gt.u32(col * 2, r * kD * 2);
      xw[r] = xt.u32(col * 2, r * kD * 2);
    }
  } else {
#pragma unroll
    for (int r = 0; r < kTile; ++r) {
      if (r < rows) {
        const int64_t off = (row0 + r) * kD + col;
        gw[r] = *reinterpret_cast<const uint32_t*>(g + off);
        xw[r] = *reinterpret_cast<const uint32_t*>(x + off);
      }
    }
  }
  float sg0 = 0.0f, cg0 = 0.0f, sg1 = 0.0f, cg1 = 0.0f;
  float sn0 = 0.0f, cn0 = 0.0f, sn1 = 0.0f, cn1 = 0.0f;
#pragma unroll
  for (int r = 0; r < kTile; ++r) {
    if (kFull || r < rows) {
      const float mu = mean[row0 + r], rs = rstd[row0 + r];
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
  constexpr int64_t kGroups = kN / kPairGroup;
  const int64_t i_scale = pair_index(b, kGroups, T0, tile, col);
  const int64_t i_shift = pair_index(b, kGroups, T0, tile, col + kD);
  st8_nt(part + i_scale, sn0, sn1);
  st8_nt(part + i_scale + kPairGroup, cn0, cn1);
  st8_nt(part + i_shift, sg0, sg1);
  st8_nt(part + i_shift + kPairGroup, cg0, cg1);
}

__device__ __forceinline__ void col_pass(const uint16_t* __restrict__ g, const uint16_t* __restrict__ x,
                                         const float* __restrict__ mean, const float* __restrict__ rstd,
                                         float* __restrict__ part, int64_t b, int64_t tile, int cb,
                                         int64_t S, int64_t T0) {
  const int64_t left = S - tile * kTile;
  if (left >= kTile) col_tile<true>(g, x, mean, rstd, part, b, tile, cb, S, T0, kTile);
  else col_tile<false>(g, x, mean, rstd, part, b, tile, cb, S, T0, static_cast<int>(left));
}

// grid: 1-D, ceil(B*T0 / 8) * 8 * blocks_per_tile blocks (blocks_per_tile = 14,
// 8 or 6 for kBoth / kRowsOnly / kColsOnly).  Block L runs on XCD L % 8; on
// that XCD its index j = L / 8 selects tile (j / bpt) * 8 + L % 8 and role j % bpt.
template <int kRole>
__global__ __launch_bounds__(kThreads) void norm_mod_bwd_kernel(
    const uint16_t* __restrict__ g, const uint16_t* __restrict__ x,
    const float* __restrict__ mean, const float* __restrict__ rstd,
    const uint16_t* __restrict__ emb, uint16_t* __restrict__ dx,
    float* __restrict__ part, int64_t B, int64_t S, int64_t T0) {
  constexpr int bpt = kRole == kBoth ? kBlocksPerTile : (kRole == kRowsOnly ? kRowBlocks : kColBlocks);
  __shared__ float4 m_lds[kD / 4];   // row blocks: m = bf16(1 + scale)
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
    col_pass(g, x, mean, rstd, part, b, tile, cb, S, T0);
  }
}

// ---- projection backward ------------------------------------------------
// dW tiles: part p of 32 (192 rows) x column block kb of 12 (256 columns),
// a write stream; 8 row slots, a thread's 8 columns per row.
constexpr int kDwParts = 32;
constexpr int kTileCols = 256;                       // columns per dW tile (32 threads x 8)
constexpr int kColThreads = kTileCols / 8;           // 32
constexpr int kSlots = 8;                            // row slots per dW tile
constexpr int kBlockThreads = kColThreads * kSlots;  // 256
constexpr int kRowsPerPart = kN / kDwParts;          // 192
constexpr int kSteps = kRowsPerPart / kSlots;        // 24 rows per thread
constexpr int kDwTiles = kDwParts * (kD / kTileCols);   // 384
constexpr int kBatchChunk = 4;

static_assert(kN % kDwParts == 0 && kRowsPerPart % kSlots == 0, "part layout");
static_assert(kD % kTileCols == 0, "column blocks");
static_assert(kBlockThreads == kThreads, "one block size for every role");

// da blocks: 16 columns of W over all 6144 rows, so each block finishes the
// sum and writes dtemb itself.  128 row slots, slot t walks rows t, t + 128,
// ... in order (fp64 accumulation of fp32 products); the 128 slots are then
// added as a pairwise tree.  The four 32-byte quarters of a 128-byte row
// segment go to blocks L, L + 8, L + 16 and L + 24, which the dispatcher
// places on the same XCD (one L2 serves all four).
constexpr int kDaCols = 16;
constexpr int kDaColThreads = kDaCols / 8;            // 2
constexpr int kDaSlots = kThreads / kDaColThreads;    // 128
constexpr int kDaBlocks = kD / kDaCols;               // 192
constexpr int kDaSteps = kN / kDaSlots;               // 48 rows per thread
constexpr int kDaShare = 128 / (kDaCols * 2);         // blocks sharing a 128-byte segment: 4

static_assert(kDaBlocks % (8 * kDaShare) == 0, "da block to column mapping");

__device__ __forceinline__ int da_first_col(int L) {
  const int g = L / (8 * kDaShare), q = (L / 8) % kDaShare, xcd = L % 8;
  return ((g * 8 + xcd) * kDaShare + q) * kDaCols;
}

// da and dtemb for samples b0 .. b0 + nb - 1 (nb <= NB) and the 32 columns of
// block L.  red: LDS, kDaSlots * NB * kDaCols doubles.
template <int NB>
__device__ __forceinline__ void da_block(const float* __restrict__ d_emb, const uint16_t* __restrict__ W,
                                         const uint16_t* __restrict__ temb, uint16_t* __restrict__ dtemb,
                                         int L, int64_t b0, int nb, double* red) {
  // rows per batch (two batches in flight), sized to keep registers <= ~128
  constexpr int U = NB == 1 ? 8 : (NB == 2 ? 6 : (NB == 3 ? 6 : 4));
  static_assert(kDaSteps % (2 * U) == 0, "batch pairs");
  static_assert(kDaSteps % U == 0, "batches");
  const int ct = threadIdx.x % kDaColThreads;
  const int slot = threadIdx.x / kDaColThreads;
  const int col0 = da_first_col(L);
  const Buffer wb(W, static_cast<uint32_t>(kN) * kD * 2);
  const Buffer eb(d_emb + b0 * kN, static_cast<uint32_t>(nb) * kN * 4);
  const uint32_t w_lane = (static_cast<uint32_t>(slot) * kD + col0 + ct * 8) * 2;
  const uint32_t e_lane = static_cast<uint32_t>(slot) * 4;
  constexpr uint32_t kWStep = kDaSlots * kD * 2;   // bytes between a slot's rows
  constexpr uint32_t kEStep = kDaSlots * 4;

  auto load = [&](int i0, uint4 (&w)[U], float (&d)[U][NB]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = wb.u128(w_lane, (i0 + u) * kWStep);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int bl = b < nb ? b : nb - 1;   // samples past nb: any in-range value, never stored
        d[u][b] = eb.f32(e_lane, bl * kN * 4 + (i0 + u) * kEStep);
      }
  };
  double acc[NB][8];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[b][e] = 0.0;
  auto accumulate = [&](const uint4 (&w)[U], const float (&d)[U][NB]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float wf[8];
      unpack8(w[u], wf);
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[b][e] += static_cast<double>(d[u][b] * wf[e]);
    }
  };

  // two register batches: the next one is in flight while one is added
  uint4 wa[U], wbt[U];
  float da_[U][NB], db_[U][NB];
  load(0, wa, da_);
  // (scheduling barriers keep the compiler from hoisting a batch's loads
  // above the adds of the batch whose registers they reuse)
#pragma unroll 1
  for (int i0 = 0; i0 < kDaSteps - 2 * U; i0 += 2 * U) {
    load(i0 + U, wbt, db_);
    __builtin_amdgcn_sched_barrier(0);
    accumulate(wa, da_);
    __builtin_amdgcn_sched_barrier(0);
    load(i0 + 2 * U, wa, da_);
    __builtin_amdgcn_sched_barrier(0);
    accumulate(wbt, db_);
    __builtin_amdgcn_sched_barrier(0);
  }
  load(kDaSteps - U, wbt, db_);
  __builtin_amdgcn_sched_barrier(0);
  accumulate(wa, da_);
  accumulate(wbt, db_);

  constexpr int kRow = NB * kDaCols;   // doubles per slot
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int e = 0; e < 8; ++e) red[slot * kRow + b * kDaCols + ct * 8 + e] = acc[b][e];
  __syncthreads();
  // pairwise tree over the slots: ((s0 + s1) + (s2 + s3)) + ...
#pragma unroll
  for (int w = 1; w < kDaSlots; w <<= 1) {
    for (int i = threadIdx.x; i < (kDaSlots / (2 * w)) * kRow; i += kThreads) {
      const int s = (i / kRow) * 2 * w, r = i % kRow;
      red[s * kRow + r] += red[(s + w) * kRow + r];
    }
    __syncthreads();
  }
  if (threadIdx.x < kRow) {
    const int b = threadIdx.x / kDaCols, c = threadIdx.x % kDaCols;
    if (b < nb) {
      const int64_t i = (b0 + b) * kD + col0 + c;
      dtemb[i] = f32_to_bf16(static_cast<float>(red[threadIdx.x]) * dsilu_f32(bf16_to_f32(temb[i])));
    }
  }
}

// dW tile (192 rows x 256 columns of part p, column block kb): a write
// stream; a = bf16(SiLU(temb)) per thread for its 8 columns.  Tiles of column
// block 0 also write db for their rows: samples in order from +0.
template <int NB>
__device__ __forceinline__ void dw_tile(const float* __restrict__ d_emb,
                                        const uint16_t* __restrict__ temb, uint16_t* __restrict__ dW,
                                        uint16_t* __restrict__ db, int p, int kb,
                                        float (*de_lds)[kRowsPerPart]) {
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
  if (kb == 0 && threadIdx.x < kRowsPerPart) {
    double s = 0.0;
#pragma unroll
    for (int b = 0; b < NB; ++b) s += static_cast<double>(de_lds[b][threadIdx.x]);
    db[jbase + threadIdx.x] = f32_to_bf16(static_cast<float>(s));
  }
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

// LDS of a projection-backward block, laid out per role.
template <int NB>
struct ProjBwdShared {
  static constexpr size_t kRed = sizeof(double) * kDaSlots * NB * kDaCols;
  static constexpr size_t kDe = sizeof(float) * NB * kRowsPerPart;
  static constexpr size_t kBytes = kRed > kDe ? kRed : kDe;
};

// Small batches (B <= 4, a template parameter): one grid, blocks [0, 192)
// are the da column blocks (they read W and write dtemb), blocks [192, 576)
// the dW tiles (they write dW and db); the two streams run side by side.
template <int NB>
__global__ __launch_bounds__(kThreads) void proj_bwd_small_kernel(
    const float* __restrict__ d_emb, const uint16_t* __restrict__ temb, const uint16_t* __restrict__ W,
    uint16_t* __restrict__ dW, uint16_t* __restrict__ db, uint16_t* __restrict__ dtemb) {
  __shared__ __align__(16) unsigned char smem[ProjBwdShared<NB>::kBytes];
  const int blk = blockIdx.x;
  if (blk < kDaBlocks) {
    da_block<NB>(d_emb, W, temb, dtemb, blk, 0, NB, reinterpret_cast<double*>(smem));
  } else {
    const int t = blk - kDaBlocks;
    dw_tile<NB>(d_emb, temb, dW, db, t % kDwParts, t / kDwParts,
                reinterpret_cast<float (*)[kRowsPerPart]>(smem));
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
// dW tile of 32 rows x 256 columns per block; samples staged through LDS 64 at
// a time (a: 32 KB, d_emb: 8 KB).  Thread (ct, rg) owns rows 4 rg .. 4 rg + 3
// and columns 8 ct .. 8 ct + 7: 32 fp64 sums, samples in ascending order.
// Blocks of column block 0 also sum db for their rows.
constexpr int kDwBRows = 32;
constexpr int kDwBCols = 256;
constexpr int kDwBSamples = 64;
constexpr int kDwBLoads = kDwBSamples * (kDwBCols / 8) / kThreads;   // 8 chunk loads per thread
static_assert(kDwBSamples * kDwBRows / kThreads == kDwBLoads, "staging layout");

__global__ __launch_bounds__(kThreads) void proj_bwd_dw_kernel(const float* __restrict__ d_emb,
                                                               const uint16_t* __restrict__ a,
                                                               uint16_t* __restrict__ dW,
                                                               uint16_t* __restrict__ db, int64_t B) {
  __shared__ uint4 a_lds[kDwBSamples][kDwBCols / 8];   // 32 KB
  __shared__ __align__(16) float d_lds[kDwBSamples][kDwBRows];   // 8 KB
  const int ct = threadIdx.x % (kDwBCols / 8);
  const int rg = threadIdx.x / (kDwBCols / 8);
  const int j0 = blockIdx.x * kDwBRows;
  const int k0 = blockIdx.y * kDwBCols;
  double acc[4][8];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = 0.0;
  double dbs = 0.0;
  for (int64_t c0 = 0; c0 < B; c0 += kDwBSamples) {
    const int nb = static_cast<int>((B - c0) < kDwBSamples ? (B - c0) : kDwBSamples);
    // unconditional loads (slots past nb repeat sample nb - 1 and are unused)
    uint4 av_r[kDwBLoads];
    float d_r[kDwBLoads];
#pragma unroll
    for (int u = 0; u < kDwBLoads; ++u) {
      const int idx = threadIdx.x + kThreads * u;
      const int sa = idx / (kDwBCols / 8) < nb ? idx / (kDwBCols / 8) : nb - 1;
      av_r[u] = ld16(a + (c0 + sa) * kD + k0 + (idx % (kDwBCols / 8)) * 8);
      const int sd = idx / kDwBRows < nb ? idx / kDwBRows : nb - 1;
      d_r[u] = d_emb[(c0 + sd) * kN + j0 + idx % kDwBRows];
    }
    __syncthreads();   // the previous chunk is consumed
#pragma unroll
    for (int u = 0; u < kDwBLoads; ++u) {
      const int idx = threadIdx.x + kThreads * u;
      a_lds[idx / (kDwBCols / 8)][idx % (kDwBCols / 8)] = av_r[u];
      d_lds[idx / kDwBRows][idx % kDwBRows] = d_r[u];
    }
    __syncthreads();
    if (blockIdx.y == 0 && threadIdx.x < kDwBRows)
      for (int b = 0; b < nb; ++b) dbs += static_cast<double>(d_lds[b][threadIdx.x]);
#pragma unroll 2
    for (int b = 0; b < nb; ++b) {
      float av[8];
      unpack8(a_lds[b][ct], av);
      const float4 d4 = *reinterpret_cast<const float4*>(&d_lds[b][rg * 4]);
      const float dd[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] += static_cast<double>(dd[r] * av[e]);
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = static_cast<float>(acc[r][e]);
    st16_nt(dW + static_cast<int64_t>(j0 + rg * 4 + r) * kD + k0 + ct * 8, pack8(o));
  }
  if (blockIdx.y == 0 && threadIdx.x < kDwBRows) db[j0 + threadIdx.x] = f32_to_bf16(static_cast<float>(dbs));
}

// da and dtemb, 4 samples per blockIdx.y
__global__ __launch_bounds__(kThreads) void proj_bwd_da_kernel(const float* __restrict__ d_emb,
                                                               const uint16_t* __restrict__ W,
                                                               const uint16_t* __restrict__ temb,
                                                               uint16_t* __restrict__ dtemb, int64_t B) {
  __shared__ __align__(16) double red[kDaSlots * kBatchChunk * kDaCols];   // 64 KB
  const int64_t b0 = static_cast<int64_t>(blockIdx.y) * kBatchChunk;
  const int nb = static_cast<int>((B - b0) < kBatchChunk ? (B - b0) : kBatchChunk);
  da_block<kBatchChunk>(d_emb, W, temb, dtemb, blockIdx.x, b0, nb, red);
}

template <int kRole>
hipError_t launch_role(const uint16_t* g, const uint16_t* x, const float* mean, const float* rstd,
                       const uint16_t* emb, uint16_t* dx, float* part, int64_t B,
                       int64_t S, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  constexpr int bpt = kRole == kBoth ? kBlocksPerTile : (kRole == kRowsOnly ? kRowBlocks : kColBlocks);
  const int64_t T0 = (S + kTile - 1) / kTile;
  const int64_t groups = (B * T0 + 7) / 8;
  const dim3 grid(static_cast<unsigned>(groups * 8 * bpt));
  if (e0 != nullptr && e1 != nullptr) {
    // events carried by the dispatch itself: no extra barrier in the stream
    hipExtLaunchKernelGGL(norm_mod_bwd_kernel<kRole>, grid, dim3(kThreads), 0, s, e0, e1, 0, g, x, mean,
                          rstd, emb, dx, part, B, S, T0);
  } else {
    hipLaunchKernelGGL(norm_mod_bwd_kernel<kRole>, grid, dim3(kThreads), 0, s, g, x, mean, rstd, emb, dx,
                       part, B, S, T0);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_norm_mod_bwd(const uint16_t* g, const uint16_t* x, const float* mean,
                               const float* rstd, const uint16_t* emb, uint16_t* dx, float* part,
                               int64_t B, int64_t S, hipStream_t s, hipEvent_t e0,
                               hipEvent_t e1) {
  static_assert(kD % kColBlockCols == 0, "column blocks must tile D");
  return launch_role<kBoth>(g, x, mean, rstd, emb, dx, part, B, S, s, e0, e1);
}

hipError_t launch_norm_mod_bwd_dx(const uint16_t* g, const uint16_t* x, const float* mean,
                                  const float* rstd, const uint16_t* emb, uint16_t* dx, int64_t B,
                                  int64_t S, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  return launch_role<kRowsOnly>(g, x, mean, rstd, emb, dx, nullptr, B, S, s, e0, e1);
}

hipError_t launch_norm_mod_bwd_tiles(const uint16_t* g, const uint16_t* x, const float* mean,
                                     const float* rstd, float* part, int64_t B,
                                     int64_t S, hipStream_t s) {
  return launch_role<kColsOnly>(g, x, mean, rstd, nullptr, nullptr, part, B, S, s, nullptr,
                                nullptr);
}

int proj_bwd_fused_max_batch() { return kBatchChunk; }

hipError_t launch_proj_bwd_fused(const float* d_emb, const uint16_t* temb, const uint16_t* W,
                                 uint16_t* dW, uint16_t* db, uint16_t* dtemb, int64_t B, hipStream_t s) {
  const dim3 grid(kDaBlocks + kDwTiles), block(kThreads);
  switch (B) {
    case 1: hipLaunchKernelGGL(proj_bwd_small_kernel<1>, grid, block, 0, s, d_emb, temb, W, dW, db, dtemb); break;
    case 2: hipLaunchKernelGGL(proj_bwd_small_kernel<2>, grid, block, 0, s, d_emb, temb, W, dW, db, dtemb); break;
    case 3: hipLaunchKernelGGL(proj_bwd_small_kernel<3>, grid, block, 0, s, d_emb, temb, W, dW, db, dtemb); break;
    case 4: hipLaunchKernelGGL(proj_bwd_small_kernel<4>, grid, block, 0, s, d_emb, temb, W, dW, db, dtemb); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_proj_bwd_dw(const float* d_emb, const uint16_t* a, uint16_t* dW, uint16_t* db, int64_t B,
                              hipStream_t s) {
  hipLaunchKernelGGL(proj_bwd_dw_kernel, dim3(kN / kDwBRows, kD / kDwBCols), dim3(kThreads), 0, s, d_emb, a,
                     dW, db, B);
  return hipGetLastError();
}

hipError_t launch_proj_bwd_da(const float* d_emb, const uint16_t* W, const uint16_t* temb, uint16_t* dtemb,
                              int64_t B, hipStream_t s) {
  const int64_t bz = (B + kBatchChunk - 1) / kBatchChunk;
  hipLaunchKernelGGL(proj_bwd_da_kernel, dim3(kDaBlocks, static_cast<unsigned>(bz)), dim3(kThreads), 0, s,
                     d_emb, W, temb, dtemb, B);
  return hipGetLastError();
}

hipError_t launch_silu(const uint16_t* temb, uint16_t* a, int64_t n, hipStream_t s) {
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(silu_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, temb, a, n);
  return hipGetLastError();
}

}  // namespace adaln
