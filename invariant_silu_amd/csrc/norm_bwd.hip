// LayerNorm + modulation backward and level 0 of the token tree (RL-Kernel
// pull request 538, "What"; token sums per the review-thread fix of
// token_sum.cu).
//
// Per row r = (b, s), with m = bf16(1 + scale) and n recomputed exactly as
// in the forward from the saved mean / rstd:
//   gy    = g * m                            (exact: bf16 x bf16)
//   alpha = fl32(sum_d gy) / D,  beta = fl32(sum_d gy * n) / D
//   dx    = bf16(rstd * ((gy - alpha) - n * beta))
//   (fp64 lane partials, chunks and columns in order, then wave_sum_f64)
// and the level-0 pairs of the token tree, per (b, 32-token tile, column):
// Neumaier (s, c) of g (-> d_shift) and of g * n (-> d_scale), tokens in
// ascending order.  Levels >= 1 are folded by tree_fold_kernel.
//
// norm_mod_bwd_kernel<role>: dx rows and/or level-0 tiles of a 32-token tile;
// the 14 blocks of a tile (8 row blocks, 6 tile blocks) run on one XCD, so
// the second read of the tile's g and x is served by that XCD's L2.  No order
// depends on the batch size or the grid.
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

  // first pass: n and gy into registers (96 values; the second pass then
  // needs four operations per element), the two row sums in fp64
  double q1 = 0.0, q2 = 0.0;
  float nv[kLaneChunks][8], gyv[kLaneChunks][8];
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
      nv[i][e] = (xf[e] - mu) * rs;
      gyv[i][e] = gf[e] * mm[e];
      q1 += static_cast<double>(gyv[i][e]);
      q2 += static_cast<double>(gyv[i][e] * nv[i][e]);
    }
  }
  const float alpha = static_cast<float>(wave_sum_f64(q1)) / static_cast<float>(kD);
  const float beta = static_cast<float>(wave_sum_f64(q2)) / static_cast<float>(kD);
  uint16_t* drow = dx + row * kD;
#pragma unroll
  for (int i = 0; i < kLaneChunks; ++i) {
    const int c = lane + 64 * i;
    float d[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) d[e] = rs * ((gyv[i][e] - alpha) - nv[i][e] * beta);
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
// Pairs go to columns scale_col0 + col (g * n) and shift_col0 + col (g) of a
// pair buffer of `groups` 64-column groups.
template <bool kFull>
__device__ __forceinline__ void col_tile(const uint16_t* __restrict__ g, const uint16_t* __restrict__ x,
                                         const float* __restrict__ mean, const float* __restrict__ rstd,
                                         float* __restrict__ part, int64_t b, int64_t tile, int cb,
                                         int64_t S, int64_t T0, int rows, int64_t groups, int scale_col0,
                                         int shift_col0) {
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
  const int64_t i_scale = pair_index(b, groups, T0, tile, scale_col0 + col);
  const int64_t i_shift = pair_index(b, groups, T0, tile, shift_col0 + col);
  st8_nt(part + i_scale, sn0, sn1);
  st8_nt(part + i_scale + kPairGroup, cn0, cn1);
  st8_nt(part + i_shift, sg0, sg1);
  st8_nt(part + i_shift + kPairGroup, cg0, cg1);
}

// columns [0, D) of d_emb: d_scale (g * n); [D, 2D): d_shift (g)
__device__ __forceinline__ void col_pass(const uint16_t* __restrict__ g, const uint16_t* __restrict__ x,
                                         const float* __restrict__ mean, const float* __restrict__ rstd,
                                         float* __restrict__ part, int64_t b, int64_t tile, int cb,
                                         int64_t S, int64_t T0, int64_t groups = kN / kPairGroup,
                                         int scale_col0 = 0, int shift_col0 = kD) {
  const int64_t left = S - tile * kTile;
  if (left >= kTile)
    col_tile<true>(g, x, mean, rstd, part, b, tile, cb, S, T0, kTile, groups, scale_col0, shift_col0);
  else
    col_tile<false>(g, x, mean, rstd, part, b, tile, cb, S, T0, static_cast<int>(left), groups, scale_col0,
                    shift_col0);
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


// ---- residual norm site ------------------------------------------------------
// Backward of h = bf16(residual + bf16(gate * x)), out = bf16(LN(h) * m + shift)
// (mod = (shift | scale | gate)), from g_out and g_h:
//   dh = bf16(bf16(rstd * ((gy - alpha) - n * beta)) + g_h),  gy = g_out * m
//   d_residual = dh,  dx = bf16(dh * gate)
// and the level-0 token tiles of d_shift (g_out), d_scale (g_out * n) and
// d_gate (dh * x) in one pair buffer of 3D columns, (shift | scale | gate).
constexpr int64_t kModGroups = 3 * kD / kPairGroup;   // 144

__device__ __forceinline__ void residual_row_pass(
    const uint16_t* __restrict__ g, const uint16_t* __restrict__ h, const float* __restrict__ mean,
    const float* __restrict__ rstd, const uint16_t* __restrict__ mod, const uint16_t* __restrict__ gh,
    const uint16_t* __restrict__ x, uint16_t* __restrict__ dres, uint16_t* __restrict__ dxo, int64_t b, int64_t s,
    int64_t S, float4* m_lds, float4* gate_lds) {
  const int lane = threadIdx.x & 63;
  const int64_t row = b * S + (s < S ? s : S - 1);   // as in row_pass
  const uint2* scale = reinterpret_cast<const uint2*>(mod + b * 3 * kD + kD);
  const uint2* gate = reinterpret_cast<const uint2*>(mod + b * 3 * kD + 2 * kD);
  uint2 sc[3], gt[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    sc[k] = scale[threadIdx.x + kThreads * k];
    gt[k] = gate[threadIdx.x + kThreads * k];
  }
  const float mu = mean[row];
  const float rs = rstd[row];
  uint4 gv[kLaneChunks], hv[kLaneChunks];
#pragma unroll
  for (int i = 0; i < kLaneChunks; ++i) {
    gv[i] = ld16(g + row * kD + (lane + 64 * i) * 8);
    hv[i] = ld16(h + row * kD + (lane + 64 * i) * 8);
  }
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    m_lds[threadIdx.x + kThreads * k] =
        make_float4(round_bf16(1.0f + bf_lo(sc[k].x)), round_bf16(1.0f + bf_hi(sc[k].x)),
                    round_bf16(1.0f + bf_lo(sc[k].y)), round_bf16(1.0f + bf_hi(sc[k].y)));
    gate_lds[threadIdx.x + kThreads * k] =
        make_float4(bf_lo(gt[k].x), bf_hi(gt[k].x), bf_lo(gt[k].y), bf_hi(gt[k].y));
  }
  __syncthreads();
  double q1 = 0.0, q2 = 0.0;
#pragma unroll
  for (int i = 0; i < kLaneChunks; ++i) {
    const int c = lane + 64 * i;
    float gf[8], hf[8];
    unpack8(gv[i], gf);
    unpack8(hv[i], hf);
    const float4 m0 = m_lds[2 * c], m1 = m_lds[2 * c + 1];
    const float mm[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float n = (hf[e] - mu) * rs;
      const float gy = gf[e] * mm[e];
      q1 += static_cast<double>(gy);
      q2 += static_cast<double>(gy * n);
    }
  }
  uint4 ghv[kLaneChunks], xv[kLaneChunks];
#pragma unroll
  for (int i = 0; i < kLaneChunks; ++i) {
    ghv[i] = ld16(gh + row * kD + (lane + 64 * i) * 8);
    xv[i] = ld16(x + row * kD + (lane + 64 * i) * 8);
  }
  const float alpha = static_cast<float>(wave_sum_f64(q1)) / static_cast<float>(kD);
  const float beta = static_cast<float>(wave_sum_f64(q2)) / static_cast<float>(kD);
#pragma unroll
  for (int i = 0; i < kLaneChunks; ++i) {
    const int c = lane + 64 * i;
    float gf[8], hf[8], ghf[8], xf[8], dh[8], dxv[8];
    unpack8(gv[i], gf);
    unpack8(hv[i], hf);
    unpack8(ghv[i], ghf);
    unpack8(xv[i], xf);
    const float4 m0 = m_lds[2 * c], m1 = m_lds[2 * c + 1];
    const float4 g0 = gate_lds[2 * c], g1 = gate_lds[2 * c + 1];
    const float mm[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
    const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float n = (hf[e] - mu) * rs;
      const float gy = gf[e] * mm[e];
      const float dh1 = round_bf16(rs * ((gy - alpha) - n * beta));
      dh[e] = round_bf16(dh1 + ghf[e]);
      dxv[e] = dh[e] * gg[e];
    }
    st16_nt(dres + row * kD + c * 8, pack8(dh));
    st16_nt(dxo + row * kD + c * 8, pack8(dxv));
  }
}

// grid as norm_mod_bwd_kernel<kBoth>: row blocks (dh, dx) and tile blocks
// (d_scale, d_shift pairs) of one 32-token tile on one XCD
__global__ __launch_bounds__(kThreads) void residual_bwd_kernel(
    const uint16_t* __restrict__ g, const uint16_t* __restrict__ gh, const uint16_t* __restrict__ x,
    const uint16_t* __restrict__ h, const float* __restrict__ mean, const float* __restrict__ rstd,
    const uint16_t* __restrict__ mod, uint16_t* __restrict__ dres, uint16_t* __restrict__ dxo,
    float* __restrict__ part, int64_t B, int64_t S, int64_t T0) {
  __shared__ float4 m_lds[kD / 4];
  __shared__ float4 gate_lds[kD / 4];
  const int64_t L = blockIdx.x;
  const int64_t j = L >> 3;
  const int64_t G = (j / kBlocksPerTile) * 8 + (L & 7);
  const int role = static_cast<int>(j % kBlocksPerTile);
  if (G >= B * T0) return;
  const int64_t b = G / T0;
  const int64_t tile = G % T0;
  if (role < kRowBlocks) {
    const int64_t s = tile * kTile + role * 4 + (threadIdx.x >> 6);
    residual_row_pass(g, h, mean, rstd, mod, gh, x, dres, dxo, b, s, S, m_lds, gate_lds);
  } else {
    col_pass(g, h, mean, rstd, part, b, tile, role - kRowBlocks, S, T0, kModGroups, kD, 0);
  }
}

// level-0 pairs of d_gate (dh * x) for one 32-token tile and 512 columns
template <bool kFull>
__device__ __forceinline__ void gate_tile(const uint16_t* __restrict__ dh, const uint16_t* __restrict__ x,
                                          float* __restrict__ part, int64_t b, int64_t tile, int cb, int64_t S,
                                          int64_t T0, int rows) {
  const int col = cb * kColBlockCols + 2 * threadIdx.x;
  const int64_t row0 = b * S + tile * kTile;
  uint32_t dw[kTile], xw[kTile];
  if (kFull) {
    constexpr uint32_t kBytes = kTile * kD * 2;
    const Buffer dt(dh + row0 * kD, kBytes), xt(x + row0 * kD, kBytes);
#pragma unroll
    for (int r = 0; r < kTile; ++r) {
      dw[r] = dt.u32(col * 2, r * kD * 2);
      xw[r] = xt.u32(col * 2, r * kD * 2);
    }
  } else {
#pragma unroll
    for (int r = 0; r < kTile; ++r) {
      if (r < rows) {
        const int64_t off = (row0 + r) * kD + col;
        dw[r] = *reinterpret_cast<const uint32_t*>(dh + off);
        xw[r] = *reinterpret_cast<const uint32_t*>(x + off);
      }
    }
  }
  float s0 = 0.0f, c0 = 0.0f, s1 = 0.0f, c1 = 0.0f;
#pragma unroll
  for (int r = 0; r < kTile; ++r) {
    if (kFull || r < rows) {
      neumaier_add(s0, c0, bf_lo(dw[r]) * bf_lo(xw[r]));
      neumaier_add(s1, c1, bf_hi(dw[r]) * bf_hi(xw[r]));
    }
  }
  const int64_t i = pair_index(b, kModGroups, T0, tile, 2 * kD + col);
  st8_nt(part + i, s0, s1);
  st8_nt(part + i + kPairGroup, c0, c1);
}

// grid: B * T0 * 6 blocks; block (G, cb) = tile G, 512-column block cb
__global__ __launch_bounds__(kThreads) void gate_tile_kernel(const uint16_t* __restrict__ dh,
                                                             const uint16_t* __restrict__ x,
                                                             float* __restrict__ part, int64_t S, int64_t T0) {
  const int64_t G = blockIdx.x / kColBlocks;
  const int cb = static_cast<int>(blockIdx.x % kColBlocks);
  const int64_t b = G / T0;
  const int64_t tile = G % T0;
  const int64_t left = S - tile * kTile;
  if (left >= kTile) gate_tile<true>(dh, x, part, b, tile, cb, S, T0, kTile);
  else gate_tile<false>(dh, x, part, b, tile, cb, S, T0, static_cast<int>(left));
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


hipError_t launch_residual_bwd(const uint16_t* g_out, const uint16_t* g_h, const uint16_t* x, const uint16_t* h,
                               const float* mean, const float* rstd, const uint16_t* mod, uint16_t* d_residual,
                               uint16_t* dx, float* part, int64_t B, int64_t S, hipStream_t s, hipEvent_t e0,
                               hipEvent_t e1) {
  const int64_t T0 = (S + kTile - 1) / kTile;
  const int64_t groups = (B * T0 + 7) / 8;
  const dim3 grid(static_cast<unsigned>(groups * 8 * kBlocksPerTile));
  if (e0 && e1) {
    hipExtLaunchKernelGGL(residual_bwd_kernel, grid, dim3(kThreads), 0, s, e0, e1, 0, g_out, g_h, x, h, mean, rstd,
                          mod, d_residual, dx, part, B, S, T0);
  } else {
    hipLaunchKernelGGL(residual_bwd_kernel, grid, dim3(kThreads), 0, s, g_out, g_h, x, h, mean, rstd, mod,
                       d_residual, dx, part, B, S, T0);
  }
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  hipLaunchKernelGGL(gate_tile_kernel, dim3(static_cast<unsigned>(B * T0 * kColBlocks)), dim3(kThreads), 0, s,
                     d_residual, x, part, S, T0);
  return hipGetLastError();
}

}  // namespace adaln
