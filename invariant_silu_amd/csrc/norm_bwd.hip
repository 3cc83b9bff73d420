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
// ascending order.  Levels >= 1 are folded by tree_fold_kernel; with one tile
// per sample (S <= 32) the kernel writes the roots, s + c, to d_emb itself.
//
// norm_mod_bwd_kernel<role>: dx rows and/or level-0 tiles of a 32-token tile;
// the 14 blocks of a tile (8 row blocks, 6 tile blocks) run on one XCD, so
// the second read of the tile's g and x is served by that XCD's L2.  No order
// depends on the batch size or the grid.
#include <hip/hip_ext.h>

#include "common.hpp"
#include "launch.hpp"
#include "norm_tiles.hpp"

namespace adaln {

namespace {

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

// grid: 1-D, ceil(B*T0 / 8) * 8 * blocks_per_tile blocks (blocks_per_tile = 14,
// 8 or 6 for kBoth / kRowsOnly / kColsOnly).  Block L runs on XCD L % 8; on
// that XCD its index j = L / 8 selects tile (j / bpt) * 8 + L % 8 and role j % bpt.
template <int kRole>
__global__ __launch_bounds__(kThreads) void norm_mod_bwd_kernel(
    const uint16_t* __restrict__ g, const uint16_t* __restrict__ x,
    const float* __restrict__ mean, const float* __restrict__ rstd,
    const uint16_t* __restrict__ emb, uint16_t* __restrict__ dx,
    float* __restrict__ part, int64_t B, int64_t S, int64_t T0, float* __restrict__ root) {
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
    col_pass(g, x, mean, rstd, part, b, tile, cb, S, T0, kN / kPairGroup, 0, kD, root, root ? root + kD : nullptr,
             kN);
  }
}


template <int kRole>
hipError_t launch_role(const uint16_t* g, const uint16_t* x, const float* mean, const float* rstd,
                       const uint16_t* emb, uint16_t* dx, float* part, int64_t B,
                       int64_t S, hipStream_t s, hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr,
                       float* root = nullptr) {
  constexpr int bpt = kRole == kBoth ? kBlocksPerTile : (kRole == kRowsOnly ? kRowBlocks : kColBlocks);
  const int64_t T0 = (S + kTile - 1) / kTile;
  const int64_t groups = (B * T0 + 7) / 8;
  const dim3 grid(static_cast<unsigned>(groups * 8 * bpt));
  // events, when given, are recorded by the dispatch itself: no packet of
  // their own in the stream
  hipExtLaunchKernelGGL(norm_mod_bwd_kernel<kRole>, grid, dim3(kThreads), 0, s, e0, e1, 0, g, x, mean, rstd, emb, dx,
                        part, B, S, T0, root);
  return hipGetLastError();
}


}  // namespace

hipError_t launch_norm_mod_bwd(const uint16_t* g, const uint16_t* x, const float* mean,
                               const float* rstd, const uint16_t* emb, uint16_t* dx, float* part,
                               int64_t B, int64_t S, hipStream_t s, hipEvent_t e0, hipEvent_t e1,
                               float* root) {
  static_assert(kD % kColBlockCols == 0, "column blocks must tile D");
  return launch_role<kBoth>(g, x, mean, rstd, emb, dx, part, B, S, s, e0, e1, root);
}

hipError_t launch_norm_mod_bwd_dx(const uint16_t* g, const uint16_t* x, const float* mean,
                                  const float* rstd, const uint16_t* emb, uint16_t* dx, int64_t B,
                                  int64_t S, hipStream_t s) {
  return launch_role<kRowsOnly>(g, x, mean, rstd, emb, dx, nullptr, B, S, s);
}

hipError_t launch_norm_mod_bwd_tiles(const uint16_t* g, const uint16_t* x, const float* mean,
                                     const float* rstd, float* part, int64_t B,
                                     int64_t S, hipStream_t s) {
  return launch_role<kColsOnly>(g, x, mean, rstd, nullptr, nullptr, part, B, S, s);
}


}  // namespace adaln
