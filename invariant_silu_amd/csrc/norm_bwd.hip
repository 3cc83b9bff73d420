// LayerNorm + modulation, backward (RL-Kernel pull request 538, "What"; token
// sums per the review-thread fix of token_sum.cu).  One launch, two kinds of
// block, both reading the g and x rows of one 32-token tile:
//
// row blocks (8 per tile, one wave per row r = (b, s)):
//   n     = (x - mean) * rstd                (recomputed exactly as the forward)
//   gy    = g * m,  m = bf16(1 + scale)      (exact: bf16 x bf16)
//   alpha = fl32(sum_d gy) / D,  beta = fl32(sum_d gy * n) / D
//   dx    = bf16(rstd * ((gy - alpha) - n * beta))
//   Row sums: fp64 lane partials (chunks in order, columns in order), then the
//   fixed lane tree of wave_sum_f64.  HBM-bound: g, x in, dx out.
//
// column blocks (6 per tile, one thread per 2 adjacent columns): the level-0
//   Neumaier pairs (s, c) of g (-> d_shift) and of g * n (-> d_scale), tokens
//   in ascending order; the 32-step recurrence of a column stays in one
//   thread.  ALU-bound.
//
// The 14 blocks of a tile get block ids congruent mod 8, so they are
// dispatched one after the other on the same XCD: the row blocks stream the
// tile from HBM while the column blocks of the same tile find it in that
// XCD's L2, and the ALU-bound and HBM-bound halves overlap.
//
// No arithmetic depends on the batch size or the grid.  Each half can also be
// launched alone (adaln_norm_mod_bwd_dx / adaln_norm_mod_bwd_tiles).
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

}  // namespace adaln
