// LayerNorm + modulation, backward (RL-Kernel pull request 538, "What"; token
// sums per the review-thread fix of token_sum.cu).  Two kernels, one per kind
// of parallelism, both reading g and x:
//
// norm_mod_bwd_dx_kernel -- rows.  One wave per row r = (b, s):
//   n     = (x - mean) * rstd                (recomputed exactly as the forward)
//   gy    = g * m,  m = bf16(1 + scale)      (exact: bf16 x bf16)
//   alpha = fl32(sum_d gy) / D,  beta = fl32(sum_d gy * n) / D
//   dx    = bf16(rstd * ((gy - alpha) - n * beta))
//   Row sums: fp64 lane partials (chunks in order, columns in order), then the
//   fixed lane tree of wave_sum_f64.  HBM-bound stream: g, x in, dx out.
//
// norm_mod_bwd_tiles_kernel -- columns.  One thread per (sample, 32-token tile,
//   2 adjacent columns): the level-0 Neumaier pairs (s, c) of g (-> d_shift)
//   and of g * n (-> d_scale), tokens in ascending order.  The 32-step
//   recurrence of a column stays in one thread; g and x are read again (the
//   row kernel has just streamed them, so they are usually still in the MALL).
//
// Neither kernel's arithmetic depends on the batch size or the grid.
#include <hip/hip_ext.h>

#include "common.hpp"
#include "launch.hpp"

namespace adaln {

namespace {

constexpr int kDxWaves = 4;
constexpr int kDxThreads = 64 * kDxWaves;
constexpr int kLaneChunks = kChunks / 64;   // 6

__global__ __launch_bounds__(kDxThreads) void norm_mod_bwd_dx_kernel(
    const uint16_t* __restrict__ g, const uint16_t* __restrict__ x,
    const float* __restrict__ mean, const float* __restrict__ rstd,
    const uint16_t* __restrict__ emb, uint16_t* __restrict__ dx, int64_t S) {
  __shared__ float4 m_lds[kD / 4];
  const int64_t b = blockIdx.y;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t s = static_cast<int64_t>(blockIdx.x) * kDxWaves + wave;
  const bool valid = s < S;
  const int64_t row = b * S + (valid ? s : 0);

  // issue the row's loads before staging m, so the two latencies overlap
  uint4 gv[kLaneChunks], xv[kLaneChunks];
#pragma unroll
  for (int i = 0; i < kLaneChunks; ++i) {
    gv[i] = ld16(g + row * kD + (lane + 64 * i) * 8);
    xv[i] = ld16(x + row * kD + (lane + 64 * i) * 8);
  }
  const float mu = mean[row];
  const float rs = rstd[row];

  const uint2* scale = reinterpret_cast<const uint2*>(emb + b * kN);
  for (int c = threadIdx.x; c < kD / 4; c += kDxThreads) {
    const uint2 w = scale[c];
    m_lds[c] = make_float4(round_bf16(1.0f + bf_lo(w.x)), round_bf16(1.0f + bf_hi(w.x)),
                           round_bf16(1.0f + bf_lo(w.y)), round_bf16(1.0f + bf_hi(w.y)));
  }
  __syncthreads();
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
    st16(drow + c * 8, pack8(d));
  }
}

constexpr int kTlThreads = 256;
constexpr int kTlCols = 2 * kTlThreads;     // 512 columns per block

__global__ __launch_bounds__(kTlThreads) void norm_mod_bwd_tiles_kernel(
    const uint16_t* __restrict__ g, const uint16_t* __restrict__ x,
    const float* __restrict__ mean, const float* __restrict__ rstd,
    float* __restrict__ part_s, float* __restrict__ part_c, int64_t S, int64_t T0) {
  __shared__ float mu_s[kTile], rs_s[kTile];
  const int col = blockIdx.x * kTlCols + 2 * threadIdx.x;
  const int64_t tile = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int rows = static_cast<int>((S - tile * kTile) < kTile ? (S - tile * kTile) : kTile);
  const int64_t row0 = b * S + tile * kTile;

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
    mu_s[threadIdx.x] = mean[row0 + threadIdx.x];
    rs_s[threadIdx.x] = rstd[row0 + threadIdx.x];
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

}  // namespace

hipError_t launch_norm_mod_bwd_dx(const uint16_t* g, const uint16_t* x, const float* mean,
                                  const float* rstd, const uint16_t* emb, uint16_t* dx, int64_t B,
                                  int64_t S, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
  const int64_t gx = (S + kDxWaves - 1) / kDxWaves;
  const dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(B));
  if (ev_start != nullptr && ev_stop != nullptr) {
    // events carried by the dispatch itself: no extra barrier in the stream
    hipExtLaunchKernelGGL(norm_mod_bwd_dx_kernel, grid, dim3(kDxThreads), 0, s, ev_start, ev_stop, 0,
                          g, x, mean, rstd, emb, dx, S);
  } else {
    hipLaunchKernelGGL(norm_mod_bwd_dx_kernel, grid, dim3(kDxThreads), 0, s, g, x, mean, rstd, emb, dx, S);
  }
  return hipGetLastError();
}

hipError_t launch_norm_mod_bwd_tiles(const uint16_t* g, const uint16_t* x, const float* mean,
                                     const float* rstd, float* part_s, float* part_c, int64_t B,
                                     int64_t S, hipStream_t s) {
  static_assert(kD % kTlCols == 0, "column blocks must tile D");
  const int64_t T0 = (S + kTile - 1) / kTile;
  hipLaunchKernelGGL(norm_mod_bwd_tiles_kernel,
                     dim3(kD / kTlCols, static_cast<unsigned>(T0), static_cast<unsigned>(B)),
                     dim3(kTlThreads), 0, s, g, x, mean, rstd, part_s, part_c, S, T0);
  return hipGetLastError();
}

}  // namespace adaln
