// Backward of a block's norm sites (the forward is site_fwd_kernel in fwd.hip;
// reading of miles_diffusion pull request 108, "Fused-norm rounding points").

#include "common.hpp"
#include "launch.hpp"
#include "norm_tiles.hpp"

namespace adaln {

namespace {

// ---- residual norm site ------------------------------------------------------
// Backward of h = bf16(residual + bf16(gate * x)), out = bf16(LN(h) * m + shift)
// (mod = (shift | scale | gate)), from g_out and g_h:
//   dh = bf16(bf16(rstd * ((gy - alpha) - n * beta)) + g_h),  gy = g_out * m
//   d_residual = dh,  dx = bf16(dh * gate)
// and the level-0 token tiles of d_shift (g_out), d_scale (g_out * n) and
// d_gate (dh * x) in one pair buffer of 3D columns, (shift | scale | gate).
constexpr int64_t kModGroups = 3 * kD / kPairGroup;   // 144

constexpr int64_t kSiteGroups = 2 * kD / kPairGroup;  // 96: the plain form's pairs (shift | scale)

// kRes: h is the LayerNorm input, dh = bf16(dh1 + g_h) goes to d_residual
// and bf16(dh * gate) to dx; plain form: h is x, dx = dh1
template <bool kRes>
__device__ __forceinline__ void site_row_pass(
    const uint16_t* __restrict__ g, const uint16_t* __restrict__ h, const float* __restrict__ mean,
    const float* __restrict__ rstd, const ModView& mv, const uint16_t* __restrict__ gh,
    uint16_t* __restrict__ dres, uint16_t* __restrict__ dxo, int64_t b, int64_t s, int64_t S, float4* m_lds,
    float4* gate_lds) {
  const int lane = threadIdx.x & 63;
  const int64_t row = b * S + (s < S ? s : S - 1);   // as in row_pass
  const uint2* scale = reinterpret_cast<const uint2*>(mv.scale + b * mv.ld);
  uint2 sc[3], gt[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) sc[k] = scale[threadIdx.x + kThreads * k];
  if (kRes) {
    const uint2* gate = reinterpret_cast<const uint2*>(mv.gate + b * mv.ld);
#pragma unroll
    for (int k = 0; k < 3; ++k) gt[k] = gate[threadIdx.x + kThreads * k];
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
    if (kRes)
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
  uint4 ghv[kLaneChunks];
  if (kRes)
#pragma unroll
    for (int i = 0; i < kLaneChunks; ++i) ghv[i] = ld16(gh + row * kD + (lane + 64 * i) * 8);
  const float alpha = static_cast<float>(wave_sum_f64(q1)) / static_cast<float>(kD);
  const float beta = static_cast<float>(wave_sum_f64(q2)) / static_cast<float>(kD);
#pragma unroll
  for (int i = 0; i < kLaneChunks; ++i) {
    const int c = lane + 64 * i;
    float gf[8], hf[8], dh[8], dxv[8];
    unpack8(gv[i], gf);
    unpack8(hv[i], hf);
    if (!kRes) {
      const float4 m0 = m_lds[2 * c], m1 = m_lds[2 * c + 1];
      const float mm[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float n = (hf[e] - mu) * rs;
        dxv[e] = rs * ((gf[e] * mm[e] - alpha) - n * beta);
      }
      st16_nt(dxo + row * kD + c * 8, pack8(dxv));
      continue;
    }
    float ghf[8];
    unpack8(ghv[i], ghf);
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
// (d_shift, d_scale pairs) of one 32-token tile on one XCD; with one tile per
// sample (S <= 32) the tile blocks write the roots into the gradient views
// (r_shift, r_scale, row stride r_ld) instead of pairs
template <bool kRes>
__global__ __launch_bounds__(kThreads) void site_bwd_kernel(
    const uint16_t* __restrict__ g, const uint16_t* __restrict__ gh, const uint16_t* __restrict__ h,
    const float* __restrict__ mean, const float* __restrict__ rstd, const ModView mv,
    uint16_t* __restrict__ dres, uint16_t* __restrict__ dxo, float* __restrict__ part, int64_t B, int64_t S,
    int64_t T0, float* __restrict__ r_shift, float* __restrict__ r_scale, int64_t r_ld) {
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
    site_row_pass<kRes>(g, h, mean, rstd, mv, gh, dres, dxo, b, s, S, m_lds, gate_lds);
  } else {
    col_pass(g, h, mean, rstd, part, b, tile, role - kRowBlocks, S, T0, kRes ? kModGroups : kSiteGroups, kD, 0,
             r_scale, r_shift, r_ld);
  }
}

// level-0 pairs of d_gate (dh * x) for one 32-token tile and 512 columns
// (with r_gate given, one tile per sample: the roots into that view)
template <bool kFull>
__device__ __forceinline__ void gate_tile(const uint16_t* __restrict__ dh, const uint16_t* __restrict__ x,
                                          float* __restrict__ part, int64_t b, int64_t tile, int cb, int64_t S,
                                          int64_t T0, int rows, float* __restrict__ r_gate, int64_t r_ld) {
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
  if (r_gate != nullptr) {
    st8(r_gate + b * r_ld + col, s0 + c0, s1 + c1);
    return;
  }
  const int64_t i = pair_index(b, kModGroups, T0, tile, 2 * kD + col);
  st8(part + i, s0, s1);
  st8(part + i + kPairGroup, c0, c1);
}

// grid: B * T0 * 6 blocks; block (G, cb) = tile G, 512-column block cb
__global__ __launch_bounds__(kThreads) void gate_tile_kernel(const uint16_t* __restrict__ dh,
                                                             const uint16_t* __restrict__ x,
                                                             float* __restrict__ part, int64_t S, int64_t T0,
                                                             float* __restrict__ r_gate, int64_t r_ld) {
  const int64_t G = blockIdx.x / kColBlocks;
  const int cb = static_cast<int>(blockIdx.x % kColBlocks);
  const int64_t b = G / T0;
  const int64_t tile = G % T0;
  const int64_t left = S - tile * kTile;
  if (left >= kTile) gate_tile<true>(dh, x, part, b, tile, cb, S, T0, kTile, r_gate, r_ld);
  else gate_tile<false>(dh, x, part, b, tile, cb, S, T0, static_cast<int>(left), r_gate, r_ld);
}

}  // namespace

namespace {
template <bool kRes>
void launch_site_bwd_kernel(dim3 grid, hipStream_t s, const uint16_t* g_out, const uint16_t* g_h,
                            const uint16_t* h, const float* mean, const float* rstd, const ModView& mv,
                            uint16_t* d_residual, uint16_t* dx, float* part, int64_t B, int64_t S, int64_t T0,
                            float* r_shift, float* r_scale, int64_t r_ld) {
  hipLaunchKernelGGL(site_bwd_kernel<kRes>, grid, dim3(kThreads), 0, s, g_out, g_h, h, mean, rstd, mv, d_residual,
                     dx, part, B, S, T0, r_shift, r_scale, r_ld);
}
}  // namespace

hipError_t launch_site_bwd(const uint16_t* g_out, const uint16_t* g_h, const uint16_t* x, const uint16_t* h,
                           const float* mean, const float* rstd, ModView mv, uint16_t* d_residual, uint16_t* dx,
                           float* part, int64_t B, int64_t S, hipStream_t s, float* r_shift, float* r_scale,
                           float* r_gate, int64_t r_ld) {
  const int64_t T0 = (S + kTile - 1) / kTile;
  const int64_t groups = (B * T0 + 7) / 8;
  const dim3 grid(static_cast<unsigned>(groups * 8 * kBlocksPerTile));
  if (!g_h) {   // plain form: the LayerNorm input is x
    launch_site_bwd_kernel<false>(grid, s, g_out, nullptr, x, mean, rstd, mv, nullptr, dx, part, B, S, T0, r_shift,
                                  r_scale, r_ld);
    return hipGetLastError();
  }
  launch_site_bwd_kernel<true>(grid, s, g_out, g_h, h, mean, rstd, mv, d_residual, dx, part, B, S, T0, r_shift,
                               r_scale, r_ld);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  hipLaunchKernelGGL(gate_tile_kernel, dim3(static_cast<unsigned>(B * T0 * kColBlocks)), dim3(kThreads), 0, s,
                     d_residual, x, part, S, T0, r_gate, r_ld);
  return hipGetLastError();
}

}  // namespace adaln
