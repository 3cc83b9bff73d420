// LayerNorm + modulation, backward, fused with level 0 of the token tree.
//
// Per row r = (b, s), with m = bf16(1 + scale) and n recomputed exactly as in
// the forward from the saved mu / rstd:
//   gy    = g * m                          (exact: bf16 x bf16)
//   alpha = fl32(sum_d gy) / D,  beta = fl32(sum_d gy * n) / D
//   dx    = bf16(rstd * ((gy - alpha) - n * beta))
// and, per (b, 32-token tile, column), the level-0 Neumaier pair (s, c) of
// g (-> d_shift) and of g * n (-> d_scale), tokens in ascending order
// (RL-Kernel pull request 538: review thread on token_sum.cu, and "What").
//
// One workgroup owns one 32-token tile of one sample, so the 32-step
// sequential Neumaier recurrence of each column never leaves a thread.
// When there are too few tiles to fill the chip, a tile is split into P
// column slices (P in {1, 2, 3, 6}); every slice still reads the whole row
// for alpha / beta, but computes dx and the column sums only for its slice.
//
// The row sums are formed the same way for every P: 8-column chunk partials
// in fp64 (columns in order), a lane tree over each block of 64 consecutive
// chunks (wave_sum_f64), then the 6 block sums as ((B0+B1)+(B2+B3))+(B4+B5).
// So dx does not depend on P, on the grid or on the batch size.
//
// Sibling slices of a tile are given block ids congruent mod 8 so they run on
// the same XCD and share its L2 for the redundant row reads.
#include "common.hpp"
#include "launch.hpp"

namespace adaln {

namespace {

template <int P>
struct BwdCfg {
  static constexpr int T = kChunks / P;       // threads per block
  static constexpr int NW = T / 64;           // waves per block
  static constexpr int RB = P == 1 ? 4 : (P == 2 ? 2 : 1);   // rows per barrier
};

template <int P>
__global__ __launch_bounds__(BwdCfg<P>::T) void norm_mod_bwd_kernel(
    const uint16_t* __restrict__ g, const uint16_t* __restrict__ x,
    const float* __restrict__ mean, const float* __restrict__ rstd,
    const uint16_t* __restrict__ emb, uint16_t* __restrict__ dx,
    float* __restrict__ part_s, float* __restrict__ part_c, int64_t S, int64_t T0) {
  using C = BwdCfg<P>;
  constexpr int T = C::T, NW = C::NW, RB = C::RB;
  __shared__ double red[2][RB][6][2];

  const int64_t b = blockIdx.y;
  const int L = blockIdx.x;
  const int xcd = L & 7;
  const int local = L >> 3;
  const int p = local % P;
  const int64_t tile = static_cast<int64_t>(local / P) * 8 + xcd;
  if (tile >= T0) return;

  const int t = threadIdx.x;
  const int wave = t >> 6;
  const int lane = t & 63;
  const int rows = static_cast<int>((S - tile * kTile) < kTile ? (S - tile * kTile) : kTile);
  const int64_t row0 = b * S + tile * kTile;

  // m for every chunk this thread reads (chunk t + T*i, i < P)
  float m[P][8];
  const uint16_t* scale = emb + b * kN;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    float sc[8];
    unpack8(ld16(scale + (t + T * i) * 8), sc);
#pragma unroll
    for (int e = 0; e < 8; ++e) m[i][e] = round_bf16(1.0f + sc[e]);
  }
  const int own_col = (t + T * p) * 8;

  float sg[8], cg[8], sgn[8], cgn[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) { sg[e] = 0.0f; cg[e] = 0.0f; sgn[e] = 0.0f; cgn[e] = 0.0f; }

  uint4 gv[RB][P], xv[RB][P];
  float mu[RB], rs[RB];
  auto load_batch = [&](int r0) {
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      const bool ok = r0 + rr < rows;
      const int64_t row = row0 + (ok ? r0 + rr : 0);
#pragma unroll
      for (int i = 0; i < P; ++i) {
        const int64_t off = row * kD + (t + T * i) * 8;
        gv[rr][i] = ok ? ld16(g + off) : make_uint4(0, 0, 0, 0);
        xv[rr][i] = ok ? ld16(x + off) : make_uint4(0, 0, 0, 0);
      }
      mu[rr] = ok ? mean[row] : 0.0f;
      rs[rr] = ok ? rstd[row] : 0.0f;
    }
  };

  load_batch(0);
  int buf = 0;
  for (int r0 = 0; r0 < rows; r0 += RB) {
    const int nr = (rows - r0) < RB ? (rows - r0) : RB;
    uint4 gcur[RB][P], xcur[RB][P];
    float mucur[RB], rscur[RB];
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      mucur[rr] = mu[rr];
      rscur[rr] = rs[rr];
#pragma unroll
      for (int i = 0; i < P; ++i) { gcur[rr][i] = gv[rr][i]; xcur[rr][i] = xv[rr][i]; }
    }
    if (r0 + RB < rows) load_batch(r0 + RB);   // prefetch; stays in flight over the barrier

    float own_n[RB][8], own_gy[RB][8], own_g[RB][8];
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
#pragma unroll
      for (int i = 0; i < P; ++i) {
        float gf[8], xf[8];
        unpack8(gcur[rr][i], gf);
        unpack8(xcur[rr][i], xf);
        double q1 = 0.0, q2 = 0.0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float n = (xf[e] - mucur[rr]) * rscur[rr];
          const float gy = gf[e] * m[i][e];
          q1 += static_cast<double>(gy);
          q2 += static_cast<double>(gy * n);
          if (i == p) { own_n[rr][e] = n; own_gy[rr][e] = gy; own_g[rr][e] = gf[e]; }
        }
        q1 = wave_sum_f64(q1);
        q2 = wave_sum_f64(q2);
        if (lane == 0) {
          red[buf][rr][wave + NW * i][0] = q1;
          red[buf][rr][wave + NW * i][1] = q2;
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      if (rr < nr) {
        const double (*q)[2] = red[buf][rr];
        const double s1 = ((q[0][0] + q[1][0]) + (q[2][0] + q[3][0])) + (q[4][0] + q[5][0]);
        const double s2 = ((q[0][1] + q[1][1]) + (q[2][1] + q[3][1])) + (q[4][1] + q[5][1]);
        const float alpha = static_cast<float>(s1) / static_cast<float>(kD);
        const float beta = static_cast<float>(s2) / static_cast<float>(kD);
        float d[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          d[e] = rscur[rr] * ((own_gy[rr][e] - alpha) - own_n[rr][e] * beta);
        st16(dx + (row0 + r0 + rr) * kD + own_col, pack8(d));
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          neumaier_add(sg[e], cg[e], own_g[rr][e]);
          neumaier_add(sgn[e], cgn[e], own_g[rr][e] * own_n[rr][e]);
        }
      }
    }
    buf ^= 1;
  }

  // level-0 pairs: columns [0, D) of d_emb are d_scale (g*n), [D, 2D) d_shift (g)
  const int64_t base = (b * T0 + tile) * kN;
  float4* ps = reinterpret_cast<float4*>(part_s + base);
  float4* pc = reinterpret_cast<float4*>(part_c + base);
  const int q0 = own_col / 4;
  ps[q0] = make_float4(sgn[0], sgn[1], sgn[2], sgn[3]);
  ps[q0 + 1] = make_float4(sgn[4], sgn[5], sgn[6], sgn[7]);
  pc[q0] = make_float4(cgn[0], cgn[1], cgn[2], cgn[3]);
  pc[q0 + 1] = make_float4(cgn[4], cgn[5], cgn[6], cgn[7]);
  ps[kD / 4 + q0] = make_float4(sg[0], sg[1], sg[2], sg[3]);
  ps[kD / 4 + q0 + 1] = make_float4(sg[4], sg[5], sg[6], sg[7]);
  pc[kD / 4 + q0] = make_float4(cg[0], cg[1], cg[2], cg[3]);
  pc[kD / 4 + q0 + 1] = make_float4(cg[4], cg[5], cg[6], cg[7]);
}

template <int P>
hipError_t launch_p(const uint16_t* g, const uint16_t* x, const float* mean, const float* rstd,
                    const uint16_t* emb, uint16_t* dx, float* part_s, float* part_c, int64_t B,
                    int64_t S, int64_t T0, hipStream_t s) {
  const int64_t groups = (T0 + 7) / 8;
  const int64_t gx = groups * 8 * P;
  hipLaunchKernelGGL(norm_mod_bwd_kernel<P>, dim3(static_cast<unsigned>(gx), static_cast<unsigned>(B)),
                     dim3(BwdCfg<P>::T), 0, s, g, x, mean, rstd, emb, dx, part_s, part_c, S, T0);
  return hipGetLastError();
}

}  // namespace

int choose_norm_bwd_split(int64_t B, int64_t T0) {
  const int64_t tiles = B * T0;
  if (tiles >= 256) return 1;
  if (tiles * 2 >= 256) return 2;
  if (tiles * 3 >= 256) return 3;
  return 6;
}

hipError_t launch_norm_mod_bwd_level0(const uint16_t* g, const uint16_t* x, const float* mean,
                                      const float* rstd, const uint16_t* emb, uint16_t* dx,
                                      float* part_s, float* part_c, int64_t B, int64_t S,
                                      int split, hipStream_t s) {
  const int64_t T0 = (S + kTile - 1) / kTile;
  switch (split) {
    case 1: return launch_p<1>(g, x, mean, rstd, emb, dx, part_s, part_c, B, S, T0, s);
    case 2: return launch_p<2>(g, x, mean, rstd, emb, dx, part_s, part_c, B, S, T0, s);
    case 3: return launch_p<3>(g, x, mean, rstd, emb, dx, part_s, part_c, B, S, T0, s);
    case 6: return launch_p<6>(g, x, mean, rstd, emb, dx, part_s, part_c, B, S, T0, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace adaln
