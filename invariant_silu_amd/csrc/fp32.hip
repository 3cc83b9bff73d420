// FP32 storage: the operator with every tensor in fp32 (the FP32 execution
// RL-Kernel pull request 538 measures beside BF16, "Prior art & reuse
// decision" and "Results").  The method is the bf16 one without the bf16
// rounding points:
//   a    = fl32(SiLU(temb))                 (float64 SiLU, rounded once)
//   emb  = fl32(sum a W) + b                (the projection's fixed tree)
//   m    = 1 + scale,  out = (n * m) + shift          (fp32 operations)
//   gy   = g * m,  dx = rstd * ((gy - alpha) - n * beta)
//   d_scale, d_shift, dW, db, da, dtemb: the same sums as with bf16 storage.
//
// Kernels here: silu_f32_kernel; proj_f32_small_kernel<NB> (the projection
// for B = NB <= 4 on the vector units); norm_mod_fwd_f32_kernel (statistics and
// modulation, one wave per row); norm_mod_bwd_f32_kernel (dx rows and the
// level-0 token tiles, the same 14 blocks per 32-token tile on one XCD as
// the bf16 kernel).  The projections run in the storage-templated matrix-core
// kernels and the vector da blocks; levels >= 1 of the token tree in
// tree_fold_kernel.
//
// Orders: a lane of a row wave holds the 16-byte chunks lane + 64 i
// (i = 0 .. 11) of its row; row sums run over them in that order in fp64,
// then wave_sum_f64.  Level-0 tiles: Neumaier over the tile's tokens in
// ascending order, per column.  No order depends on the batch size.

#include "common.hpp"
#include "launch.hpp"

namespace adaln {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kRowChunks = kD / 4 / 64;            // 12 chunks of 4 floats per lane
constexpr int kRowBlocks = kTile / 4;              // 8 row blocks of 4 rows per tile
constexpr int kColBlockCols = 2 * kThreads;        // 512 columns per tile block
constexpr int kColBlocks = kD / kColBlockCols;     // 6
constexpr int kBlocksPerTile = kRowBlocks + kColBlocks;

__device__ __forceinline__ void load_row_f32(const float* __restrict__ x, int64_t row, int lane,
                                             float4 (&xv)[kRowChunks]) {
  const float4* p = reinterpret_cast<const float4*>(x + row * kD);
#pragma unroll
  for (int i = 0; i < kRowChunks; ++i) xv[i] = p[lane + 64 * i];
}

typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void st4_nt(float* p, const float (&f)[4]) {
  const f32x4_t v = {f[0], f[1], f[2], f[3]};
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(p));
}

__device__ __forceinline__ void unpack4(const float4& v, float (&f)[4]) {
  f[0] = v.x;
  f[1] = v.y;
  f[2] = v.z;
  f[3] = v.w;
}

// m = 1 + scale (and, with kShift, shift) of sample b into LDS (768 float4
// each); all loads are issued before the first LDS write
template <bool kShift>
__device__ __forceinline__ void stage_mod_f32(const float* __restrict__ emb, int64_t b, float4* m_lds,
                                              float4* sh_lds) {
  const float4* scale = reinterpret_cast<const float4*>(emb + b * kN);
  const float4* shift = reinterpret_cast<const float4*>(emb + b * kN + kD);
  float4 sc[3], sh[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    sc[k] = scale[threadIdx.x + kThreads * k];
    if constexpr (kShift) sh[k] = shift[threadIdx.x + kThreads * k];
  }
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int c = threadIdx.x + kThreads * k;
    m_lds[c] = make_float4(1.0f + sc[k].x, 1.0f + sc[k].y, 1.0f + sc[k].z, 1.0f + sc[k].w);
    if constexpr (kShift) sh_lds[c] = sh[k];
  }
}

__global__ __launch_bounds__(256) void silu_f32_kernel(const float* __restrict__ temb, float* __restrict__ a,
                                                       int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) a[i] = silu_f32(temb[i]);
}

// Projection for B = NB <= 4, fp32 storage: the sum for one (sample, row of
// W) is the matrix-core kernel's: 64 leaves, leaf l over k in [48 l, 48 l +
// 48) as k = 48 l + 12 g + s (s = 0..11 outer, g = 0..3 inner), each term an
// fp64 fused multiply-add of the fp32 operands (exact product) from +0, the
// leaves then added pairwise in index order (wave_sum_f64); emb = fl32(sum) +
// bias.  Lane l holds leaf l of two rows of W (48 floats each, 16-byte
// loads); a (from silu_f32_kernel) is staged in LDS as [s][l][g] so a step
// reads the four terms of a leaf with one conflict-free 16-byte load.  Block:
// 4 waves x 2 rows.
constexpr int kF32Rows = 2;
constexpr int kF32LeafK = kD / 64;          // 48
constexpr int kF32Steps = kF32LeafK / 4;    // 12

template <int NB>
__global__ __launch_bounds__(kThreads) void proj_f32_small_kernel(const float* __restrict__ a,
                                                                  const float* __restrict__ W,
                                                                  const float* __restrict__ bias,
                                                                  float* __restrict__ emb) {
  __shared__ float4 a_lds[NB][kF32Steps * 64];      // NB x 12 KB
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int row0 = (blockIdx.x * (kThreads / 64) + wave) * kF32Rows;
  // W first: the long stream, in flight while a is staged
  float4 w[kF32Rows][kF32LeafK / 4];
#pragma unroll
  for (int r = 0; r < kF32Rows; ++r)
#pragma unroll
    for (int q = 0; q < kF32LeafK / 4; ++q)
      w[r][q] = *reinterpret_cast<const float4*>(W + static_cast<int64_t>(row0 + r) * kD + lane * kF32LeafK + 4 * q);
  float* al = reinterpret_cast<float*>(a_lds);
#pragma unroll
  for (int it = 0; it < NB * kD / kThreads; ++it) {
    const int i = threadIdx.x + kThreads * it;
    const int bb = i / kD, k = i % kD;
    const int l = k / kF32LeafK, rem = k % kF32LeafK;
    al[(bb * kF32Steps * 64 + (rem % kF32Steps) * 64 + l) * 4 + rem / kF32Steps] = a[i];
  }
  __syncthreads();
  const float* wf = reinterpret_cast<const float*>(w);
  double acc[kF32Rows][NB];
#pragma unroll
  for (int r = 0; r < kF32Rows; ++r)
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) acc[r][bb] = 0.0;
#pragma unroll
  for (int st = 0; st < kF32Steps; ++st) {
    float4 av[NB];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) av[bb] = a_lds[bb][st * 64 + lane];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
      for (int r = 0; r < kF32Rows; ++r) {
        const double wv = static_cast<double>(wf[r * kF32LeafK + 12 * g + st]);
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
          const float ag = g == 0 ? av[bb].x : g == 1 ? av[bb].y : g == 2 ? av[bb].z : av[bb].w;
          acc[r][bb] = __builtin_fma(static_cast<double>(ag), wv, acc[r][bb]);
        }
      }
    }
    // the accumulators are materialised after every step, so the step's
    // LDS reads and fp64 conversions stay next to their uses
#pragma unroll
    for (int r = 0; r < kF32Rows; ++r)
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) asm volatile("" : "+v"(acc[r][bb]));
  }
#pragma unroll
  for (int r = 0; r < kF32Rows; ++r)
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      const double tot = wave_sum_f64(acc[r][bb]);
      if (lane == r * NB + bb) emb[bb * kN + row0 + r] = static_cast<float>(tot) + bias[row0 + r];
    }
}

// 4 rows of one sample per block (one per wave): statistics and modulation
__global__ __launch_bounds__(kThreads) void norm_mod_fwd_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ emb, float* __restrict__ out,
    float* __restrict__ mean, float* __restrict__ rstd, int64_t S, float eps) {
  __shared__ float4 m_lds[kD / 4];
  __shared__ float4 sh_lds[kD / 4];
  const int64_t b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int64_t s = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  // a wave past the end redoes row S - 1 (same bytes as its owner): no branch
  // after the barrier
  const int64_t row = b * S + (s < S ? s : S - 1);
  float4 xv[kRowChunks];
  load_row_f32(x, row, lane, xv);
  stage_mod_f32<true>(emb, b, m_lds, sh_lds);
  __syncthreads();
  double acc = 0.0;
#pragma unroll
  for (int i = 0; i < kRowChunks; ++i) {
    float v[4];
    unpack4(xv[i], v);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc += static_cast<double>(v[e]);
  }
  const float mu = static_cast<float>(wave_sum_f64(acc)) / static_cast<float>(kD);
  double acc2 = 0.0;
#pragma unroll
  for (int i = 0; i < kRowChunks; ++i) {
    float v[4];
    unpack4(xv[i], v);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float d = v[e] - mu;
      acc2 += static_cast<double>(d * d);
    }
  }
  const float var = static_cast<float>(wave_sum_f64(acc2)) / static_cast<float>(kD);
  const float rs = 1.0f / __builtin_sqrtf(var + eps);
  float* orow = out + row * kD;
#pragma unroll
  for (int i = 0; i < kRowChunks; ++i) {
    const int c = lane + 64 * i;
    float v[4], mm[4], hh[4], o[4];
    unpack4(xv[i], v);
    unpack4(m_lds[c], mm);
    unpack4(sh_lds[c], hh);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float n = (v[e] - mu) * rs;
      o[e] = n * mm[e] + hh[e];
    }
    st4_nt(orow + 4 * c, o);
  }
  if (lane == 0) {
    mean[row] = mu;
    rstd[row] = rs;
  }
}

// dx of one row (one wave): two passes over the row held in registers
__device__ __forceinline__ void row_pass_f32(const float* __restrict__ g, const float* __restrict__ x,
                                             const float* __restrict__ mean, const float* __restrict__ rstd,
                                             const float* __restrict__ emb, float* __restrict__ dx, int64_t b,
                                             int64_t s, int64_t S, float4* m_lds) {
  const int lane = threadIdx.x & 63;
  const int64_t row = b * S + (s < S ? s : S - 1);   // as in the forward
  const float mu = mean[row];
  const float rs = rstd[row];
  float4 gv[kRowChunks], xv[kRowChunks];
  load_row_f32(g, row, lane, gv);
  load_row_f32(x, row, lane, xv);
  stage_mod_f32<false>(emb, b, m_lds, nullptr);
  __syncthreads();
  double q1 = 0.0, q2 = 0.0;
#pragma unroll
  for (int i = 0; i < kRowChunks; ++i) {
    float gf[4], xf[4], mm[4];
    unpack4(gv[i], gf);
    unpack4(xv[i], xf);
    unpack4(m_lds[lane + 64 * i], mm);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float n = (xf[e] - mu) * rs;
      const float gy = gf[e] * mm[e];
      q1 += static_cast<double>(gy);
      q2 += static_cast<double>(gy * n);
    }
  }
  const float alpha = static_cast<float>(wave_sum_f64(q1)) / static_cast<float>(kD);
  const float beta = static_cast<float>(wave_sum_f64(q2)) / static_cast<float>(kD);
  float* drow = dx + row * kD;
#pragma unroll
  for (int i = 0; i < kRowChunks; ++i) {
    const int c = lane + 64 * i;
    float gf[4], xf[4], mm[4], d[4];
    unpack4(gv[i], gf);
    unpack4(xv[i], xf);
    unpack4(m_lds[c], mm);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float n = (xf[e] - mu) * rs;
      const float gy = gf[e] * mm[e];
      d[e] = rs * ((gy - alpha) - n * beta);
    }
    st4_nt(drow + 4 * c, d);
  }
}

// Level-0 pairs of one 32-token tile for 512 columns (2 per thread); a full
// tile uses buffer loads (column in a VGPR, row in an SGPR), the last ragged
// tile of a sample a guarded loop.  With one tile per sample (S <= 32) and
// `root` given, s + c (the fold's one add at that size) goes straight to
// root = d_emb [B, 2D] instead of the pair.
template <bool kFull>
__device__ __forceinline__ void col_tile_f32(const float* __restrict__ g, const float* __restrict__ x,
                                             const float* __restrict__ mean, const float* __restrict__ rstd,
                                             float* __restrict__ part, int64_t b, int64_t tile, int cb,
                                             int64_t S, int64_t T0, int rows, float* __restrict__ root) {
  const int col = cb * kColBlockCols + 2 * threadIdx.x;
  const int64_t row0 = b * S + tile * kTile;
  float2 gw[kTile], xw[kTile];
  if (kFull) {
    constexpr uint32_t kBytes = kTile * kD * 4;
    const Buffer gt(g + row0 * kD, kBytes), xt(x + row0 * kD, kBytes);
#pragma unroll
    for (int r = 0; r < kTile; ++r) {
      const auto gg = __builtin_amdgcn_raw_buffer_load_b64(gt.rsrc, col * 4, r * kD * 4, 0);
      const auto xx = __builtin_amdgcn_raw_buffer_load_b64(xt.rsrc, col * 4, r * kD * 4, 0);
      gw[r] = make_float2(__uint_as_float(gg[0]), __uint_as_float(gg[1]));
      xw[r] = make_float2(__uint_as_float(xx[0]), __uint_as_float(xx[1]));
    }
  } else {
#pragma unroll
    for (int r = 0; r < kTile; ++r) {
      if (r < rows) {
        const int64_t off = (row0 + r) * kD + col;
        gw[r] = *reinterpret_cast<const float2*>(g + off);
        xw[r] = *reinterpret_cast<const float2*>(x + off);
      }
    }
  }
  float sg0 = 0.0f, cg0 = 0.0f, sg1 = 0.0f, cg1 = 0.0f;
  float sn0 = 0.0f, cn0 = 0.0f, sn1 = 0.0f, cn1 = 0.0f;
#pragma unroll
  for (int r = 0; r < kTile; ++r) {
    if (kFull || r < rows) {
      const float mu = mean[row0 + r], rs = rstd[row0 + r];
      const float g0 = gw[r].x, g1 = gw[r].y;
      const float n0 = (xw[r].x - mu) * rs;
      const float n1 = (xw[r].y - mu) * rs;
      neumaier_add(sg0, cg0, g0);
      neumaier_add(sg1, cg1, g1);
      neumaier_add(sn0, cn0, g0 * n0);
      neumaier_add(sn1, cn1, g1 * n1);
    }
  }
  if (root != nullptr) {
    st8(root + b * kN + col, sn0 + cn0, sn1 + cn1);
    st8(root + b * kN + kD + col, sg0 + cg0, sg1 + cg1);
    return;
  }
  constexpr int64_t kGroups = kN / kPairGroup;
  const int64_t i_scale = pair_index(b, kGroups, T0, tile, col);
  const int64_t i_shift = pair_index(b, kGroups, T0, tile, col + kD);
  st8(part + i_scale, sn0, sn1);
  st8(part + i_scale + kPairGroup, cn0, cn1);
  st8(part + i_shift, sg0, sg1);
  st8(part + i_shift + kPairGroup, cg0, cg1);
}

// grid: 1-D, ceil(B*T0 / 8) * 8 * 14 blocks.  Block L runs on XCD L % 8; on
// that XCD its index j = L / 8 selects tile (j / 14) * 8 + L % 8 and role j % 14
// (8 row blocks, then 6 tile blocks), so the second read of a tile's g and x
// is served by that XCD's L2.
__global__ __launch_bounds__(kThreads) void norm_mod_bwd_f32_kernel(
    const float* __restrict__ g, const float* __restrict__ x, const float* __restrict__ mean,
    const float* __restrict__ rstd, const float* __restrict__ emb, float* __restrict__ dx,
    float* __restrict__ part, int64_t B, int64_t S, int64_t T0, float* __restrict__ root) {
  __shared__ float4 m_lds[kD / 4];
  const int64_t L = blockIdx.x;
  const int64_t j = L >> 3;
  const int64_t G = (j / kBlocksPerTile) * 8 + (L & 7);
  const int role = static_cast<int>(j % kBlocksPerTile);
  if (G >= B * T0) return;
  const int64_t b = G / T0;
  const int64_t tile = G % T0;
  if (role < kRowBlocks) {
    const int64_t s = tile * kTile + role * 4 + (threadIdx.x >> 6);
    row_pass_f32(g, x, mean, rstd, emb, dx, b, s, S, m_lds);
  } else {
    const int cb = role - kRowBlocks;
    const int64_t left = S - tile * kTile;
    if (left >= kTile) col_tile_f32<true>(g, x, mean, rstd, part, b, tile, cb, S, T0, kTile, root);
    else col_tile_f32<false>(g, x, mean, rstd, part, b, tile, cb, S, T0, static_cast<int>(left), root);
  }
}

}  // namespace

hipError_t launch_proj_f32_small(const float* a, const float* W, const float* bias, float* emb, int64_t B,
                                 hipStream_t s) {
  const dim3 grid(kN / ((kThreads / 64) * kF32Rows)), block(kThreads);
  switch (B) {
    case 1: hipLaunchKernelGGL(proj_f32_small_kernel<1>, grid, block, 0, s, a, W, bias, emb); break;
    case 2: hipLaunchKernelGGL(proj_f32_small_kernel<2>, grid, block, 0, s, a, W, bias, emb); break;
    case 3: hipLaunchKernelGGL(proj_f32_small_kernel<3>, grid, block, 0, s, a, W, bias, emb); break;
    case 4: hipLaunchKernelGGL(proj_f32_small_kernel<4>, grid, block, 0, s, a, W, bias, emb); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_silu_f32(const float* temb, float* a, int64_t n, hipStream_t s) {
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(silu_f32_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, temb, a, n);
  return hipGetLastError();
}

hipError_t launch_norm_mod_fwd_f32(const float* x, const float* emb, float* out, float* mean, float* rstd,
                                   int64_t B, int64_t S, float eps, hipStream_t s) {
  const int64_t gx = (S + kWaves - 1) / kWaves;
  hipLaunchKernelGGL(norm_mod_fwd_f32_kernel, dim3(static_cast<unsigned>(gx), static_cast<unsigned>(B)),
                     dim3(kThreads), 0, s, x, emb, out, mean, rstd, S, eps);
  return hipGetLastError();
}

hipError_t launch_norm_mod_bwd_f32(const float* g, const float* x, const float* mean, const float* rstd,
                                   const float* emb, float* dx, float* part, int64_t B, int64_t S,
                                   hipStream_t s, float* root) {
  static_assert(kD % kColBlockCols == 0, "column blocks must tile D");
  const int64_t T0 = (S + kTile - 1) / kTile;
  const int64_t groups = (B * T0 + 7) / 8;
  const dim3 grid(static_cast<unsigned>(groups * 8 * kBlocksPerTile));
  hipLaunchKernelGGL(norm_mod_bwd_f32_kernel, grid, dim3(kThreads), 0, s, g, x, mean, rstd, emb, dx, part, B, S,
                     T0, root);
  return hipGetLastError();
}

}  // namespace adaln
