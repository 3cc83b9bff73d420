// Forward of the AdaLN final modulation (RL-Kernel pull request 538, "What";
// rounding points of miles_diffusion pull request 108):
//
//   emb  = bf16(fl32(SiLU(temb) W^T) + b)          (scale | shift), 3072 -> 6144
//   mu   = fl32(sum_d x_d) / D,  var = fl32(sum_d (x_d - mu)^2) / D
//   rstd = 1 / sqrt(var + eps),  n = (x - mu) * rstd
//   out  = bf16((n * m) + shift),  m = bf16(1 + scale)
//
// Device pieces shared by every kernel below, so the standalone entry points
// and the overlapped stage kernels compute identical bits:
//
// proj_block<NB> (B = NB <= 4): 8 rows of W (4 waves x 2 rows) held in
//   registers; lane l holds the 16-byte chunks l, l+64, ..., l+320 of a row,
//   loaded chunk-major.  The temb loads are issued first; their SiLU
//   (silu8_fast, with the rare near-tie elements redone by silu_bf16_exact:
//   identical bits to the float64 definition) goes to LDS while W is in
//   flight.  bf16 x bf16 products (exact in fp32) are accumulated in fp64
//   (mac_exact): chunk-major within the lane, then the fixed lane tree of
//   wave_sum_f64; one rounding to fp32, the bias added in fp32, one rounding
//   to bf16.  One accumulator per sample: emb of a sample does not depend on
//   B or the grid.
// proj_wide_kernel (B > 4): the same rows, lanes, chunks and order for 8
//   samples per block, so the same bits.
// row_stats: one wave per row, the lane's 48 values summed in fp64 in order,
//   then wave_sum_f64; (x - mu) and its square in fp32; correctly rounded
//   sqrt and divide.
// modulate: two fp32 operations per element, one bf16 rounding.
//
// Kernels: proj_fwd_kernel / proj_wide_kernel (adaln_proj_fwd),
// norm_mod_fwd_kernel (statistics and modulation, adaln_norm_mod_fwd), and
// for the one-call forward adaln_fwd with B <= 4: fwd_stage1_kernel
// (projection blocks and statistics blocks in one grid: two independent HBM
// streams, W and x) then norm_modulate_kernel; with B > 4, proj_wide_kernel
// then norm_mod_fwd_kernel.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace adaln {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kLaneChunks = kChunks / 64;                  // 6
constexpr int kRows = 2;                                   // rows of W per wave
constexpr int kProjRowsPerBlock = kWaves * kRows;          // 8
constexpr int kProjBlocks = kN / kProjRowsPerBlock;        // 768
constexpr int kMaxNarrowBatch = 4;                         // proj_block up to here
static_assert(kN % kProjRowsPerBlock == 0, "rows per block must divide N");

// ----------------------------------------------------------- projection ----
template <int NB>
struct ProjShared {
  uint4 a[NB * kChunks];
};

// Projection blocks for B = NB <= 4 (one pass over the samples).
template <int NB>
__device__ __forceinline__ void proj_block(const uint16_t* __restrict__ temb,
                                           const uint16_t* __restrict__ W,
                                           const uint16_t* __restrict__ bias,
                                           uint16_t* __restrict__ emb, int blk, uint4* a_lds) {
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
  uint4 w[kLaneChunks][kRows];
#pragma unroll
  for (int i = 0; i < kLaneChunks; ++i)
#pragma unroll
    for (int r = 0; r < kRows; ++r)
      w[i][r] = ld16(W + static_cast<int64_t>(row0 + r) * kD + (lane + 64 * i) * 8);

  // SiLU of the NB samples into LDS; elements the fast path flags are redone
  // from memory in a separate, rarely taken loop
  uint64_t redo = 0;
#pragma unroll
  for (int k = 0; k < kStage; ++k) {
    const int c = threadIdx.x + kThreads * k;
    if (c < NB * kChunks) {
      uint32_t m;
      a_lds[c] = silu8_fast(tz[k], m);
      redo |= static_cast<uint64_t>(m) << (8 * k);
    }
  }
  while (redo != 0) {
    const int bit = __builtin_ctzll(redo);
    redo &= redo - 1;
    const int c = threadIdx.x + kThreads * (bit / 8);
    const int e = bit % 8;
    reinterpret_cast<uint16_t*>(a_lds)[c * 8 + e] =
        silu_bf16_exact(bf16_to_f32(temb[(c / kChunks) * kD + (c % kChunks) * 8 + e]));
  }
  __syncthreads();

  double acc[kRows][NB];
#pragma unroll
  for (int r = 0; r < kRows; ++r)
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) acc[r][bb] = 0.0;
#pragma unroll
  for (int i = 0; i < kLaneChunks; ++i) {
    float av[NB][8];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) unpack8(a_lds[bb * kChunks + lane + 64 * i], av[bb]);
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      float wv[8];
      unpack8(w[i][r], wv);
#pragma unroll
      for (int bb = 0; bb < NB; ++bb)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][bb] = mac_exact(av[bb][e], wv[e], acc[r][bb]);
    }
  }
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      const double tot = wave_sum_f64(acc[r][bb]);
      if (lane == r * NB + bb) {
        const float v = static_cast<float>(tot) + bias_f[r];
        emb[bb * kN + row0 + r] = f32_to_bf16(v);
      }
    }
  }
}

// Projection for B > 4: the same 8 rows of W per block (same lanes, chunks
// and order), kWideBT samples per blockIdx.y.  Per (sample, row) the lane's
// partial sum and the wave tree are exactly those of proj_block, so emb has
// the same bits whatever B.
constexpr int kWideBT = 8;
constexpr int kWideSB = 1;

// kHaveA: `src` already holds a = bf16(SiLU(temb)) [B, 3072] (computed once
// by silu_kernel); otherwise `src` is temb and every block computes the SiLU
// of its samples (768-fold redundant, which the arithmetic-bound large-batch
// case cannot hide).  a has the same bits either way.
template <bool kHaveA>
__global__ __launch_bounds__(kThreads) void proj_wide_kernel(const uint16_t* __restrict__ src,
                                                             const uint16_t* __restrict__ W,
                                                             const uint16_t* __restrict__ bias,
                                                             uint16_t* __restrict__ emb, int64_t B) {
  const uint16_t* __restrict__ temb = src;
  constexpr int kStage = kWideBT * kChunks / kThreads;   // 12 chunks of 8 per thread
  static_assert(kWideBT * kChunks % kThreads == 0, "staging layout");
  __shared__ uint4 a_lds[kWideBT * kChunks];            // 48 KB
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int row0 = (static_cast<int>(blockIdx.x) * kWaves + wave) * kRows;
  const int64_t b0 = static_cast<int64_t>(blockIdx.y) * kWideBT;
  const int nb = static_cast<int>((B - b0) < kWideBT ? (B - b0) : kWideBT);

  uint4 tz[kStage];
#pragma unroll
  for (int k = 0; k < kStage; ++k) {
    const int c = threadIdx.x + kThreads * k;
    if (c / kChunks < nb) tz[k] = ld16(temb + (b0 + c / kChunks) * kD + (c % kChunks) * 8);
  }
  float bias_f[kRows];
#pragma unroll
  for (int r = 0; r < kRows; ++r) bias_f[r] = bf16_to_f32(bias[row0 + r]);
  uint4 w[kLaneChunks][kRows];
#pragma unroll
  for (int i = 0; i < kLaneChunks; ++i)
#pragma unroll
    for (int r = 0; r < kRows; ++r)
      w[i][r] = ld16(W + static_cast<int64_t>(row0 + r) * kD + (lane + 64 * i) * 8);

  // SiLU into LDS one chunk at a time (a scheduling barrier per chunk keeps
  // the temporaries of only one chunk live next to the W registers); the
  // elements the fast path cannot decide are redone from memory afterwards
  uint64_t redo[2] = {0, 0};
#pragma unroll
  for (int k = 0; k < kStage; ++k) {
    if (kHaveA) {
      const int c = threadIdx.x + kThreads * k;
      if (c / kChunks < nb) a_lds[c] = tz[k];
      continue;
    }
    const int c = threadIdx.x + kThreads * k;
    if (c / kChunks < nb) {
      uint32_t m;
      a_lds[c] = silu8_fast(tz[k], m);
      redo[k / 8] |= static_cast<uint64_t>(m) << (8 * (k % 8));
    }
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    while (redo[h] != 0) {
      const int bit = __builtin_ctzll(redo[h]);
      redo[h] &= redo[h] - 1;
      const int c = threadIdx.x + kThreads * (8 * h + bit / 8);
      const int e = bit % 8;
      reinterpret_cast<uint16_t*>(a_lds)[c * 8 + e] =
          silu_bf16_exact(bf16_to_f32(temb[(b0 + c / kChunks) * kD + (c % kChunks) * 8 + e]));
    }
  }
  __syncthreads();

  // W unpacked to fp32 once (96 registers); then per group of samples the
  // lane's partial per row, chunk-major as in proj_block, and the wave tree
  float wf[kLaneChunks][kRows][8];
#pragma unroll
  for (int i = 0; i < kLaneChunks; ++i)
#pragma unroll
    for (int r = 0; r < kRows; ++r) unpack8(w[i][r], wf[i][r]);
#pragma unroll 1
  for (int s0 = 0; s0 < kWideBT; s0 += kWideSB) {
    // kWideSB samples at a time: 2 * kWideSB independent fp64 chains per wave
    // (one per sample and row) hide the add latency.  Slots past nb hold
    // stale LDS data; their sums are never stored.
    double acc[kWideSB][kRows];
#pragma unroll
    for (int q = 0; q < kWideSB; ++q)
#pragma unroll
      for (int r = 0; r < kRows; ++r) acc[q][r] = 0.0;
#pragma unroll
    for (int i = 0; i < kLaneChunks; ++i) {
#pragma unroll
      for (int q = 0; q < kWideSB; ++q) {
        float av[8];
        unpack8(a_lds[(s0 + q) * kChunks + lane + 64 * i], av);
#pragma unroll
        for (int r = 0; r < kRows; ++r)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[q][r] = mac_exact(av[e], wf[i][r][e], acc[q][r]);
      }
    }
#pragma unroll
    for (int q = 0; q < kWideSB; ++q) {
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        const double tot = wave_sum_f64(acc[q][r]);
        if (lane == r && s0 + q < nb) {
          const float v = static_cast<float>(tot) + bias_f[r];
          emb[(b0 + s0 + q) * kN + row0 + r] = f32_to_bf16(v);
        }
      }
    }
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
template <int NB>
__global__ __launch_bounds__(kThreads) void proj_fwd_kernel(const uint16_t* __restrict__ temb,
                                                            const uint16_t* __restrict__ W,
                                                            const uint16_t* __restrict__ bias,
                                                            uint16_t* __restrict__ emb) {
  __shared__ ProjShared<NB> sh;
  proj_block<NB>(temb, W, bias, emb, blockIdx.x, sh.a);
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
// modulation block for the same rows right after, which then finds x in that
// XCD's L2 (3.1 MB of x per XCD at S = 4096 against a 4 MB L2).
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

// B <= 4: proj_block with NB = B; larger batches: proj_wide_kernel
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

hipError_t launch_wide(const uint16_t* temb, const uint16_t* W, const uint16_t* bias, uint16_t* emb,
                       int64_t B, hipStream_t s) {
  const int64_t by = (B + kWideBT - 1) / kWideBT;
  hipLaunchKernelGGL(proj_wide_kernel<false>, dim3(kProjBlocks, static_cast<unsigned>(by)), dim3(kThreads), 0,
                     s, temb, W, bias, emb, B);
  return hipGetLastError();
}

// a = bf16(SiLU(temb)) computed once into `a`, then the projection from it
hipError_t launch_wide_from_a(const uint16_t* temb, uint16_t* a, const uint16_t* W, const uint16_t* bias,
                              uint16_t* emb, int64_t B, hipStream_t s) {
  if (hipError_t e = launch_silu(temb, a, B * kD, s); e != hipSuccess) return e;
  const int64_t by = (B + kWideBT - 1) / kWideBT;
  hipLaunchKernelGGL(proj_wide_kernel<true>, dim3(kProjBlocks, static_cast<unsigned>(by)), dim3(kThreads), 0,
                     s, a, W, bias, emb, B);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_proj_fwd(const uint16_t* temb, const uint16_t* W, const uint16_t* bias,
                           uint16_t* emb, int64_t B, hipStream_t s) {
  if (B > kMaxNarrowBatch) return launch_wide(temb, W, bias, emb, B, s);
  return by_batch(B, [&](auto nb) {
    hipLaunchKernelGGL(proj_fwd_kernel<decltype(nb)::value>, dim3(kProjBlocks), dim3(kThreads), 0, s, temb,
                       W, bias, emb);
    return hipGetLastError();
  });
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
    // the projection is arithmetic-bound here: SiLU once (into the first
    // B * 3072 elements of `out`, which the modulation overwrites later),
    // the projection, then statistics and modulation in one pass over x
    if (hipError_t e = launch_wide_from_a(temb, out, W, bias, emb, B, s); e != hipSuccess) return e;
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

}  // namespace adaln
