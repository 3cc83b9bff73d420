// Modulation projection, backward, from the fp32 d_emb = (d_scale | d_shift):
//   dW[j,k]  = bf16(fl32(sum_b d_emb[b,j] * a[b,k]))      (fp32 products)
//   db[j]    = bf16(fl32(sum_b d_emb[b,j]))
//   da[b,k]  = fl32(sum_j d_emb[b,j] * W[j,k])             (fp32 products)
//   dtemb    = bf16(da * silu'(temb))
// (RL-Kernel pull request 538: "What" -- projection backward behind the
// fixed-order projection -- and the review thread's SiLU VJP.)
// All sums accumulate fp32 products in fp64 in a fixed order:
//   dW, db  : samples in ascending order (trailing zero samples change nothing);
//   da      : 32 fixed parts of 192 rows; in a part, 8 row slots each walk
//             every 8th row in order, slots combined as a pairwise tree; the
//             32 part sums are added in order by the final kernel.
// None of these orders depends on the batch size, so dtemb of a sample is the
// same bytes alone or in any batch.
//
// B <= 4: proj_bwd_small_kernel, one grid with a dW-writing and a W-reading
//   half over the same (192-row, 256-column) tiles; the dW half computes
//   a = bf16(SiLU(temb)) per thread for its own 8 columns.
// B > 4:  silu_kernel (a into the workspace), proj_bwd_dw_kernel, then
//   proj_bwd_da_kernel in batch chunks of 4 (same arithmetic per element).
// proj_bwd_final_kernel: dtemb from the 32 partials, and db.
#include "common.hpp"
#include "launch.hpp"

namespace adaln {

namespace {

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

// Small batches (B <= 4, a template parameter): one grid, two kinds of block
// over the same (192-row part, 256-column block) tiles.  blockIdx.z = 0 writes
// dW (a write stream; each thread computes a = bf16(SiLU(temb)) for its 8
// columns), blockIdx.z = 1 reads W and forms the fp64 da partials (a read
// stream).  The two streams run side by side.
template <int NB>
__global__ __launch_bounds__(kBlockThreads) void proj_bwd_small_kernel(
    const float* __restrict__ d_emb, const uint16_t* __restrict__ temb,
    const uint16_t* __restrict__ W, uint16_t* __restrict__ dW, double* __restrict__ part) {
  __shared__ double red[kSlots][NB][kTileCols];
  __shared__ float de_lds[NB][kRowsPerPart];
  const int p = blockIdx.x;
  const int kb = blockIdx.y;
  const bool write_dw = blockIdx.z == 0;
  const int ct = threadIdx.x % kColThreads;
  const int slot = threadIdx.x / kColThreads;
  const int col = kb * kTileCols + ct * 8;
  const int jbase = p * kRowsPerPart;
  constexpr int kDeLoads = (NB * kRowsPerPart + kBlockThreads - 1) / kBlockThreads;

  // small loads first (the memory counter drains in issue order)
  float de_r[kDeLoads];
#pragma unroll
  for (int k = 0; k < kDeLoads; ++k) {
    const int idx = threadIdx.x + kBlockThreads * k;
    if (idx < NB * kRowsPerPart)
      de_r[k] = d_emb[static_cast<int64_t>(idx / kRowsPerPart) * kN + jbase + idx % kRowsPerPart];
  }
  if (write_dw) {
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
    return;
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

}  // namespace

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

}  // namespace adaln
