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
//             32 part sums are added in order by the dtemb kernel.
// None of these orders depends on the batch size, so dtemb of a sample is the
// same bytes alone or in any batch.
#include "common.hpp"
#include "launch.hpp"

namespace adaln {

namespace {

// ---- dW / db: a write stream over dW (37.75 MB), 4 rows per block ----------
constexpr int kDwRows = 4;
constexpr int kDwThreads = kChunks;     // 384: one 16-byte chunk of a row each
constexpr int kDwBatch = 8;

__global__ __launch_bounds__(kDwThreads) void proj_bwd_dw_kernel(const float* __restrict__ d_emb,
                                                                 const uint16_t* __restrict__ a,
                                                                 uint16_t* __restrict__ dW,
                                                                 uint16_t* __restrict__ db,
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
    for (int bb = 0; bb < kDwBatch; ++bb) {
      if (bb < nb) unpack8(ld16(a + (b0 + bb) * kD + t * 8), av[bb]);
    }
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
  if (t < kDwRows) {
    double s = 0.0;
    for (int64_t b = 0; b < B; ++b) s += static_cast<double>(d_emb[b * kN + j0 + t]);
    db[j0 + t] = f32_to_bf16(static_cast<float>(s));
  }
}

// ---- da partials: a read stream over W (37.75 MB) ---------------------------
constexpr int kDaCols = 256;                        // columns per block (32 threads x 8)
constexpr int kDaColThreads = kDaCols / 8;          // 32
constexpr int kDaSlots = 8;                         // row slots per block
constexpr int kDaThreads = kDaColThreads * kDaSlots;   // 256
constexpr int kDaRowsPerPart = kN / kProjBwdParts;  // 192
constexpr int kDaBatch = 4;                         // samples per block

__global__ __launch_bounds__(kDaThreads) void proj_bwd_da_kernel(const float* __restrict__ d_emb,
                                                                 const uint16_t* __restrict__ W,
                                                                 double* __restrict__ part,
                                                                 int64_t B) {
  __shared__ double red[kDaSlots][kDaBatch][kDaCols];   // 64 KB
  const int p = blockIdx.x;
  const int kb = blockIdx.y;
  const int64_t b0 = static_cast<int64_t>(blockIdx.z) * kDaBatch;
  const int nb = static_cast<int>((B - b0) < kDaBatch ? (B - b0) : kDaBatch);
  const int ct = threadIdx.x % kDaColThreads;
  const int slot = threadIdx.x / kDaColThreads;
  const int col = kb * kDaCols + ct * 8;
  const int jbase = p * kDaRowsPerPart;

  double acc[kDaBatch][8];
#pragma unroll
  for (int bb = 0; bb < kDaBatch; ++bb)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[bb][e] = 0.0;

  constexpr int kSteps = kDaRowsPerPart / kDaSlots;   // 24
  uint4 wcur = ld16(W + static_cast<int64_t>(jbase + slot) * kD + col);
  for (int i = 0; i < kSteps; ++i) {
    const int j = jbase + slot + kDaSlots * i;
    uint4 wnext = wcur;
    if (i + 1 < kSteps) wnext = ld16(W + static_cast<int64_t>(j + kDaSlots) * kD + col);
    float wv[8];
    unpack8(wcur, wv);
#pragma unroll
    for (int bb = 0; bb < kDaBatch; ++bb) {
      if (bb < nb) {
        const float d = d_emb[(b0 + bb) * kN + j];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[bb][e] += static_cast<double>(d * wv[e]);
      }
    }
    wcur = wnext;
  }
#pragma unroll
  for (int bb = 0; bb < kDaBatch; ++bb)
#pragma unroll
    for (int e = 0; e < 8; ++e) red[slot][bb][ct * 8 + e] = acc[bb][e];
  __syncthreads();
  for (int o = threadIdx.x; o < kDaBatch * kDaCols; o += kDaThreads) {
    const int bb = o / kDaCols;
    const int c = o % kDaCols;
    if (bb < nb) {
      const double v = ((red[0][bb][c] + red[1][bb][c]) + (red[2][bb][c] + red[3][bb][c])) +
                       ((red[4][bb][c] + red[5][bb][c]) + (red[6][bb][c] + red[7][bb][c]));
      part[(static_cast<int64_t>(p) * B + b0 + bb) * kD + kb * kDaCols + c] = v;
    }
  }
}

// ---- dtemb: sum the 32 parts in order, apply silu' ---------------------------
__global__ __launch_bounds__(256) void proj_bwd_dtemb_kernel(const double* __restrict__ part,
                                                             const uint16_t* __restrict__ temb,
                                                             uint16_t* __restrict__ dtemb,
                                                             int64_t B) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= B * kD) return;
  double s = 0.0;
#pragma unroll 8
  for (int p = 0; p < kProjBwdParts; ++p) s += part[static_cast<int64_t>(p) * B * kD + i];
  const float da = static_cast<float>(s);
  dtemb[i] = f32_to_bf16(da * dsilu_f32(bf16_to_f32(temb[i])));
}

}  // namespace

hipError_t launch_proj_bwd_dw(const float* d_emb, const uint16_t* a, uint16_t* dW, uint16_t* db,
                              int64_t B, hipStream_t s) {
  hipLaunchKernelGGL(proj_bwd_dw_kernel, dim3(kN / kDwRows), dim3(kDwThreads), 0, s, d_emb, a, dW,
                     db, B);
  return hipGetLastError();
}

hipError_t launch_proj_bwd_da(const float* d_emb, const uint16_t* W, double* part, int64_t B,
                              hipStream_t s) {
  static_assert(kN % kProjBwdParts == 0 && kDaRowsPerPart % kDaSlots == 0, "part layout");
  static_assert(kD % kDaCols == 0, "column blocks");
  const int64_t bz = (B + kDaBatch - 1) / kDaBatch;
  hipLaunchKernelGGL(proj_bwd_da_kernel,
                     dim3(kProjBwdParts, kD / kDaCols, static_cast<unsigned>(bz)), dim3(kDaThreads), 0,
                     s, d_emb, W, part, B);
  return hipGetLastError();
}

hipError_t launch_proj_bwd_dtemb(const double* part, const uint16_t* temb, uint16_t* dtemb,
                                 int64_t B, hipStream_t s) {
  const int64_t n = B * kD;
  hipLaunchKernelGGL(proj_bwd_dtemb_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256),
                     0, s, part, temb, dtemb, B);
  return hipGetLastError();
}

}  // namespace adaln
