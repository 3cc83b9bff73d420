// Modulation projection, forward:  emb = bf16(SiLU(temb) W^T + b)
// (RL-Kernel pull request 538, "What": 3072 -> 6144, chunk(2) = (scale, shift)).
//
// One kernel, an HBM-bound pass over W (37.75 MB).  Each wave owns
// kRowsPerWave rows of W and keeps them in registers; lane l holds the 16-byte
// chunks l, l+64, ..., l+320 of each row.  The W loads are issued first; while
// they are in flight the block computes a = bf16(SiLU(temb)) for up to 4
// samples into LDS (silu_bf16: identical bits to the float64 definition).
// bf16 x bf16 products are exact in fp32; they are accumulated in fp64 in a
// fixed order (chunk-major within the lane, then the lane tree of
// wave_sum_f64), rounded once to fp32, the bias added in fp32 and the result
// rounded once to bf16.  The arithmetic of every (b, j) is the same for any
// batch size and any grid, so a sample's emb bytes do not depend on B.
#include "common.hpp"
#include "launch.hpp"

namespace adaln {

namespace {

constexpr int kPfWaves = 4;
constexpr int kRowsPerWave = 4;
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kPfRowsPerBlock = kPfWaves * kRowsPerWave;   // 16 -> 384 blocks
constexpr int kPfBatchChunk = 4;                           // samples of a staged in LDS
constexpr int kLaneChunks = kChunks / 64;                  // 6

__global__ __launch_bounds__(256) void silu_kernel(const uint16_t* __restrict__ temb,
                                                   uint16_t* __restrict__ a, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) a[i] = silu_bf16(bf16_to_f32(temb[i]));
}

__global__ __launch_bounds__(kPfThreads) void proj_fwd_kernel(const uint16_t* __restrict__ temb,
                                                              const uint16_t* __restrict__ W,
                                                              const uint16_t* __restrict__ bias,
                                                              uint16_t* __restrict__ emb,
                                                              int64_t B) {
  __shared__ uint4 a_lds[kPfBatchChunk * kChunks];   // 24 KB
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int row0 = (blockIdx.x * kPfWaves + wave) * kRowsPerWave;

  uint4 w[kRowsPerWave][kLaneChunks];
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
    for (int i = 0; i < kLaneChunks; ++i)
      w[r][i] = ld16(W + static_cast<int64_t>(row0 + r) * kD + (lane + 64 * i) * 8);
  float bias_f[kRowsPerWave];
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) bias_f[r] = bf16_to_f32(bias[row0 + r]);

#pragma unroll 1
  for (int64_t b0 = 0; b0 < B; b0 += kPfBatchChunk) {
    const int nb = static_cast<int>((B - b0) < kPfBatchChunk ? (B - b0) : kPfBatchChunk);
    __syncthreads();
    for (int c = threadIdx.x; c < nb * kChunks; c += kPfThreads) {
      float z[8];
      unpack8(ld16(temb + (b0 + c / kChunks) * kD + (c % kChunks) * 8), z);
      uint4 v;
      v.x = static_cast<uint32_t>(silu_bf16(z[0])) | (static_cast<uint32_t>(silu_bf16(z[1])) << 16);
      v.y = static_cast<uint32_t>(silu_bf16(z[2])) | (static_cast<uint32_t>(silu_bf16(z[3])) << 16);
      v.z = static_cast<uint32_t>(silu_bf16(z[4])) | (static_cast<uint32_t>(silu_bf16(z[5])) << 16);
      v.w = static_cast<uint32_t>(silu_bf16(z[6])) | (static_cast<uint32_t>(silu_bf16(z[7])) << 16);
      a_lds[c] = v;
    }
    __syncthreads();
    // the W registers are opaque to the compiler here, so their unpacking is
    // not hoisted out of this loop into 192 extra registers
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
      for (int i = 0; i < kLaneChunks; ++i)
        asm volatile("" : "+v"(w[r][i].x), "+v"(w[r][i].y), "+v"(w[r][i].z), "+v"(w[r][i].w));

    double acc[kRowsPerWave][kPfBatchChunk];
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
      for (int bb = 0; bb < kPfBatchChunk; ++bb) acc[r][bb] = 0.0;
#pragma unroll
    for (int i = 0; i < kLaneChunks; ++i) {
      float av[kPfBatchChunk][8];
#pragma unroll
      for (int bb = 0; bb < kPfBatchChunk; ++bb)
        if (bb < nb) unpack8(a_lds[bb * kChunks + lane + 64 * i], av[bb]);
#pragma unroll
      for (int r = 0; r < kRowsPerWave; ++r) {
        float wv[8];
        unpack8(w[r][i], wv);
#pragma unroll
        for (int bb = 0; bb < kPfBatchChunk; ++bb)
          if (bb < nb)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[r][bb] += static_cast<double>(av[bb][e] * wv[e]);
      }
    }
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
#pragma unroll
      for (int bb = 0; bb < kPfBatchChunk; ++bb) {
        if (bb < nb) {
          const double tot = wave_sum_f64(acc[r][bb]);
          if (lane == r * kPfBatchChunk + bb) {
            const float v = static_cast<float>(tot) + bias_f[r];
            emb[(b0 + bb) * kN + row0 + r] = f32_to_bf16(v);
          }
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_silu(const uint16_t* temb, uint16_t* a, int64_t n, hipStream_t s) {
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(silu_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, temb, a, n);
  return hipGetLastError();
}

hipError_t launch_proj_fwd(const uint16_t* temb, const uint16_t* W, const uint16_t* bias,
                           uint16_t* emb, int64_t B, hipStream_t s) {
  static_assert(kN % kPfRowsPerBlock == 0, "rows per block must divide N");
  hipLaunchKernelGGL(proj_fwd_kernel, dim3(kN / kPfRowsPerBlock), dim3(kPfThreads), 0, s, temb, W,
                     bias, emb, B);
  return hipGetLastError();
}

}  // namespace adaln
