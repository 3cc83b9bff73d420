// Modulation projection, forward:  emb = bf16(SiLU(temb) W^T + b)
// (RL-Kernel pull request 538, "What": 3072 -> 6144, chunk(2) = (scale, shift)).
//
// One kernel, an HBM-bound pass over W (37.75 MB).  Each wave owns kRows rows
// of W and keeps them in registers; lane l holds the 16-byte chunks l, l+64,
// ..., l+320 of each row, loaded chunk-major so the products of chunk 0 can
// start while later chunks are still arriving.  Before the W loads, the block
// issues the loads of its first NB samples of temb; their SiLU
// (silu8_fast + silu_bf16_exact: identical bits to the float64 definition)
// is computed into LDS while W is in flight.  bf16 x bf16 products are exact
// in fp32; they are accumulated in fp64 in a fixed order (chunk-major within
// the lane, then the lane tree of wave_sum_f64), rounded once to fp32, the
// bias added in fp32 and the result rounded once to bf16.  The kernel is
// instantiated for NB = 1, 2 and 4 samples per pass; each sample has its own
// accumulator, so the arithmetic of every (b, j) is the same for any NB, any
// batch size and any grid: a sample's emb bytes do not depend on B.
#include "common.hpp"
#include "launch.hpp"

namespace adaln {

namespace {

constexpr int kPfWaves = 4;
constexpr int kRows = 2;                                   // rows of W per wave
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kPfRowsPerBlock = kPfWaves * kRows;          // 8 -> 768 blocks
constexpr int kLaneChunks = kChunks / 64;                  // 6

__global__ __launch_bounds__(256) void silu_kernel(const uint16_t* __restrict__ temb,
                                                   uint16_t* __restrict__ a, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) {
    const float z = bf16_to_f32(temb[i]);
    bool redo;
    const uint32_t v = silu_bf16_fast(z, redo);
    a[i] = redo ? silu_bf16_exact(z) : static_cast<uint16_t>(v);
  }
}

template <int NB>
__global__ __launch_bounds__(kPfThreads) void proj_fwd_kernel(const uint16_t* __restrict__ temb,
                                                              const uint16_t* __restrict__ W,
                                                              const uint16_t* __restrict__ bias,
                                                              uint16_t* __restrict__ emb,
                                                              int64_t B) {
  constexpr int kStage = (NB * kChunks + kPfThreads - 1) / kPfThreads;
  __shared__ uint4 a_lds[NB * kChunks];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int row0 = (blockIdx.x * kPfWaves + wave) * kRows;

  // SiLU of samples [b0, b0 + NB) into LDS; elements the fast path flags
  // are redone from memory in a separate, rarely taken loop
  auto stage = [&](const uint4 (&tz)[kStage], int64_t b0) __attribute__((always_inline)) {
    static_assert(kStage <= 8, "redo mask holds 8 chunks of 8 elements");
    uint64_t redo = 0;
#pragma unroll
    for (int k = 0; k < kStage; ++k) {
      const int c = threadIdx.x + kPfThreads * k;
      if (c < NB * kChunks) {
        uint32_t m;
        a_lds[c] = silu8_fast(tz[k], m);
        redo |= static_cast<uint64_t>(m) << (8 * k);
      }
    }
    while (redo != 0) {
      const int bit = __builtin_ctzll(redo);
      redo &= redo - 1;
      const int c = threadIdx.x + kPfThreads * (bit / 8);
      const int e = bit % 8;
      reinterpret_cast<uint16_t*>(a_lds)[c * 8 + e] =
          silu_bf16_exact(bf16_to_f32(temb[(b0 + c / kChunks) * kD + (c % kChunks) * 8 + e]));
    }
  };
  auto load_temb = [&](uint4 (&tz)[kStage], int64_t b0) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < kStage; ++k) {
      const int c = threadIdx.x + kPfThreads * k;
      if (c < NB * kChunks) tz[k] = ld16(temb + (b0 + c / kChunks) * kD + (c % kChunks) * 8);
    }
  };

  // small loads first: the memory counter drains in issue order, so the
  // first SiLU needs only these while the W rows stay in flight
  uint4 tz[kStage];
  load_temb(tz, 0);
  float bias_f[kRows];
#pragma unroll
  for (int r = 0; r < kRows; ++r) bias_f[r] = bf16_to_f32(bias[row0 + r]);
  uint4 w[kLaneChunks][kRows];
#pragma unroll
  for (int i = 0; i < kLaneChunks; ++i)
#pragma unroll
    for (int r = 0; r < kRows; ++r)
      w[i][r] = ld16(W + static_cast<int64_t>(row0 + r) * kD + (lane + 64 * i) * 8);
  stage(tz, 0);

#pragma unroll 1
  for (int64_t b0 = 0; b0 < B; b0 += NB) {
    if (b0 > 0) {
      __syncthreads();   // the previous pass is done reading a_lds
      load_temb(tz, b0);
      stage(tz, b0);
      // the W registers are opaque here, so their unpacking is not hoisted
      // out of this loop into extra registers
#pragma unroll
      for (int i = 0; i < kLaneChunks; ++i)
#pragma unroll
        for (int r = 0; r < kRows; ++r)
          asm volatile("" : "+v"(w[i][r].x), "+v"(w[i][r].y), "+v"(w[i][r].z), "+v"(w[i][r].w));
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
          for (int e = 0; e < 8; ++e) acc[r][bb] += static_cast<double>(av[bb][e] * wv[e]);
      }
    }
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) {
        const double tot = wave_sum_f64(acc[r][bb]);
        if (lane == r * NB + bb) {
          const float v = static_cast<float>(tot) + bias_f[r];
          emb[(b0 + bb) * kN + row0 + r] = f32_to_bf16(v);
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

// NB = the largest of 4, 2, 1 that divides B, so every pass is a full one.
hipError_t launch_proj_fwd(const uint16_t* temb, const uint16_t* W, const uint16_t* bias,
                           uint16_t* emb, int64_t B, hipStream_t s) {
  static_assert(kN % kPfRowsPerBlock == 0, "rows per block must divide N");
  const dim3 grid(kN / kPfRowsPerBlock), block(kPfThreads);
  if (B % 4 == 0) {
    hipLaunchKernelGGL(proj_fwd_kernel<4>, grid, block, 0, s, temb, W, bias, emb, B);
  } else if (B % 2 == 0) {
    hipLaunchKernelGGL(proj_fwd_kernel<2>, grid, block, 0, s, temb, W, bias, emb, B);
  } else {
    hipLaunchKernelGGL(proj_fwd_kernel<1>, grid, block, 0, s, temb, W, bias, emb, B);
  }
  return hipGetLastError();
}

}  // namespace adaln
