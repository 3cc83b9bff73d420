// LayerNorm + modulation, forward (RL-Kernel pull request 538, "What";
// rounding points of miles_diffusion pull request 108):
//   mu   = fl32(sum_d x_d) / D                  (sum exact in fp64, rounded once)
//   var  = fl32(sum_d (x_d - mu)^2) / D         ((x-mu) and its square in fp32)
//   rstd = 1 / sqrt(var + eps)                  (correctly rounded sqrt and divide)
//   n_d  = (x_d - mu) * rstd                    (fp32)
//   out  = bf16((n_d * m_d) + shift_d),  m = bf16(1 + scale)
// One wave per row: lane l holds the 16-byte chunks l, l+64, ..., l+320 of the
// row; row sums are fp64 lane partials reduced by wave_sum_f64 (fixed lane
// tree, no LDS, no atomics).  A block of 4 waves handles 4 rows of ONE sample;
// (1 + scale) and shift for that sample are staged in LDS while the row loads
// are in flight.  mu and rstd are written for the
// backward pass (8 bytes per row).
#include "common.hpp"
#include "launch.hpp"

namespace adaln {

namespace {

constexpr int kNfWaves = 4;
constexpr int kNfThreads = 64 * kNfWaves;
constexpr int kNfRowsPerBlock = kNfWaves;
constexpr int kLaneChunks = kChunks / 64;   // 6

__global__ __launch_bounds__(kNfThreads) void norm_mod_fwd_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ emb, uint16_t* __restrict__ out,
    float* __restrict__ mean, float* __restrict__ rstd, int64_t S, float eps) {
  __shared__ float4 m_lds[kD / 4];
  __shared__ float4 sh_lds[kD / 4];
  const int64_t b = blockIdx.y;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t s = static_cast<int64_t>(blockIdx.x) * kNfRowsPerBlock + wave;
  const bool valid = s < S;
  const int64_t row = b * S + (valid ? s : 0);

  // small loads first: the memory counter drains in issue order, so staging
  // needs only these, while the row loads below stay in flight
  const uint2* scale = reinterpret_cast<const uint2*>(emb + b * kN);
  const uint2* shift = reinterpret_cast<const uint2*>(emb + b * kN + kD);
  uint2 sc[3], sh[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    sc[k] = scale[threadIdx.x + kNfThreads * k];
    sh[k] = shift[threadIdx.x + kNfThreads * k];
  }
  uint4 xv[kLaneChunks];
#pragma unroll
  for (int i = 0; i < kLaneChunks; ++i) xv[i] = ld16(x + row * kD + (lane + 64 * i) * 8);
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int c = threadIdx.x + kNfThreads * k;
    m_lds[c] = make_float4(round_bf16(1.0f + bf_lo(sc[k].x)), round_bf16(1.0f + bf_hi(sc[k].x)),
                           round_bf16(1.0f + bf_lo(sc[k].y)), round_bf16(1.0f + bf_hi(sc[k].y)));
    sh_lds[c] = make_float4(bf_lo(sh[k].x), bf_hi(sh[k].x), bf_lo(sh[k].y), bf_hi(sh[k].y));
  }
  __syncthreads();
  if (!valid) return;   // whole wave

  double acc = 0.0;
#pragma unroll
  for (int i = 0; i < kLaneChunks; ++i) {
    float v[8];
    unpack8(xv[i], v);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += static_cast<double>(v[e]);
  }
  const float mu = static_cast<float>(wave_sum_f64(acc)) / static_cast<float>(kD);
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
  const float rs = 1.0f / __builtin_sqrtf(var + eps);
  uint16_t* orow = out + row * kD;
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
  if (lane == 0) {
    mean[row] = mu;
    rstd[row] = rs;
  }
}

}  // namespace

hipError_t launch_norm_mod_fwd(const uint16_t* x, const uint16_t* emb, uint16_t* out, float* mean,
                               float* rstd, int64_t B, int64_t S, float eps, hipStream_t s) {
  const int64_t gx = (S + kNfRowsPerBlock - 1) / kNfRowsPerBlock;
  hipLaunchKernelGGL(norm_mod_fwd_kernel, dim3(static_cast<unsigned>(gx), static_cast<unsigned>(B)),
                     dim3(kNfThreads), 0, s, x, emb, out, mean, rstd, S, eps);
  return hipGetLastError();
}

}  // namespace adaln
