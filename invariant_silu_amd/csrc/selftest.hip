// Strict-math probe kernel: the operations the rounding points rely on.
//   out[4i]   = sqrt(v)        (must be correctly rounded)
//   out[4i+1] = 1 / v          (must be correctly rounded)
//   out[4i+2] = v * w + c      (two roundings: must not be contracted to fma)
//   out[4i+3] = fp32(fp64(v) / fp64(w))
//   bits[i]   = bf16(v)        (round to nearest, ties to even)
#include "common.hpp"
#include "launch.hpp"

namespace adaln {

namespace {

__global__ __launch_bounds__(256) void probe_kernel(const float* __restrict__ in,
                                                    float* __restrict__ out,
                                                    uint32_t* __restrict__ bits, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float v = in[i];
  const float w = in[(i + 1) % n];
  const float c = in[(i + 2) % n];
  out[4 * i + 0] = __builtin_sqrtf(__builtin_fabsf(v));
  out[4 * i + 1] = 1.0f / v;
  out[4 * i + 2] = v * w + c;
  out[4 * i + 3] = static_cast<float>(static_cast<double>(v) / static_cast<double>(w));
  bits[i] = f32_to_bf16(v);
}

}  // namespace

hipError_t launch_selftest_probe(const float* in, float* out, uint32_t* bits, int n,
                                 hipStream_t s) {
  hipLaunchKernelGGL(probe_kernel, dim3((n + 255) / 256), dim3(256), 0, s, in, out, bits, n);
  return hipGetLastError();
}

}  // namespace adaln
