// Measurement helpers for bench.py, built into a library of their own
// (libadaln_bench.so): nothing in the operator's library uses them.
//
// bench_flush: evicts the caches before a timed phase.  It writes every byte
//   of a caller buffer, then reads it all back, so that whatever the L2s and
//   the 256 MB memory-side cache held before is gone and the dirty lines the
//   write left behind are written back during the flush, not during the
//   phase that follows.  Pass a buffer of at least twice the memory-side
//   cache.  Optional caller events are recorded by the flush's own dispatches
//   (the start of its first kernel, the end of its last), so a phase between
//   two flushes is timed with no event packet inside it.
// bench_stream_copy: a plain device copy, 16 bytes per lane, four loads in
//   flight per lane before the four stores: the bandwidth a stream of equal
//   bytes reaches on this part, the ceiling the step is set against.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kThreads) void fill_kernel(uint4* __restrict__ p, int64_t n16, uint32_t v) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  const uint4 w = make_uint4(v, v ^ 1u, v ^ 2u, v ^ 3u);
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n16; i += stride) p[i] = w;
}

// Reads every 16-byte chunk; the xor of all of them is stored only when it
// equals a value the fill never produces, so the loads cannot be dropped and
// nothing is written in practice.
__global__ __launch_bounds__(kThreads) void read_kernel(const uint4* __restrict__ p, int64_t n16,
                                                        uint32_t* __restrict__ sink) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  uint32_t acc = 0;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n16; i += stride) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x5a5a5a5bu) sink[threadIdx.x] = acc;
}

__global__ __launch_bounds__(kThreads) void copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                        int64_t n16) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) dst[i + u * stride] = v[u];
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

unsigned grid_for(int64_t n16) {
  // 8 blocks per compute unit on 256 compute units, fewer for small buffers
  const int64_t want = (n16 + kThreads - 1) / kThreads;
  return static_cast<unsigned>(want < 2048 ? (want > 0 ? want : 1) : 2048);
}

}  // namespace

extern "C" {

// 0 on success, -1 for a bad argument (NULL, size not a positive multiple of
// 16 bytes, pointer not 16-byte aligned), -7 for a launch error.
int bench_flush(void* buf, size_t bytes, void* ev_start, void* ev_end, void* stream) {
  if (!buf || bytes == 0 || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(buf) % 16 != 0) return -1;
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const uint32_t v = 0x5a5a5a5au;
  hipExtLaunchKernelGGL(fill_kernel, dim3(grid_for(n16)), dim3(kThreads), 0, s,
                        reinterpret_cast<hipEvent_t>(ev_start), nullptr, 0, static_cast<uint4*>(buf), n16, v);
  hipExtLaunchKernelGGL(read_kernel, dim3(grid_for(n16)), dim3(kThreads), 0, s, nullptr,
                        reinterpret_cast<hipEvent_t>(ev_end), 0, static_cast<const uint4*>(buf), n16,
                        static_cast<uint32_t*>(buf));
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

// Optional caller events are recorded by the copy's own dispatch (the start
// and the end of the kernel), as for the kernel they are compared with.
int bench_stream_copy(const void* src, void* dst, size_t bytes, void* ev_start, void* ev_end, void* stream) {
  if (!src || !dst || bytes == 0 || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(src) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(dst) % 16 != 0)
    return -1;
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  hipExtLaunchKernelGGL(copy_kernel, dim3(grid_for(n16)), dim3(kThreads), 0, reinterpret_cast<hipStream_t>(stream),
                        reinterpret_cast<hipEvent_t>(ev_start), reinterpret_cast<hipEvent_t>(ev_end), 0,
                        static_cast<const uint4*>(src), static_cast<uint4*>(dst), n16);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

// Timing events for the flushes and for adaln_norm_mod_bwd_level0 (created
// with timing enabled; milliseconds between two recorded events after the
// stream has reached both).
int bench_event_create(void** ev) {
  hipEvent_t e = nullptr;
  if (!ev || hipEventCreate(&e) != hipSuccess) return -7;
  *ev = e;
  return 0;
}
int bench_event_elapsed(void* a, void* b, float* ms) {
  if (hipEventSynchronize(reinterpret_cast<hipEvent_t>(b)) != hipSuccess) return -7;
  return hipEventElapsedTime(ms, reinterpret_cast<hipEvent_t>(a), reinterpret_cast<hipEvent_t>(b)) == hipSuccess ? 0
                                                                                                                   : -7;
}
int bench_event_destroy(void* ev) { return hipEventDestroy(reinterpret_cast<hipEvent_t>(ev)) == hipSuccess ? 0 : -7; }

}  // extern "C"
