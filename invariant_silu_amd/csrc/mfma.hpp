// Helpers for the fp64 matrix-core kernels (gfx950).
//
// v_mfma_f64_16x16x4f64: lane L supplies A[L % 16][L / 16] and
// B[L / 16][L % 16]; lane L holds D[L / 16 + 4 v][L % 16] in component v.
// Each output is the chain acc = fma(A[i][k], B[k][j], acc) for k = 0, 1, 2, 3
// in that order (fused: one rounding per step), which the vector units
// reproduce bit for bit with __builtin_fma in the same order.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace adaln {

typedef double f64x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f64x4_t mfma_f64(double a, double b, f64x4_t acc) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc, 0, 0, 0);
}

__device__ __forceinline__ double bf_lo64(uint32_t w) { return static_cast<double>(bf_lo(w)); }
__device__ __forceinline__ double bf_hi64(uint32_t w) { return static_cast<double>(bf_hi(w)); }
__device__ __forceinline__ double bf_half64(uint32_t w, int h) { return h ? bf_hi64(w) : bf_lo64(w); }

// n consecutive elements of one row held raw in registers (loaded with
// buffer loads of 8 or 16 bytes); at(i) is element i widened exactly to fp64.
template <int n, typename T>
struct RowRun;
template <int n>
struct RowRun<n, uint16_t> {
  static_assert(n % 4 == 0, "8-byte loads");
  uint32_t v[n / 2];
  __device__ __forceinline__ void load(const Buffer& b, uint32_t lane_off, uint32_t off) {
#pragma unroll
    for (int q = 0; q < n / 4; ++q) {
      const auto t = __builtin_amdgcn_raw_buffer_load_b64(b.rsrc, lane_off, off + 8 * q, 0);
      v[2 * q] = t[0];
      v[2 * q + 1] = t[1];
    }
  }
  __device__ __forceinline__ double at(int i) const { return bf_half64(v[i / 2], i & 1); }
};
template <int n>
struct RowRun<n, float> {
  static_assert(n % 4 == 0, "16-byte loads");
  float v[n];
  __device__ __forceinline__ void load(const Buffer& b, uint32_t lane_off, uint32_t off) {
#pragma unroll
    for (int q = 0; q < n / 4; ++q) {
      const uint4 t = b.u128(lane_off, off + 16 * q);
      v[4 * q] = __uint_as_float(t.x);
      v[4 * q + 1] = __uint_as_float(t.y);
      v[4 * q + 2] = __uint_as_float(t.z);
      v[4 * q + 3] = __uint_as_float(t.w);
    }
  }
  __device__ __forceinline__ double at(int i) const { return static_cast<double>(v[i]); }
};

// Pairwise tree over values pushed in index order (0 + 1, 2 + 3, then pairs of
// pairs, ...); node[kLevels] is the root once 2^kLevels values are in.
template <int kLevels, typename T>
struct PairTree {
  T node[kLevels + 1];
  template <int kLeaf, int kLvl = 0>
  __device__ __forceinline__ void push(T t) {
    if constexpr (kLvl < kLevels && ((kLeaf >> kLvl) & 1)) push<kLeaf, kLvl + 1>(node[kLvl] + t);
    else node[kLvl] = t;
  }
};

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

constexpr int ilog2(int n) { return n <= 1 ? 0 : 1 + ilog2(n / 2); }

// Pairwise combination of kCount subtrees v[0 .. kCount) in index order.
template <int kCount, typename T>
__device__ __forceinline__ T pair_reduce(T (&v)[kCount]) {
#pragma unroll
  for (int step = 1; step < kCount; step *= 2)
#pragma unroll
    for (int w = 0; w + step < kCount; w += 2 * step) v[w] = v[w] + v[w + step];
  return v[0];
}

}  // namespace adaln
