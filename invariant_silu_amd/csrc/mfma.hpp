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
