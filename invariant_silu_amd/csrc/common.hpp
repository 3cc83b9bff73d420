// Shared device helpers for the AdaLN final-modulation kernels (gfx950).
//
// Numerics follow the autocast rounding points described in miles_diffusion
// pull request 108 ("Fused-norm rounding points"): fp32 LayerNorm, (1 + scale)
// rounded once to bf16, fp32 modulation, one bf16 rounding of the output.
// Everything is built with -ffp-contract=off: every float operation below is
// one IEEE operation, and a fused multiply-add appears only where it is
// written out.  bf16 stores use the hardware round-to-nearest-even conversion.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace adaln {

constexpr int kD = 3072;            // hidden width D (= conditioning width K)
constexpr int kN = 2 * kD;          // projection width N: (scale | shift)
constexpr int kN6 = 6 * kD;         // a block's 6-way modulation projection: 2 x (shift | scale | gate)
constexpr int kChunks = kD / 8;     // 16-byte chunks (8 bf16) per row: 384
constexpr int kTile = 32;           // tokens per level-0 tile of the token tree
constexpr int kMaxFoldLevels = 5;   // S <= 32^6 tokens

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round-to-nearest-even float -> bf16 (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t v = {lo, hi};
  bf16x2_t r = __builtin_convertvector(v, bf16x2_t);
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return static_cast<uint16_t>(pack_bf16x2(f, 0.0f) & 0xffffu);
}
// bf16 value of an fp32 number, as fp32 (round to nearest even).
__device__ __forceinline__ float round_bf16(float f) { return bf_lo(f32_to_bf16(f)); }

__device__ __forceinline__ void unpack8(const uint4& v, float (&f)[8]) {
  f[0] = bf_lo(v.x); f[1] = bf_hi(v.x);
  f[2] = bf_lo(v.y); f[3] = bf_hi(v.y);
  f[4] = bf_lo(v.z); f[5] = bf_hi(v.z);
  f[6] = bf_lo(v.w); f[7] = bf_hi(v.w);
}
__device__ __forceinline__ uint4 pack8(const float (&f)[8]) {
  uint4 r;
  r.x = pack_bf16x2(f[0], f[1]);
  r.y = pack_bf16x2(f[2], f[3]);
  r.z = pack_bf16x2(f[4], f[5]);
  r.w = pack_bf16x2(f[6], f[7]);
  return r;
}

__device__ __forceinline__ uint4 ld16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void st16(uint16_t* p, const uint4& v) {
  *reinterpret_cast<uint4*>(p) = v;
}
// Streaming (nontemporal) 16-byte store for outputs nothing in the step reads
// back soon.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void st16_nt(uint16_t* p, const uint4& v) {
  u32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
}

// A byte range read through a raw buffer resource.  The base is uniform; a
// load takes a per-lane byte offset in a VGPR and a uniform one in an SGPR,
// so a run of loads at fixed strides needs no per-load address arithmetic.
// Callers keep every load inside [0, bytes): nothing relies on the range
// check.  The third descriptor word is the gfx9-family raw-buffer format.
struct Buffer {
  __amdgpu_buffer_rsrc_t rsrc;
  __device__ __forceinline__ Buffer(const void* base, uint32_t bytes)
      : rsrc(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                               0x00020000)) {}
  __device__ __forceinline__ uint32_t u32(uint32_t lane_off, uint32_t uni_off) const {
    return __builtin_amdgcn_raw_buffer_load_b32(rsrc, lane_off, uni_off, 0);
  }
  __device__ __forceinline__ float f32(uint32_t lane_off, uint32_t uni_off) const {
    return __uint_as_float(u32(lane_off, uni_off));
  }
  __device__ __forceinline__ uint4 u128(uint32_t lane_off, uint32_t uni_off) const {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, lane_off, uni_off, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
  }
};

// Level-0 pairs of the token tree in memory: columns in groups of 64; per
// (sample, group, tile) 64 sums s followed by their 64 corrections c, tiles
// of a group consecutive.  The fold then reads each node's 32 children as one
// contiguous 16 KB run.  pair_index gives the index of s; c is 64 later.
constexpr int kPairGroup = 64;
__device__ __forceinline__ int64_t pair_index(int64_t b, int64_t groups, int64_t T0, int64_t tile,
                                              int64_t col) {
  return ((b * groups + col / kPairGroup) * T0 + tile) * (2 * kPairGroup) + col % kPairGroup;
}

// Level-0 token-tree pairs: plain stores, so the fold that reads them next
// finds them in the caches.
__device__ __forceinline__ void st8(float* p, float a, float b) {
  *reinterpret_cast<f32x2_t*>(p) = f32x2_t{a, b};
}

// Sum over the 64 lanes of a wave as a pairwise tree over lane index
// (xor 1, 2, 4, ..., 32).  IEEE addition commutes, so every lane ends with
// the same bits; the tree depends only on which value sits in which lane.
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// SiLU and its derivative, evaluated in float64 and rounded once to float32
// (RL-Kernel pull request 538, review thread: silu'(z) = s (1 + z (1 - s))).
__device__ __forceinline__ float silu_f32(float z) {
  const double zd = z;
  return static_cast<float>(zd / (1.0 + exp(-zd)));
}

__device__ __forceinline__ float dsilu_f32(float z) {
  const double zd = z;
  const double s = 1.0 / (1.0 + exp(-zd));
  return static_cast<float>(s * (1.0 + zd * (1.0 - s)));
}

// bf16(fl32(SiLU_f64(z))) computed mostly in fp32.  expf is accurate to about
// 1 ulp and the add and the correctly rounded divide add half an ulp each, so
// the fp32 value lies within 3 ulp of the float64 result.  bf16 rounding can
// only differ between the two if a rounding tie (low 16 bits 0x8000) lies in
// that window.  silu_bf16_fast returns the bf16 bits of the fp32 value and
// reports whether the float64 path must decide instead: within 8 ulp of a
// tie, a non-finite value, or |z| >= 64 (where expf(-z) approaches overflow
// and the result approaches the denormal range).  Callers redo the flagged
// elements with silu_bf16_exact in a separate, rarely taken loop.  Checked
// exhaustively over all finite bf16 inputs against the float64 definition.
__device__ __forceinline__ uint32_t silu_bf16_fast(float z, bool& redo) {
  const float y = z / (1.0f + expf(-z));
  const uint32_t u = __float_as_uint(y);
  const uint32_t lo = u & 0xffffu;
  const bool near_tie = (lo > 0x8000u - 8u) && (lo < 0x8000u + 8u);
  const bool finite = (u & 0x7f800000u) != 0x7f800000u;
  redo = near_tie || !finite || __builtin_fabsf(z) >= 64.0f;
  return f32_to_bf16(y);
}
__device__ __forceinline__ uint16_t silu_bf16_exact(float z) { return f32_to_bf16(silu_f32(z)); }

// SiLU of 8 consecutive bf16 inputs (one 16-byte chunk) -> 8 bf16 outputs.
// Bit i of the returned mask is set when element i needs silu_bf16_exact.
__device__ __forceinline__ uint4 silu8_fast(const uint4& in, uint32_t& redo_mask) {
  float z[8];
  unpack8(in, z);
  uint32_t o[8];
  redo_mask = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    bool r;
    o[e] = silu_bf16_fast(z[e], r);
    redo_mask |= static_cast<uint32_t>(r) << e;
  }
  return make_uint4(o[0] | (o[1] << 16), o[2] | (o[3] << 16), o[4] | (o[5] << 16), o[6] | (o[7] << 16));
}

// Element access for the two storage types of the operator's tensors: bf16
// (bit patterns in uint16_t; stores round to nearest even) and fp32.
template <typename T>
struct Storage;
template <>
struct Storage<uint16_t> {
  __device__ __forceinline__ static float load1(uint16_t v) { return bf16_to_f32(v); }
  __device__ __forceinline__ static uint16_t store1(float v) { return f32_to_bf16(v); }
};
template <>
struct Storage<float> {
  __device__ __forceinline__ static float load1(float v) { return v; }
  __device__ __forceinline__ static float store1(float v) { return v; }
};

// One Neumaier step: t = s + x; c += exact rounding error of that add.
// The branch-free form picks the larger-magnitude operand for Fast2Sum, so
// c gets the same exact error term as the textbook |s| >= |x| branch.
__device__ __forceinline__ void neumaier_add(float& s, float& c, float x) {
  const float t = s + x;
  const bool big = __builtin_fabsf(s) >= __builtin_fabsf(x);
  const float hi = big ? s : x;
  const float lo = big ? x : s;
  c = c + ((hi - t) + lo);
  s = t;
}

}  // namespace adaln
