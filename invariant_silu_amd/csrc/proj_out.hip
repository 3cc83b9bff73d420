// The output projection after the final modulation, proj_out: 3072 -> 64 per
// token (RL-Kernel pull request 538, "What" and "Scope / Known limitations":
// the step after the operator, run by its own GEMM; miles_diffusion pull
// request 108, "Fused-norm rounding points": the bf16 rounding of the
// modulated output is this matmul's input), forward and backward:
//   latent[t, o] = bf16(fl32(sum_k out[t, k] Wp[o, k]) + bp[o])
//   d_out[t, k]  = bf16(sum_o d_lat[t, o] Wp[o, k])
//   dWp[o, k]    = bf16(sum_t d_lat[t, o] out[t, k]),  dbp[o] = bf16(sum_t d_lat[t, o])
//
// A dense contraction with bf16 operands: every product runs on the bf16
// matrix cores (v_mfma_f32_16x16x32_bf16: products exact, fp32 accumulation
// inside the instruction, fp32 accumulator).  A token's results come from the
// same instruction sequence wherever the token sits in a tile (the unit gives
// every output position the same arithmetic), so per-token outputs do not
// depend on the batch.  Sums:
//   latent: four chains per output, one per quarter of K, each 24
//           instructions of 32 consecutive k from +0; then ((q0 + q1) +
//           (q2 + q3)) + bias in fp32 (a second launch) and one bf16 rounding;
//   d_out:  one chain per output over o in 2 instructions of 32;
//   dWp:    per fixed chunk of 512 tokens a chain over 16 instructions of 32
//           tokens, from +0; the chunks added in fp64 in ascending order
//           (a second launch), then rounded to fp32 and to bf16; dbp the
//           same with fp64 sums of the chunk's tokens.  Trailing tokens whose
//           d_lat is zero add exact zeros.
#include <hip/hip_ext.h>

#include "common.hpp"
#include "launch.hpp"

namespace adaln {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_bf16(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

constexpr int kO = 64;                 // latent channels
constexpr int kChunk = 512;            // tokens per dWp partial
constexpr int kRound = 64;             // tokens staged in LDS at a time
constexpr int kLdsStride = 72;         // bf16 elements per transposed LDS row (64 + pad; 144 bytes)
constexpr int kLdsStride2 = kLdsStride / 2;

// the last valid row for t >= T (T >= 1)
__device__ __forceinline__ int64_t clamp_row(int64_t t, int64_t T) { return t < T ? t : T - 1; }

__device__ __forceinline__ uint32_t lo16(uint32_t w) { return w & 0xffffu; }
__device__ __forceinline__ uint32_t hi16(uint32_t w) { return w >> 16; }

// two rows' 8 consecutive elements -> 8 dwords (element e of row 0 | of row 1 << 16)
__device__ __forceinline__ void interleave8(const uint4& r0, const uint4& r1, uint32_t (&o)[8]) {
  const uint32_t a[4] = {r0.x, r0.y, r0.z, r0.w}, b[4] = {r1.x, r1.y, r1.z, r1.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = lo16(a[i]) | (lo16(b[i]) << 16);
    o[2 * i + 1] = hi16(a[i]) | (hi16(b[i]) << 16);
  }
}

// ---- forward ---------------------------------------------------------------
// Partials: block = 64 tokens (t0 ..) x one quarter of K (kq: k in [768 kq,
// 768 kq + 768)), 4 waves; wave w owns outputs 16 w .. + 15 and holds its B
// operand, Wp[16 w + r][768 kq + 32 s + 8 g .. + 7] for the 24 steps s, in
// registers.  The block stages its 64 x 768 slice of out in LDS once (rows
// padded to 1552 bytes: 16 lanes reading 16 rows hit distinct banks); token
// tile tt's A operand is out[t0 + 16 tt + r][same k].  Each partial is one
// chain of 24 instructions from +0.  Tokens past T are staged as zeros and
// never stored.  The quarters' partials go to part[kq][t][o].
constexpr int kQuarters = 4;
constexpr int kQK = kD / kQuarters;            // 768
constexpr int kQSteps = kQK / 32;              // 24
constexpr int kFwdTokens = 64;
constexpr int kARow32 = (kQK * 2 + 16) / 4;    // 388 dwords per staged row

// Zero the staged rows of tokens t >= T (the last block only), after the
// block's own writes of those rows.
template <int kRows>
__device__ __forceinline__ void zero_tail_rows(uint32_t* as, int64_t t0, int64_t T) {
  if (t0 + kRows <= T) return;
  constexpr int kChunksPerRow = kQK / 8;
  for (int q = threadIdx.x; q < kRows * kChunksPerRow; q += 256) {   // the staging loops' thread mapping
    const int row = q / kChunksPerRow;
    if (t0 + row >= T)
      *reinterpret_cast<uint4*>(as + row * kARow32 + 4 * (q % kChunksPerRow)) = make_uint4(0u, 0u, 0u, 0u);
  }
}

__global__ __launch_bounds__(256) void proj_out_fwd_part_kernel(const uint16_t* __restrict__ out,
                                                                const uint16_t* __restrict__ W,
                                                                float* __restrict__ part, int64_t T) {
  __shared__ __align__(16) uint32_t as[kFwdTokens * kARow32];   // 97 KB
  const int kq = blockIdx.y;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kFwdTokens;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  // stage: 64 rows x 96 chunks of 16 bytes, consecutive threads on consecutive chunks
  const uint16_t* abase = out + kq * kQK;
  constexpr int kChunksPerRow = kQK / 8;   // 96
  constexpr int kIt = kFwdTokens * kChunksPerRow / 256;
  uint4 av[kIt];
#pragma unroll
  for (int it = 0; it < kIt; ++it) {
    const int q = threadIdx.x + 256 * it;
    const int row = q / kChunksPerRow, c = q % kChunksPerRow;
    // rows past T load row T - 1 (in bounds) and are zeroed after the LDS
    // writes: a load under a branch, or a select on its value (which the
    // compiler turns into one), makes it wait for every load issued before
    av[it] = ld16(abase + clamp_row(t0 + row, T) * kD + 8 * c);
  }
  // all 24 loads stay in flight before the first LDS write (one block per CU:
  // the slice's bytes in flight are what keeps HBM busy)
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int it = 0; it < kIt; ++it) {
    const int q = threadIdx.x + 256 * it;
    const int row = q / kChunksPerRow, c = q % kChunksPerRow;
    *reinterpret_cast<uint4*>(as + row * kARow32 + 4 * c) = av[it];
  }
  zero_tail_rows<kFwdTokens>(as, t0, T);
  uint4 wv[kQSteps];
  const uint16_t* wrow = W + static_cast<int64_t>(16 * wave + r) * kD + kq * kQK + 8 * g;
#pragma unroll
  for (int st = 0; st < kQSteps; ++st) wv[st] = ld16(wrow + 32 * st);
  __syncthreads();
  f32x4_t acc[kFwdTokens / 16];
#pragma unroll
  for (int tt = 0; tt < kFwdTokens / 16; ++tt) {
    acc[tt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    const uint32_t* arow = as + (16 * tt + r) * kARow32 + 4 * g;
#pragma unroll
    for (int st = 0; st < kQSteps; ++st)
      acc[tt] = mfma_bf16(*reinterpret_cast<const uint4*>(arow + 16 * st), wv[st], acc[tt]);
  }
  // lane holds tokens t0 + 16 tt + 4 g + v, output 16 w + r
  float* pq = part + static_cast<int64_t>(kq) * T * kO;
#pragma unroll
  for (int tt = 0; tt < kFwdTokens / 16; ++tt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t t = t0 + 16 * tt + 4 * g + v;
      if (t < T) pq[t * kO + 16 * wave + r] = acc[tt][v];
    }
}

// The same partials with the final modulation computed on the fly: the
// block's slice of out, out[t][k] = bf16(((x - mean) * rstd) * bf16(1 + scale)
// + shift) with t's sample's (scale | shift) from emb -- the final
// modulation's expression, operation for operation -- goes straight into
// LDS, so out never reaches HBM.  32 tokens per block.
// kOneSample (S a multiple of 32: a block's tokens share one sample): the
// sample's slice of scale and shift is staged once in LDS, which frees the
// registers to issue Wp's quarter (from L2) ahead of x, so it has arrived by
// the time the chains start.  Otherwise each row looks its sample up.
constexpr int kFuseTokens = 32;

template <bool kOneSample>
__global__ __launch_bounds__(256) void proj_out_fused_part_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ emb, const float* __restrict__ mean,
    const float* __restrict__ rstd, const uint16_t* __restrict__ W, float* __restrict__ part, int64_t T,
    int64_t S) {
  __shared__ __align__(16) uint32_t as[kFuseTokens * kARow32];   // 48.5 KB
  const int kq = blockIdx.y;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kFuseTokens;
  constexpr int kChunksPerRow = kQK / 8;                          // 96
  constexpr int kIt = kFuseTokens * kChunksPerRow / 256;          // 12
  const int kbase = kq * kQK;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const uint16_t* wrow = W + static_cast<int64_t>(16 * wave + r) * kD + kbase + 8 * g;
  uint4 wv[kQSteps];
  uint4 xv[kIt];
  float mu[kIt], rs[kIt];
  if constexpr (kOneSample) {
    // the sample's bf16(1 + scale) and shift slices as fp32, 8 columns per
    // 16-byte chunk pair: threads [0, 128) take chunk tid of scale, threads
    // [128, 256) chunk tid - 128 of shift; chunks past 95 reload chunk 95 into
    // spare entries (every thread loads and stores: no branch around a load)
    __shared__ float4 m_lds[2 * 2 * 128];
    const int64_t b = static_cast<uint32_t>(t0) / static_cast<uint32_t>(S);
    const int half = threadIdx.x >> 7, ec = threadIdx.x & 127;
    const uint4 ev = ld16(emb + b * kN + half * kD + kbase + 8 * min(ec, kChunksPerRow - 1));
#pragma unroll
    for (int st = 0; st < kQSteps; ++st) wv[st] = ld16(wrow + 32 * st);
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int q = threadIdx.x + 256 * it;
      const int64_t t = clamp_row(t0 + q / kChunksPerRow, T);
      xv[it] = ld16(x + t * kD + kbase + 8 * (q % kChunksPerRow));
      mu[it] = mean[t];
      rs[it] = rstd[t];
    }
    __builtin_amdgcn_sched_barrier(0);
    {
      float f[8];
      unpack8(ev, f);
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = half ? f[e] : round_bf16(1.0f + f[e]);
      m_lds[2 * threadIdx.x] = make_float4(f[0], f[1], f[2], f[3]);
      m_lds[2 * threadIdx.x + 1] = make_float4(f[4], f[5], f[6], f[7]);
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int q = threadIdx.x + 256 * it;
      const int row = q / kChunksPerRow, c = q % kChunksPerRow;
      float xf[8], o[8];
      unpack8(xv[it], xf);
      const float4 m0 = m_lds[2 * c], m1 = m_lds[2 * c + 1];
      const float4 h0 = m_lds[256 + 2 * c], h1 = m_lds[256 + 2 * c + 1];
      const float mm[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
      const float hh[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float n = (xf[e] - mu[it]) * rs[it];
        o[e] = n * mm[e] + hh[e];
      }
      *reinterpret_cast<uint4*>(as + row * kARow32 + 4 * c) = pack8(o);
    }
    zero_tail_rows<kFuseTokens>(as, t0, T);
  } else {
    uint4 sc[kIt], sh[kIt];
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int q = threadIdx.x + 256 * it;
      const int row = q / kChunksPerRow, c = q % kChunksPerRow;
      const int64_t t = clamp_row(t0 + row, T);
      // token index and sample fit 32 bits (T <= 65535 * 512)
      const int64_t b = static_cast<uint32_t>(t) / static_cast<uint32_t>(S);
      xv[it] = ld16(x + t * kD + kbase + 8 * c);
      sc[it] = ld16(emb + b * kN + kbase + 8 * c);
      sh[it] = ld16(emb + b * kN + kD + kbase + 8 * c);
      mu[it] = mean[t];
      rs[it] = rstd[t];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int q = threadIdx.x + 256 * it;
      const int row = q / kChunksPerRow, c = q % kChunksPerRow;
      float xf[8], sf[8], hf[8], o[8];
      unpack8(xv[it], xf);
      unpack8(sc[it], sf);
      unpack8(sh[it], hf);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float n = (xf[e] - mu[it]) * rs[it];
        o[e] = n * round_bf16(1.0f + sf[e]) + hf[e];
      }
      *reinterpret_cast<uint4*>(as + row * kARow32 + 4 * c) = pack8(o);
    }
    zero_tail_rows<kFuseTokens>(as, t0, T);
#pragma unroll
    for (int st = 0; st < kQSteps; ++st) wv[st] = ld16(wrow + 32 * st);
  }
  __syncthreads();
  f32x4_t acc[kFuseTokens / 16];
#pragma unroll
  for (int tt = 0; tt < kFuseTokens / 16; ++tt) {
    acc[tt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    const uint32_t* arow = as + (16 * tt + r) * kARow32 + 4 * g;
#pragma unroll
    for (int st = 0; st < kQSteps; ++st)
      acc[tt] = mfma_bf16(*reinterpret_cast<const uint4*>(arow + 16 * st), wv[st], acc[tt]);
  }
  float* pq = part + static_cast<int64_t>(kq) * T * kO;
#pragma unroll
  for (int tt = 0; tt < kFuseTokens / 16; ++tt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t t = t0 + 16 * tt + 4 * g + v;
      if (t < T) pq[t * kO + 16 * wave + r] = acc[tt][v];
    }
}

// latent = bf16(((q0 + q1) + (q2 + q3)) + bias) per element, in fp32
__global__ __launch_bounds__(256) void proj_out_fwd_combine_kernel(const float* __restrict__ part,
                                                                   const uint16_t* __restrict__ bias,
                                                                   uint16_t* __restrict__ latent, int64_t T) {
  // 4 consecutive outputs of one token per thread (64 outputs per token)
  const int64_t n = T * kO;
  const int64_t i = 4 * (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x);
  if (i >= n) return;
  const float4 q0 = *reinterpret_cast<const float4*>(part + i);
  const float4 q1 = *reinterpret_cast<const float4*>(part + n + i);
  const float4 q2 = *reinterpret_cast<const float4*>(part + 2 * n + i);
  const float4 q3 = *reinterpret_cast<const float4*>(part + 3 * n + i);
  const uint2 bw = *reinterpret_cast<const uint2*>(bias + i % kO);
  const float l0 = ((q0.x + q1.x) + (q2.x + q3.x)) + bf_lo(bw.x);
  const float l1 = ((q0.y + q1.y) + (q2.y + q3.y)) + bf_hi(bw.x);
  const float l2 = ((q0.z + q1.z) + (q2.z + q3.z)) + bf_lo(bw.y);
  const float l3 = ((q0.w + q1.w) + (q2.w + q3.w)) + bf_hi(bw.y);
  *reinterpret_cast<uint2*>(latent + i) = make_uint2(pack_bf16x2(l0, l1), pack_bf16x2(l2, l3));
}

// ---- backward: d_out ---------------------------------------------------------
// Block: 64 tokens (wave w: tokens t0 + 16 w ..) x 256 columns (k0 ..).  Wp's
// 64 x 256 slab is staged in LDS transposed (row k holds the 64 outputs'
// weights).  Output tiles come in pairs (m, h = 0, 1) over 32 columns: tile
// row i = 4 q + v is column 32 m + 8 q + 4 h + v, so A = the slab's rows for
// those columns (outputs 8 g .. + 7, then 32 + 8 g ..), B = d_lat[t][8 g ..]
// (the same outputs), and a lane holds 8 consecutive columns of one token
// after the pair: one 16-byte store.
constexpr int kDxCols = 256;

// d_out for 64 tokens (token block bx) x 256 columns (column block by)
__device__ __forceinline__ void dx_block(const uint16_t* __restrict__ d_lat, const uint16_t* __restrict__ W,
                                         uint16_t* __restrict__ d_out, int64_t T, int64_t bx, int by,
                                         uint32_t* wt) {
  const int k0 = by * kDxCols;
  // stage: row pair p (outputs 2p, 2p + 1) x column octet c8: 32 x 32 items
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int item = threadIdx.x + 256 * it;
    const int p = item % 32, c8 = item / 32;
    const uint4 r0 = ld16(W + static_cast<int64_t>(2 * p) * kD + k0 + 8 * c8);
    const uint4 r1 = ld16(W + static_cast<int64_t>(2 * p + 1) * kD + k0 + 8 * c8);
    uint32_t o[8];
    interleave8(r0, r1, o);
#pragma unroll
    for (int e = 0; e < 8; ++e) wt[(8 * c8 + e) * kLdsStride2 + p] = o[e];
  }
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int64_t tw = bx * 64 + 16 * wave;
  const int64_t tr = tw + r < T ? tw + r : T - 1;
  const uint4 b0 = ld16(d_lat + tr * kO + 8 * g);
  const uint4 b1 = ld16(d_lat + tr * kO + 32 + 8 * g);
  __syncthreads();
  const bool store = tw + r < T;
  uint16_t* orow = d_out + tr * kD + k0 + 8 * g;   // stored only when tw + r < T
#pragma unroll 2
  for (int m = 0; m < kDxCols / 32; ++m) {
    f32x4_t acc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // A row r of tile (m, h): column 32 m + 8 (r / 4) + 4 h + r % 4
      const uint32_t* wr = wt + (32 * m + 8 * (r / 4) + 4 * h + r % 4) * kLdsStride2;
      const uint4 a0 = *reinterpret_cast<const uint4*>(wr + 4 * g);
      const uint4 a1 = *reinterpret_cast<const uint4*>(wr + 16 + 4 * g);
      acc[h] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      acc[h] = mfma_bf16(a0, b0, acc[h]);
      acc[h] = mfma_bf16(a1, b1, acc[h]);
    }
    // lane holds columns k0 + 32 m + 8 g + 4 h + v of token tw + r
    if (store) {
      uint4 v;
      v.x = pack_bf16x2(acc[0][0], acc[0][1]);
      v.y = pack_bf16x2(acc[0][2], acc[0][3]);
      v.z = pack_bf16x2(acc[1][0], acc[1][1]);
      v.w = pack_bf16x2(acc[1][2], acc[1][3]);
      st16_nt(orow + 32 * m, v);
    }
  }
}

// ---- backward: dWp and dbp partials ------------------------------------------
// Block: 64 columns (k0 ..) x one chunk of 512 tokens, in 8 rounds of 64
// tokens staged in LDS transposed (out: row k holds the round's 64 tokens;
// d_lat: row o likewise); tokens past T are staged as zeros.  Wave w owns
// outputs 16 w .. (A = d_lat rows), 4 column tiles n (B = out rows k0 + 16 n +
// r); each instruction adds 32 tokens.  Blocks of column block 0 also sum
// d_lat per output (wave 0, fp64, tokens ascending).
// One block: 64 columns of out x one 512-token chunk.  A full chunk (all
// tokens < T) loads unconditionally, two rounds ahead of the one being
// added; the last, partial chunk takes the guarded loads (zeros past T).
template <bool kFull>
__device__ __forceinline__ void dw_chunk(const uint16_t* __restrict__ d_lat, const uint16_t* __restrict__ out,
                                         float* __restrict__ part, double* __restrict__ part_db, int64_t T,
                                         int bx, int64_t c, uint32_t* xs, uint32_t* ds) {
  constexpr int kRounds = kChunk / kRound;   // 8
  const int k0 = bx * 64;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int p = threadIdx.x % 32, c8 = threadIdx.x / 32;   // staging: token pair p, octet c8
  f32x4_t acc[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) acc[n] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  double sdb = 0.0;
  // a round's four rows per thread: out and d_lat of tokens tb, tb + 1
  uint4 buf[kRounds][4];
  auto load = [&](int rd) {
    const int64_t tb = c * kChunk + rd * kRound + 2 * p;
    if constexpr (kFull) {
      buf[rd][0] = ld16(out + tb * kD + k0 + 8 * c8);
      buf[rd][1] = ld16(out + (tb + 1) * kD + k0 + 8 * c8);
      buf[rd][2] = ld16(d_lat + tb * kO + 8 * c8);
      buf[rd][3] = ld16(d_lat + (tb + 1) * kO + 8 * c8);
    } else {
      const uint4 z = make_uint4(0u, 0u, 0u, 0u);
      buf[rd][0] = tb < T ? ld16(out + tb * kD + k0 + 8 * c8) : z;
      buf[rd][1] = tb + 1 < T ? ld16(out + (tb + 1) * kD + k0 + 8 * c8) : z;
      buf[rd][2] = tb < T ? ld16(d_lat + tb * kO + 8 * c8) : z;
      buf[rd][3] = tb + 1 < T ? ld16(d_lat + (tb + 1) * kO + 8 * c8) : z;
    }
  };
  load(0);
  load(1);
#pragma unroll
  for (int rd = 0; rd < kRounds; ++rd) {
    uint32_t ox[8], od[8];
    interleave8(buf[rd][0], buf[rd][1], ox);
    interleave8(buf[rd][2], buf[rd][3], od);
    if (rd + 2 < kRounds) load(rd + 2);
    __syncthreads();   // the previous round's reads are done
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      xs[(8 * c8 + e) * kLdsStride2 + p] = ox[e];
      ds[(8 * c8 + e) * kLdsStride2 + p] = od[e];
    }
    __syncthreads();
#pragma unroll
    for (int sub = 0; sub < kRound / 32; ++sub) {
      const uint4 a = *reinterpret_cast<const uint4*>(ds + (16 * wave + r) * kLdsStride2 + 16 * sub + 4 * g);
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const uint4 b = *reinterpret_cast<const uint4*>(xs + (16 * n + r) * kLdsStride2 + 16 * sub + 4 * g);
        acc[n] = mfma_bf16(a, b, acc[n]);
      }
    }
    if (bx == 0 && wave == 0) {
      const uint32_t* row = ds + lane * kLdsStride2;
      for (int q = 0; q < kRound / 2; ++q) {
        sdb += static_cast<double>(bf_lo(row[q]));
        sdb += static_cast<double>(bf_hi(row[q]));
      }
    }
  }
  // lane holds outputs 16 w + 4 g + v, columns k0 + 16 n + r
  float* pc = part + c * kO * kD;
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int v = 0; v < 4; ++v) pc[static_cast<int64_t>(16 * wave + 4 * g + v) * kD + k0 + 16 * n + r] = acc[n][v];
  if (bx == 0 && wave == 0) part_db[c * kO + lane] = sdb;
}

// The backward's two independent products in one launch: blocks [0, 48 C)
// take a 64-column x 512-token chunk of the dWp partial sums (chunk-major, so
// the longer blocks start first), the rest take 64 tokens x 256 columns of
// d_out.
constexpr int kDwColBlocks = kD / 64;   // 48

__global__ __launch_bounds__(256) void proj_out_bwd_kernel(const uint16_t* __restrict__ d_lat,
                                                           const uint16_t* __restrict__ out,
                                                           const uint16_t* __restrict__ W,
                                                           uint16_t* __restrict__ d_out, float* __restrict__ part,
                                                           double* __restrict__ part_db, int64_t T,
                                                           int64_t dw_blocks) {
  __shared__ __align__(16) uint32_t lds[kDxCols * kLdsStride2];   // 36 KB: dx's Wp slab, or dw's two tiles
  static_assert(2 * 64 * kLdsStride2 <= kDxCols * kLdsStride2, "dw tiles must fit the shared buffer");
  const int64_t blk = blockIdx.x;
  if (blk < dw_blocks) {
    const int bx = static_cast<int>(blk % kDwColBlocks);
    const int64_t c = blk / kDwColBlocks;
    if ((c + 1) * kChunk <= T)
      dw_chunk<true>(d_lat, out, part, part_db, T, bx, c, lds, lds + 64 * kLdsStride2);
    else
      dw_chunk<false>(d_lat, out, part, part_db, T, bx, c, lds, lds + 64 * kLdsStride2);
  } else {
    constexpr int kDxColBlocks = kD / kDxCols;
    const int64_t q = blk - dw_blocks;
    dx_block(d_lat, W, d_out, T, q / kDxColBlocks, static_cast<int>(q % kDxColBlocks), lds);
  }
}

// dWp and dbp: the chunks' partials added in ascending order in fp64
// 4 consecutive elements of dWp per thread; the chunks' partials are loaded
// 8 at a time (indices clamped to the last chunk, so every load is in
// bounds and none sits under a branch) and added in ascending chunk order
__global__ __launch_bounds__(256) void proj_out_dw_combine_kernel(const float* __restrict__ part,
                                                                  const double* __restrict__ part_db,
                                                                  uint16_t* __restrict__ dW, uint16_t* __restrict__ db,
                                                                  int64_t chunks) {
  const int64_t i = 4 * (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x);   // < 64 * 3072 by the grid
  double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
  for (int64_t c0 = 0; c0 < chunks; c0 += 8) {
    float4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t c = c0 + j < chunks ? c0 + j : chunks - 1;
      v[j] = *reinterpret_cast<const float4*>(part + c * kO * kD + i);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool in = c0 + j < chunks;
      s0 = in ? s0 + static_cast<double>(v[j].x) : s0;
      s1 = in ? s1 + static_cast<double>(v[j].y) : s1;
      s2 = in ? s2 + static_cast<double>(v[j].z) : s2;
      s3 = in ? s3 + static_cast<double>(v[j].w) : s3;
    }
  }
  const uint2 w = make_uint2(pack_bf16x2(static_cast<float>(s0), static_cast<float>(s1)),
                             pack_bf16x2(static_cast<float>(s2), static_cast<float>(s3)));
  *reinterpret_cast<uint2*>(dW + i) = w;
  if (blockIdx.x == 0 && threadIdx.x < kO) {
    double t = 0.0;
    for (int64_t c = 0; c < chunks; ++c) t += part_db[c * kO + threadIdx.x];
    db[threadIdx.x] = f32_to_bf16(static_cast<float>(t));
  }
}

}  // namespace

int64_t proj_out_chunks(int64_t T) { return (T + kChunk - 1) / kChunk; }

hipError_t launch_proj_out_fwd(const uint16_t* out, const uint16_t* W, const uint16_t* bias, uint16_t* latent,
                               float* part, int64_t T, hipStream_t s) {
  hipLaunchKernelGGL(proj_out_fwd_part_kernel, dim3(static_cast<unsigned>((T + kFwdTokens - 1) / kFwdTokens), kQuarters),
                     dim3(256), 0, s, out, W, part, T);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  hipLaunchKernelGGL(proj_out_fwd_combine_kernel, dim3(static_cast<unsigned>((T * kO / 4 + 255) / 256)), dim3(256), 0, s,
                     part, bias, latent, T);
  return hipGetLastError();
}

hipError_t launch_proj_out_fwd_fused(const uint16_t* x, const uint16_t* emb, const float* mean, const float* rstd,
                                     const uint16_t* W, const uint16_t* bias, uint16_t* latent, float* part,
                                     int64_t B, int64_t S, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const int64_t T = B * S;
  const dim3 grid(static_cast<unsigned>((T + kFuseTokens - 1) / kFuseTokens), kQuarters);
  // S a multiple of 32: every block's tokens belong to one sample
  auto k = S % kFuseTokens == 0 ? proj_out_fused_part_kernel<true> : proj_out_fused_part_kernel<false>;
  if (e0 && e1)
    hipExtLaunchKernelGGL(k, grid, dim3(256), 0, s, e0, e1, 0, x, emb, mean, rstd, W, part, T, S);
  else
    hipLaunchKernelGGL(k, grid, dim3(256), 0, s, x, emb, mean, rstd, W, part, T, S);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  hipLaunchKernelGGL(proj_out_fwd_combine_kernel, dim3(static_cast<unsigned>((T * kO / 4 + 255) / 256)), dim3(256), 0, s,
                     part, bias, latent, T);
  return hipGetLastError();
}

hipError_t launch_proj_out_bwd(const uint16_t* d_lat, const uint16_t* out, const uint16_t* W, uint16_t* d_out,
                               uint16_t* dW, uint16_t* db, float* part, double* part_db, int64_t T, hipStream_t s,
                               hipEvent_t e0, hipEvent_t e1) {
  const int64_t chunks = proj_out_chunks(T);
  const int64_t dw_blocks = kDwColBlocks * chunks;
  const int64_t dx_blocks = (T + 63) / 64 * (kD / kDxCols);
  const dim3 grid(static_cast<unsigned>(dw_blocks + dx_blocks));
  if (e0 && e1)
    hipExtLaunchKernelGGL(proj_out_bwd_kernel, grid, dim3(256), 0, s, e0, e1, 0, d_lat, out, W, d_out, part, part_db,
                          T, dw_blocks);
  else
    hipLaunchKernelGGL(proj_out_bwd_kernel, grid, dim3(256), 0, s, d_lat, out, W, d_out, part, part_db, T, dw_blocks);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  hipLaunchKernelGGL(proj_out_dw_combine_kernel, dim3(kO * kD / 4 / 256), dim3(256), 0, s, part, part_db, dW, db,
                     chunks);
  return hipGetLastError();
}

}  // namespace adaln
