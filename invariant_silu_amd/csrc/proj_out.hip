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
//   latent: two chains per output, k in [0, 1536) and [1536, 3072), each 48
//           instructions of 32 (a lane's 8 operands: k = 64 s + 16 g + 8 h + e)
//           from +0, then added (first half + second half) and the bias added;
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
constexpr int kHalves = 2;             // forward: waves per output tile, each half of K
constexpr int kSteps = kD / 64 / kHalves;   // 24 steps of 64 k (two instructions each) per wave
constexpr int kAhead = 8;              // steps in flight
constexpr int kChunk = 512;            // tokens per dWp partial
constexpr int kRound = 64;             // tokens staged in LDS at a time
constexpr int kLdsStride = 72;         // bf16 elements per transposed LDS row (64 + pad; 144 bytes)
constexpr int kLdsStride2 = kLdsStride / 2;

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
// Block: kTT tiles of 16 tokens (t0 ..) x all 64 outputs, 8 waves: wave w owns
// outputs 16 (w % 4) .. + 15 over the K half w / 4 (k0 = 1536 (w / 4)).  Lane
// (r = lane % 16, g = lane / 16) feeds the A operand with out[t0 + 16 tt +
// r][k0 + 64 s + 16 g + 8 h .. + 7] and the B operand with Wp[16 (w % 4) +
// r][same k] for the two instructions h = 0, 1 of step s; eight steps of
// loads are in flight (one wave per SIMD at T = 4096 hides the memory latency
// only with many).  The second half's waves pass their sums through LDS.
// Rows past T load row T - 1 and are never stored.
template <int kTT>
struct FwdStep {
  uint4 w[2];
  uint4 a[kTT][2];
};

template <int kTT>
__global__ __launch_bounds__(512) void proj_out_fwd_kernel(const uint16_t* __restrict__ out,
                                                           const uint16_t* __restrict__ W,
                                                           const uint16_t* __restrict__ bias,
                                                           uint16_t* __restrict__ latent, int64_t T) {
  __shared__ f32x4_t half1[4][kTT][64];
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int ot = wave % 4, kh = wave / 4;
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * 16 * kTT;
  const int k0 = kh * (kD / kHalves);
  const uint16_t* wrow = W + static_cast<int64_t>(16 * ot + r) * kD + k0 + 16 * g;
  const uint16_t* arow[kTT];
#pragma unroll
  for (int tt = 0; tt < kTT; ++tt) {
    const int64_t t = t0 + 16 * tt + r;
    arow[tt] = out + (t < T ? t : T - 1) * kD + k0 + 16 * g;
  }
  FwdStep<kTT> buf[kAhead + 1];
  auto load = [&](FwdStep<kTT>& d, int s) {
#pragma unroll
    for (int h = 0; h < 2; ++h) d.w[h] = ld16(wrow + 64 * s + 8 * h);
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt)
#pragma unroll
      for (int h = 0; h < 2; ++h) d.a[tt][h] = ld16(arow[tt] + 64 * s + 8 * h);
  };
#pragma unroll
  for (int s = 0; s < kAhead; ++s) load(buf[s], s);
  f32x4_t acc[kTT];
#pragma unroll
  for (int tt = 0; tt < kTT; ++tt) acc[tt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    if (s + kAhead < kSteps) load(buf[(s + kAhead) % (kAhead + 1)], s + kAhead);
    // keeps the loads above issued here: the scheduler would otherwise sink
    // them next to their use and leave only a few steps in flight
    __builtin_amdgcn_sched_barrier(0);
    const FwdStep<kTT>& cur = buf[s % (kAhead + 1)];
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt) {
      acc[tt] = mfma_bf16(cur.a[tt][0], cur.w[0], acc[tt]);
      acc[tt] = mfma_bf16(cur.a[tt][1], cur.w[1], acc[tt]);
    }
  }
  if (kh == 1)
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt) half1[ot][tt][lane] = acc[tt];
  __syncthreads();
  if (kh == 1) return;
  // lane holds tokens t0 + 16 tt + 4 g + v, output 16 ot + r
  const float bf = bf16_to_f32(bias[16 * ot + r]);
#pragma unroll
  for (int tt = 0; tt < kTT; ++tt) {
    const f32x4_t h1 = half1[ot][tt][lane];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t t = t0 + 16 * tt + 4 * g + v;
      if (t < T) latent[t * kO + 16 * ot + r] = f32_to_bf16((acc[tt][v] + h1[v]) + bf);
    }
  }
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

__global__ __launch_bounds__(256) void proj_out_dx_kernel(const uint16_t* __restrict__ d_lat,
                                                          const uint16_t* __restrict__ W,
                                                          uint16_t* __restrict__ d_out, int64_t T) {
  __shared__ __align__(16) uint32_t wt[kDxCols * kLdsStride2];   // 36 KB
  const int k0 = static_cast<int>(blockIdx.y) * kDxCols;
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
  const int64_t tw = static_cast<int64_t>(blockIdx.x) * 64 + 16 * wave;
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
      *reinterpret_cast<uint4*>(orow + 32 * m) = v;
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
__global__ __launch_bounds__(256) void proj_out_dw_kernel(const uint16_t* __restrict__ d_lat,
                                                          const uint16_t* __restrict__ out,
                                                          float* __restrict__ part, double* __restrict__ part_db,
                                                          int64_t T) {
  __shared__ __align__(16) uint32_t xs[64 * kLdsStride2];   // [k][token]
  __shared__ __align__(16) uint32_t ds[64 * kLdsStride2];   // [o][token]
  const int k0 = static_cast<int>(blockIdx.x) * 64;
  const int64_t c = blockIdx.y;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int p = threadIdx.x % 32, c8 = threadIdx.x / 32;   // staging: token pair p, octet c8
  f32x4_t acc[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) acc[n] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  double sdb = 0.0;
  // the round's four rows: out and d_lat of tokens tb, tb + 1 (zeros past T);
  // the next round's are loaded while this one is added
  uint4 x0, x1, d0, d1;
  auto load = [&](int rd) {
    const int64_t tb = c * kChunk + rd * kRound + 2 * p;
    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
    x0 = tb < T ? ld16(out + tb * kD + k0 + 8 * c8) : z;
    x1 = tb + 1 < T ? ld16(out + (tb + 1) * kD + k0 + 8 * c8) : z;
    d0 = tb < T ? ld16(d_lat + tb * kO + 8 * c8) : z;
    d1 = tb + 1 < T ? ld16(d_lat + (tb + 1) * kO + 8 * c8) : z;
  };
  load(0);
  for (int rd = 0; rd < kChunk / kRound; ++rd) {
    uint32_t ox[8], od[8];
    interleave8(x0, x1, ox);
    interleave8(d0, d1, od);
    if (rd + 1 < kChunk / kRound) load(rd + 1);
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
    if (blockIdx.x == 0 && wave == 0) {
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
  if (blockIdx.x == 0 && wave == 0) part_db[c * kO + lane] = sdb;
}

// dWp and dbp: the chunks' partials added in ascending order in fp64
__global__ __launch_bounds__(256) void proj_out_dw_combine_kernel(const float* __restrict__ part,
                                                                  const double* __restrict__ part_db,
                                                                  uint16_t* __restrict__ dW, uint16_t* __restrict__ db,
                                                                  int64_t chunks) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;   // < 64 * 3072 by the grid
  double s = 0.0;
  for (int64_t c = 0; c < chunks; ++c) s += static_cast<double>(part[c * kO * kD + i]);
  dW[i] = f32_to_bf16(static_cast<float>(s));
  if (blockIdx.x == 0 && threadIdx.x < kO) {
    double t = 0.0;
    for (int64_t c = 0; c < chunks; ++c) t += part_db[c * kO + threadIdx.x];
    db[threadIdx.x] = f32_to_bf16(static_cast<float>(t));
  }
}

}  // namespace

int64_t proj_out_chunks(int64_t T) { return (T + kChunk - 1) / kChunk; }

hipError_t launch_proj_out_fwd(const uint16_t* out, const uint16_t* W, const uint16_t* bias, uint16_t* latent,
                               int64_t T, hipStream_t s) {
  const int64_t blocks = (T + 15) / 16;
  hipLaunchKernelGGL(proj_out_fwd_kernel<1>, dim3(static_cast<unsigned>(blocks)), dim3(512), 0, s, out, W, bias,
                     latent, T);
  return hipGetLastError();
}

hipError_t launch_proj_out_bwd(const uint16_t* d_lat, const uint16_t* out, const uint16_t* W, uint16_t* d_out,
                               uint16_t* dW, uint16_t* db, float* part, double* part_db, int64_t T, hipStream_t s,
                               hipEvent_t e0, hipEvent_t e1) {
  const int64_t chunks = proj_out_chunks(T);
  const dim3 gdx(static_cast<unsigned>((T + 63) / 64), kD / kDxCols);
  if (e0 && e1)
    hipExtLaunchKernelGGL(proj_out_dx_kernel, gdx, dim3(256), 0, s, e0, e1, 0, d_lat, W, d_out, T);
  else
    hipLaunchKernelGGL(proj_out_dx_kernel, gdx, dim3(256), 0, s, d_lat, W, d_out, T);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  hipLaunchKernelGGL(proj_out_dw_kernel, dim3(kD / 64, static_cast<unsigned>(chunks)), dim3(256), 0, s, d_lat, out,
                     part, part_db, T);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  hipLaunchKernelGGL(proj_out_dw_combine_kernel, dim3(kO * kD / 256), dim3(256), 0, s, part, part_db, dW, db,
                     chunks);
  return hipGetLastError();
}

}  // namespace adaln
