// The output projection after the final modulation, proj_out: 3072 -> 64 per
// token (RL-Kernel pull request 538, "What" and "Scope / Known limitations":
// the step after the operator, run by its own GEMM; miles_diffusion pull
// request 108, "Fused-norm rounding points": the bf16 rounding of the
// modulated output is this matmul's input), forward and backward:
//   latent[t, o] = bf16(fl32(sum_k out[t, k] Wp[o, k]) + bp[o])
//   d_out[t, k]  = bf16(sum_o d_lat[t, o] Wp[o, k])
//   dWp[o, k]    = bf16(sum_t d_lat[t, o] out[t, k]),  dbp[o] = bf16(sum_t d_lat[t, o])
//
// A dense contraction, so it runs on the matrix cores -- the fp64 ones
// (v_mfma_f64_16x16x4f64, a chain of fused multiply-adds): every product of
// two bf16 numbers is exact in fp64 and the sums accumulate in fp64 in fixed
// orders, so each result, rounded once to fp32 (then to bf16), is the
// correctly rounded sum unless the sum sits within about 2^-40 of its size
// from a rounding boundary.  The bf16 matrix cores were the first design
// here; their fp32 accumulation inside the instruction left cancelling sums
// several bf16 ulps from the correctly rounded result.
//
// Orders (the same for a token wherever it sits, so per-token results do not
// depend on T):
//   latent: eight parts of K (384 consecutive k each), one chain per part,
//           step s of part p taking k = 384 p + 32 (s / 8) + 8 g + s % 8 for
//           slots g = 0 .. 3 in order; the parts added as ((p0 + p1) +
//           (p2 + p3)) + ((p4 + p5) + (p6 + p7)) in fp64, rounded to fp32,
//           bias added in fp32, one bf16 rounding;
//   d_out:  one chain per output over o, step s taking o = 16 g + s;
//   dWp:    per fixed chunk of 512 tokens one chain over the chunk's tokens
//           in ascending order (4 per step), from +0; the chunks added in
//           fp64 in ascending order (a second launch), then rounded to fp32
//           and to bf16; dbp the same with fp64 sums of the chunk's tokens.
//           Trailing tokens whose d_lat is zero add exact zeros.
#include "common.hpp"
#include "launch.hpp"
#include "mfma.hpp"

namespace adaln {

namespace {

constexpr int kO = 64;                 // latent channels
constexpr int kChunk = 512;            // tokens per dWp partial

// the last valid row for t >= T (T >= 1)
__device__ __forceinline__ int64_t clamp_row(int64_t t, int64_t T) { return t < T ? t : T - 1; }

// element e (0 .. 7) of 8 consecutive bf16 in a 16-byte word, widened to fp64
__device__ __forceinline__ double el8(const uint4& v, int e) {
  const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
  return bf_half64(w, e & 1);
}

// ---- forward ---------------------------------------------------------------
// Block: 16 tokens (t0 ..) x all 64 outputs, 8 waves; wave p runs part p of K
// for the four 16-output tiles.  Lane (r, g) takes A = out[t0 + r][k] and B =
// Wp[16 j + r][k] (Wp is 384 KB: it stays in L2), 16 bytes per 8 steps each,
// one group of 8 steps ahead: from memory in proj_out_fwd_kernel (no staging,
// so two blocks share a CU), from the rows the block computed into LDS in
// proj_out_fused_kernel (rows padded by 16 bytes).  The parts then meet in
// LDS.  Tokens past T use row T - 1 and are never stored.
constexpr int kFT = 16;                      // tokens per block
constexpr int kParts = 8;                    // parts of K, one per wave
constexpr int kPK = kD / kParts;             // 384
constexpr int kPGroups = kPK / 32;           // 12 groups of 8 steps
constexpr int kARowDw = kD / 2 + 4;          // LDS dwords per staged row (1540)
constexpr int kFwdThreads = 64 * kParts;     // 512
constexpr size_t kFwdLds = sizeof(uint32_t) * kFT * kARowDw;   // 98.6 KB
static_assert(sizeof(double) * kParts * kFT * kO <= kFwdLds, "the parts' results reuse the staged rows");

// The chains of part p over the staged rows; acc[j] = output tile j.
__device__ __forceinline__ void fwd_chains(const uint32_t* __restrict__ a_lds, const uint16_t* __restrict__ W,
                                           int p, f64x4_t (&acc)[4]) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const uint16_t* wrow = W + static_cast<int64_t>(r) * kD + kPK * p + 8 * g;
  const uint32_t* arow = a_lds + r * kARowDw + (kPK * p + 8 * g) / 2;
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f64x4_t{0.0, 0.0, 0.0, 0.0};
  uint4 wb[2][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) wb[0][j] = ld16(wrow + static_cast<int64_t>(16 * j) * kD);
#pragma unroll
  for (int q = 0; q < kPGroups; ++q) {
    if (q + 1 < kPGroups) {
#pragma unroll
      for (int j = 0; j < 4; ++j) wb[(q + 1) & 1][j] = ld16(wrow + static_cast<int64_t>(16 * j) * kD + 32 * (q + 1));
    }
    const uint4 av = *reinterpret_cast<const uint4*>(arow + 16 * q);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double a = el8(av, e);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = mfma_f64(a, el8(wb[q & 1][j], e), acc[j]);
    }
  }
}

// The parts' results into LDS (the staged rows are dead by then), then
// latent for the block's tokens: 2 consecutive outputs per thread.
__device__ __forceinline__ void fwd_combine(uint32_t* lds, const f64x4_t (&acc)[4], const uint16_t* __restrict__ bias,
                                            uint16_t* __restrict__ latent, int64_t t0, int64_t T) {
  const int p = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  double* cmb = reinterpret_cast<double*>(lds);   // [part][token][output]
  __syncthreads();   // every wave is done reading the staged rows
  // lane holds token g + 4 v, output 16 j + r of tile j
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) cmb[(p * kFT + g + 4 * v) * kO + 16 * j + r] = acc[j][v];
  __syncthreads();
  const int i = threadIdx.x >> 5, o = 2 * (threadIdx.x & 31);   // token i, outputs o, o + 1
  float res[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    double c[kParts];
#pragma unroll
    for (int q = 0; q < kParts; ++q) c[q] = cmb[(q * kFT + i) * kO + o + h];
    const double s = ((c[0] + c[1]) + (c[2] + c[3])) + ((c[4] + c[5]) + (c[6] + c[7]));
    res[h] = static_cast<float>(s) + bf16_to_f32(bias[o + h]);
  }
  if (t0 + i < T) *reinterpret_cast<uint32_t*>(latent + (t0 + i) * kO + o) = pack_bf16x2(res[0], res[1]);
}

// The same chains with A from memory: lane (r, g) reads out[t0 + r][384 p +
// 32 q + 8 g ..] (16 bytes per 8 steps, one group ahead), as it reads Wp.
__device__ __forceinline__ void fwd_chains_direct(const uint16_t* __restrict__ out, const uint16_t* __restrict__ W,
                                                  int64_t t0, int64_t T, int p, f64x4_t (&acc)[4]) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const uint16_t* wrow = W + static_cast<int64_t>(r) * kD + kPK * p + 8 * g;
  const uint16_t* arow = out + clamp_row(t0 + r, T) * kD + kPK * p + 8 * g;
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f64x4_t{0.0, 0.0, 0.0, 0.0};
  uint4 wb[2][4], ab[2];
#pragma unroll
  for (int j = 0; j < 4; ++j) wb[0][j] = ld16(wrow + static_cast<int64_t>(16 * j) * kD);
  ab[0] = ld16(arow);
#pragma unroll
  for (int q = 0; q < kPGroups; ++q) {
    if (q + 1 < kPGroups) {
#pragma unroll
      for (int j = 0; j < 4; ++j) wb[(q + 1) & 1][j] = ld16(wrow + static_cast<int64_t>(16 * j) * kD + 32 * (q + 1));
      ab[(q + 1) & 1] = ld16(arow + 32 * (q + 1));
    }
    const uint4 av = ab[q & 1];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double a = el8(av, e);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = mfma_f64(a, el8(wb[q & 1][j], e), acc[j]);
    }
  }
}

constexpr size_t kCmbLds = sizeof(double) * kParts * kFT * kO;   // 64 KB

__global__ __launch_bounds__(kFwdThreads) void proj_out_fwd_kernel(const uint16_t* __restrict__ out,
                                                                  const uint16_t* __restrict__ W,
                                                                  const uint16_t* __restrict__ bias,
                                                                  uint16_t* __restrict__ latent, int64_t T) {
  __shared__ __align__(16) uint32_t lds[kCmbLds / 4];
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kFT;
  f64x4_t acc[4];
  fwd_chains_direct(out, W, t0, T, threadIdx.x >> 6, acc);
  fwd_combine(lds, acc, bias, latent, t0, T);
}

// The same with the final modulation computed on the fly: the block's rows
// of out, out[t][k] = bf16(((x - mean) * rstd) * bf16(1 + scale) + shift)
// with t's sample's (scale | shift) from emb -- the final modulation's
// expression, operation for operation -- go straight into LDS, so out never
// reaches HBM.
__global__ __launch_bounds__(kFwdThreads) void proj_out_fused_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ emb, const float* __restrict__ mean,
    const float* __restrict__ rstd, const uint16_t* __restrict__ W, const uint16_t* __restrict__ bias,
    uint16_t* __restrict__ latent, int64_t T, int64_t S) {
  __shared__ __align__(16) uint32_t lds[kFwdLds / 4];
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kFT;
  constexpr int kChunksPerRow = kD / 8;
  constexpr int kIt = kFT * kChunksPerRow / kFwdThreads;
#pragma unroll 4
  for (int it = 0; it < kIt; ++it) {
    const int q = threadIdx.x + kFwdThreads * it;
    const int row = q / kChunksPerRow, c = q % kChunksPerRow;
    const int64_t t = clamp_row(t0 + row, T);
    // token index and sample fit 32 bits (T <= 65535 * 512)
    const int64_t b = static_cast<uint32_t>(t) / static_cast<uint32_t>(S);
    const uint4 xv = ld16(x + t * kD + 8 * c);
    const uint4 sc = ld16(emb + b * kN + 8 * c);
    const uint4 sh = ld16(emb + b * kN + kD + 8 * c);
    const float mu = mean[t], rs = rstd[t];
    float xf[8], sf[8], hf[8], o[8];
    unpack8(xv, xf);
    unpack8(sc, sf);
    unpack8(sh, hf);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float n = (xf[e] - mu) * rs;
      o[e] = n * round_bf16(1.0f + sf[e]) + hf[e];
    }
    *reinterpret_cast<uint4*>(lds + row * kARowDw + 4 * c) = pack8(o);
  }
  __syncthreads();
  f64x4_t acc[4];
  fwd_chains(lds, W, threadIdx.x >> 6, acc);
  fwd_combine(lds, acc, bias, latent, t0, T);
}

// ---- backward ------------------------------------------------------------------
// One launch, two roles of 512 threads: blocks [0, dw_blocks) the dWp chunk
// partials, the rest d_out.
constexpr int kBwdThreads = 512;
constexpr int kWtStride2 = 36;               // dwords per LDS row of the transposed Wp slab (64 + 8 bf16)
constexpr int kDxCols = 256;                 // d_out columns per block
constexpr int kDxTokens = 64;                // d_out tokens per block
constexpr int kDwCols = 128;                 // dWp columns per block
constexpr int kDwColBlocks = kD / kDwCols;   // 24
constexpr int kRound = 64;                   // tokens staged per round
constexpr int kStRow2 = kDwCols / 2 + 4;     // dwords per staged token row of out (128 + 8 bf16)
constexpr int kDlRow2 = kO / 2 + 4;          // dwords per staged token row of d_lat (64 + 8 bf16)
constexpr size_t kBwdLds = sizeof(uint32_t) * kDxCols * kWtStride2;   // 36 KB
static_assert(sizeof(uint32_t) * kRound * (kStRow2 + kDlRow2) <= kBwdLds, "dWp rounds fit the shared buffer");
static_assert(sizeof(uint16_t) * 8 * 16 * 128 <= kBwdLds, "d_out staging fits the shared buffer");

// two rows' 8 consecutive elements -> 8 dwords (element e of row 0 | of row 1 << 16)
__device__ __forceinline__ void interleave8(const uint4& r0, const uint4& r1, uint32_t (&o)[8]) {
  const uint32_t a[4] = {r0.x, r0.y, r0.z, r0.w}, b[4] = {r1.x, r1.y, r1.z, r1.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = (a[i] & 0xffffu) | (b[i] << 16);
    o[2 * i + 1] = (a[i] >> 16) | (b[i] & 0xffff0000u);
  }
}

// d_out for 64 tokens (tb ..) x 256 columns (k0 ..).  Wp's 64 x 256 slab is
// staged transposed (row k holds the 64 outputs' weights).  Wave w: token
// tile w % 4, columns 128 (w / 4) .. + 127 as 8 column tiles run side by
// side.  Lane (r, g): A = d_lat[t][16 g + s] (its 16 values loaded once), B =
// the slab's row of column 16 kt + r at outputs 16 g .. + 15 (32 bytes per
// tile).  The results go through LDS so each lane stores 16 contiguous bytes.
__device__ __forceinline__ void dx_block(const uint16_t* __restrict__ d_lat, const uint16_t* __restrict__ W,
                                         uint16_t* __restrict__ d_out, int64_t T, int64_t tb, int k0,
                                         uint32_t* lds) {
  // stage: row pair p (outputs 2 p, 2 p + 1) x column octet c8: 32 x 32 items, 2 per thread
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int item = threadIdx.x + kBwdThreads * it;
    const int p = item % 32, c8 = item / 32;
    const uint4 r0 = ld16(W + static_cast<int64_t>(2 * p) * kD + k0 + 8 * c8);
    const uint4 r1 = ld16(W + static_cast<int64_t>(2 * p + 1) * kD + k0 + 8 * c8);
    uint32_t o[8];
    interleave8(r0, r1, o);
#pragma unroll
    for (int e = 0; e < 8; ++e) lds[(8 * c8 + e) * kWtStride2 + p] = o[e];
  }
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int tt = wave & 3, half = wave >> 2;
  const int64_t tw = tb + 16 * tt;
  const int64_t tr = clamp_row(tw + r, T);
  const uint4 a0 = ld16(d_lat + tr * kO + 16 * g);
  const uint4 a1 = ld16(d_lat + tr * kO + 16 * g + 8);
  __syncthreads();
  f64x4_t acc[8];
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) acc[kt] = f64x4_t{0.0, 0.0, 0.0, 0.0};
  // outputs 16 g + s for s = 0 .. 7, then 8 .. 15: half of the slab's row in registers at a time
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint4 b[8];
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
      b[kt] = *reinterpret_cast<const uint4*>(lds + (128 * half + 16 * kt + r) * kWtStride2 + 8 * g + 4 * h);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const double a = el8(h == 0 ? a0 : a1, s);
#pragma unroll
      for (int kt = 0; kt < 8; ++kt) acc[kt] = mfma_f64(a, el8(b[kt], s), acc[kt]);
    }
  }
  __syncthreads();   // the slab is read; its space now stages the results
  // lane holds token tw + g + 4 v, column k0 + 128 half + 16 kt + r
  uint16_t* st = reinterpret_cast<uint16_t*>(lds) + wave * (16 * 128);
#pragma unroll
  for (int kt = 0; kt < 8; ++kt)
#pragma unroll
    for (int v = 0; v < 4; ++v) st[(g + 4 * v) * 128 + 16 * kt + r] = f32_to_bf16(static_cast<float>(acc[kt][v]));
  __syncthreads();
  // 16 tokens x 16 chunks of 16 bytes per wave, 4 per lane
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int q = lane + 64 * it;
    const int row = q / 16, c = q % 16;
    if (tw + row < T)
      st16_nt(d_out + (tw + row) * kD + k0 + 128 * half + 8 * c, *reinterpret_cast<const uint4*>(st + row * 128 + 8 * c));
  }
}

// dWp and dbp partials of one 512-token chunk (c) for 128 columns (k0 ..): 8
// rounds of 64 tokens staged in LDS as they are (token rows of out and
// d_lat; tokens past T staged as zeros).  Wave w: output tile w % 4, column
// tiles 4 (w / 4) .. + 3.  Lane (r, g) at step s of a round: A = d_lat[4 s +
// g][16 (w % 4) + r], B = out[4 s + g][16 n + r]: the chunk's tokens in
// ascending order.  Wave 0 of column block 0 also adds d_lat per output (lane
// o, fp64, tokens ascending) for dbp.
template <bool kFull>
__device__ __forceinline__ void dw_chunk(const uint16_t* __restrict__ d_lat, const uint16_t* __restrict__ out,
                                         double* __restrict__ part, double* __restrict__ part_db, int64_t T,
                                         int bx, int64_t c, uint32_t* lds) {
  constexpr int kRounds = kChunk / kRound;   // 8
  const int k0 = bx * kDwCols;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int ot = wave & 3, n0 = 4 * (wave >> 2);
  uint32_t* xs = lds;                        // [64 tokens][kStRow2]
  uint32_t* ds = lds + kRound * kStRow2;     // [64 tokens][kDlRow2]
  // staging items: out 64 tokens x 16 chunks (2 per thread), d_lat 64 x 8 (1 per thread)
  const int xt = threadIdx.x / 16, xc = threadIdx.x % 16;     // + 32 tokens for the second
  const int dt = threadIdx.x / 8, dc = threadIdx.x % 8;
  f64x4_t acc[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) acc[n] = f64x4_t{0.0, 0.0, 0.0, 0.0};
  double sdb = 0.0;
  uint4 bx0[2], bx1[2], bd[2];
  auto load = [&](int rd, int slot) {
    const int64_t tbase = c * kChunk + rd * kRound;
    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
    const int64_t ta = tbase + xt, tb2 = tbase + xt + 32, td = tbase + dt;
    if constexpr (kFull) {
      bx0[slot] = ld16(out + ta * kD + k0 + 8 * xc);
      bx1[slot] = ld16(out + tb2 * kD + k0 + 8 * xc);
      bd[slot] = ld16(d_lat + td * kO + 8 * dc);
    } else {
      bx0[slot] = ta < T ? ld16(out + ta * kD + k0 + 8 * xc) : z;
      bx1[slot] = tb2 < T ? ld16(out + tb2 * kD + k0 + 8 * xc) : z;
      bd[slot] = td < T ? ld16(d_lat + td * kO + 8 * dc) : z;
    }
  };
  auto round = [&](int rd, auto slot_c) __attribute__((always_inline)) {
    constexpr int cur = decltype(slot_c)::value;
    if (rd + 1 < kRounds) load(rd + 1, cur ^ 1);
    __syncthreads();   // the previous round's reads are done
    *reinterpret_cast<uint4*>(xs + xt * kStRow2 + 4 * xc) = bx0[cur];
    *reinterpret_cast<uint4*>(xs + (xt + 32) * kStRow2 + 4 * xc) = bx1[cur];
    *reinterpret_cast<uint4*>(ds + dt * kDlRow2 + 4 * dc) = bd[cur];
    __syncthreads();
    const uint16_t* xh = reinterpret_cast<const uint16_t*>(xs);
    const uint16_t* dh = reinterpret_cast<const uint16_t*>(ds);
#pragma unroll
    for (int s = 0; s < kRound / 4; ++s) {
      const int t = 4 * s + g;
      const double a = static_cast<double>(bf16_to_f32(dh[t * (2 * kDlRow2) + 16 * ot + r]));
#pragma unroll
      for (int n = 0; n < 4; ++n)
        acc[n] = mfma_f64(a, static_cast<double>(bf16_to_f32(xh[t * (2 * kStRow2) + 16 * (n0 + n) + r])), acc[n]);
    }
    if (bx == 0 && wave == 0) {
      for (int t = 0; t < kRound; ++t) sdb += static_cast<double>(bf16_to_f32(dh[t * (2 * kDlRow2) + lane]));
    }
  };
  load(0, 0);
#pragma unroll 1
  for (int rp = 0; rp < kRounds / 2; ++rp) {
    round(2 * rp, std::integral_constant<int, 0>{});
    round(2 * rp + 1, std::integral_constant<int, 1>{});
  }
  // lane holds outputs 16 ot + g + 4 v, columns k0 + 16 (n0 + n) + r
  double* pc = part + c * kO * kD;
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int v = 0; v < 4; ++v)
      pc[static_cast<int64_t>(16 * ot + g + 4 * v) * kD + k0 + 16 * (n0 + n) + r] = acc[n][v];
  if (bx == 0 && wave == 0) part_db[c * kO + lane] = sdb;
}

__global__ __launch_bounds__(kBwdThreads) void proj_out_bwd_kernel(const uint16_t* __restrict__ d_lat,
                                                                  const uint16_t* __restrict__ out,
                                                                  const uint16_t* __restrict__ W,
                                                                  uint16_t* __restrict__ d_out,
                                                                  double* __restrict__ part,
                                                                  double* __restrict__ part_db, int64_t T,
                                                                  int64_t dw_blocks) {
  __shared__ __align__(16) uint32_t lds[kBwdLds / 4];
  const int64_t blk = blockIdx.x;
  if (blk < dw_blocks) {
    const int bx = static_cast<int>(blk % kDwColBlocks);
    const int64_t c = blk / kDwColBlocks;
    if ((c + 1) * kChunk <= T)
      dw_chunk<true>(d_lat, out, part, part_db, T, bx, c, lds);
    else
      dw_chunk<false>(d_lat, out, part, part_db, T, bx, c, lds);
  } else {
    constexpr int kDxColBlocks = kD / kDxCols;
    const int64_t q = blk - dw_blocks;
    dx_block(d_lat, W, d_out, T, (q / kDxColBlocks) * kDxTokens, static_cast<int>(q % kDxColBlocks) * kDxCols, lds);
  }
}

// dWp and dbp: the chunks' partials added in ascending order in fp64, then
// rounded to fp32 and to bf16.  2 consecutive elements of dWp per thread;
// the partials are loaded 8 chunks at a time (indices clamped to the last
// chunk, so every load is in bounds and none sits under a branch).
__global__ __launch_bounds__(256) void proj_out_dw_combine_kernel(const double* __restrict__ part,
                                                                  const double* __restrict__ part_db,
                                                                  uint16_t* __restrict__ dW, uint16_t* __restrict__ db,
                                                                  int64_t chunks) {
  const int64_t i = 2 * (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x);   // < 64 * 3072 by the grid
  double s0 = 0.0, s1 = 0.0;
  for (int64_t c0 = 0; c0 < chunks; c0 += 8) {
    double2 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t c = c0 + j < chunks ? c0 + j : chunks - 1;
      v[j] = *reinterpret_cast<const double2*>(part + c * kO * kD + i);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool in = c0 + j < chunks;
      s0 = in ? s0 + v[j].x : s0;
      s1 = in ? s1 + v[j].y : s1;
    }
  }
  *reinterpret_cast<uint32_t*>(dW + i) = pack_bf16x2(static_cast<float>(s0), static_cast<float>(s1));
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
  hipLaunchKernelGGL(proj_out_fwd_kernel, dim3(static_cast<unsigned>((T + kFT - 1) / kFT)), dim3(kFwdThreads), 0, s,
                     out, W, bias, latent, T);
  return hipGetLastError();
}

hipError_t launch_proj_out_fwd_fused(const uint16_t* x, const uint16_t* emb, const float* mean, const float* rstd,
                                     const uint16_t* W, const uint16_t* bias, uint16_t* latent, int64_t B, int64_t S,
                                     hipStream_t s) {
  const int64_t T = B * S;
  hipLaunchKernelGGL(proj_out_fused_kernel, dim3(static_cast<unsigned>((T + kFT - 1) / kFT)), dim3(kFwdThreads), 0, s,
                     x, emb, mean, rstd, W, bias, latent, T, S);
  return hipGetLastError();
}

hipError_t launch_proj_out_bwd(const uint16_t* d_lat, const uint16_t* out, const uint16_t* W, uint16_t* d_out,
                               uint16_t* dW, uint16_t* db, double* part, double* part_db, int64_t T, hipStream_t s) {
  const int64_t chunks = proj_out_chunks(T);
  const int64_t dw_blocks = kDwColBlocks * chunks;
  const int64_t dx_blocks = (T + kDxTokens - 1) / kDxTokens * (kD / kDxCols);
  const dim3 grid(static_cast<unsigned>(dw_blocks + dx_blocks));
  hipLaunchKernelGGL(proj_out_bwd_kernel, grid, dim3(kBwdThreads), 0, s, d_lat, out, W, d_out, part, part_db, T,
                     dw_blocks);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  hipLaunchKernelGGL(proj_out_dw_combine_kernel, dim3(kO * kD / 2 / 256), dim3(256), 0, s, part, part_db, dW, db,
                     chunks);
  return hipGetLastError();
}

}  // namespace adaln
