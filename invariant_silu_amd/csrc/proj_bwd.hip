// Projection backward of the AdaLN final modulation (RL-Kernel pull request
// 538, "What"; SiLU VJP per the review thread), from the fp32
// d_emb = (d_scale | d_shift):
//   dW[j,k]  = bf16(fl32(sum_b d_emb[b,j] * a[b,k]))      (fp32 products)
//   db[j]    = bf16(fl32(sum_b d_emb[b,j]))
//   da[b,k]  = fl32(sum_j d_emb[b,j] * W[j,k])             (fp32 products)
//   dtemb    = bf16(da * silu'(temb))
// Sums accumulate fp32 products in fp64 in fixed orders: samples ascending
// for dW and db; for da, 128 row slots (slot t: rows t, t + 128, ... in
// order) added as a pairwise tree.  Device pieces are shared by every
// kernel, so every entry point computes identical bits, and no order depends
// on the batch size or the grid.
//
// Kernels:
//   proj_bwd_small_kernel<NB>  B <= 4: da column blocks (-> dtemb) and dW
//                              tiles (-> dW, db) in one grid
//   silu_kernel, proj_bwd_dw_kernel, proj_bwd_da_kernel   B > 4
#include "common.hpp"
#include "launch.hpp"

namespace adaln {

namespace {

constexpr int kThreads = 256;

// ---- projection backward ------------------------------------------------
// dW tiles: part p of 32 (192 rows) x column block kb of 12 (256 columns),
// a write stream; 8 row slots, a thread's 8 columns per row.
constexpr int kDwParts = 32;
constexpr int kTileCols = 256;                       // columns per dW tile (32 threads x 8)
constexpr int kColThreads = kTileCols / 8;           // 32
constexpr int kSlots = 8;                            // row slots per dW tile
constexpr int kBlockThreads = kColThreads * kSlots;  // 256
constexpr int kRowsPerPart = kN / kDwParts;          // 192
constexpr int kSteps = kRowsPerPart / kSlots;        // 24 rows per thread
constexpr int kDwTiles = kDwParts * (kD / kTileCols);   // 384
constexpr int kBatchChunk = 4;

static_assert(kN % kDwParts == 0 && kRowsPerPart % kSlots == 0, "part layout");
static_assert(kD % kTileCols == 0, "column blocks");
static_assert(kBlockThreads == kThreads, "one block size for every role");

// da blocks: 16 columns of W over all 6144 rows, so each block finishes the
// sum and writes dtemb itself.  128 row slots, slot t walks rows t, t + 128,
// ... in order (fp64 accumulation of fp32 products); the 128 slots are then
// added as a pairwise tree.  The four 32-byte quarters of a 128-byte row
// segment go to blocks L, L + 8, L + 16 and L + 24, which the dispatcher
// places on the same XCD (one L2 serves all four).
constexpr int kDaCols = 16;
constexpr int kDaColThreads = kDaCols / 8;            // 2
constexpr int kDaSlots = kThreads / kDaColThreads;    // 128
constexpr int kDaBlocks = kD / kDaCols;               // 192
constexpr int kDaSteps = kN / kDaSlots;               // 48 rows per thread
constexpr int kDaShare = 128 / (kDaCols * 2);         // blocks sharing a 128-byte segment: 4

static_assert(kDaBlocks % (8 * kDaShare) == 0, "da block to column mapping");

__device__ __forceinline__ int da_first_col(int L) {
  const int g = L / (8 * kDaShare), q = (L / 8) % kDaShare, xcd = L % 8;
  return ((g * 8 + xcd) * kDaShare + q) * kDaCols;
}

// da and dtemb for samples b0 .. b0 + nb - 1 (nb <= NB) and the 32 columns of
// block L.  red: LDS, kDaSlots * NB * kDaCols doubles.
template <int NB>
__device__ __forceinline__ void da_block(const float* __restrict__ d_emb, const uint16_t* __restrict__ W,
                                         const uint16_t* __restrict__ temb, uint16_t* __restrict__ dtemb,
                                         int L, int64_t b0, int nb, double* red) {
  // rows per batch (two batches in flight), sized to keep registers <= ~128
  constexpr int U = NB == 1 ? 8 : (NB == 2 ? 6 : (NB == 3 ? 6 : 4));
  static_assert(kDaSteps % (2 * U) == 0, "batch pairs");
  static_assert(kDaSteps % U == 0, "batches");
  const int ct = threadIdx.x % kDaColThreads;
  const int slot = threadIdx.x / kDaColThreads;
  const int col0 = da_first_col(L);
  const Buffer wb(W, static_cast<uint32_t>(kN) * kD * 2);
  const Buffer eb(d_emb + b0 * kN, static_cast<uint32_t>(nb) * kN * 4);
  const uint32_t w_lane = (static_cast<uint32_t>(slot) * kD + col0 + ct * 8) * 2;
  const uint32_t e_lane = static_cast<uint32_t>(slot) * 4;
  constexpr uint32_t kWStep = kDaSlots * kD * 2;   // bytes between a slot's rows
  constexpr uint32_t kEStep = kDaSlots * 4;

  auto load = [&](int i0, uint4 (&w)[U], float (&d)[U][NB]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = wb.u128(w_lane, (i0 + u) * kWStep);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int bl = b < nb ? b : nb - 1;   // samples past nb: any in-range value, never stored
        d[u][b] = eb.f32(e_lane, bl * kN * 4 + (i0 + u) * kEStep);
      }
  };
  double acc[NB][8];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[b][e] = 0.0;
  auto accumulate = [&](const uint4 (&w)[U], const float (&d)[U][NB]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float wf[8];
      unpack8(w[u], wf);
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[b][e] += static_cast<double>(d[u][b] * wf[e]);
    }
  };

  // two register batches: the next one is in flight while one is added
  uint4 wa[U], wbt[U];
  float da_[U][NB], db_[U][NB];
  load(0, wa, da_);
  // (scheduling barriers keep the compiler from hoisting a batch's loads
  // above the adds of the batch whose registers they reuse)
#pragma unroll 1
  for (int i0 = 0; i0 < kDaSteps - 2 * U; i0 += 2 * U) {
    load(i0 + U, wbt, db_);
    __builtin_amdgcn_sched_barrier(0);
    accumulate(wa, da_);
    __builtin_amdgcn_sched_barrier(0);
    load(i0 + 2 * U, wa, da_);
    __builtin_amdgcn_sched_barrier(0);
    accumulate(wbt, db_);
    __builtin_amdgcn_sched_barrier(0);
  }
  load(kDaSteps - U, wbt, db_);
  __builtin_amdgcn_sched_barrier(0);
  accumulate(wa, da_);
  accumulate(wbt, db_);

  constexpr int kRow = NB * kDaCols;   // doubles per slot
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int e = 0; e < 8; ++e) red[slot * kRow + b * kDaCols + ct * 8 + e] = acc[b][e];
  __syncthreads();
  // pairwise tree over the slots: ((s0 + s1) + (s2 + s3)) + ...
#pragma unroll
  for (int w = 1; w < kDaSlots; w <<= 1) {
    for (int i = threadIdx.x; i < (kDaSlots / (2 * w)) * kRow; i += kThreads) {
      const int s = (i / kRow) * 2 * w, r = i % kRow;
      red[s * kRow + r] += red[(s + w) * kRow + r];
    }
    __syncthreads();
  }
  if (threadIdx.x < kRow) {
    const int b = threadIdx.x / kDaCols, c = threadIdx.x % kDaCols;
    if (b < nb) {
      const int64_t i = (b0 + b) * kD + col0 + c;
      dtemb[i] = f32_to_bf16(static_cast<float>(red[threadIdx.x]) * dsilu_f32(bf16_to_f32(temb[i])));
    }
  }
}

// dW tile (192 rows x 256 columns of part p, column block kb): a write
// stream; a = bf16(SiLU(temb)) per thread for its 8 columns.  Tiles of column
// block 0 also write db for their rows: samples in order from +0.
template <int NB>
__device__ __forceinline__ void dw_tile(const float* __restrict__ d_emb,
                                        const uint16_t* __restrict__ temb, uint16_t* __restrict__ dW,
                                        uint16_t* __restrict__ db, int p, int kb,
                                        float (*de_lds)[kRowsPerPart]) {
  const int ct = threadIdx.x % kColThreads;
  const int slot = threadIdx.x / kColThreads;
  const int col = kb * kTileCols + ct * 8;
  const int jbase = p * kRowsPerPart;
  constexpr int kDeLoads = (NB * kRowsPerPart + kBlockThreads - 1) / kBlockThreads;
  float de_r[kDeLoads];
#pragma unroll
  for (int k = 0; k < kDeLoads; ++k) {
    const int idx = threadIdx.x + kBlockThreads * k;
    if (idx < NB * kRowsPerPart)
      de_r[k] = d_emb[static_cast<int64_t>(idx / kRowsPerPart) * kN + jbase + idx % kRowsPerPart];
  }
  uint4 tz[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) tz[b] = ld16(temb + static_cast<int64_t>(b) * kD + col);
#pragma unroll
  for (int k = 0; k < kDeLoads; ++k) {
    const int idx = threadIdx.x + kBlockThreads * k;
    if (idx < NB * kRowsPerPart) de_lds[idx / kRowsPerPart][idx % kRowsPerPart] = de_r[k];
  }
  float av[NB][8];
  uint32_t redo = 0;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    uint32_t m;
    unpack8(silu8_fast(tz[b], m), av[b]);
    redo |= m << (8 * b);
  }
  while (redo != 0) {   // rarely taken: elements the fast SiLU cannot decide
    const int bit = __builtin_ctz(redo);
    redo &= redo - 1;
    const int b = bit / 8, e = bit % 8;
    const float v = bf16_to_f32(silu_bf16_exact(bf16_to_f32(temb[static_cast<int64_t>(b) * kD + col + e])));
#pragma unroll
    for (int bb = 0; bb < NB; ++bb)
#pragma unroll
      for (int ee = 0; ee < 8; ++ee)
        if (bb == b && ee == e) av[bb][ee] = v;
  }
  __syncthreads();
  if (kb == 0 && threadIdx.x < kRowsPerPart) {
    double s = 0.0;
#pragma unroll
    for (int b = 0; b < NB; ++b) s += static_cast<double>(de_lds[b][threadIdx.x]);
    db[jbase + threadIdx.x] = f32_to_bf16(static_cast<float>(s));
  }
#pragma unroll 4
  for (int i = 0; i < kSteps; ++i) {
    const int jl = slot + kSlots * i;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      double s = 0.0;
#pragma unroll
      for (int b = 0; b < NB; ++b) s += static_cast<double>(de_lds[b][jl] * av[b][e]);
      o[e] = static_cast<float>(s);
    }
    st16_nt(dW + static_cast<int64_t>(jbase + jl) * kD + col, pack8(o));
  }
}

// LDS of a projection-backward block, laid out per role.
template <int NB>
struct ProjBwdShared {
  static constexpr size_t kRed = sizeof(double) * kDaSlots * NB * kDaCols;
  static constexpr size_t kDe = sizeof(float) * NB * kRowsPerPart;
  static constexpr size_t kBytes = kRed > kDe ? kRed : kDe;
};

// Small batches (B <= 4, a template parameter): one grid, blocks [0, 192)
// are the da column blocks (they read W and write dtemb), blocks [192, 576)
// the dW tiles (they write dW and db); the two streams run side by side.
template <int NB>
__global__ __launch_bounds__(kThreads) void proj_bwd_small_kernel(
    const float* __restrict__ d_emb, const uint16_t* __restrict__ temb, const uint16_t* __restrict__ W,
    uint16_t* __restrict__ dW, uint16_t* __restrict__ db, uint16_t* __restrict__ dtemb) {
  __shared__ __align__(16) unsigned char smem[ProjBwdShared<NB>::kBytes];
  const int blk = blockIdx.x;
  if (blk < kDaBlocks) {
    da_block<NB>(d_emb, W, temb, dtemb, blk, 0, NB, reinterpret_cast<double*>(smem));
  } else {
    const int t = blk - kDaBlocks;
    dw_tile<NB>(d_emb, temb, dW, db, t % kDwParts, t / kDwParts,
                reinterpret_cast<float (*)[kRowsPerPart]>(smem));
  }
}

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

// ---- B > 4 ------------------------------------------------------------------
// dW tile of 32 rows x 256 columns per block; samples staged through LDS 64 at
// a time (a: 32 KB, d_emb: 8 KB).  Thread (ct, rg) owns rows 4 rg .. 4 rg + 3
// and columns 8 ct .. 8 ct + 7: 32 fp64 sums, samples in ascending order.
// Blocks of column block 0 also sum db for their rows.
constexpr int kDwBRows = 32;
constexpr int kDwBCols = 256;
constexpr int kDwBSamples = 64;
constexpr int kDwBLoads = kDwBSamples * (kDwBCols / 8) / kThreads;   // 8 chunk loads per thread
static_assert(kDwBSamples * kDwBRows / kThreads == kDwBLoads, "staging layout");

__global__ __launch_bounds__(kThreads) void proj_bwd_dw_kernel(const float* __restrict__ d_emb,
                                                               const uint16_t* __restrict__ a,
                                                               uint16_t* __restrict__ dW,
                                                               uint16_t* __restrict__ db, int64_t B) {
  __shared__ uint4 a_lds[kDwBSamples][kDwBCols / 8];   // 32 KB
  __shared__ __align__(16) float d_lds[kDwBSamples][kDwBRows];   // 8 KB
  const int ct = threadIdx.x % (kDwBCols / 8);
  const int rg = threadIdx.x / (kDwBCols / 8);
  const int j0 = blockIdx.x * kDwBRows;
  const int k0 = blockIdx.y * kDwBCols;
  double acc[4][8];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = 0.0;
  double dbs = 0.0;
  for (int64_t c0 = 0; c0 < B; c0 += kDwBSamples) {
    const int nb = static_cast<int>((B - c0) < kDwBSamples ? (B - c0) : kDwBSamples);
    // unconditional loads (slots past nb repeat sample nb - 1 and are unused)
    uint4 av_r[kDwBLoads];
    float d_r[kDwBLoads];
#pragma unroll
    for (int u = 0; u < kDwBLoads; ++u) {
      const int idx = threadIdx.x + kThreads * u;
      const int sa = idx / (kDwBCols / 8) < nb ? idx / (kDwBCols / 8) : nb - 1;
      av_r[u] = ld16(a + (c0 + sa) * kD + k0 + (idx % (kDwBCols / 8)) * 8);
      const int sd = idx / kDwBRows < nb ? idx / kDwBRows : nb - 1;
      d_r[u] = d_emb[(c0 + sd) * kN + j0 + idx % kDwBRows];
    }
    __syncthreads();   // the previous chunk is consumed
#pragma unroll
    for (int u = 0; u < kDwBLoads; ++u) {
      const int idx = threadIdx.x + kThreads * u;
      a_lds[idx / (kDwBCols / 8)][idx % (kDwBCols / 8)] = av_r[u];
      d_lds[idx / kDwBRows][idx % kDwBRows] = d_r[u];
    }
    __syncthreads();
    if (blockIdx.y == 0 && threadIdx.x < kDwBRows)
      for (int b = 0; b < nb; ++b) dbs += static_cast<double>(d_lds[b][threadIdx.x]);
#pragma unroll 2
    for (int b = 0; b < nb; ++b) {
      float av[8];
      unpack8(a_lds[b][ct], av);
      const float4 d4 = *reinterpret_cast<const float4*>(&d_lds[b][rg * 4]);
      const float dd[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] += static_cast<double>(dd[r] * av[e]);
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = static_cast<float>(acc[r][e]);
    st16_nt(dW + static_cast<int64_t>(j0 + rg * 4 + r) * kD + k0 + ct * 8, pack8(o));
  }
  if (blockIdx.y == 0 && threadIdx.x < kDwBRows) db[j0 + threadIdx.x] = f32_to_bf16(static_cast<float>(dbs));
}

// da and dtemb, 4 samples per blockIdx.y
__global__ __launch_bounds__(kThreads) void proj_bwd_da_kernel(const float* __restrict__ d_emb,
                                                               const uint16_t* __restrict__ W,
                                                               const uint16_t* __restrict__ temb,
                                                               uint16_t* __restrict__ dtemb, int64_t B) {
  __shared__ __align__(16) double red[kDaSlots * kBatchChunk * kDaCols];   // 64 KB
  const int64_t b0 = static_cast<int64_t>(blockIdx.y) * kBatchChunk;
  const int nb = static_cast<int>((B - b0) < kBatchChunk ? (B - b0) : kBatchChunk);
  da_block<kBatchChunk>(d_emb, W, temb, dtemb, blockIdx.x, b0, nb, red);
}


}  // namespace

int proj_bwd_fused_max_batch() { return kBatchChunk; }

hipError_t launch_proj_bwd_fused(const float* d_emb, const uint16_t* temb, const uint16_t* W,
                                 uint16_t* dW, uint16_t* db, uint16_t* dtemb, int64_t B, hipStream_t s) {
  const dim3 grid(kDaBlocks + kDwTiles), block(kThreads);
  switch (B) {
    case 1: hipLaunchKernelGGL(proj_bwd_small_kernel<1>, grid, block, 0, s, d_emb, temb, W, dW, db, dtemb); break;
    case 2: hipLaunchKernelGGL(proj_bwd_small_kernel<2>, grid, block, 0, s, d_emb, temb, W, dW, db, dtemb); break;
    case 3: hipLaunchKernelGGL(proj_bwd_small_kernel<3>, grid, block, 0, s, d_emb, temb, W, dW, db, dtemb); break;
    case 4: hipLaunchKernelGGL(proj_bwd_small_kernel<4>, grid, block, 0, s, d_emb, temb, W, dW, db, dtemb); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_proj_bwd_dw(const float* d_emb, const uint16_t* a, uint16_t* dW, uint16_t* db, int64_t B,
                              hipStream_t s) {
  hipLaunchKernelGGL(proj_bwd_dw_kernel, dim3(kN / kDwBRows, kD / kDwBCols), dim3(kThreads), 0, s, d_emb, a,
                     dW, db, B);
  return hipGetLastError();
}

hipError_t launch_proj_bwd_da(const float* d_emb, const uint16_t* W, const uint16_t* temb, uint16_t* dtemb,
                              int64_t B, hipStream_t s) {
  const int64_t bz = (B + kBatchChunk - 1) / kBatchChunk;
  hipLaunchKernelGGL(proj_bwd_da_kernel, dim3(kDaBlocks, static_cast<unsigned>(bz)), dim3(kThreads), 0, s,
                     d_emb, W, temb, dtemb, B);
  return hipGetLastError();
}

hipError_t launch_silu(const uint16_t* temb, uint16_t* a, int64_t n, hipStream_t s) {
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(silu_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, temb, a, n);
  return hipGetLastError();
}


}  // namespace adaln
