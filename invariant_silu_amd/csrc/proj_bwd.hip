// Projection backward of the AdaLN final modulation (RL-Kernel pull request
// 538, "What"; SiLU VJP per the review thread), from the fp32
// d_emb = (d_scale | d_shift):
//   dW[j,k]  = bf16(fl32(sum_b d_emb[b,j] * a[b,k]))
//   db[j]    = bf16(fl32(sum_b d_emb[b,j]))
//   da[b,k]  = fl32(sum_j d_emb[b,j] * W[j,k])
//   dtemb    = bf16(da * silu'(temb))
// Every product is exact (an fp64 fused multiply-add of the fp32 and bf16
// operands) and the sums run in fp64 in fixed orders:
//   dW: samples ascending from +0, one fused multiply-add each;
//   db: samples ascending from +0 (plain adds);
//   da: 128 leaves, leaf t over rows t, t + 128, ..., t + 128 (N / 128 - 1)
//       in that order from +0; then the leaves added pairwise in index order.
// N is the projection width: 6144 for the final modulation, 18432 for a
// block's 6-way modulation (a template parameter of every kernel here).
// The vector-unit kernels (B <= 4) and the matrix-core kernels (B > 4; a
// v_mfma_f64_16x16x4f64 is that same chain of four fused multiply-adds) run
// these orders exactly, so no result depends on the batch size or the grid.
//
// Kernels:
//   proj_bwd_small_kernel<NB>  B <= 6: da leaf-group blocks (-> the 32
//                              4-leaf subtrees of every column) and dW tiles
//                              (-> dW, db) in one grid
//   da_finish_kernel<NB>       B <= 6: the subtrees added pairwise (-> dtemb)
//   proj_bwd_f32_small_kernel<NB>  fp32 storage, B <= 4: the leaf-group blocks
//                              and the matrix-core dW tiles in one grid (then
//                              da_finish_kernel<NB, float>)
//   silu_kernel, dw_mfma_kernel, da_mfma_kernel   B > 6 (fp32 storage: B > 4)
//   proj_bwd_mid_kernel        da's leaf runs and the dW
//                              tiles in one grid (fp32 storage: 17 <= B)
//   da_parts_kernel            the leaf runs' subtrees added
//                              pairwise (-> dtemb)
// With kAcc (adaln_proj_bwd_acc) the bf16 kernels also store the fp32 values
// they round to bf16 -- fl32 of the dW and db sums, and da * silu'(temb) in
// fp32 -- into whichever of the caller's fp32 arrays are not NULL; the
// arithmetic is the same instructions either way.

#include "common.hpp"
#include "launch.hpp"
#include "mfma.hpp"

#include <type_traits>

namespace adaln {

namespace {

constexpr int kThreads = 256;

// ---- projection backward ------------------------------------------------
// dW tiles: part p of N / 192 (192 rows) x column block kb of 12 (256
// columns), a write stream; 8 row slots, a thread's 8 columns per row.
constexpr int kTileCols = 256;                       // columns per dW tile (32 threads x 8)
constexpr int kColThreads = kTileCols / 8;           // 32
constexpr int kSlots = 8;                            // row slots per dW tile
constexpr int kBlockThreads = kColThreads * kSlots;  // 256
constexpr int kRowsPerPart = 192;
constexpr int kSteps = kRowsPerPart / kSlots;        // 24 rows per thread
template <int N>
constexpr int kDwParts = N / kRowsPerPart;           // 32 at N = 6144
template <int N>
constexpr int kDwTiles = kDwParts<N> * (kD / kTileCols);   // 384 at N = 6144
// largest B on the vector units (the matrix-core path from 7 samples: backward
// -4 to -6 us at B = 7 and 8 for S = 3 ... 4096; at B = 6 it is no faster)
constexpr int kBatchChunk = 6;

static_assert(kN % kRowsPerPart == 0 && kN6 % kRowsPerPart == 0 && kRowsPerPart % kSlots == 0, "part layout");
static_assert(kD % kTileCols == 0, "column blocks");
static_assert(kBlockThreads == kThreads, "one block size for every role");

// da: 128 leaves per column, leaf t = rows t, t + 128, ... in that order
// from +0 (N / 128 rows each); the leaves are then added pairwise in index
// order.
constexpr int kDaSlots = 128;
template <int N>
constexpr int kDaSteps = N / kDaSlots;                // rows per leaf: 48 at N = 6144
static_assert(kDaSteps<kN> == 48 && kN6 % kDaSlots == 0, "leaf rows");

// 2 consecutive elements of one row
template <typename T>
struct Pair;
template <>
struct Pair<uint16_t> {
  uint32_t v;
  __device__ __forceinline__ void load(const Buffer& b, uint32_t lane_off, uint32_t off) { v = b.u32(lane_off, off); }
  __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const uint32_t*>(p); }
  __device__ __forceinline__ float lo() const { return bf_lo(v); }
  __device__ __forceinline__ float hi() const { return bf_hi(v); }
  __device__ __forceinline__ static void store(uint16_t* p, float a, float b) {
    *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(a, b);
  }
};
template <>
struct Pair<float> {
  uint32_t v[2];
  __device__ __forceinline__ void load(const Buffer& b, uint32_t lane_off, uint32_t off) {
    const auto t = __builtin_amdgcn_raw_buffer_load_b64(b.rsrc, lane_off, off, 0);
    v[0] = t[0];
    v[1] = t[1];
  }
  __device__ __forceinline__ void load(const float* p) {
    const uint2 t = *reinterpret_cast<const uint2*>(p);
    v[0] = t.x;
    v[1] = t.y;
  }
  __device__ __forceinline__ float lo() const { return __uint_as_float(v[0]); }
  __device__ __forceinline__ float hi() const { return __uint_as_float(v[1]); }
  __device__ __forceinline__ static void store(float* p, float a, float b) {
    *reinterpret_cast<float2*>(p) = make_float2(a, b);
  }
};

// da for B <= 4 in two steps.  A leaf-group block (gq, cg) runs the 4
// leaves 4 gq .. 4 gq + 3 over the 256 columns 256 cg .. 256 cg + 255 of W;
// wave w is leaf 4 gq + w and its lane holds column quad lane (4 columns), so
// one wave load is 512 contiguous bytes of one row of W (a 16-leaf block of 64
// columns, each wave load 4 rows x 128 bytes, took 2 us longer with W cold in
// HBM).  The W stream is spread over 384 blocks.  The block then adds its 4
// leaves pairwise in leaf order -- the subtree those leaves form in the
// 128-leaf pairwise tree -- and writes one fp64 value per (sample, column) to
// sub[gq][b][col].  da_finish_kernel adds the 32 subtrees pairwise in order
// (the tree's top five levels): the 128-leaf pairwise tree exactly.
constexpr int kDaGroupLeaves = 4;
constexpr int kDaGroups = kDaSlots / kDaGroupLeaves;            // 32
constexpr int kDaQuadCols = 256;                                // columns per leaf-group block
constexpr int kDaQuads = kDaQuadCols / 4;                       // 64 column quads
constexpr int kDaLeafBlocks = kDaGroups * (kD / kDaQuadCols);   // 384
static_assert(kDaGroupLeaves * kDaQuads == kThreads, "leaf-group block shape");
static_assert(kD % kDaQuadCols == 0, "leaf-group columns");

// 4 consecutive elements of one row of W: one 8-byte load (bf16) or one
// 16-byte load (fp32)
template <typename T>
struct Quad;
template <>
struct Quad<uint16_t> {
  uint32_t v[2];
  __device__ __forceinline__ void load(const Buffer& b, uint32_t lane_off, uint32_t off) {
    const auto t = __builtin_amdgcn_raw_buffer_load_b64(b.rsrc, lane_off, off, 0);
    v[0] = t[0];
    v[1] = t[1];
  }
  __device__ __forceinline__ void unpack(float (&f)[4]) const {
    f[0] = bf_lo(v[0]); f[1] = bf_hi(v[0]); f[2] = bf_lo(v[1]); f[3] = bf_hi(v[1]);
  }
};
template <>
struct Quad<float> {
  uint32_t v[4];
  __device__ __forceinline__ void load(const Buffer& b, uint32_t lane_off, uint32_t off) {
    const uint4 t = b.u128(lane_off, off);
    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
  }
  __device__ __forceinline__ void unpack(float (&f)[4]) const {
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(v[e]);
  }
};

template <int NB, typename T, int N = kN>
__device__ __forceinline__ void da_leaf_group(const float* __restrict__ d_emb, const T* __restrict__ W,
                                              double* __restrict__ sub, int L, double* red) {
  // rows per batch (two batches in flight, registers <= ~128); N / 128 rows
  // per leaf (48 or 144)
  constexpr int U = sizeof(T) == 4 ? (NB == 1 ? 8 : (NB == 2 ? 6 : 4)) : (NB == 1 ? 12 : (NB == 2 ? 8 : (NB <= 4 ? 6 : 4)));
  constexpr int kLeafRows = kDaSteps<N>;
  static_assert(kLeafRows % (2 * U) == 0, "batch pairs");
  const int gq = L % kDaGroups, cg = L / kDaGroups;
  const int l = threadIdx.x / kDaQuads, cq = threadIdx.x % kDaQuads;
  const int leaf = gq * kDaGroupLeaves + l;
  const int col0 = cg * kDaQuadCols;
  const Buffer wb(W, static_cast<uint32_t>(N) * kD * sizeof(T));
  const Buffer eb(d_emb, static_cast<uint32_t>(NB) * N * 4);
  const uint32_t w_lane = (static_cast<uint32_t>(leaf) * kD + col0 + cq * 4) * sizeof(T);
  const uint32_t e_lane = static_cast<uint32_t>(leaf) * 4;
  constexpr uint32_t kWStep = kDaSlots * kD * sizeof(T);   // bytes between a leaf's rows
  constexpr uint32_t kEStep = kDaSlots * 4;

  auto load = [&](int i0, Quad<T> (&w)[U], float (&d)[U][NB]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) w[u].load(wb, w_lane, (i0 + u) * kWStep);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int b = 0; b < NB; ++b) d[u][b] = eb.f32(e_lane, b * N * 4 + (i0 + u) * kEStep);
  };
  double acc[NB][4];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[b][e] = 0.0;
  auto accumulate = [&](const Quad<T> (&w)[U], const float (&d)[U][NB]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float wf[4];
      w[u].unpack(wf);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const double dd = static_cast<double>(d[u][b]);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[b][e] = __builtin_fma(dd, static_cast<double>(wf[e]), acc[b][e]);
      }
    }
  };

  // two register batches: the next one is in flight while one is added
  Quad<T> wa[U], wbt[U];
  float da_[U][NB], db_[U][NB];
  load(0, wa, da_);
#pragma unroll 1
  for (int i0 = 0; i0 < kLeafRows - 2 * U; i0 += 2 * U) {
    load(i0 + U, wbt, db_);
    __builtin_amdgcn_sched_barrier(0);
    accumulate(wa, da_);
    __builtin_amdgcn_sched_barrier(0);
    load(i0 + 2 * U, wa, da_);
    __builtin_amdgcn_sched_barrier(0);
    accumulate(wbt, db_);
    __builtin_amdgcn_sched_barrier(0);
  }
  load(kLeafRows - U, wbt, db_);
  __builtin_amdgcn_sched_barrier(0);
  accumulate(wa, da_);
  accumulate(wbt, db_);

  // the block's 4 leaves, pairwise in leaf order: (l0 + l1) + (l2 + l3)
  constexpr int kRow = NB * kDaQuadCols;   // doubles per leaf
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[l * kRow + b * kDaQuadCols + cq * 4 + e] = acc[b][e];
  __syncthreads();
#pragma unroll
  for (int w = 1; w < kDaGroupLeaves; w <<= 1) {
    for (int i = threadIdx.x; i < (kDaGroupLeaves / (2 * w)) * kRow; i += kThreads) {
      const int s = (i / kRow) * 2 * w, r = i % kRow;
      red[s * kRow + r] += red[(s + w) * kRow + r];
    }
    __syncthreads();
  }
  for (int i = threadIdx.x; i < kRow; i += kThreads) {
    const int b = i / kDaQuadCols, c = i % kDaQuadCols;
    sub[(static_cast<int64_t>(gq) * NB + b) * kD + col0 + c] = red[i];
  }
}

// da = the 32 subtrees of a (sample, column) added pairwise in order, then
// dtemb = da * silu'(temb) in the storage type (bf16: one rounding); one
// thread per (sample, column)
// da_finish_kernel: block of 64 (sample, column) elements, 8 waves; wave w
// adds subtrees 4 w .. 4 w + 3 pairwise (two levels of the 32-subtree top),
// wave 0 then the 8 results pairwise through LDS (three more): the same tree
// as one thread over all 32, with four loads per thread in flight instead of
// one thread's 32
constexpr int kFinishWaves = 8;

template <int NB, typename T = uint16_t, bool kAcc = false>
__global__ __launch_bounds__(64 * kFinishWaves) void da_finish_kernel(const double* __restrict__ sub,
                                                                      const T* __restrict__ temb,
                                                                      T* __restrict__ dtemb,
                                                                      float* __restrict__ dtemb32) {
  constexpr int kPer = kDaGroups / kFinishWaves;   // subtrees per wave
  static_assert(kPer == 4 && kD % 64 == 0, "two levels per wave, whole 64-column blocks");
  __shared__ double node[kFinishWaves][64];
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * 64 + lane;   // b * D + column
  double v[kPer];
#pragma unroll
  for (int q = 0; q < kPer; ++q) v[q] = sub[static_cast<int64_t>(w * kPer + q) * NB * kD + i];
  node[w][lane] = (v[0] + v[1]) + (v[2] + v[3]);
  __syncthreads();
  if (w != 0) return;
  double u[kFinishWaves];
#pragma unroll
  for (int j = 0; j < kFinishWaves; ++j) u[j] = node[j][lane];
  const float d = static_cast<float>(pair_reduce(u)) * dsilu_f32(Storage<T>::load1(temb[i]));
  dtemb[i] = Storage<T>::store1(d);
  if constexpr (kAcc) {
    if (dtemb32) dtemb32[i] = d;
  }
}

// 8 consecutive fp32 values, two 16-byte stores
__device__ __forceinline__ void st32f(float* p, const float (&f)[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(f[4], f[5], f[6], f[7]);
}

// dW tile (192 rows x 256 columns of part p, column block kb): a write
// stream; a = bf16(SiLU(temb)) per thread for its 8 columns.  Tiles of column
// block 0 also write db for their rows: samples in order from +0.
template <int NB, int N = kN, bool kAcc = false>
__device__ __forceinline__ void dw_tile(const float* __restrict__ d_emb,
                                        const uint16_t* __restrict__ temb, uint16_t* __restrict__ dW,
                                        uint16_t* __restrict__ db, float* __restrict__ dW32,
                                        float* __restrict__ db32, int p, int kb,
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
      de_r[k] = d_emb[static_cast<int64_t>(idx / kRowsPerPart) * N + jbase + idx % kRowsPerPart];
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
  // 8 flag bits per sample: the mask holds NB * 8 bits
  using Mask = std::conditional_t<(NB > 4), uint64_t, uint32_t>;
  static_assert(NB <= 8, "redo mask holds 8 samples of 8 elements");
  Mask redo = 0;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    uint32_t m;
    unpack8(silu8_fast(tz[b], m), av[b]);
    redo |= static_cast<Mask>(m) << (8 * b);
  }
  while (redo != 0) {   // rarely taken: elements the fast SiLU cannot decide
    const int bit = sizeof(Mask) == 8 ? __builtin_ctzll(redo) : __builtin_ctz(static_cast<uint32_t>(redo));
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
    const float v = static_cast<float>(s);
    db[jbase + threadIdx.x] = f32_to_bf16(v);
    if constexpr (kAcc) {
      if (db32) db32[jbase + threadIdx.x] = v;
    }
  }
#pragma unroll 4
  for (int i = 0; i < kSteps; ++i) {
    const int jl = slot + kSlots * i;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      double s = 0.0;
#pragma unroll
      for (int b = 0; b < NB; ++b)
        s = __builtin_fma(static_cast<double>(de_lds[b][jl]), static_cast<double>(av[b][e]), s);
      o[e] = static_cast<float>(s);
    }
    st16(dW + static_cast<int64_t>(jbase + jl) * kD + col, pack8(o));
    if constexpr (kAcc) {
      if (dW32) st32f(dW32 + static_cast<int64_t>(jbase + jl) * kD + col, o);
    }
  }
}

// LDS of a projection-backward block, laid out per role.
template <int NB>
struct ProjBwdShared {
  static constexpr size_t kRed = sizeof(double) * kDaGroupLeaves * NB * kDaQuadCols;
  static constexpr size_t kDe = sizeof(float) * NB * kRowsPerPart;
  static constexpr size_t kBytes = kRed > kDe ? kRed : kDe;
};

// Small batches (B <= 4, a template parameter): one grid, blocks [0, 384)
// are the da leaf-group blocks (they read W and write the subtrees), the
// rest the dW tiles (they write dW and db): [384, 768) at N = 6144; the two
// streams run side by side.  da_finish_kernel follows.  The kAcc form (its
// own kernel, so the plain one keeps its argument list) also stores the fp32
// dW and db.
template <int NB, int N, bool kAcc>
__device__ __forceinline__ void proj_bwd_small_body(const float* __restrict__ d_emb,
                                                    const uint16_t* __restrict__ temb,
                                                    const uint16_t* __restrict__ W, uint16_t* __restrict__ dW,
                                                    uint16_t* __restrict__ db, double* __restrict__ sub,
                                                    float* __restrict__ dW32, float* __restrict__ db32) {
  __shared__ __align__(16) unsigned char smem[ProjBwdShared<NB>::kBytes];
  const int blk = blockIdx.x;
  if (blk < kDaLeafBlocks) {
    da_leaf_group<NB, uint16_t, N>(d_emb, W, sub, blk, reinterpret_cast<double*>(smem));
  } else {
    const int t = blk - kDaLeafBlocks;
    dw_tile<NB, N, kAcc>(d_emb, temb, dW, db, dW32, db32, t % kDwParts<N>, t / kDwParts<N>,
                         reinterpret_cast<float (*)[kRowsPerPart]>(smem));
  }
}

template <int NB, int N = kN>
__global__ __launch_bounds__(kThreads) void proj_bwd_small_kernel(
    const float* __restrict__ d_emb, const uint16_t* __restrict__ temb, const uint16_t* __restrict__ W,
    uint16_t* __restrict__ dW, uint16_t* __restrict__ db, double* __restrict__ sub) {
  proj_bwd_small_body<NB, N, false>(d_emb, temb, W, dW, db, sub, nullptr, nullptr);
}

template <int NB, int N = kN>
__global__ __launch_bounds__(kThreads) void proj_bwd_small_acc_kernel(
    const float* __restrict__ d_emb, const uint16_t* __restrict__ temb, const uint16_t* __restrict__ W,
    uint16_t* __restrict__ dW, uint16_t* __restrict__ db, double* __restrict__ sub, float* __restrict__ dW32,
    float* __restrict__ db32) {
  proj_bwd_small_body<NB, N, true>(d_emb, temb, W, dW, db, sub, dW32, db32);
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

// ---- matrix cores -------------------------------------------------------------
// dW: a wave computes 64 rows x 32 columns as 4 x 2 output tiles; tile (m, n)
// holds rows j0 + 4 i + m and columns k0 + 2 c + n (i, c = 0 .. 15), so a
// lane's operands per sample are 16 contiguous bytes of d_emb (4 rows) and
// two contiguous elements of a.  Step s feeds samples 4 s .. 4 s + 3 (slot g =
// sample 4 s + g): each sum is the chain over samples in ascending order from
// +0, as in dw_tile.  Samples past B enter with d_emb = 0, which leaves every
// sum unchanged (the chain never holds -0).  Waves of column block 0 also sum
// db for their 64 rows.  T: storage type of a, dW and db; N rows.
constexpr int kDwMRows = 64;
constexpr int kDwMCols = 32;
constexpr int kDwMWaves = 4;

// block (bx, by): rows bx * 64 .., columns by * 128 .. (32 per wave)
template <typename T, int N, bool kAcc>
__device__ __forceinline__ void dw_block(const float* __restrict__ d_emb, const T* __restrict__ a,
                                         T* __restrict__ dW, T* __restrict__ db, int64_t B,
                                         float* __restrict__ dW32, float* __restrict__ db32, int bx, int by) {
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int j0 = bx * kDwMRows;
  const int k0 = (by * kDwMWaves + wave) * kDwMCols;
  const int64_t steps = (B + 3) / 4;

  f64x4_t acc[4][2];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n) acc[m][n] = f64x4_t{0.0, 0.0, 0.0, 0.0};

  const float* dp = d_emb + j0 + 4 * r;
  const T* ap = a + k0 + 2 * r;
  auto load = [&](int64_t st, float4& dv, Pair<T>& av) {
    const int64_t b = 4 * st + g;
    const int64_t bc = b < B ? b : B - 1;
    dv = *reinterpret_cast<const float4*>(dp + bc * N);
    av.load(ap + bc * kD);
    if (b >= B) dv = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  };
  auto step = [&](const float4& dv, const Pair<T>& av) {
    const double dd[4] = {static_cast<double>(dv.x), static_cast<double>(dv.y), static_cast<double>(dv.z),
                          static_cast<double>(dv.w)};
    const double aa[2] = {static_cast<double>(av.lo()), static_cast<double>(av.hi())};
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int n = 0; n < 2; ++n) acc[m][n] = mfma_f64(dd[m], aa[n], acc[m][n]);
  };
  float4 d0, d1;
  Pair<T> a0, a1;
  load(0, d0, a0);
  int64_t st = 0;
  for (; st + 2 <= steps; st += 2) {
    load(st + 1, d1, a1);
    step(d0, a0);
    load(st + 2 < steps ? st + 2 : st + 1, d0, a0);
    step(d1, a1);
  }
  if (st < steps) step(d0, a0);

  // lane holds rows j0 + 4 (g + 4 v) + m, columns k0 + 2 r + n
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t i = static_cast<int64_t>(j0 + 4 * (g + 4 * v) + m) * kD + k0 + 2 * r;
      const float f0 = static_cast<float>(acc[m][0][v]), f1 = static_cast<float>(acc[m][1][v]);
      Pair<T>::store(dW + i, f0, f1);
      if constexpr (kAcc) {
        if (dW32) *reinterpret_cast<float2*>(dW32 + i) = make_float2(f0, f1);
      }
    }
  if (by == 0 && wave == 0) {
    double sdb = 0.0;
    for (int64_t b = 0; b < B; ++b) sdb += static_cast<double>(d_emb[b * N + j0 + lane]);
    const float v = static_cast<float>(sdb);
    db[j0 + lane] = Storage<T>::store1(v);
    if constexpr (kAcc) {
      if (db32) db32[j0 + lane] = v;
    }
  }
}

template <typename T, int N = kN, bool kAcc = false>
__global__ __launch_bounds__(64 * kDwMWaves) void dw_mfma_kernel(const float* __restrict__ d_emb,
                                                                 const T* __restrict__ a,
                                                                 T* __restrict__ dW,
                                                                 T* __restrict__ db, int64_t B,
                                                                 float* __restrict__ dW32,
                                                                 float* __restrict__ db32) {
  dw_block<T, N, kAcc>(d_emb, a, dW, db, B, dW32, db32, blockIdx.x, blockIdx.y);
}

// da and dtemb: block of 16 samples (b0 ..) x 32 columns (k0 ..), 8 waves;
// wave w takes leaves 16 w .. 16 w + 15 in four groups of four consecutive
// leaves t0 .. t0 + 3, run side by side (8 chains: 4 leaves x 2 column
// tiles).  Step s of a leaf feeds rows t + 128 (4 s + g) at slot g, so a
// leaf's N / 512 steps (12 at N = 6144) are its rows in order.  Output tile n (0, 1) holds
// columns k0 + 2 c + n.  Lane (r, g) loads d_emb[b0 + r][t0 + 128 (4 s + g)
// .. + 3] (16 bytes: the four leaves) and W[t0 + l + 128 (4 s + g)][k0 + 2 r ..
// + 1] for l = 0 .. 3.  Leaf results go into the wave's leaf tree in order;
// the 8 subtrees meet in LDS, pairwise in leaf order.  At most 128 VGPRs,
// so two blocks fit a CU.  Blocks x and x + 8
// (same XCD) take the two halves of one 128-byte row segment of W.  Rows
// past B load sample B - 1 and are never stored.
// Split form (kParts = 8, 4 or 2, by da_runs): the 128 leaves fall into kParts aligned
// runs of 128 / kParts, one per blockIdx.z, each run on 4 waves; a block
// stores its run's subtree (fp64, 2 tiles x 64 lanes) in `parts` and
// da_parts_kernel adds the kParts subtrees pairwise in run order, which is
// the tree the one-block form builds.  With 96 x ceil(B / 16) blocks the
// one-block form leaves CUs idle; the split fills them (at every B measured).
template <int N>
constexpr int kLeafSteps = N / (4 * kDaSlots);   // a leaf's rows, 4 per matrix-core step
constexpr int kDaMWaves = 8;
constexpr int kDaMGroup = 4;                   // leaves run side by side
constexpr int kDaMCols = 32;
constexpr int kDaBlocksX = kD / kDaMCols;        // column blocks
constexpr int kDaMAhead = 1;                   // steps in flight

template <typename T>
struct DaStep {
  uint4 d;          // d_emb of the group's 4 leaves
  Pair<T> w[4];     // W, 2 columns, per leaf
};

// T: storage type of W, temb and dtemb; N rows of W
// blocks for kParts runs: 4 waves; one run: kDaMWaves
template <int kParts>
constexpr int kDaWavesFor = kParts == 1 ? kDaMWaves : 4;

// block x's first column and the block's samples b0 .. b0 + rows - 1
__device__ __forceinline__ int da_col0(int x) { return ((x / 16) * 8 + x % 8) * 64 + ((x / 8) % 2) * kDaMCols; }

// dtemb from the root tiles: lane (r, g) holds samples b0 + g + 4 v, columns
// k0 + 2 r + n
template <typename T, bool kAcc>
__device__ __forceinline__ void da_store(const f64x4_t (&tot)[2], const T* __restrict__ temb,
                                         T* __restrict__ dtemb, float* __restrict__ dtemb32, int64_t b0,
                                         int rows_here, int k0, int r, int g) {
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int sr = g + 4 * v;
    if (sr < rows_here) {
      const int64_t i = (b0 + sr) * kD + k0 + 2 * r;
      Pair<T> z;
      z.load(temb + i);
      const float d0 = static_cast<float>(tot[0][v]) * dsilu_f32(z.lo());
      const float d1 = static_cast<float>(tot[1][v]) * dsilu_f32(z.hi());
      Pair<T>::store(dtemb + i, d0, d1);
      if constexpr (kAcc) {
        if (dtemb32) *reinterpret_cast<float2*>(dtemb32 + i) = make_float2(d0, d1);
      }
    }
  }
}

// da block (x, y) of run z (z = 0 with one run); sub: the block's LDS for
// its waves' subtrees
template <int kParts>
using DaSub = f64x4_t[kDaWavesFor<kParts> - 1][2][64];   // 28 KB at 8 waves

template <typename T, int N, bool kAcc, int kParts>
__device__ __forceinline__ void da_block(const float* __restrict__ d_emb, const T* __restrict__ W,
                                         const T* __restrict__ temb, T* __restrict__ dtemb, int64_t B,
                                         float* __restrict__ dtemb32, f64x4_t* __restrict__ parts, int x, int y,
                                         int z, DaSub<kParts>& sub) {
  constexpr int kWaves = kDaWavesFor<kParts>;
  constexpr int kLeaves = 128 / (kParts * kWaves);   // per wave
  static_assert(kLeaves >= kDaMGroup && kLeaves % kDaMGroup == 0, "a wave runs whole leaf groups");
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int k0 = da_col0(x);
  const int64_t b0 = static_cast<int64_t>(y) * 16;
  const int rows_here = static_cast<int>((B - b0) < 16 ? (B - b0) : 16);
  const int br = r < rows_here ? r : rows_here - 1;

  const Buffer eb(d_emb + b0 * N, static_cast<uint32_t>(rows_here) * N * 4);
  const Buffer wbuf(W, static_cast<uint32_t>(N) * kD * sizeof(T));
  const uint32_t e_off = (static_cast<uint32_t>(br) * N + kDaSlots * g) * 4;
  const uint32_t w_off = (static_cast<uint32_t>(kDaSlots * g) * kD + k0 + 2 * r) * sizeof(T);
  const int leaf0 = (z * kWaves + wave) * kLeaves;

  PairTree<ilog2(kLeaves), f64x4_t> tree[2];
  static_for<0, kLeaves / kDaMGroup>([&](auto qc) {
    constexpr int q = decltype(qc)::value;
    const int t0 = leaf0 + kDaMGroup * q;
    auto load = [&](DaStep<T>& d, int st) {
      const uint32_t row = static_cast<uint32_t>(t0 + kDaSlots * 4 * st);   // + 128 g in the lane offset
      d.d = eb.u128(e_off, row * 4);
#pragma unroll
      for (int l = 0; l < kDaMGroup; ++l) d.w[l].load(wbuf, w_off, (row + l) * kD * sizeof(T));
    };
    DaStep<T> buf[kDaMAhead + 1];
#pragma unroll
    for (int st = 0; st < kDaMAhead; ++st) load(buf[st], st);
    f64x4_t acc[kDaMGroup][2];
#pragma unroll
    for (int l = 0; l < kDaMGroup; ++l) acc[l][0] = acc[l][1] = f64x4_t{0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int st = 0; st < kLeafSteps<N>; ++st) {
      if (st + kDaMAhead < kLeafSteps<N>) load(buf[(st + kDaMAhead) % (kDaMAhead + 1)], st + kDaMAhead);
      const DaStep<T>& cur = buf[st % (kDaMAhead + 1)];
      const uint32_t dv[4] = {cur.d.x, cur.d.y, cur.d.z, cur.d.w};
#pragma unroll
      for (int l = 0; l < kDaMGroup; ++l) {
        const double dd = static_cast<double>(__uint_as_float(dv[l]));
        acc[l][0] = mfma_f64(dd, static_cast<double>(cur.w[l].lo()), acc[l][0]);
        acc[l][1] = mfma_f64(dd, static_cast<double>(cur.w[l].hi()), acc[l][1]);
      }
    }
    static_for<0, kDaMGroup>([&](auto lc) {
      constexpr int l = decltype(lc)::value;
      tree[0].template push<kDaMGroup * q + l>(acc[l][0]);
      tree[1].template push<kDaMGroup * q + l>(acc[l][1]);
    });
  });
  constexpr int kTop = ilog2(kLeaves);
  if (wave > 0) {
    sub[wave - 1][0][lane] = tree[0].node[kTop];
    sub[wave - 1][1][lane] = tree[1].node[kTop];
  }
  __syncthreads();
  if (wave > 0) return;
  f64x4_t tot[2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    f64x4_t v[kWaves];
    v[0] = tree[n].node[kTop];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) v[w] = sub[w - 1][n][lane];
    tot[n] = pair_reduce(v);
  }
  if constexpr (kParts > 1) {
    // run z of block (x, y): its two tiles, lane-major
    const int64_t at = ((static_cast<int64_t>(y) * kDaBlocksX + x) * kParts + z) * 2;
#pragma unroll
    for (int n = 0; n < 2; ++n) parts[(at + n) * 64 + lane] = tot[n];
  } else {
    da_store<T, kAcc>(tot, temb, dtemb, dtemb32, b0, rows_here, k0, r, g);
  }
}

template <typename T, int N = kN, bool kAcc = false, int kParts = 1>
__global__ __launch_bounds__(64 * kDaMWaves) void da_mfma_kernel(const float* __restrict__ d_emb,
                                                                 const T* __restrict__ W,
                                                                 const T* __restrict__ temb,
                                                                 T* __restrict__ dtemb, int64_t B,
                                                                 float* __restrict__ dtemb32,
                                                                 f64x4_t* __restrict__ parts) {
  __shared__ DaSub<kParts> sub;
  da_block<T, N, kAcc, kParts>(d_emb, W, temb, dtemb, B, dtemb32, parts, blockIdx.x, blockIdx.y, blockIdx.z, sub);
}

// The split form: the da run blocks (ids [0, n_da), x fastest,
// then the sample row, then the run) and the dW tiles (row block fastest) in
// one grid of 4-wave blocks, so each fills the CUs the other leaves idle.
// n_da is a multiple of 8, so both keep their XCD placement.
template <typename T, int N, bool kAcc, int kParts>
__global__ __launch_bounds__(256) void proj_bwd_mid_kernel(const float* __restrict__ d_emb,
                                                           const T* __restrict__ a, const T* __restrict__ W,
                                                           T* __restrict__ dW, T* __restrict__ db, int64_t B,
                                                           f64x4_t* __restrict__ parts, float* __restrict__ dW32,
                                                           float* __restrict__ db32) {
  static_assert(kParts > 1 && kDaWavesFor<kParts> == 4 && kDwMWaves == 4, "both roles run 4-wave blocks");
  __shared__ DaSub<kParts> sub;
  const int rows = static_cast<int>((B + 15) / 16);
  const int n_da = kDaBlocksX * rows * kParts;
  const int id = blockIdx.x;
  if (id < n_da) {
    da_block<T, N, kAcc, kParts>(d_emb, W, nullptr, nullptr, B, nullptr, parts, id % kDaBlocksX,
                                 (id / kDaBlocksX) % rows, id / (kDaBlocksX * rows), sub);
  } else {
    const int t = id - n_da;
    dw_block<T, N, kAcc>(d_emb, a, dW, db, B, dW32, db32, t % (N / kDwMRows), t / (N / kDwMRows));
  }
}

// the split form's second launch: block (x, y) of 4 x 64 threads; thread
// (v, lane) adds component v (sample g + 4 v of the lane's tiles) of its
// kParts run subtrees pairwise in run order and writes that sample's dtemb
template <typename T, int kParts, bool kAcc>
__global__ __launch_bounds__(256) void da_parts_kernel(const f64x4_t* __restrict__ parts,
                                                       const T* __restrict__ temb, T* __restrict__ dtemb,
                                                       int64_t B, float* __restrict__ dtemb32) {
  const int lane = threadIdx.x & 63;
  const int v = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int k0 = da_col0(blockIdx.x);
  const int64_t b0 = static_cast<int64_t>(blockIdx.y) * 16;
  const int rows_here = static_cast<int>((B - b0) < 16 ? (B - b0) : 16);
  const int64_t blk = static_cast<int64_t>(blockIdx.y) * gridDim.x + blockIdx.x;
  const double* pd = reinterpret_cast<const double*>(parts);
  double tot[2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    double w[kParts];
#pragma unroll
    for (int q = 0; q < kParts; ++q) w[q] = pd[(((blk * kParts + q) * 2 + n) * 64 + lane) * 4 + v];
    tot[n] = pair_reduce(w);
  }
  const int sr = g + 4 * v;
  if (sr < rows_here) {
    const int64_t i = (b0 + sr) * kD + k0 + 2 * r;
    Pair<T> z;
    z.load(temb + i);
    const float d0 = static_cast<float>(tot[0]) * dsilu_f32(z.lo());
    const float d1 = static_cast<float>(tot[1]) * dsilu_f32(z.hi());
    Pair<T>::store(dtemb + i, d0, d1);
    if constexpr (kAcc) {
      if (dtemb32) *reinterpret_cast<float2*>(dtemb32 + i) = make_float2(d0, d1);
    }
  }
}

// runs per da block for B samples: 8 for one row of blocks (B <= 16), 4 up
// to four rows (B <= 64), 2 beyond (with the dW tiles in the same grid:
// backward -8 to -25 us at B = 72 ... 256, S = 1024; -106 us at B = 2048,
// S = 3) than one block over all 128 leaves (kParts = 1), the form those
// figures compare against.
int da_runs(int64_t B) {
  const int64_t by = (B + 15) / 16;
  return by == 1 ? 8 : by <= 4 ? 4 : 2;
}

// dW, db, da and dtemb on the matrix cores, a = SiLU(temb) already in `a`:
// the dW tiles, then one block over all 128 leaves per tile (kParts = 1); or
// the leaf runs and the dW tiles in one grid, then da_parts_kernel (parts:
// proj_bwd_da_parts_bytes(B) bytes).  fp32 storage with 8 runs keeps the
// two grids apart: its combined blocks hold more registers than the dW
// tiles alone and measured slower (B = 8: 103.6 -> 106.0 us backward).
template <typename T, int N, bool kAcc, int kParts>
hipError_t mfma_launch(const float* d_emb, const T* a, const T* W, const T* temb, T* dW, T* db, T* dtemb,
                       int64_t B, const AccOut& acc, f64x4_t* parts, hipStream_t s) {
  constexpr bool kCombined = kParts > 1 && !(sizeof(T) == 4 && kParts == 8);
  const unsigned rows = static_cast<unsigned>((B + 15) / 16);
  const dim3 dw_grid(N / kDwMRows, kD / (kDwMCols * kDwMWaves));
  if constexpr (kCombined) {
    const unsigned blocks = kDaBlocksX * rows * kParts + dw_grid.x * dw_grid.y;
    hipLaunchKernelGGL((proj_bwd_mid_kernel<T, N, kAcc, kParts>), dim3(blocks), dim3(256), 0, s, d_emb, a, W, dW,
                       db, B, parts, acc.dW, acc.db);
  } else {
    hipLaunchKernelGGL((dw_mfma_kernel<T, N, kAcc>), dw_grid, dim3(64 * kDwMWaves), 0, s, d_emb, a, dW, db, B,
                       acc.dW, acc.db);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    hipLaunchKernelGGL((da_mfma_kernel<T, N, kAcc, kParts>), dim3(kDaBlocksX, rows, kParts),
                       dim3(64 * kDaWavesFor<kParts>), 0, s, d_emb, W, temb, dtemb, B, acc.dtemb, parts);
  }
  if constexpr (kParts > 1) {
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    hipLaunchKernelGGL((da_parts_kernel<T, kParts, kAcc>), dim3(kDaBlocksX, rows), dim3(256), 0, s, parts, temb,
                       dtemb, B, acc.dtemb);
  }
  return hipGetLastError();
}

template <typename T, int N, bool kAcc>
hipError_t mfma_rows(const float* d_emb, const T* a, const T* W, const T* temb, T* dW, T* db, T* dtemb,
                     double* parts, int64_t B, const AccOut& acc, hipStream_t s) {
  f64x4_t* p = reinterpret_cast<f64x4_t*>(parts);
  switch (da_runs(B)) {
    case 8: return mfma_launch<T, N, kAcc, 8>(d_emb, a, W, temb, dW, db, dtemb, B, acc, p, s);
    case 4: return mfma_launch<T, N, kAcc, 4>(d_emb, a, W, temb, dW, db, dtemb, B, acc, p, s);
    default: return mfma_launch<T, N, kAcc, 2>(d_emb, a, W, temb, dW, db, dtemb, B, acc, p, s);
  }
}

// fp32 storage, B = NB <= 4: the da leaf-group blocks (blocks [0, 384))
// beside the matrix-core dW tiles (the rest, row block fastest) in one grid,
// as proj_bwd_small_kernel does for bf16; da_finish_kernel<NB, float> follows
template <int NB>
__global__ __launch_bounds__(kThreads) void proj_bwd_f32_small_kernel(const float* __restrict__ d_emb,
                                                                      const float* __restrict__ a,
                                                                      const float* __restrict__ W,
                                                                      float* __restrict__ dW, float* __restrict__ db,
                                                                      double* __restrict__ sub) {
  static_assert(kThreads == 64 * kDwMWaves && kDaLeafBlocks % 8 == 0, "one block shape; XCD placement kept");
  __shared__ __align__(16) double red[kDaGroupLeaves * NB * kDaQuadCols];
  if (blockIdx.x < kDaLeafBlocks) {
    da_leaf_group<NB, float>(d_emb, W, sub, blockIdx.x, red);
    return;
  }
  const int t = static_cast<int>(blockIdx.x) - kDaLeafBlocks;
  dw_block<float, kN, false>(d_emb, a, dW, db, NB, nullptr, nullptr, t % (kN / kDwMRows), t / (kN / kDwMRows));
}

}  // namespace

int proj_bwd_fused_max_batch() { return kBatchChunk; }
int proj_bwd_f32_max_batch() { return 4; }

namespace {

template <int NB, int N, bool kAcc>
hipError_t launch_small(const float* d_emb, const uint16_t* temb, const uint16_t* W, uint16_t* dW, uint16_t* db,
                        uint16_t* dtemb, double* sub, const AccOut& acc, hipStream_t s) {
  const dim3 grid(kDaLeafBlocks + kDwTiles<N>), block(kThreads);
  if constexpr (kAcc)
    hipLaunchKernelGGL((proj_bwd_small_acc_kernel<NB, N>), grid, block, 0, s, d_emb, temb, W, dW, db, sub, acc.dW,
                       acc.db);
  else
    hipLaunchKernelGGL((proj_bwd_small_kernel<NB, N>), grid, block, 0, s, d_emb, temb, W, dW, db, sub);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  hipLaunchKernelGGL((da_finish_kernel<NB, uint16_t, kAcc>), dim3(NB * kD / 64), dim3(64 * kFinishWaves), 0, s, sub,
                     temb, dtemb, acc.dtemb);
  return hipGetLastError();
}

template <int N, bool kAcc>
hipError_t proj_bwd_fused_rows(const float* d_emb, const uint16_t* temb, const uint16_t* W, uint16_t* dW,
                               uint16_t* db, uint16_t* dtemb, double* sub, int64_t B, const AccOut& acc,
                               hipStream_t s) {
  switch (B) {
    case 1: return launch_small<1, N, kAcc>(d_emb, temb, W, dW, db, dtemb, sub, acc, s);
    case 2: return launch_small<2, N, kAcc>(d_emb, temb, W, dW, db, dtemb, sub, acc, s);
    case 3: return launch_small<3, N, kAcc>(d_emb, temb, W, dW, db, dtemb, sub, acc, s);
    case 4: return launch_small<4, N, kAcc>(d_emb, temb, W, dW, db, dtemb, sub, acc, s);
    case 5: return launch_small<5, N, kAcc>(d_emb, temb, W, dW, db, dtemb, sub, acc, s);
    case 6: return launch_small<6, N, kAcc>(d_emb, temb, W, dW, db, dtemb, sub, acc, s);
    default: return hipErrorInvalidValue;
  }
}

bool any(const AccOut& acc) { return acc.dW || acc.db || acc.dtemb; }

}  // namespace

size_t proj_bwd_fused_sub_bytes(int64_t B) { return static_cast<size_t>(kDaGroups * B * kD * 8); }

size_t proj_bwd_da_parts_bytes(int64_t B) {
  const int runs = da_runs(B);
  return runs == 1 ? 0 : static_cast<size_t>((B + 15) / 16) * (kD / kDaMCols) * runs * 2 * 64 * sizeof(f64x4_t);
}

hipError_t launch_proj_bwd_fused(const float* d_emb, const uint16_t* temb, const uint16_t* W,
                                 uint16_t* dW, uint16_t* db, uint16_t* dtemb, double* sub, int64_t B, int64_t N,
                                 hipStream_t s, const AccOut& acc) {
  const bool a = any(acc);
  if (N == kN)
    return a ? proj_bwd_fused_rows<kN, true>(d_emb, temb, W, dW, db, dtemb, sub, B, acc, s)
             : proj_bwd_fused_rows<kN, false>(d_emb, temb, W, dW, db, dtemb, sub, B, acc, s);
  if (N == kN6)
    return a ? proj_bwd_fused_rows<kN6, true>(d_emb, temb, W, dW, db, dtemb, sub, B, acc, s)
             : proj_bwd_fused_rows<kN6, false>(d_emb, temb, W, dW, db, dtemb, sub, B, acc, s);
  return hipErrorInvalidValue;
}

hipError_t launch_proj_bwd_mfma(const float* d_emb, const uint16_t* a, const uint16_t* W, const uint16_t* temb,
                                uint16_t* dW, uint16_t* db, uint16_t* dtemb, double* parts, int64_t B, int64_t N,
                                hipStream_t s, const AccOut& acc) {
  const bool f = any(acc);
  if (N == kN)
    return f ? mfma_rows<uint16_t, kN, true>(d_emb, a, W, temb, dW, db, dtemb, parts, B, acc, s)
             : mfma_rows<uint16_t, kN, false>(d_emb, a, W, temb, dW, db, dtemb, parts, B, acc, s);
  if (N == kN6)
    return f ? mfma_rows<uint16_t, kN6, true>(d_emb, a, W, temb, dW, db, dtemb, parts, B, acc, s)
             : mfma_rows<uint16_t, kN6, false>(d_emb, a, W, temb, dW, db, dtemb, parts, B, acc, s);
  return hipErrorInvalidValue;
}

hipError_t launch_silu(const uint16_t* temb, uint16_t* a, int64_t n, hipStream_t s) {
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(silu_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, temb, a, n);
  return hipGetLastError();
}


namespace {

template <int NB>
hipError_t proj_f32_small(const float* d_emb, const float* a, const float* W, const float* temb, float* dW,
                          float* db, float* dtemb, double* sub, hipStream_t s) {
  const unsigned blocks = kDaLeafBlocks + (kN / kDwMRows) * (kD / (kDwMCols * kDwMWaves));
  hipLaunchKernelGGL(proj_bwd_f32_small_kernel<NB>, dim3(blocks), dim3(kThreads), 0, s, d_emb, a, W, dW, db, sub);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  hipLaunchKernelGGL((da_finish_kernel<NB, float>), dim3(NB * kD / 64), dim3(64 * kFinishWaves), 0, s, sub, temb, dtemb,
                     nullptr);
  return hipGetLastError();
}

}  // namespace

// fp32 storage: a = SiLU(temb) into `a` (unless a_ready), dW and db on the
// matrix cores for every B, da and dtemb on the vector units for B <= 4 and
// the matrix cores beyond (the same leaves and order either way)
hipError_t launch_proj_bwd_f32(const float* d_emb, const float* temb, const float* W, float* a, float* dW,
                               float* db, float* dtemb, double* sub, int64_t B, hipStream_t s, bool a_ready) {
  if (!a_ready)
    if (hipError_t e = launch_silu_f32(temb, a, B * kD, s); e != hipSuccess) return e;
  switch (B) {
    case 1: return proj_f32_small<1>(d_emb, a, W, temb, dW, db, dtemb, sub, s);
    case 2: return proj_f32_small<2>(d_emb, a, W, temb, dW, db, dtemb, sub, s);
    case 3: return proj_f32_small<3>(d_emb, a, W, temb, dW, db, dtemb, sub, s);
    case 4: return proj_f32_small<4>(d_emb, a, W, temb, dW, db, dtemb, sub, s);
    default: return mfma_rows<float, kN, false>(d_emb, a, W, temb, dW, db, dtemb, sub, B, AccOut{}, s);
  }
}

}  // namespace adaln
