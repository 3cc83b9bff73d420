// Fixed token-sum tree (RL-Kernel pull request 538: "What" -- fixed 32-way
// trees whose shape depends only on S -- and the review-thread fix of
// token_sum.cu -- 32-token tiles summed in ascending order with Neumaier
// compensation, sums and corrections folded level by level, one final add).
//
// Level 0 turns every 32-token tile of every sample into a pair (s, c).
// Level k >= 1 turns every run of 32 consecutive level-(k-1) nodes into one
// node: for each child in ascending order, one Neumaier step on the child's s,
// then the child's c is added to the node's c.  The root's s + c is the sum.
// Tiles restart at token 0 of each sample, so a sample's sum is the same bytes
// whatever the batch size or the sample's position in the batch.
//
// Level-0 pairs are stored in groups of 64 columns (pair_index): the 32
// children of a level-1 node are one contiguous run per group.
//
// token_level0_kernel: one thread per (sample, tile, column), for the
//   stand-alone token_tree_sum (the norm backward computes its own level 0).
// tree_fold_kernel: one block per (sample, 64-column group); its 4 waves
//   compute the level-1 nodes 4 at a time (one per wave); the first wave then
//   streams them through levels 2.. with per-level running nodes kept in
//   registers, which is the same arithmetic as building each level in turn.
//   Rows of blocks past the last sample (blockIdx.y >= B), when asked for,
//   compute a = SiLU(temb) (bf16 or fp32 storage) for the projection backward
//   that follows, so that pass needs no launch of its own.
#include "common.hpp"
#include "launch.hpp"

namespace adaln {

namespace {

constexpr int kFoldCols = kPairGroup;
constexpr int kFoldLanes = 4;

__global__ __launch_bounds__(256) void token_level0_kernel(const float* __restrict__ x,
                                                           float* __restrict__ part, int64_t S,
                                                           int64_t H, int64_t T0) {
  const int64_t col = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t tile = blockIdx.y;
  const int64_t b = blockIdx.z;
  if (col >= H) return;
  const int64_t s0 = tile * kTile;
  const int n = static_cast<int>((S - s0) < kTile ? (S - s0) : kTile);
  const float* xp = x + (b * S + s0) * H + col;
  float s = 0.0f, c = 0.0f;
  for (int i = 0; i < n; ++i) neumaier_add(s, c, xp[static_cast<int64_t>(i) * H]);
  const int64_t i = pair_index(b, (H + kPairGroup - 1) / kPairGroup, T0, tile, col);
  part[i] = s;
  part[i + kPairGroup] = c;
}

// Where the roots go: a dense [B, H] array, or up to three [B, D] views with
// one row stride (columns [0, D) to the first, [D, 2D) to the second, ...).
struct DenseOut {
  float* out;
  int64_t H;
  __device__ __forceinline__ float* at(int64_t b, int64_t col) const { return out + b * H + col; }
};
struct ViewOut {
  float* seg[3];
  int64_t ld;
  __device__ __forceinline__ float* at(int64_t b, int64_t col) const {
    const int64_t k = col / kD;
    return (k == 0 ? seg[0] : k == 1 ? seg[1] : seg[2]) + b * ld + (col - k * kD);
  }
};

// a = bf16(SiLU(temb)) for the 8 elements of chunk i (n = B * D elements in
// all, a multiple of 8): the same bits as silu_kernel
__device__ __forceinline__ void silu_chunk(const uint16_t* __restrict__ temb, uint16_t* __restrict__ act,
                                           int64_t i) {
  uint32_t redo;
  const uint4 v = silu8_fast(*reinterpret_cast<const uint4*>(temb + 8 * i), redo);
  *reinterpret_cast<uint4*>(act + 8 * i) = v;
  while (redo != 0) {
    const int e = __builtin_ctz(redo);
    redo &= redo - 1;
    act[8 * i + e] = silu_bf16_exact(bf16_to_f32(temb[8 * i + e]));
  }
}

// fp32 storage: a = silu_f32(temb) for the 4 elements of chunk i, as silu_f32_kernel
__device__ __forceinline__ void silu_chunk_f32(const float* __restrict__ temb, float* __restrict__ act, int64_t i) {
  const float4 t = *reinterpret_cast<const float4*>(temb + 4 * i);
  *reinterpret_cast<float4*>(act + 4 * i) = make_float4(silu_f32(t.x), silu_f32(t.y), silu_f32(t.z), silu_f32(t.w));
}

template <typename Out>
__global__ __launch_bounds__(kFoldCols * kFoldLanes) void tree_fold_kernel(
    const float* __restrict__ part, Out out, int64_t T0, int64_t H, int levels, int64_t B,
    const uint16_t* __restrict__ temb, uint16_t* __restrict__ act, const float* __restrict__ temb32,
    float* __restrict__ act32, int64_t n_chunks) {
  if (blockIdx.y >= B) {   // SiLU rows: one chunk (8 bf16 or 4 fp32 elements) per thread
    const int64_t i = (static_cast<int64_t>(blockIdx.y - B) * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n_chunks) {
      if (act32) silu_chunk_f32(temb32, act32, i);
      else silu_chunk(temb, act, i);
    }
    return;
  }
  __shared__ float lds_s[kFoldLanes][kFoldCols];
  __shared__ float lds_c[kFoldLanes][kFoldCols];
  // node lane = wave index; readfirstlane tells the compiler it is uniform,
  // so the buffer descriptors built from it live in SGPRs (no per-load loop)
  const int q = __builtin_amdgcn_readfirstlane(threadIdx.x / kFoldCols);
  const int cl = threadIdx.x % kFoldCols;
  const int64_t col = static_cast<int64_t>(blockIdx.x) * kFoldCols + cl;
  const bool ok = col < H;
  const int64_t b = blockIdx.y;
  // this column's tile t: s at ps[t * 128], c at ps[t * 128 + 64]
  const float* ps = part + pair_index(b, gridDim.x, T0, 0, col);

  if (levels == 0) {                                // one tile: s + c
    if (q == 0 && ok) *out.at(b, col) = ps[0] + ps[kPairGroup];
    return;
  }
  const int64_t T1 = (T0 + kTile - 1) / kTile;

  // running nodes of levels 2 .. levels (index 0 = level 2)
  float rs[kMaxFoldLevels - 1], rc[kMaxFoldLevels - 1];
  int rn[kMaxFoldLevels - 1];
#pragma unroll
  for (int l = 0; l < kMaxFoldLevels - 1; ++l) { rs[l] = 0.0f; rc[l] = 0.0f; rn[l] = 0; }
  const int top = levels - 2;                       // index of the root level (levels >= 2)

  // push a finished node into level (2 + start); cascades up through full nodes
  auto push = [&](int start, float s, float c) {
    bool active = true;
#pragma unroll
    for (int l = 0; l < kMaxFoldLevels - 1; ++l) {
      if (active && l >= start) {
        neumaier_add(rs[l], rc[l], s);
        rc[l] = rc[l] + c;
        rn[l] += 1;
        if (l == top || rn[l] < kTile) {
          active = false;
        } else {
          s = rs[l]; c = rc[l];
          rs[l] = 0.0f; rc[l] = 0.0f; rn[l] = 0;
        }
      }
    }
  };

  float root_s = 0.0f, root_c = 0.0f;
  for (int64_t n0 = 0; n0 < T1; n0 += kFoldLanes) {
    const int64_t node = n0 + q;                    // q is the wave: uniform per wave
    float s = 0.0f, c = 0.0f;
    if (node < T1) {
      const int64_t t0 = node * kTile;
      const int cnt = static_cast<int>((T0 - t0) < kTile ? (T0 - t0) : kTile);
      if (cnt == kTile) {
        // a full node: its 32 children are one contiguous 16 KB run; buffer
        // loads with the lane's column in a VGPR and the child in an SGPR
        // (lanes past H read the group's unused slots, never stored)
        const Buffer run(part + pair_index(b, gridDim.x, T0, t0, static_cast<int64_t>(blockIdx.x) * kFoldCols),
                         kTile * 2 * kPairGroup * 4);
        float vs[kTile], vc[kTile];
#pragma unroll
        for (int i = 0; i < kTile; ++i) {
          vs[i] = run.f32(cl * 4, i * 2 * kPairGroup * 4);
          vc[i] = run.f32(cl * 4, i * 2 * kPairGroup * 4 + kPairGroup * 4);
        }
#pragma unroll
        for (int i = 0; i < kTile; ++i) {
          neumaier_add(s, c, vs[i]);
          c = c + vc[i];
        }
      } else {
        for (int i = 0; i < cnt; ++i) {
          neumaier_add(s, c, ps[(t0 + i) * 2 * kPairGroup]);
          c = c + ps[(t0 + i) * 2 * kPairGroup + kPairGroup];
        }
      }
    }
    __syncthreads();
    lds_s[q][cl] = s;
    lds_c[q][cl] = c;
    __syncthreads();
    if (q == 0) {
      const int nn = static_cast<int>((T1 - n0) < kFoldLanes ? (T1 - n0) : kFoldLanes);
      for (int k = 0; k < nn; ++k) {
        if (levels == 1) { root_s = lds_s[k][cl]; root_c = lds_c[k][cl]; }
        else push(0, lds_s[k][cl], lds_c[k][cl]);
      }
    }
  }
  if (q != 0 || !ok) return;
  if (levels >= 2) {
    // flush partial nodes bottom-up
#pragma unroll
    for (int l = 0; l < kMaxFoldLevels - 2; ++l) {
      if (l < top && rn[l] > 0) {
        const float s = rs[l], c = rc[l];
        rs[l] = 0.0f; rc[l] = 0.0f; rn[l] = 0;
        push(l + 1, s, c);
      }
    }
#pragma unroll
    for (int l = 0; l < kMaxFoldLevels - 1; ++l)
      if (l == top) { root_s = rs[l]; root_c = rc[l]; }
  }
  *out.at(b, col) = root_s + root_c;
}

// with temb and act (or their fp32 forms): also a = SiLU(temb) over B * D
// elements in extra rows of blocks, unless they would take the grid past
// 65535 rows (*act_done says which)
template <typename Out>
hipError_t fold(const float* part, Out out, int64_t B, int64_t T0, int64_t H, hipStream_t s,
                const uint16_t* temb = nullptr, uint16_t* act = nullptr, bool* act_done = nullptr,
                const float* temb32 = nullptr, float* act32 = nullptr) {
  int levels = 0;
  for (int64_t n = T0; n > 1; n = (n + kTile - 1) / kTile) ++levels;
  if (levels > kMaxFoldLevels) return hipErrorInvalidValue;
  const int64_t gx = (H + kFoldCols - 1) / kFoldCols;
  constexpr int64_t kBlock = kFoldCols * kFoldLanes;
  int64_t n_chunks = 0, rows = 0;
  if ((temb && act) || (temb32 && act32)) {
    n_chunks = B * kD / (act32 ? 4 : 8);
    rows = (n_chunks + gx * kBlock - 1) / (gx * kBlock);
    if (B + rows > 65535) n_chunks = rows = 0;
  }
  if (act_done) *act_done = rows > 0;
  hipLaunchKernelGGL(tree_fold_kernel<Out>, dim3(static_cast<unsigned>(gx), static_cast<unsigned>(B + rows)),
                     dim3(kBlock), 0, s, part, out, T0, H, levels, B, temb, act, temb32, act32, n_chunks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_token_level0(const float* x, float* part, int64_t B, int64_t S, int64_t H,
                               hipStream_t s) {
  const int64_t T0 = (S + kTile - 1) / kTile;
  hipLaunchKernelGGL(token_level0_kernel,
                     dim3(static_cast<unsigned>((H + 255) / 256), static_cast<unsigned>(T0),
                          static_cast<unsigned>(B)),
                     dim3(256), 0, s, x, part, S, H, T0);
  return hipGetLastError();
}

hipError_t launch_tree_fold(const float* part, float* out, int64_t B, int64_t T0, int64_t H,
                            hipStream_t s, const uint16_t* temb, uint16_t* act, bool* act_done,
                            const float* temb32, float* act32) {
  return fold(part, DenseOut{out, H}, B, T0, H, s, temb, act, act_done, temb32, act32);
}

hipError_t launch_tree_fold_views(const float* part, float* d0, float* d1, float* d2, int64_t ld, int64_t B,
                                  int64_t T0, int64_t nseg, hipStream_t s) {
  return fold(part, ViewOut{{d0, d1, d2}, ld}, B, T0, nseg * kD, s);
}

}  // namespace adaln
