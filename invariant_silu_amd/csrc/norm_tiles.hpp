// Level 0 of the token tree for a LayerNorm + modulation backward, shared by
// the final modulation's backward (norm_bwd.hip) and a block's norm sites
// (site.hip): per (sample, 32-token tile, column) the Neumaier (s, c) of g
// (-> d_shift) and of g * n (-> d_scale), tokens in ascending order, n
// recomputed from the saved mean / rstd.  Layout of the blocks of a tile:
// kRowBlocks row blocks of 4 rows, kColBlocks tile blocks of 512 columns.
#pragma once

#include "common.hpp"

namespace adaln {

namespace {

constexpr int kThreads = 256;
constexpr int kLaneChunks = kChunks / 64;          // 6
constexpr int kRowBlocks = kTile / 4;              // 8 row blocks of 4 rows per tile
constexpr int kColPairs = kThreads;                // 256 column pairs per column block
constexpr int kColBlockCols = 2 * kColPairs;       // 512 columns
constexpr int kColBlocks = kD / kColBlockCols;     // 6
constexpr int kBlocksPerTile = kRowBlocks + kColBlocks;   // 14

// Level-0 pairs of one 32-token tile for 512 columns (2 per thread).  The
// tile's statistics are the same for the whole block (scalar loads, no LDS,
// no barrier).  A full tile takes the branch-free form: buffer loads (the
// lane's column offset in a VGPR, the row's in an SGPR, no per-load address
// arithmetic), and the memory counter lets the chains start on row 0 while
// later rows are in flight.  Only the last, ragged tile of a sample takes the
// guarded form.
// Pairs go to columns scale_col0 + col (g * n) and shift_col0 + col (g) of a
// pair buffer of `groups` 64-column groups.  A sample of one tile (S <= 32)
// has its roots here already: with root_scale / root_shift given, s + c (the
// fold's one add at that size) goes to root_scale[b * root_ld + col] and
// root_shift[b * root_ld + col] instead of the pairs.
template <bool kFull>
__device__ __forceinline__ void col_tile(const uint16_t* __restrict__ g, const uint16_t* __restrict__ x,
                                         const float* __restrict__ mean, const float* __restrict__ rstd,
                                         float* __restrict__ part, int64_t b, int64_t tile, int cb,
                                         int64_t S, int64_t T0, int rows, int64_t groups, int scale_col0,
                                         int shift_col0, float* __restrict__ root_scale,
                                         float* __restrict__ root_shift, int64_t root_ld) {
  const int col = cb * kColBlockCols + 2 * threadIdx.x;
  const int64_t row0 = b * S + tile * kTile;
  uint32_t gw[kTile], xw[kTile];
  if (kFull) {
    constexpr uint32_t kBytes = kTile * kD * 2;
    const Buffer gt(g + row0 * kD, kBytes), xt(x + row0 * kD, kBytes);
#pragma unroll
    for (int r = 0; r < kTile; ++r) {
      gw[r] = gt.u32(col * 2, r * kD * 2);
      xw[r] = xt.u32(col * 2, r * kD * 2);
    }
  } else {
#pragma unroll
    for (int r = 0; r < kTile; ++r) {
      if (r < rows) {
        const int64_t off = (row0 + r) * kD + col;
        gw[r] = *reinterpret_cast<const uint32_t*>(g + off);
        xw[r] = *reinterpret_cast<const uint32_t*>(x + off);
      }
    }
  }
  float sg0 = 0.0f, cg0 = 0.0f, sg1 = 0.0f, cg1 = 0.0f;
  float sn0 = 0.0f, cn0 = 0.0f, sn1 = 0.0f, cn1 = 0.0f;
#pragma unroll
  for (int r = 0; r < kTile; ++r) {
    if (kFull || r < rows) {
      const float mu = mean[row0 + r], rs = rstd[row0 + r];
      const float g0 = bf_lo(gw[r]), g1 = bf_hi(gw[r]);
      const float n0 = (bf_lo(xw[r]) - mu) * rs;
      const float n1 = (bf_hi(xw[r]) - mu) * rs;
      neumaier_add(sg0, cg0, g0);
      neumaier_add(sg1, cg1, g1);
      neumaier_add(sn0, cn0, g0 * n0);
      neumaier_add(sn1, cn1, g1 * n1);
    }
  }
  if (root_scale != nullptr) {
    st8(root_scale + b * root_ld + col, sn0 + cn0, sn1 + cn1);
    st8(root_shift + b * root_ld + col, sg0 + cg0, sg1 + cg1);
    return;
  }
  const int64_t i_scale = pair_index(b, groups, T0, tile, scale_col0 + col);
  const int64_t i_shift = pair_index(b, groups, T0, tile, shift_col0 + col);
  st8(part + i_scale, sn0, sn1);
  st8(part + i_scale + kPairGroup, cn0, cn1);
  st8(part + i_shift, sg0, sg1);
  st8(part + i_shift + kPairGroup, cg0, cg1);
}

// columns [0, D) of d_emb: d_scale (g * n); [D, 2D): d_shift (g)
__device__ __forceinline__ void col_pass(const uint16_t* __restrict__ g, const uint16_t* __restrict__ x,
                                         const float* __restrict__ mean, const float* __restrict__ rstd,
                                         float* __restrict__ part, int64_t b, int64_t tile, int cb,
                                         int64_t S, int64_t T0, int64_t groups = kN / kPairGroup,
                                         int scale_col0 = 0, int shift_col0 = kD, float* root_scale = nullptr,
                                         float* root_shift = nullptr, int64_t root_ld = 0) {
  const int64_t left = S - tile * kTile;
  if (left >= kTile)
    col_tile<true>(g, x, mean, rstd, part, b, tile, cb, S, T0, kTile, groups, scale_col0, shift_col0, root_scale,
                   root_shift, root_ld);
  else
    col_tile<false>(g, x, mean, rstd, part, b, tile, cb, S, T0, static_cast<int>(left), groups, scale_col0,
                    shift_col0, root_scale, root_shift, root_ld);
}

}  // namespace

}  // namespace adaln
