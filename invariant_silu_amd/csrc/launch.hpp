// Kernel launchers (internal).  Shapes and pointers are validated by the
// C-ABI layer before any of these is called; each returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace adaln {

hipError_t launch_silu(const uint16_t* temb, uint16_t* a, int64_t n, hipStream_t s);
hipError_t launch_fwd(const uint16_t* temb, const uint16_t* W, const uint16_t* bias,
                      const uint16_t* x, uint16_t* emb, uint16_t* out, float* mean, float* rstd,
                      int64_t B, int64_t S, float eps, hipStream_t s);
// the one-call forward's emb, mean, rstd without the modulation (a: B * D
// bf16, used when B > 4)
hipError_t launch_fwd_stats(const uint16_t* temb, const uint16_t* W, const uint16_t* bias, const uint16_t* x,
                            uint16_t* emb, float* mean, float* rstd, uint16_t* a, int64_t B, int64_t S, float eps,
                            hipStream_t s);
// projections: N = kN (final modulation) or kN6 (a block's 6-way modulation)
hipError_t launch_proj_fwd(const uint16_t* temb, const uint16_t* W, const uint16_t* bias,
                           uint16_t* emb, uint16_t* a, int64_t B, int64_t N, hipStream_t s);
hipError_t launch_norm_mod_fwd(const uint16_t* x, const uint16_t* emb, uint16_t* out,
                               float* mean, float* rstd, int64_t B, int64_t S, float eps,
                               hipStream_t s);
hipError_t launch_norm_mod_bwd(const uint16_t* g, const uint16_t* x, const float* mean,
                               const float* rstd, const uint16_t* emb, uint16_t* dx, float* part,
                               int64_t B, int64_t S, hipStream_t s, hipEvent_t ev_start = nullptr,
                               hipEvent_t ev_stop = nullptr, float* root = nullptr);
hipError_t launch_norm_mod_bwd_dx(const uint16_t* g, const uint16_t* x, const float* mean,
                                  const float* rstd, const uint16_t* emb, uint16_t* dx, int64_t B,
                                  int64_t S, hipStream_t s);
hipError_t launch_norm_mod_bwd_tiles(const uint16_t* g, const uint16_t* x, const float* mean,
                                     const float* rstd, float* part, int64_t B,
                                     int64_t S, hipStream_t s);
hipError_t launch_token_level0(const float* x, float* part, int64_t B,
                               int64_t S, int64_t H, hipStream_t s);
// with temb and act (bf16) or temb32 and act32 (fp32 storage): the same
// launch also writes act = SiLU(temb) ([B, D]; *act_done = false when it
// could not, B near the grid's limit)
hipError_t launch_tree_fold(const float* part, float* out, int64_t B,
                            int64_t T0, int64_t H, hipStream_t s, const uint16_t* temb = nullptr,
                            uint16_t* act = nullptr, bool* act_done = nullptr, const float* temb32 = nullptr,
                            float* act32 = nullptr);
// the same fold, roots of columns [k D, (k + 1) D) to view k (row stride ld), nseg views
hipError_t launch_tree_fold_views(const float* part, float* d0, float* d1, float* d2, int64_t ld, int64_t B,
                                  int64_t T0, int64_t nseg, hipStream_t s);
int proj_bwd_fused_max_batch();
// the same for the fp32-storage projection backward
int proj_bwd_f32_max_batch();
// bytes of fp64 da subtrees the B <= 4 path keeps between its two launches
size_t proj_bwd_fused_sub_bytes(int64_t B);
// B > 6 (bf16) or B > 4 (fp32 storage): the da run subtrees (0: none)
size_t proj_bwd_da_parts_bytes(int64_t B);
// Optional fp32 copies of the projection backward's bf16 outputs (the values
// rounded to bf16); any member may be NULL.
struct AccOut {
  float* dW = nullptr;
  float* db = nullptr;
  float* dtemb = nullptr;
};
hipError_t launch_proj_bwd_fused(const float* d_emb, const uint16_t* temb, const uint16_t* W,
                                 uint16_t* dW, uint16_t* db, uint16_t* dtemb, double* sub, int64_t B, int64_t N,
                                 hipStream_t s, const AccOut& acc = AccOut{});
// B > 6: dW, db, da and dtemb on the matrix cores from a = SiLU(temb);
// parts: proj_bwd_da_parts_bytes(B) bytes
hipError_t launch_proj_bwd_mfma(const float* d_emb, const uint16_t* a, const uint16_t* W, const uint16_t* temb,
                                uint16_t* dW, uint16_t* db, uint16_t* dtemb, double* parts, int64_t B, int64_t N,
                                hipStream_t s, const AccOut& acc = AccOut{});
// A block's norm site.  Its modulation as three [B, D] bf16 views with one
// row stride ld (elements, a multiple of 8); gate is used only with the
// residual add.
struct ModView {
  const uint16_t* shift;
  const uint16_t* scale;
  const uint16_t* gate;
  int64_t ld;
};
// residual != nullptr: h = bf16(residual + bf16(gate * x)) is stored and
// normalized; else x is normalized (h unused)
hipError_t launch_site_fwd(const uint16_t* x, const uint16_t* residual, ModView mv, uint16_t* h, uint16_t* out,
                           float* mean, float* rstd, int64_t B, int64_t S, float eps, hipStream_t s);
// g_h != nullptr: the residual form (d_residual, dx, pairs of 3D columns:
// shift | scale | gate); else the plain form (dx, pairs of 2D columns: shift |
// scale; the LayerNorm input is x, h and d_residual unused)
hipError_t launch_site_bwd(const uint16_t* g_out, const uint16_t* g_h, const uint16_t* x, const uint16_t* h,
                           const float* mean, const float* rstd, ModView mv, uint16_t* d_residual, uint16_t* dx,
                           float* part, int64_t B, int64_t S, hipStream_t s, float* r_shift = nullptr,
                           float* r_scale = nullptr, float* r_gate = nullptr, int64_t r_ld = 0);
// proj_out (3072 -> 64 per token) on the fp64 matrix cores.  Backward part:
// proj_out_chunks(T) x 64 x 3072 fp64 (the dWp chunk partials), part_db:
// proj_out_chunks(T) x 64 fp64
int64_t proj_out_chunks(int64_t T);
// latent from x with the final modulation computed on the fly (out is never
// stored): the same bytes as launch_proj_out_fwd on the modulated output
hipError_t launch_proj_out_fwd_fused(const uint16_t* x, const uint16_t* emb, const float* mean, const float* rstd,
                                     const uint16_t* W, const uint16_t* bias, uint16_t* latent, int64_t B, int64_t S,
                                     hipStream_t s);
hipError_t launch_proj_out_fwd(const uint16_t* out, const uint16_t* W, const uint16_t* bias, uint16_t* latent,
                               int64_t T, hipStream_t s);
hipError_t launch_proj_out_bwd(const uint16_t* d_lat, const uint16_t* out, const uint16_t* W, uint16_t* d_out,
                               uint16_t* dW, uint16_t* db, double* part, double* part_db, int64_t T, hipStream_t s);
// fp32 storage
hipError_t launch_silu_f32(const float* temb, float* a, int64_t n, hipStream_t s);
// B <= 4: the fp32-storage projection on the vector units (same bits as the matrix-core kernel)
hipError_t launch_proj_f32_small(const float* a, const float* W, const float* bias, float* emb, int64_t B,
                                 hipStream_t s);
hipError_t launch_proj_fwd_f32(const float* temb, float* a, const float* W, const float* bias, float* emb,
                               int64_t B, hipStream_t s);
hipError_t launch_norm_mod_fwd_f32(const float* x, const float* emb, float* out, float* mean, float* rstd,
                                   int64_t B, int64_t S, float eps, hipStream_t s);
hipError_t launch_norm_mod_bwd_f32(const float* g, const float* x, const float* mean, const float* rstd,
                                   const float* emb, float* dx, float* part, int64_t B, int64_t S,
                                   hipStream_t s, float* root = nullptr);
hipError_t launch_proj_bwd_f32(const float* d_emb, const float* temb, const float* W, float* a, float* dW,
                               float* db, float* dtemb, double* sub, int64_t B, hipStream_t s,
                               bool a_ready = false);   // a_ready: a = SiLU(temb) already in `a`
// sub: B <= 4, the da subtrees (proj_bwd_fused_sub_bytes); B > 4, the da run
// subtrees (proj_bwd_da_parts_bytes)
hipError_t launch_selftest_probe(const float* in, float* out, uint32_t* bits, int n,
                                 hipStream_t s);

}  // namespace adaln
