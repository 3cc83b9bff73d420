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
// projections: N = kN (final modulation) or kN6 (a block's 6-way modulation)
hipError_t launch_proj_fwd(const uint16_t* temb, const uint16_t* W, const uint16_t* bias,
                           uint16_t* emb, uint16_t* a, int64_t B, int64_t N, hipStream_t s);
hipError_t launch_norm_mod_fwd(const uint16_t* x, const uint16_t* emb, uint16_t* out,
                               float* mean, float* rstd, int64_t B, int64_t S, float eps,
                               hipStream_t s);
hipError_t launch_norm_mod_bwd(const uint16_t* g, const uint16_t* x, const float* mean,
                               const float* rstd, const uint16_t* emb, uint16_t* dx, float* part,
                               int64_t B, int64_t S, hipStream_t s,
                               hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);
hipError_t launch_norm_mod_bwd_dx(const uint16_t* g, const uint16_t* x, const float* mean,
                                  const float* rstd, const uint16_t* emb, uint16_t* dx, int64_t B,
                                  int64_t S, hipStream_t s, hipEvent_t ev_start = nullptr,
                                  hipEvent_t ev_stop = nullptr);
hipError_t launch_norm_mod_bwd_tiles(const uint16_t* g, const uint16_t* x, const float* mean,
                                     const float* rstd, float* part, int64_t B,
                                     int64_t S, hipStream_t s);
hipError_t launch_token_level0(const float* x, float* part, int64_t B,
                               int64_t S, int64_t H, hipStream_t s);
hipError_t launch_tree_fold(const float* part, float* out, int64_t B,
                            int64_t T0, int64_t H, hipStream_t s);
int proj_bwd_fused_max_batch();
hipError_t launch_proj_bwd_fused(const float* d_emb, const uint16_t* temb, const uint16_t* W,
                                 uint16_t* dW, uint16_t* db, uint16_t* dtemb, int64_t B, int64_t N,
                                 hipStream_t s, hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);
hipError_t launch_proj_bwd_dw(const float* d_emb, const uint16_t* a, uint16_t* dW, uint16_t* db,
                              int64_t B, int64_t N, hipStream_t s);
hipError_t launch_proj_bwd_da(const float* d_emb, const uint16_t* W, const uint16_t* temb,
                              uint16_t* dtemb, int64_t B, int64_t N, hipStream_t s);
// residual norm site (mod = shift | scale | gate); part: pairs of 3D columns
hipError_t launch_residual_fwd(const uint16_t* x, const uint16_t* residual, const uint16_t* mod, uint16_t* h,
                               uint16_t* out, float* mean, float* rstd, int64_t B, int64_t S, float eps,
                               hipStream_t s);
hipError_t launch_residual_bwd(const uint16_t* g_out, const uint16_t* g_h, const uint16_t* x, const uint16_t* h,
                               const float* mean, const float* rstd, const uint16_t* mod, uint16_t* d_residual,
                               uint16_t* dx, float* part, int64_t B, int64_t S, hipStream_t s,
                               hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);
// proj_out (3072 -> 64 per token).  Forward part: 4 x T x 64 fp32 (the K
// quarters' partial sums); backward part: proj_out_chunks(T) x 64 x 3072 fp32,
// part_db: proj_out_chunks(T) x 64 fp64
int64_t proj_out_chunks(int64_t T);
hipError_t launch_proj_out_fwd(const uint16_t* out, const uint16_t* W, const uint16_t* bias, uint16_t* latent,
                               float* part, int64_t T, hipStream_t s);
hipError_t launch_proj_out_bwd(const uint16_t* d_lat, const uint16_t* out, const uint16_t* W, uint16_t* d_out,
                               uint16_t* dW, uint16_t* db, float* part, double* part_db, int64_t T, hipStream_t s,
                               hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);
// fp32 storage
hipError_t launch_silu_f32(const float* temb, float* a, int64_t n, hipStream_t s);
hipError_t launch_proj_fwd_f32(const float* temb, float* a, const float* W, const float* bias, float* emb,
                               int64_t B, hipStream_t s);
hipError_t launch_norm_mod_fwd_f32(const float* x, const float* emb, float* out, float* mean, float* rstd,
                                   int64_t B, int64_t S, float eps, hipStream_t s);
hipError_t launch_norm_mod_bwd_f32(const float* g, const float* x, const float* mean, const float* rstd,
                                   const float* emb, float* dx, float* part, int64_t B, int64_t S,
                                   hipStream_t s, hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);
hipError_t launch_proj_bwd_f32(const float* d_emb, const float* temb, const float* W, float* a, float* dW,
                               float* db, float* dtemb, int64_t B, hipStream_t s);
hipError_t launch_selftest_probe(const float* in, float* out, uint32_t* bits, int n,
                                 hipStream_t s);

}  // namespace adaln
