/*
 * adaln.h -- C ABI of the batch-invariant AdaLN final modulation for MI355X (gfx950).
 *
 * The operation is Qwen-Image's final image-stream modulation `norm_out`
 * (RL-Kernel pull request 538, section "What"):
 *
 *     scale, shift = (SiLU(temb) @ W^T + b).chunk(2)        3072 -> 6144, scale first
 *     out          = LayerNorm(x, eps, no affine) * (1 + scale) + shift
 *
 * at the autocast rounding points of miles_diffusion pull request 108
 * ("Fused-norm rounding points"): fp32 LayerNorm, (1 + scale) rounded once to
 * bf16, fp32 modulation, one bf16 rounding of the output.  The backward gives
 * dx, d_scale / d_shift as fp32 token sums over a fixed 32-token compensated
 * tree whose shape depends only on S (pull request 538, review thread on
 * token_sum.cu), and dW, db, dtemb through the projection.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - bf16 tensors are passed as `adaln_bf16` (uint16_t bit patterns); fp32 as
 *   float; the only fp64 data lives in workspaces.
 * - Every pointer is a DEVICE pointer on the current HIP device and must be
 *   16-byte aligned.  Tensors are dense, row-major and contiguous.
 * - The caller owns every buffer, workspaces included.  Apart from
 *   adaln_selftest the library allocates no device memory, keeps no per-call
 *   state and never synchronizes: the work is enqueued on `stream` (a
 *   hipStream_t; NULL means the null stream).
 * - Outputs are always written in full (never aliases or views of an input)
 *   and must not overlap any input, any other output or the workspace.
 * - Fixed widths: D = K = 3072 and N = 2 * D = 6144.  B >= 1, S >= 1.
 * - Every check runs before anything is enqueued; a non-zero status means
 *   nothing was launched (except ADALN_ERR_LAUNCH).
 * - Determinism: identical inputs give identical bytes; every per-sample /
 *   per-row output (emb, out, mean, rstd, dx, d_emb, dtemb) has the same bytes
 *   for any batch size B and any position of the sample in the batch.  dW and
 *   db are batch sums in ascending sample order; trailing all-zero gradient
 *   samples leave them byte-identical.
 * - Unsupported devices (anything but gfx950) fail closed with
 *   ADALN_ERR_DEVICE (pull request 538: other platforms fail closed); so does
 *   a stream that belongs to another device than the current one.
 */
#ifndef ADALN_H
#define ADALN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t adaln_bf16;

#define ADALN_ABI_VERSION 17

enum adaln_status {
  ADALN_OK = 0,
  ADALN_ERR_NULL = -1,       /* a required pointer is NULL                        */
  ADALN_ERR_SHAPE = -2,      /* B, S, H out of range or D/K/N not 3072/3072/6144  */
  ADALN_ERR_ALIGN = -3,      /* a pointer is not 16-byte aligned                  */
  ADALN_ERR_DEVICE = -4,     /* current device not gfx950, no HIP device, or the
                                stream is on another device                       */
  ADALN_ERR_WORKSPACE = -5,  /* ws_bytes < adaln_workspace_bytes(...)             */
  ADALN_ERR_OVERLAP = -6,    /* an output overlaps an input, output or workspace  */
  ADALN_ERR_LAUNCH = -7,     /* a kernel launch failed (hipGetLastError)          */
  ADALN_ERR_SCRATCH = -8     /* the problem needs more than the no-alloc scratch   */
};

/* Size of the fixed device array behind adaln_norm_mod_bwd_noalloc (per GPU). */
#define ADALN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

enum adaln_op {
  ADALN_OP_PROJ_FWD = 1,
  ADALN_OP_NORM_MOD_BWD = 2,
  ADALN_OP_PROJ_BWD = 3,
  ADALN_OP_TOKEN_TREE_SUM = 4,
  ADALN_OP_BWD = 5,
  ADALN_OP_BWD_F32 = 6,
  ADALN_OP_RESIDUAL_BWD = 7,
  ADALN_OP_PROJ_OUT_BWD = 8,
  ADALN_OP_PROJ_OUT_FWD = 9,
  ADALN_OP_FWD_PROJ_OUT = 10
};

/* Workspace bytes an entry point needs (0 for an unknown op or bad sizes).
 * The pages' operator allocates its scratch itself (pull request 538, review
 * thread on det_linear.cu: checks that run after its torch::empty
 * allocations); this library leaves every allocation to the caller, who sizes
 * each entry point's scratch with this call.
 *   PROJ_FWD:       H = K (3072), S ignored.  B*K*2 (SiLU activations, used when
 *                   B > 4).
 *   NORM_MOD_BWD:   H = D (3072).  B * ceil(S/32) * 2D * 8 bytes (level-0 pairs).
 *   PROJ_BWD:       H = K (3072), S ignored.  B <= 6: 32*B*K*8 (the fp64 da
 *                   subtrees, 32 per sample and column); B > 6: B*K*2 (SiLU
 *                   activations), then the fp64 subtrees of the da leaf runs,
 *                   ceil(B/16) * 96 * R * 2 * 64 * 32 bytes with R = 8 runs for
 *                   B <= 16, 4 for B <= 64 and 2 beyond.
 *   TOKEN_TREE_SUM: B * ceil(S/32) * ceil(H/64) * 64 * 8 bytes (level-0 pairs).
 *   BWD:            H = D (3072).  NORM_MOD_BWD + PROJ_BWD, in that order.
 *   BWD_F32:        H = D (3072).  NORM_MOD_BWD + B*K*4 (fp32 activations),
 *                   then for B <= 4 32*B*K*8 (the fp64 da subtrees), for
 *                   B > 4 the da runs' subtrees as for PROJ_BWD.
 *   (Every part is rounded up to a multiple of 256 bytes.)
 *   RESIDUAL_BWD:   H = D (3072).  B * ceil(S/32) * 3D * 8 bytes (level-0 pairs).
 *   PROJ_OUT_BWD:   H = K (3072), T = B * S tokens (T <= 65535 * 512; only the
 *                   product is checked, so B = 1, S = T is fine).
 *                   C * 64 * K * 8 bytes (fp64 dWp partials) + C * 64 * 8
 *                   (dbp partials), C = ceil(T / 512).
 *   PROJ_OUT_FWD:   H = K (3072), T = B * S tokens.  256 bytes (nothing is
 *                   kept there; the parts of each sum meet on chip).
 *   FWD_PROJ_OUT:   H = D (3072), B and S within the modulation's limits.
 *                   PROJ_FWD + PROJ_OUT_FWD (T = B * S), in that order.
 * Each region is padded to 256 bytes. */
size_t adaln_workspace_bytes(int op, int64_t B, int64_t S, int64_t H);

/* Projection forward (pull request 538, "What": SiLU(temb) @ W^T + b, chunk(2)).
 *   temb [B, K] bf16 (in), W [N, K] bf16 (in, row-major), bias [N] bf16 (in),
 *   emb  [B, N] bf16 (out).  K = 3072; N = 6144, the final modulation, emb =
 *   (scale | shift), or N = 18432, a block's 6-way modulation (pull request
 *   537, named in 538's "What" and "Prior art & reuse decision": the six
 *   chunks of temb.chunk(6)), emb = (shift1 | scale1 | gate1 | shift2 | scale2 |
 *   gate2) for the block's two norm sites.  Any other N: ADALN_ERR_SHAPE.
 *   emb = bf16(fp32(sum_k a_k W_jk) + bias_j), a = bf16(fp32(SiLU(temb))),
 *   SiLU evaluated in float64.  The sum is one fixed tree whatever B: 64 leaves
 *   of 48 consecutive k, each accumulated from +0 by fp64 fused multiply-adds
 *   (exact products, one rounding per add) in the order k = 48 l + 12 g + s
 *   (s = 0..11 outer, g = 0..3 inner), the leaves then added pairwise in index
 *   order.  B <= 4 runs it on the vector units, B > 4 on the fp64 matrix cores
 *   (a chain of fused multiply-adds in k order): the same bits either way.
 *   ws: adaln_workspace_bytes(ADALN_OP_PROJ_FWD, B, 1, K) bytes, 16-byte
 *   aligned; holds a when B > 4. */
int adaln_proj_fwd(const adaln_bf16* temb, const adaln_bf16* W, const adaln_bf16* bias,
                   adaln_bf16* emb, void* ws, size_t ws_bytes, int64_t B, int64_t K, int64_t N,
                   void* stream);

/* LayerNorm + modulation forward (pull request 538, "What"; rounding points of
 * miles_diffusion pull request 108).
 *   x [B, S, D] bf16 (in), emb [B, 2D] bf16 (in, from adaln_proj_fwd),
 *   out [B, S, D] bf16 (out), mean [B, S] fp32 (out), rstd [B, S] fp32 (out).
 *   mean = fp32(sum x)/D, var = fp32(sum (x-mean)^2)/D (biased), rstd =
 *   1/sqrt(var + eps) correctly rounded, n = (x - mean) * rstd,
 *   out = bf16((n * bf16(1 + scale)) + shift).  Pass eps = 1e-6f. */
int adaln_norm_mod_fwd(const adaln_bf16* x, const adaln_bf16* emb, adaln_bf16* out, float* mean,
                       float* rstd, int64_t B, int64_t S, int64_t D, float eps, void* stream);

/* LayerNorm + modulation backward with the token-sum tree (pull request 538,
 * "What" and the token_sum.cu review fix).
 *   gout [B, S, D] bf16 (in, upstream gradient), x [B, S, D] bf16 (in),
 *   mean, rstd [B, S] fp32 (in, from adaln_norm_mod_fwd), emb [B, 2D] bf16 (in),
 *   dx [B, S, D] bf16 (out), d_emb [B, 2D] fp32 (out) = (d_scale | d_shift).
 *   gy = g * m, dx = bf16(rstd * ((gy - mean(gy)) - n * mean(gy * n)));
 *   d_scale = tree_S(g * n), d_shift = tree_S(g), kept in fp32 (the gradient
 *   passes straight through the bf16 rounding of 1 + scale). */
int adaln_norm_mod_bwd(const adaln_bf16* gout, const adaln_bf16* x, const float* mean,
                       const float* rstd, const adaln_bf16* emb, adaln_bf16* dx, float* d_emb,
                       void* ws, size_t ws_bytes, int64_t B, int64_t S, int64_t D, void* stream);

/* The three stages of adaln_norm_mod_bwd, exported separately (each can then be
 * timed, overlapped or reused on its own).
 *
 * adaln_norm_mod_bwd_dx: dx only (arguments as in adaln_norm_mod_bwd).
 * adaln_norm_mod_bwd_tiles: level 0 of the token tree over H = 2D columns
 *   (columns [0, D) of g * n for d_scale, [D, 2D) of g for d_shift).  `part`
 *   receives fp32 [B, ceil(H/64), T0, 2, 64] with T0 = ceil(S/32): for sample b,
 *   64-column group k and tile t, the 64 sums s of columns 64k .. 64k+63, then
 *   their 64 corrections c; part_bytes must be at least
 *   adaln_workspace_bytes(ADALN_OP_NORM_MOD_BWD, B, S, D).
 * token_tree_fold: levels >= 1 of the tree from such pairs: `part` as written by
 *   adaln_norm_mod_bwd_tiles (H = 2D) or by level 0 of token_tree_sum (any H, in
 *   the same layout), T0 tiles per sample; out [B, H] fp32.  part_bytes is the
 *   size of the caller's pair buffer: it must hold B * ceil(H/64) * T0 * 128
 *   floats (rounded up to 256 bytes), else ADALN_ERR_WORKSPACE and nothing is
 *   read. */
int adaln_norm_mod_bwd_dx(const adaln_bf16* gout, const adaln_bf16* x, const float* mean,
                          const float* rstd, const adaln_bf16* emb, adaln_bf16* dx, int64_t B,
                          int64_t S, int64_t D, void* stream);
int adaln_norm_mod_bwd_tiles(const adaln_bf16* gout, const adaln_bf16* x, const float* mean,
                             const float* rstd, void* part, size_t part_bytes, int64_t B, int64_t S,
                             int64_t D, void* stream);
int token_tree_fold(const void* part, size_t part_bytes, float* out, int64_t B, int64_t T0, int64_t H,
                    void* stream);

/* adaln_norm_mod_bwd_level0: the first launch of adaln_norm_mod_bwd alone --
 * dx and the level-0 pairs of the token tree in one pass over g and x (the
 * same kernel, the same bytes as adaln_norm_mod_bwd_dx and
 * adaln_norm_mod_bwd_tiles together); token_tree_fold on `part` then gives
 * d_emb.  Arguments as in adaln_norm_mod_bwd_dx and _tiles.  ev_start /
 * ev_stop: optional caller-owned hipEvent_t handles (NULL for none) that the
 * kernel's dispatch records when it starts and ends -- a timing of this
 * kernel alone with no event packet in the stream.  The library keeps no
 * state for them. */
int adaln_norm_mod_bwd_level0(const adaln_bf16* gout, const adaln_bf16* x, const float* mean, const float* rstd,
                              const adaln_bf16* emb, adaln_bf16* dx, void* part, size_t part_bytes, int64_t B,
                              int64_t S, int64_t D, void* ev_start, void* ev_stop, void* stream);

/* Projection backward (pull request 538, "What": projection backward; review
 * thread: silu'(z) = sigmoid(z) * (1 + z * (1 - sigmoid(z)))).
 *   d_emb [B, N] fp32 (in), temb [B, K] bf16 (in), W [N, K] bf16 (in),
 *   dW [N, K] bf16 (out), db [N] bf16 (out), dtemb [B, K] bf16 (out);
 *   K = 3072, N = 6144 or 18432 as for adaln_proj_fwd.
 *   dW = bf16(fp32(sum_b d_emb_bj * a_bk)), db = bf16(fp32(sum_b d_emb_bj)),
 *   dtemb = bf16(fp32(sum_j d_emb_bj * W_jk) * silu'(temb)).  Every product is
 *   exact (an fp64 fused multiply-add) and the sums run in fp64 in orders that
 *   do not depend on B: dW and db over samples ascending from +0; da as 128
 *   leaves (leaf t: rows t, t + 128, ..., ascending, from +0; N / 128 rows
 *   each) added pairwise in leaf order.  B <= 6 runs on the vector units, B > 6 on the fp64 matrix
 *   cores: the same bits either way.
 *   ws: adaln_workspace_bytes(ADALN_OP_PROJ_BWD, B, 1, K) bytes (B <= 6: the
 *   sums of leaves 4g .. 4g + 3 for g = 0 .. 31, added pairwise by a second
 *   launch; B > 6: a, then the subtrees of aligned runs of the 128 leaves --
 *   8 runs of 16 for B <= 16, 4 runs of 32 up to 64, 2 of 64 beyond -- added
 *   pairwise by a second launch: the same tree, spread over more blocks). */
int adaln_proj_bwd(const float* d_emb, const adaln_bf16* temb, const adaln_bf16* W,
                   adaln_bf16* dW, adaln_bf16* db, adaln_bf16* dtemb, void* ws, size_t ws_bytes,
                   int64_t B, int64_t K, int64_t N, void* stream);

/* adaln_proj_bwd that also returns the fp32 values its bf16 outputs are
 * rounded from (pull request 538, "What": dW, db and dtemb accumulate in
 * fp32 before their single bf16 rounding; these are those fp32 results):
 *   dW_f32 [N, K] = fp32(sum_b d_emb_bj * a_bk), db_f32 [N] = fp32(sum_b d_emb_bj),
 *   dtemb_f32 [B, K] = fp32(sum_j d_emb_bj * W_jk) * silu'(temb) (one fp32 product),
 * all fp32, 16-byte aligned.  Each may be NULL (not written); with all three
 * NULL this is adaln_proj_bwd.  The bf16 outputs are the same bytes as
 * adaln_proj_bwd's and are bf16(the fp32 outputs) exactly.  The fp32 outputs
 * must not overlap any input, output or the workspace (ADALN_ERR_OVERLAP).
 * Same shapes, workspace and errors as adaln_proj_bwd. */
int adaln_proj_bwd_acc(const float* d_emb, const adaln_bf16* temb, const adaln_bf16* W,
                       adaln_bf16* dW, adaln_bf16* db, adaln_bf16* dtemb, float* dW_f32, float* db_f32,
                       float* dtemb_f32, void* ws, size_t ws_bytes, int64_t B, int64_t K, int64_t N,
                       void* stream);

/* Token-sum tree (pull request 538: fixed 32-way tree that depends only on S;
 * review thread: 32-token Neumaier tiles folded level by level, one final add).
 *   x [B, S, H] fp32 (in), out [B, H] fp32 (out).  Any H >= 1.  S = 1 still
 *   computes (out is a fresh buffer, never a view of x). */
int token_tree_sum(const float* x, float* out, void* ws, size_t ws_bytes, int64_t B, int64_t S,
                   int64_t H, void* stream);

/* Device check plus strict-math probe (pull request 538, "Results (H100
 * sm90 ...)": the build's strict-math probe must report true; its review
 * thread asks that the probe's verdict be cached on failure as well as on
 * success, so a refused device is not probed again on every call):
 * correctly rounded sqrt and divide, no contraction into fused multiply-add,
 * bf16 round-to-nearest-even, run synchronously on the current device.  It is the one entry point that
 * allocates: 80 KB of device memory for the probe, freed before it returns.
 * The verdict is cached per device, both ways.  Returns ADALN_OK,
 * ADALN_ERR_DEVICE, or a positive count of failed probe values. */
int adaln_selftest(void);

/* One-call forward: adaln_proj_fwd then adaln_norm_mod_fwd, same results bit
 * for bit.  B <= 4 with x of at most 32 MiB: the projection's pass over W and
 * the LayerNorm statistics pass over x run side by side (one launch), then the
 * modulation, which re-reads x from the caches; B <= 4 with a larger x: the
 * projection, then statistics and modulation in one pass over x.  B > 4: the
 * SiLU once (into the first B * 3072 elements of `out`, which the modulation
 * overwrites afterwards), the projection, then statistics and modulation in
 * one pass over x.
 *   temb, W, bias, x in; emb, out, mean, rstd out (layouts as above). */
int adaln_fwd(const adaln_bf16* temb, const adaln_bf16* W, const adaln_bf16* bias, const adaln_bf16* x,
              adaln_bf16* emb, adaln_bf16* out, float* mean, float* rstd, int64_t B, int64_t S,
              int64_t D, float eps, void* stream);

/* One-call backward: adaln_norm_mod_bwd then adaln_proj_bwd (same launches,
 * same results bit for bit) with one workspace and one validation pass.
 * ws: adaln_workspace_bytes(ADALN_OP_BWD, B, S, D) bytes. */
int adaln_bwd(const adaln_bf16* gout, const adaln_bf16* x, const float* mean, const float* rstd,
              const adaln_bf16* emb, const adaln_bf16* temb, const adaln_bf16* W, adaln_bf16* dx,
              float* d_emb, adaln_bf16* dW, adaln_bf16* db, adaln_bf16* dtemb, void* ws, size_t ws_bytes,
              int64_t B, int64_t S, int64_t D, void* stream);

/* FP32 storage (the FP32 execution RL-Kernel pull request 538 measures beside
 * BF16): every tensor fp32, the same method without the bf16 rounding points --
 * a = fp32(SiLU(temb)), emb = fp32(sum a W) + b, m = 1 + scale in fp32,
 * out = (n * m) + shift, dx, dtemb, dW, db stored in fp32 -- and the same
 * summation orders as with bf16 storage.  Layouts as above with fp32 elements;
 * mean, rstd, d_emb as above.  The projection and dW run on the fp64 matrix
 * cores for every B, da on the vector units for B <= 4 and the matrix cores
 * beyond (the same order, the same bits).
 * adaln_fwd_f32 uses the first B * 3072 elements of `out` as scratch before
 * writing it.  adaln_bwd_f32: ws = adaln_workspace_bytes(ADALN_OP_BWD_F32,
 * B, S, D) bytes. */
int adaln_fwd_f32(const float* temb, const float* W, const float* bias, const float* x, float* emb, float* out,
                  float* mean, float* rstd, int64_t B, int64_t S, int64_t D, float eps, void* stream);
int adaln_bwd_f32(const float* gout, const float* x, const float* mean, const float* rstd, const float* emb,
                  const float* temb, const float* W, float* dx, float* d_emb, float* dW, float* db, float* dtemb,
                  void* ws, size_t ws_bytes, int64_t B, int64_t S, int64_t D, void* stream);

/* Residual norm site of a transformer block (ScaleResidualLayerNormScaleShift:
 * miles_diffusion pull request 108 names it beside LayerNormScaleShift with the
 * same autocast rounding points; its formula is the reading below).
 *   x, residual [B, S, D] bf16 (in), mod [B, 3D] bf16 (in) = (shift | scale |
 *   gate), h [B, S, D] bf16 (out), out [B, S, D] bf16 (out), mean, rstd [B, S]
 *   fp32 (out):
 *   h = bf16(residual + bf16(gate * x)),  out = bf16((n * bf16(1 + scale)) + shift),
 *   n = LayerNorm(h) as in adaln_norm_mod_fwd.
 * Backward, from g_out = dL/dout and g_h = dL/dh (bf16 [B, S, D], in):
 *   dh = bf16(bf16(rstd * ((gy - alpha) - n * beta)) + g_h), gy = g_out * m;
 *   d_residual = dh, dx = bf16(dh * gate) (bf16 [B, S, D], out);
 *   d_mod [B, 3D] fp32 (out) = (sum_S g_out | sum_S g_out * n | sum_S dh * x),
 *   each the 32-token Neumaier tree of token_tree_sum.
 *   ws: adaln_workspace_bytes(ADALN_OP_RESIDUAL_BWD, B, S, D) bytes.
 * Per-sample outputs are the same bytes whatever B.  These are adaln_site_fwd /
 * adaln_site_bwd with the views mod, mod + D, mod + 2D (and d_mod likewise),
 * row stride 3D. */
int adaln_residual_fwd(const adaln_bf16* x, const adaln_bf16* residual, const adaln_bf16* mod, adaln_bf16* h,
                       adaln_bf16* out, float* mean, float* rstd, int64_t B, int64_t S, int64_t D, float eps,
                       void* stream);
int adaln_residual_bwd(const adaln_bf16* g_out, const adaln_bf16* g_h, const adaln_bf16* x, const adaln_bf16* h,
                       const float* mean, const float* rstd, const adaln_bf16* mod, adaln_bf16* d_residual,
                       adaln_bf16* dx, float* d_mod, void* ws, size_t ws_bytes, int64_t B, int64_t S, int64_t D,
                       void* stream);

/* A block's norm site with its modulation as views (pull request 108: the
 * LayerNormScaleShift and ScaleResidualLayerNormScaleShift sites; pull request
 * 538, "Prior art & reuse decision": scale / shift as views of the 6-way
 * modulation temb.chunk(6)), so each site reads its chunks straight out of
 * adaln_proj_fwd's N = 18432 output and writes its gradients into the 6-way
 * d_emb.  shift, scale, gate: [B, D] bf16 views, row b at view + b * mod_ld;
 * d_shift, d_scale, d_gate: [B, D] fp32 views, row stride dmod_ld.  Strides
 * are elements, >= D and multiples of 8; every pointer 16-byte aligned.  Views
 * of one tensor may interleave (their rows must not share bytes).
 * adaln_site_fwd: residual == NULL: the plain site (LayerNormScaleShift), out =
 *   bf16((LayerNorm(x) * bf16(1 + scale)) + shift), gate and h unused (may be
 *   NULL); residual != NULL: adaln_residual_fwd's site, h written.
 * adaln_site_bwd: g_h == NULL: the plain site's backward from g_out: dx =
 *   bf16(rstd * ((gy - alpha) - n * beta)) with n from x, d_shift and d_scale;
 *   h, gate, d_residual, d_gate unused (may be NULL).  g_h != NULL:
 *   adaln_residual_bwd's outputs (h = the forward's h).
 *   ws: adaln_workspace_bytes(ADALN_OP_RESIDUAL_BWD, B, S, D) bytes (either form).
 * The plain site gives the same bytes as adaln_norm_mod_fwd / _bwd with emb =
 * (scale | shift).  In a block: site 1 takes shift1, scale1 (and, fused with
 * the previous block's residual add, that block's gate2); site 2 takes gate1,
 * shift2, scale2. */
int adaln_site_fwd(const adaln_bf16* x, const adaln_bf16* residual, const adaln_bf16* shift, const adaln_bf16* scale,
                   const adaln_bf16* gate, int64_t mod_ld, adaln_bf16* h, adaln_bf16* out, float* mean, float* rstd,
                   int64_t B, int64_t S, int64_t D, float eps, void* stream);
int adaln_site_bwd(const adaln_bf16* g_out, const adaln_bf16* g_h, const adaln_bf16* x, const adaln_bf16* h,
                   const float* mean, const float* rstd, const adaln_bf16* scale, const adaln_bf16* gate,
                   int64_t mod_ld, adaln_bf16* d_residual, adaln_bf16* dx, float* d_shift, float* d_scale,
                   float* d_gate, int64_t dmod_ld, void* ws, size_t ws_bytes, int64_t B, int64_t S, int64_t D,
                   void* stream);

/* proj_out, the 3072 -> 64 projection after the final modulation (pull
 * request 538, "What" and "Scope / Known limitations": a separate GEMM that
 * takes the modulated output; pull request 108, "Fused-norm rounding points":
 * that output's single bf16 rounding is this matmul's input).  T tokens, each
 * on its own (T = B * S of the modulation, 1 <= T <= 65535 * 512), K = 3072,
 * O = 64.
 * adaln_proj_out_fwd: out [T, K] bf16 (in), W [O, K] bf16 (in), bias [O] bf16
 *   (in), latent [T, O] bf16 (out) = bf16(fp32(sum_k out_tk W_ok) + bias_o);
 *   ws: adaln_workspace_bytes(ADALN_OP_PROJ_OUT_FWD, 1, T, K) bytes.
 * adaln_proj_out_bwd: d_lat [T, O] bf16 (in), out, W as above (in); d_out
 *   [T, K] bf16 (out) = bf16(sum_o d_lat_to W_ok), dW [O, K] bf16 (out) =
 *   bf16(sum_t d_lat_to out_tk), db [O] bf16 (out) = bf16(sum_t d_lat_to);
 *   ws: adaln_workspace_bytes(ADALN_OP_PROJ_OUT_BWD, 1, T, K) bytes.
 * Products run on the fp64 matrix cores: every product of two bf16 numbers is
 * exact and the sums accumulate in fp64 in fixed orders -- latent as eight
 * chains over 384 consecutive k each, added ((p0 + p1) + (p2 + p3)) + ((p4 +
 * p5) + (p6 + p7)), rounded to fp32, plus the bias in fp32; d_out one chain
 * over the 64 outputs; dW and db over fixed 512-token chunks, the chunks then
 * added in ascending order -- so every result is the correctly rounded sum
 * except where the exact sum lies within about 2^-40 of its magnitude from an
 * fp32 rounding boundary.  A token's results do not depend on T or on where
 * the token sits; trailing tokens with d_lat = 0 leave dW and db unchanged. */
int adaln_proj_out_fwd(const adaln_bf16* out, const adaln_bf16* W, const adaln_bf16* bias, adaln_bf16* latent,
                       void* ws, size_t ws_bytes, int64_t T, int64_t K, int64_t O, void* stream);
int adaln_proj_out_bwd(const adaln_bf16* d_lat, const adaln_bf16* out, const adaln_bf16* W, adaln_bf16* d_out,
                       adaln_bf16* dW, adaln_bf16* db, void* ws, size_t ws_bytes, int64_t T, int64_t K, int64_t O,
                       void* stream);

/* Serving forward of the final layer: the final modulation followed by
 * proj_out (pull request 538, "What" and "Scope / Known limitations"; pull
 * request 108, "Fused-norm rounding points": the modulated output is rounded to
 * bf16 once, as the projection's input) without the modulated output in
 * memory.  latent, emb, mean and rstd are bit for bit those of adaln_fwd
 * followed by adaln_proj_out_fwd on its `out`: emb, mean and rstd come from the
 * same kernels as adaln_fwd's, and proj_out's blocks compute their slice of
 * out from x, mean, rstd and emb with the final modulation's expression
 * straight into on-chip memory, then run adaln_proj_out_fwd's matrix-core
 * chains on it.
 *   temb [B, D], W [2D, D], bias [2D], x [B, S, D], Wp [O, D], bp [O] bf16 (in);
 *   emb [B, 2D] bf16, latent [B, S, O] bf16, mean, rstd [B, S] fp32 (out);
 *   D = 3072, O = 64, B and S within adaln_fwd's limits, eps >= 0 finite.
 *   ws: adaln_workspace_bytes(ADALN_OP_FWD_PROJ_OUT, B, S, D) bytes, 16-byte
 *   aligned, contents on entry ignored. */
int adaln_fwd_proj_out(const adaln_bf16* temb, const adaln_bf16* W, const adaln_bf16* bias, const adaln_bf16* x,
                       const adaln_bf16* Wp, const adaln_bf16* bp, adaln_bf16* emb, adaln_bf16* latent, float* mean,
                       float* rstd, void* ws, size_t ws_bytes, int64_t B, int64_t S, int64_t D, int64_t O, float eps,
                       void* stream);

/* adaln_norm_mod_bwd for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Arguments, results and kernels are adaln_norm_mod_bwd's (the same
 * bytes); there is no workspace argument: the level-0 pairs of the token tree
 * live in a fixed file-scope device array of ADALN_NOALLOC_SCRATCH_BYTES
 * (64 MiB) that every GPU the library runs on holds until the process ends.
 * The call allocates nothing; its first call on a device looks up that
 * device's copy of the array (hipGetSymbolAddress) and keeps the address.
 * Limit: adaln_workspace_bytes(ADALN_OP_NORM_MOD_BWD, B, S, D) <= 64 MiB, i.e.
 * B * ceil(S / 32) <= 1365 tiles (B = 1: S <= 43680; B = 4: S <= 10912);
 * larger problems return ADALN_ERR_SCRATCH before anything is launched.
 * Nothing in the array needs to start at zero (every byte read is written
 * earlier in the same call).  All calls on one GPU share its array: calls
 * that overlap in time on one GPU (two streams, or two host threads) race on
 * it and must be ordered by the caller. */
int adaln_norm_mod_bwd_noalloc(const adaln_bf16* gout, const adaln_bf16* x, const float* mean,
                               const float* rstd, const adaln_bf16* emb, adaln_bf16* dx, float* d_emb,
                               int64_t B, int64_t S, int64_t D, void* stream);

/* Static description of a status code (pull request 538, "What": the
 * operator has no fallback and other platforms fail closed, so every refusal
 * reaches the caller; this names its reason). */
const char* adaln_strerror(int status);

/* ADALN_ABI_VERSION of the loaded library. */
int adaln_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ADALN_H */
