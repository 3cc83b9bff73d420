// C-ABI layer: argument validation, device check, workspace carving and
// kernel sequencing.  Every check runs before anything is enqueued
// (RL-Kernel pull request 538, automated review: capability checks before
// allocation; width-correct 16-byte load guards; outputs never alias inputs;
// probe verdicts cached both ways).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstring>
#include <vector>

#include "../../include/adaln.h"
#include "launch.hpp"

namespace {


constexpr int64_t kD = 3072;
constexpr int64_t kN = 6144;
constexpr int64_t kN6 = 18432;   // a block's 6-way modulation projection
constexpr int64_t kTile = 32;
constexpr int64_t kMaxB = 65535;
constexpr int64_t kMaxS = kTile * 65535;
constexpr int kMaxDevices = 64;

std::atomic<int> g_arch_verdict[kMaxDevices];    // 0 unknown, 1 gfx950, 2 other
std::atomic<int> g_probe_verdict[kMaxDevices];   // 0 unknown, 1 pass, 2 fail
std::atomic<int> g_probe_failures[kMaxDevices];

inline size_t pad256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
  const void* p;
  size_t n;
};
inline bool overlaps(const Range& a, const Range& b) {
  if (a.n == 0 || b.n == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.n && b0 < a0 + a.n;
}
// every output against every input, every other output and the workspace
int check_overlap(const std::vector<Range>& outs, const std::vector<Range>& ins) {
  for (size_t i = 0; i < outs.size(); ++i) {
    for (const Range& r : ins)
      if (overlaps(outs[i], r)) return ADALN_ERR_OVERLAP;
    for (size_t j = i + 1; j < outs.size(); ++j)
      if (overlaps(outs[i], outs[j])) return ADALN_ERR_OVERLAP;
  }
  return ADALN_OK;
}

// Two [B rows x row_bytes] views with one row stride (ld_bytes): do any two
// of their rows share a byte?  (Views of one tensor's column chunks do not.)
bool views_overlap(const void* a, const void* b, int64_t row_bytes, int64_t ld_bytes, int64_t B) {
  const int64_t delta = static_cast<int64_t>(reinterpret_cast<uintptr_t>(b)) -
                        static_cast<int64_t>(reinterpret_cast<uintptr_t>(a));
  // rows i of a and j of b overlap iff |delta + (j - i) ld| < row_bytes, |j - i| < B
  const int64_t k0 = -delta / ld_bytes;
  for (int64_t k = k0 - 1; k <= k0 + 1; ++k) {
    if (k <= -B || k >= B) continue;
    const int64_t d = delta + k * ld_bytes;
    if (d > -row_bytes && d < row_bytes) return true;
  }
  return false;
}
// bytes a [B, D] view with row stride ld (elements of el bytes) spans
size_t view_span(int64_t B, int64_t ld, size_t el) { return static_cast<size_t>((B - 1) * ld + kD) * el; }

// The current device must be a gfx950, and the caller's stream (when one is
// given) must belong to it: the kernels run on the stream's device, while the
// per-device state (the verdicts, the allocation-free entry point's array)
// is looked up on the current one.
int check_device(void* stream = nullptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return ADALN_ERR_DEVICE;
  }
  if (stream != nullptr) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(reinterpret_cast<hipStream_t>(stream), &sdev) != hipSuccess || sdev != dev) {
      (void)hipGetLastError();
      return ADALN_ERR_DEVICE;
    }
  }
  int v = g_arch_verdict[dev].load(std::memory_order_acquire);
  if (v == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      v = 2;
    } else {
      v = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    }
    g_arch_verdict[dev].store(v, std::memory_order_release);
  }
  return v == 1 ? ADALN_OK : ADALN_ERR_DEVICE;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline int launched(hipError_t e) { return e == hipSuccess ? ADALN_OK : ADALN_ERR_LAUNCH; }

// level-0 pairs: per (sample, 64-column group, tile) 64 sums and 64 corrections
size_t ws_pairs(int64_t B, int64_t S, int64_t H) {
  return pad256(static_cast<size_t>(B * ceil_div(S, kTile) * ceil_div(H, 64) * 128 * 4));
}
size_t ws_norm_bwd(int64_t B, int64_t S) { return ws_pairs(B, S, kN); }
size_t ws_proj_fwd(int64_t B) {
  return pad256(static_cast<size_t>(B * kD * 2));   // SiLU activations (B > 4)
}
size_t ws_proj_bwd(int64_t B) {
  // B <= 6: the fp64 da subtrees (32 per sample and column) between the two
  // launches; B > 6: the SiLU activations, then the fp64 subtrees
  // of the da leaf runs
  if (B <= adaln::proj_bwd_fused_max_batch()) return pad256(adaln::proj_bwd_fused_sub_bytes(B));
  return pad256(static_cast<size_t>(B * kD * 2)) + pad256(adaln::proj_bwd_da_parts_bytes(B));
}
// the da run subtrees: after the SiLU activations a (bf16, B > 6)
double* da_parts(void* a, int64_t B) {
  return reinterpret_cast<double*>(static_cast<char*>(a) + pad256(static_cast<size_t>(B * kD * 2)));
}
size_t ws_tree(int64_t B, int64_t S, int64_t H) { return ws_pairs(B, S, H); }
constexpr int64_t kMaxTokens = int64_t{65535} * 512;   // proj_out: token indices (and a token's sample) fit 32 bits
constexpr int64_t kProjOutO = 64;
bool tokens_ok(int64_t T) { return T >= 1 && T <= kMaxTokens; }
size_t ws_proj_out_db_offset(int64_t T) {
  return pad256(static_cast<size_t>(adaln::proj_out_chunks(T) * kProjOutO * kD * 8));
}
// the forward keeps its partial sums on chip: a nominal 256 bytes (the
// argument stays, so a later design can use it without an ABI change)
size_t ws_proj_out_fwd(int64_t) { return 256; }
size_t ws_proj_out(int64_t T) {
  return ws_proj_out_db_offset(T) + pad256(static_cast<size_t>(adaln::proj_out_chunks(T) * kProjOutO * 8));
}
size_t ws_fwd_proj_out(int64_t B, int64_t S) { return ws_proj_fwd(B) + ws_proj_out_fwd(B * S); }
size_t ws_proj_bwd_f32(int64_t B) {
  // SiLU activations (fp32 storage), then the fp64 da subtrees: B <= 4, the
  // leaf groups'; B > 4, the leaf runs' (none beyond B = 64)
  return pad256(static_cast<size_t>(B * kD * 4)) +
         pad256(B <= adaln::proj_bwd_f32_max_batch() ? adaln::proj_bwd_fused_sub_bytes(B)
                                                      : adaln::proj_bwd_da_parts_bytes(B));
}
bool batch_ok(int64_t B) { return B >= 1 && B <= kMaxB; }
bool seq_ok(int64_t S) { return S >= 1 && S <= kMaxS; }
// projection widths: the final modulation (2D) and a block's 6-way modulation (6D)
bool proj_width_ok(int64_t N) { return N == kN || N == kN6; }

// host reference values for the strict-math probe
uint32_t host_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
float from_bits(uint32_t u) {
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}
uint32_t to_bits(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return u;
}

int run_probe() {
  constexpr int n = 4096;
  std::vector<float> in(n);
  // an fma would give 2^-24 here; two roundings give exactly 0
  in[0] = 1.0f + 0x1p-12f;
  in[1] = 1.0f + 0x1p-12f;
  in[2] = -(1.0f + 0x1p-11f);
  uint64_t st = 0x9e3779b97f4a7c15ull;
  for (int i = 3; i < n; ++i) {
    st = st * 6364136223846793005ull + 1442695040888963407ull;
    const uint32_t r = static_cast<uint32_t>(st >> 32);
    if (i % 4 == 0) {
      // bf16 ties and near-ties
      const uint32_t u = (0x3f800000u + ((r & 0xffu) << 16)) | 0x8000u | (r & 0x10000u ? 1u : 0u);
      in[i] = from_bits(i % 8 == 0 ? (u & ~1u) : u);
    } else {
      const uint32_t mant = r & 0x7fffffu;
      const uint32_t ex = 64u + ((r >> 23) & 127u);   // 2^-63 .. 2^63
      in[i] = from_bits((ex << 23) | mant | ((r >> 31) << 31));
    }
  }
  float *d_in = nullptr, *d_out = nullptr;
  uint32_t* d_bits = nullptr;
  int fails = -1;
  if (hipMalloc(&d_in, n * 4) == hipSuccess && hipMalloc(&d_out, n * 16) == hipSuccess &&
      hipMalloc(&d_bits, n * 4) == hipSuccess &&
      hipMemcpy(d_in, in.data(), n * 4, hipMemcpyHostToDevice) == hipSuccess &&
      adaln::launch_selftest_probe(d_in, d_out, d_bits, n, nullptr) == hipSuccess &&
      hipDeviceSynchronize() == hipSuccess) {
    std::vector<float> out(4 * n);
    std::vector<uint32_t> bits(n);
    if (hipMemcpy(out.data(), d_out, n * 16, hipMemcpyDeviceToHost) == hipSuccess &&
        hipMemcpy(bits.data(), d_bits, n * 4, hipMemcpyDeviceToHost) == hipSuccess) {
      fails = 0;
      for (int i = 0; i < n; ++i) {
        const float v = in[i], w = in[(i + 1) % n], c = in[(i + 2) % n];
        volatile float prod = v * w;   // keep the host from contracting
        const float want[4] = {std::sqrt(std::fabs(v)), 1.0f / v, prod + c,
                               static_cast<float>(static_cast<double>(v) / static_cast<double>(w))};
        for (int k = 0; k < 4; ++k)
          if (to_bits(out[4 * i + k]) != to_bits(want[k])) ++fails;
        if (bits[i] != host_bf16(v)) ++fails;
      }
      if (to_bits(out[2]) != 0u) ++fails;   // the fma detector must read +0
    }
  }
  (void)hipGetLastError();
  if (d_in) (void)hipFree(d_in);
  if (d_out) (void)hipFree(d_out);
  if (d_bits) (void)hipFree(d_bits);
  return fails;
}

}  // namespace

extern "C" {

int adaln_abi_version(void) { return ADALN_ABI_VERSION; }

const char* adaln_strerror(int status) {
  switch (status) {
    case ADALN_OK: return "ok";
    case ADALN_ERR_NULL: return "a required pointer is NULL";
    case ADALN_ERR_SHAPE: return "bad shape (need B, S >= 1 within limits and D = K = 3072, N = 6144)";
    case ADALN_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case ADALN_ERR_DEVICE:
      return "unsupported or missing device (gfx950 required), or a stream of another device than the current one";
    case ADALN_ERR_WORKSPACE: return "workspace too small";
    case ADALN_ERR_OVERLAP: return "an output overlaps an input, another output or the workspace";
    case ADALN_ERR_LAUNCH: return "kernel launch failed";
    case ADALN_ERR_SCRATCH: return "problem too large for the fixed scratch array of the no-alloc entry point";
    default: return status > 0 ? "strict-math probe mismatches" : "unknown status";
  }
}

size_t adaln_workspace_bytes(int op, int64_t B, int64_t S, int64_t H) {
  if (!batch_ok(B)) return 0;
  switch (op) {
    case ADALN_OP_NORM_MOD_BWD: return (H == kD && seq_ok(S)) ? ws_norm_bwd(B, S) : 0;
    case ADALN_OP_PROJ_FWD: return H == kD ? ws_proj_fwd(B) : 0;
    case ADALN_OP_PROJ_BWD: return H == kD ? ws_proj_bwd(B) : 0;
    case ADALN_OP_BWD: return (H == kD && seq_ok(S)) ? ws_norm_bwd(B, S) + ws_proj_bwd(B) : 0;
    case ADALN_OP_BWD_F32: return (H == kD && seq_ok(S)) ? ws_norm_bwd(B, S) + ws_proj_bwd_f32(B) : 0;
    case ADALN_OP_RESIDUAL_BWD: return (H == kD && seq_ok(S)) ? ws_pairs(B, S, 3 * kD) : 0;
    // proj_out: only the token count T = B * S matters (S may exceed the
    // modulation's sequence limit, e.g. B = 1, S = T)
    case ADALN_OP_PROJ_OUT_BWD:
      return (H == kD && S >= 1 && S <= kMaxTokens && tokens_ok(B * S)) ? ws_proj_out(B * S) : 0;
    case ADALN_OP_PROJ_OUT_FWD:
      return (H == kD && S >= 1 && S <= kMaxTokens && tokens_ok(B * S)) ? ws_proj_out_fwd(B * S) : 0;
    case ADALN_OP_FWD_PROJ_OUT: return (H == kD && seq_ok(S)) ? ws_fwd_proj_out(B, S) : 0;
    case ADALN_OP_TOKEN_TREE_SUM:
      return (seq_ok(S) && H >= 1 && H <= (int64_t{1} << 24)) ? ws_tree(B, S, H) : 0;
    default: return 0;
  }
}

int adaln_proj_fwd(const adaln_bf16* temb, const adaln_bf16* W, const adaln_bf16* bias,
                   adaln_bf16* emb, void* ws, size_t ws_bytes, int64_t B, int64_t K, int64_t N,
                   void* stream) {
  if (!temb || !W || !bias || !emb || !ws) return ADALN_ERR_NULL;
  if (!batch_ok(B) || K != kD || !proj_width_ok(N)) return ADALN_ERR_SHAPE;
  if (!aligned16(temb) || !aligned16(W) || !aligned16(bias) || !aligned16(emb) || !aligned16(ws))
    return ADALN_ERR_ALIGN;
  const size_t need = ws_proj_fwd(B);
  if (ws_bytes < need) return ADALN_ERR_WORKSPACE;
  if (int rc = check_overlap({{emb, static_cast<size_t>(B * N * 2)}, {ws, need}},
                             {{temb, static_cast<size_t>(B * kD * 2)}, {W, static_cast<size_t>(N * kD * 2)},
                              {bias, static_cast<size_t>(N * 2)}}))
    return rc;
  if (int rc = check_device(stream)) return rc;
  (void)hipGetLastError();
  return launched(adaln::launch_proj_fwd(temb, W, bias, emb, static_cast<uint16_t*>(ws), B, N,
                                         as_stream(stream)));
}

int adaln_norm_mod_fwd(const adaln_bf16* x, const adaln_bf16* emb, adaln_bf16* out, float* mean,
                       float* rstd, int64_t B, int64_t S, int64_t D, float eps, void* stream) {
  if (!x || !emb || !out || !mean || !rstd) return ADALN_ERR_NULL;
  if (!batch_ok(B) || !seq_ok(S) || D != kD) return ADALN_ERR_SHAPE;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return ADALN_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(emb) || !aligned16(out) || !aligned16(mean) || !aligned16(rstd))
    return ADALN_ERR_ALIGN;
  const size_t rows = static_cast<size_t>(B * S);
  if (int rc = check_overlap({{out, rows * kD * 2}, {mean, rows * 4}, {rstd, rows * 4}},
                             {{x, rows * kD * 2}, {emb, static_cast<size_t>(B * kN * 2)}}))
    return rc;
  if (int rc = check_device(stream)) return rc;
  (void)hipGetLastError();
  return launched(adaln::launch_norm_mod_fwd(x, emb, out, mean, rstd, B, S, eps, as_stream(stream)));
}

int adaln_norm_mod_bwd_dx(const adaln_bf16* gout, const adaln_bf16* x, const float* mean,
                          const float* rstd, const adaln_bf16* emb, adaln_bf16* dx, int64_t B,
                          int64_t S, int64_t D, void* stream) {
  if (!gout || !x || !mean || !rstd || !emb || !dx) return ADALN_ERR_NULL;
  if (!batch_ok(B) || !seq_ok(S) || D != kD) return ADALN_ERR_SHAPE;
  if (!aligned16(gout) || !aligned16(x) || !aligned16(mean) || !aligned16(rstd) ||
      !aligned16(emb) || !aligned16(dx))
    return ADALN_ERR_ALIGN;
  const size_t rows = static_cast<size_t>(B * S);
  if (int rc = check_overlap({{dx, rows * kD * 2}},
                             {{gout, rows * kD * 2}, {x, rows * kD * 2}, {mean, rows * 4},
                              {rstd, rows * 4}, {emb, static_cast<size_t>(B * kN * 2)}}))
    return rc;
  if (int rc = check_device(stream)) return rc;
  (void)hipGetLastError();
  return launched(adaln::launch_norm_mod_bwd_dx(gout, x, mean, rstd, emb, dx, B, S, as_stream(stream)));
}

int adaln_norm_mod_bwd_tiles(const adaln_bf16* gout, const adaln_bf16* x, const float* mean,
                             const float* rstd, void* part, size_t part_bytes, int64_t B, int64_t S,
                             int64_t D, void* stream) {
  if (!gout || !x || !mean || !rstd || !part) return ADALN_ERR_NULL;
  if (!batch_ok(B) || !seq_ok(S) || D != kD) return ADALN_ERR_SHAPE;
  if (!aligned16(gout) || !aligned16(x) || !aligned16(mean) || !aligned16(rstd) || !aligned16(part))
    return ADALN_ERR_ALIGN;
  const size_t need = ws_norm_bwd(B, S);
  if (part_bytes < need) return ADALN_ERR_WORKSPACE;
  const size_t rows = static_cast<size_t>(B * S);
  if (int rc = check_overlap({{part, need}}, {{gout, rows * kD * 2}, {x, rows * kD * 2},
                                              {mean, rows * 4}, {rstd, rows * 4}}))
    return rc;
  if (int rc = check_device(stream)) return rc;
  (void)hipGetLastError();
  return launched(adaln::launch_norm_mod_bwd_tiles(gout, x, mean, rstd, static_cast<float*>(part), B, S,
                                                   as_stream(stream)));
}

int adaln_norm_mod_bwd_level0(const adaln_bf16* gout, const adaln_bf16* x, const float* mean, const float* rstd,
                              const adaln_bf16* emb, adaln_bf16* dx, void* part, size_t part_bytes, int64_t B,
                              int64_t S, int64_t D, void* ev_start, void* ev_stop, void* stream) {
  if (!gout || !x || !mean || !rstd || !emb || !dx || !part) return ADALN_ERR_NULL;
  if (!batch_ok(B) || !seq_ok(S) || D != kD) return ADALN_ERR_SHAPE;
  if (!aligned16(gout) || !aligned16(x) || !aligned16(mean) || !aligned16(rstd) || !aligned16(emb) ||
      !aligned16(dx) || !aligned16(part))
    return ADALN_ERR_ALIGN;
  const size_t need = ws_norm_bwd(B, S);
  if (part_bytes < need) return ADALN_ERR_WORKSPACE;
  const size_t rows = static_cast<size_t>(B * S);
  if (int rc = check_overlap({{dx, rows * kD * 2}, {part, need}},
                             {{gout, rows * kD * 2}, {x, rows * kD * 2}, {mean, rows * 4}, {rstd, rows * 4},
                              {emb, static_cast<size_t>(B * kN * 2)}}))
    return rc;
  if (int rc = check_device(stream)) return rc;
  (void)hipGetLastError();
  return launched(adaln::launch_norm_mod_bwd(gout, x, mean, rstd, emb, dx, static_cast<float*>(part), B, S,
                                             as_stream(stream), static_cast<hipEvent_t>(ev_start),
                                             static_cast<hipEvent_t>(ev_stop)));
}

int token_tree_fold(const void* part, size_t part_bytes, float* out, int64_t B, int64_t T0, int64_t H,
                    void* stream) {
  if (!part || !out) return ADALN_ERR_NULL;
  if (!batch_ok(B) || T0 < 1 || T0 > kMaxS / kTile || H < 1 || H > (int64_t{1} << 24))
    return ADALN_ERR_SHAPE;
  if (!aligned16(part) || !aligned16(out)) return ADALN_ERR_ALIGN;
  const size_t bytes = ws_pairs(B, T0 * kTile, H);
  if (part_bytes < bytes) return ADALN_ERR_WORKSPACE;
  if (int rc = check_overlap({{out, static_cast<size_t>(B * H * 4)}}, {{part, bytes}})) return rc;
  if (int rc = check_device(stream)) return rc;
  (void)hipGetLastError();
  return launched(adaln::launch_tree_fold(static_cast<const float*>(part), out, B, T0, H, as_stream(stream)));
}

int adaln_norm_mod_bwd(const adaln_bf16* gout, const adaln_bf16* x, const float* mean,
                       const float* rstd, const adaln_bf16* emb, adaln_bf16* dx, float* d_emb,
                       void* ws, size_t ws_bytes, int64_t B, int64_t S, int64_t D, void* stream) {
  if (!gout || !x || !mean || !rstd || !emb || !dx || !d_emb || !ws) return ADALN_ERR_NULL;
  if (!batch_ok(B) || !seq_ok(S) || D != kD) return ADALN_ERR_SHAPE;
  if (!aligned16(gout) || !aligned16(x) || !aligned16(mean) || !aligned16(rstd) ||
      !aligned16(emb) || !aligned16(dx) || !aligned16(d_emb) || !aligned16(ws))
    return ADALN_ERR_ALIGN;
  const size_t need = ws_norm_bwd(B, S);
  if (ws_bytes < need) return ADALN_ERR_WORKSPACE;
  const size_t rows = static_cast<size_t>(B * S);
  if (int rc = check_overlap({{dx, rows * kD * 2}, {d_emb, static_cast<size_t>(B * kN * 4)}, {ws, need}},
                             {{gout, rows * kD * 2}, {x, rows * kD * 2}, {mean, rows * 4},
                              {rstd, rows * 4}, {emb, static_cast<size_t>(B * kN * 2)}}))
    return rc;
  if (int rc = check_device(stream)) return rc;
  (void)hipGetLastError();
  // one tile per sample: the LayerNorm backward writes the roots itself
  const bool one_tile = S <= kTile;
  if (int rc = launched(adaln::launch_norm_mod_bwd(gout, x, mean, rstd, emb, dx, static_cast<float*>(ws), B, S,
                                                   as_stream(stream), nullptr, nullptr,
                                                   one_tile ? d_emb : nullptr)))
    return rc;
  if (one_tile) return ADALN_OK;
  return token_tree_fold(ws, need, d_emb, B, ceil_div(S, kTile), kN, stream);
}

int adaln_proj_bwd_acc(const float* d_emb, const adaln_bf16* temb, const adaln_bf16* W,
                       adaln_bf16* dW, adaln_bf16* db, adaln_bf16* dtemb, float* dW_f32, float* db_f32,
                       float* dtemb_f32, void* ws, size_t ws_bytes, int64_t B, int64_t K, int64_t N,
                       void* stream) {
  if (!d_emb || !temb || !W || !dW || !db || !dtemb || !ws) return ADALN_ERR_NULL;
  if (!batch_ok(B) || K != kD || !proj_width_ok(N)) return ADALN_ERR_SHAPE;
  if (!aligned16(d_emb) || !aligned16(temb) || !aligned16(W) || !aligned16(dW) || !aligned16(db) ||
      !aligned16(dtemb) || !aligned16(ws) || (dW_f32 && !aligned16(dW_f32)) || (db_f32 && !aligned16(db_f32)) ||
      (dtemb_f32 && !aligned16(dtemb_f32)))
    return ADALN_ERR_ALIGN;
  const size_t need = ws_proj_bwd(B);
  if (ws_bytes < need) return ADALN_ERR_WORKSPACE;
  std::vector<Range> outs = {{dW, static_cast<size_t>(N * kD * 2)}, {db, static_cast<size_t>(N * 2)},
                             {dtemb, static_cast<size_t>(B * kD * 2)}, {ws, need}};
  if (dW_f32) outs.push_back({dW_f32, static_cast<size_t>(N * kD * 4)});
  if (db_f32) outs.push_back({db_f32, static_cast<size_t>(N * 4)});
  if (dtemb_f32) outs.push_back({dtemb_f32, static_cast<size_t>(B * kD * 4)});
  if (int rc = check_overlap(outs, {{d_emb, static_cast<size_t>(B * N * 4)},
                                    {temb, static_cast<size_t>(B * kD * 2)},
                                    {W, static_cast<size_t>(N * kD * 2)}}))
    return rc;
  if (int rc = check_device(stream)) return rc;
  (void)hipGetLastError();
  adaln::AccOut acc;
  acc.dW = dW_f32;
  acc.db = db_f32;
  acc.dtemb = dtemb_f32;
  uint16_t* a = static_cast<uint16_t*>(ws);
  const hipStream_t s = as_stream(stream);
  if (B <= adaln::proj_bwd_fused_max_batch()) {
    return launched(
        adaln::launch_proj_bwd_fused(d_emb, temb, W, dW, db, dtemb, static_cast<double*>(ws), B, N, s, acc));
  }
  if (int rc = launched(adaln::launch_silu(temb, a, B * kD, s))) return rc;
  return launched(adaln::launch_proj_bwd_mfma(d_emb, a, W, temb, dW, db, dtemb, da_parts(a, B), B, N, s, acc));
}

int adaln_proj_bwd(const float* d_emb, const adaln_bf16* temb, const adaln_bf16* W,
                   adaln_bf16* dW, adaln_bf16* db, adaln_bf16* dtemb, void* ws, size_t ws_bytes,
                   int64_t B, int64_t K, int64_t N, void* stream) {
  return adaln_proj_bwd_acc(d_emb, temb, W, dW, db, dtemb, nullptr, nullptr, nullptr, ws, ws_bytes, B, K, N,
                            stream);
}

int token_tree_sum(const float* x, float* out, void* ws, size_t ws_bytes, int64_t B, int64_t S,
                   int64_t H, void* stream) {
  if (!x || !out || !ws) return ADALN_ERR_NULL;
  if (!batch_ok(B) || !seq_ok(S) || H < 1 || H > (int64_t{1} << 24)) return ADALN_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(out) || !aligned16(ws)) return ADALN_ERR_ALIGN;
  const size_t need = ws_tree(B, S, H);
  if (ws_bytes < need) return ADALN_ERR_WORKSPACE;
  if (int rc = check_overlap({{out, static_cast<size_t>(B * H * 4)}, {ws, need}},
                             {{x, static_cast<size_t>(B * S * H * 4)}}))
    return rc;
  if (int rc = check_device(stream)) return rc;
  (void)hipGetLastError();
  const int64_t T0 = ceil_div(S, kTile);
  float* part = static_cast<float*>(ws);
  const hipStream_t s = as_stream(stream);
  if (int rc = launched(adaln::launch_token_level0(x, part, B, S, H, s))) return rc;
  return launched(adaln::launch_tree_fold(part, out, B, T0, H, s));
}

int adaln_fwd(const adaln_bf16* temb, const adaln_bf16* W, const adaln_bf16* bias, const adaln_bf16* x,
              adaln_bf16* emb, adaln_bf16* out, float* mean, float* rstd, int64_t B, int64_t S,
              int64_t D, float eps, void* stream) {
  if (!temb || !W || !bias || !x || !emb || !out || !mean || !rstd) return ADALN_ERR_NULL;
  if (!batch_ok(B) || !seq_ok(S) || D != kD) return ADALN_ERR_SHAPE;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return ADALN_ERR_SHAPE;
  if (!aligned16(temb) || !aligned16(W) || !aligned16(bias) || !aligned16(x) || !aligned16(emb) ||
      !aligned16(out) || !aligned16(mean) || !aligned16(rstd))
    return ADALN_ERR_ALIGN;
  const size_t rows = static_cast<size_t>(B * S);
  if (int rc = check_overlap({{emb, static_cast<size_t>(B * kN * 2)}, {out, rows * kD * 2}, {mean, rows * 4},
                              {rstd, rows * 4}},
                             {{temb, static_cast<size_t>(B * kD * 2)}, {W, static_cast<size_t>(kN * kD * 2)},
                              {bias, static_cast<size_t>(kN * 2)}, {x, rows * kD * 2}}))
    return rc;
  if (int rc = check_device(stream)) return rc;
  (void)hipGetLastError();
  return launched(adaln::launch_fwd(temb, W, bias, x, emb, out, mean, rstd, B, S, eps, as_stream(stream)));
}

int adaln_bwd(const adaln_bf16* gout, const adaln_bf16* x, const float* mean, const float* rstd,
              const adaln_bf16* emb, const adaln_bf16* temb, const adaln_bf16* W, adaln_bf16* dx,
              float* d_emb, adaln_bf16* dW, adaln_bf16* db, adaln_bf16* dtemb, void* ws, size_t ws_bytes,
              int64_t B, int64_t S, int64_t D, void* stream) {
  if (!gout || !x || !mean || !rstd || !emb || !temb || !W || !dx || !d_emb || !dW || !db || !dtemb || !ws)
    return ADALN_ERR_NULL;
  if (!batch_ok(B) || !seq_ok(S) || D != kD) return ADALN_ERR_SHAPE;
  if (!aligned16(gout) || !aligned16(x) || !aligned16(mean) || !aligned16(rstd) || !aligned16(emb) ||
      !aligned16(temb) || !aligned16(W) || !aligned16(dx) || !aligned16(d_emb) || !aligned16(dW) ||
      !aligned16(db) || !aligned16(dtemb) || !aligned16(ws))
    return ADALN_ERR_ALIGN;
  const size_t n_norm = ws_norm_bwd(B, S);
  const size_t need = n_norm + ws_proj_bwd(B);
  if (ws_bytes < need) return ADALN_ERR_WORKSPACE;
  const size_t rows = static_cast<size_t>(B * S);
  if (int rc = check_overlap(
          {{dx, rows * kD * 2}, {d_emb, static_cast<size_t>(B * kN * 4)}, {dW, static_cast<size_t>(kN * kD * 2)},
           {db, static_cast<size_t>(kN * 2)}, {dtemb, static_cast<size_t>(B * kD * 2)}, {ws, need}},
          {{gout, rows * kD * 2}, {x, rows * kD * 2}, {mean, rows * 4}, {rstd, rows * 4},
           {emb, static_cast<size_t>(B * kN * 2)}, {temb, static_cast<size_t>(B * kD * 2)},
           {W, static_cast<size_t>(kN * kD * 2)}}))
    return rc;
  if (int rc = check_device(stream)) return rc;
  (void)hipGetLastError();
  const hipStream_t s = as_stream(stream);
  const int64_t T0 = ceil_div(S, kTile);
  float* part = static_cast<float*>(ws);
  uint16_t* a = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + n_norm);
  // dx rows and level-0 tiles in one launch (g and x read once), the fold,
  // then the projection backward: adaln_norm_mod_bwd then adaln_proj_bwd
  // one tile per sample (S <= 32): the LayerNorm backward writes d_emb's roots itself
  if (int rc = launched(adaln::launch_norm_mod_bwd(gout, x, mean, rstd, emb, dx, part, B, S, s, nullptr, nullptr,
                                                   T0 == 1 ? d_emb : nullptr)))
    return rc;
  // B > 6: the fold's launch also computes a = SiLU(temb) for the matrix cores
  const bool vec = B <= adaln::proj_bwd_fused_max_batch();
  bool act_done = false;
  if (T0 > 1)
    if (int rc = launched(adaln::launch_tree_fold(part, d_emb, B, T0, kN, s, vec ? nullptr : temb, vec ? nullptr : a,
                                                  &act_done)))
      return rc;
  if (vec)
    return launched(adaln::launch_proj_bwd_fused(d_emb, temb, W, dW, db, dtemb, reinterpret_cast<double*>(a), B, kN,
                                                 s));
  if (!act_done)
    if (int rc = launched(adaln::launch_silu(temb, a, B * kD, s))) return rc;
  return launched(adaln::launch_proj_bwd_mfma(d_emb, a, W, temb, dW, db, dtemb, da_parts(a, B), B, kN, s));
}

int adaln_fwd_f32(const float* temb, const float* W, const float* bias, const float* x, float* emb, float* out,
                  float* mean, float* rstd, int64_t B, int64_t S, int64_t D, float eps, void* stream) {
  if (!temb || !W || !bias || !x || !emb || !out || !mean || !rstd) return ADALN_ERR_NULL;
  if (!batch_ok(B) || !seq_ok(S) || D != kD) return ADALN_ERR_SHAPE;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return ADALN_ERR_SHAPE;
  if (!aligned16(temb) || !aligned16(W) || !aligned16(bias) || !aligned16(x) || !aligned16(emb) ||
      !aligned16(out) || !aligned16(mean) || !aligned16(rstd))
    return ADALN_ERR_ALIGN;
  const size_t rows = static_cast<size_t>(B * S);
  if (int rc = check_overlap({{emb, static_cast<size_t>(B * kN * 4)}, {out, rows * kD * 4}, {mean, rows * 4},
                              {rstd, rows * 4}},
                             {{temb, static_cast<size_t>(B * kD * 4)}, {W, static_cast<size_t>(kN * kD * 4)},
                              {bias, static_cast<size_t>(kN * 4)}, {x, rows * kD * 4}}))
    return rc;
  if (int rc = check_device(stream)) return rc;
  (void)hipGetLastError();
  const hipStream_t s = as_stream(stream);
  // SiLU into the first B * 3072 elements of `out` (overwritten by the
  // modulation afterwards), the projection, then statistics and modulation
  if (int rc = launched(adaln::launch_proj_fwd_f32(temb, out, W, bias, emb, B, s))) return rc;
  return launched(adaln::launch_norm_mod_fwd_f32(x, emb, out, mean, rstd, B, S, eps, s));
}

int adaln_bwd_f32(const float* gout, const float* x, const float* mean, const float* rstd, const float* emb,
                  const float* temb, const float* W, float* dx, float* d_emb, float* dW, float* db, float* dtemb,
                  void* ws, size_t ws_bytes, int64_t B, int64_t S, int64_t D, void* stream) {
  if (!gout || !x || !mean || !rstd || !emb || !temb || !W || !dx || !d_emb || !dW || !db || !dtemb || !ws)
    return ADALN_ERR_NULL;
  if (!batch_ok(B) || !seq_ok(S) || D != kD) return ADALN_ERR_SHAPE;
  if (!aligned16(gout) || !aligned16(x) || !aligned16(mean) || !aligned16(rstd) || !aligned16(emb) ||
      !aligned16(temb) || !aligned16(W) || !aligned16(dx) || !aligned16(d_emb) || !aligned16(dW) ||
      !aligned16(db) || !aligned16(dtemb) || !aligned16(ws))
    return ADALN_ERR_ALIGN;
  const size_t n_norm = ws_norm_bwd(B, S);
  const size_t need = n_norm + ws_proj_bwd_f32(B);
  if (ws_bytes < need) return ADALN_ERR_WORKSPACE;
  const size_t rows = static_cast<size_t>(B * S);
  if (int rc = check_overlap(
          {{dx, rows * kD * 4}, {d_emb, static_cast<size_t>(B * kN * 4)}, {dW, static_cast<size_t>(kN * kD * 4)},
           {db, static_cast<size_t>(kN * 4)}, {dtemb, static_cast<size_t>(B * kD * 4)}, {ws, need}},
          {{gout, rows * kD * 4}, {x, rows * kD * 4}, {mean, rows * 4}, {rstd, rows * 4},
           {emb, static_cast<size_t>(B * kN * 4)}, {temb, static_cast<size_t>(B * kD * 4)},
           {W, static_cast<size_t>(kN * kD * 4)}}))
    return rc;
  if (int rc = check_device(stream)) return rc;
  (void)hipGetLastError();
  const hipStream_t s = as_stream(stream);
  const int64_t T0 = ceil_div(S, kTile);
  float* part = static_cast<float*>(ws);
  float* a = reinterpret_cast<float*>(static_cast<char*>(ws) + n_norm);
  // one tile per sample (S <= 32): the LayerNorm backward writes d_emb's roots itself
  if (int rc = launched(adaln::launch_norm_mod_bwd_f32(gout, x, mean, rstd, emb, dx, part, B, S, s,
                                                       T0 == 1 ? d_emb : nullptr)))
    return rc;
  // the fold's launch also computes a = SiLU(temb) for the projection backward
  bool act_done = false;
  if (T0 > 1)
    if (int rc = launched(adaln::launch_tree_fold(part, d_emb, B, T0, kN, s, nullptr, nullptr, &act_done, temb, a)))
      return rc;
  double* sub = reinterpret_cast<double*>(reinterpret_cast<char*>(a) + pad256(static_cast<size_t>(B * kD * 4)));
  return launched(adaln::launch_proj_bwd_f32(d_emb, temb, W, a, dW, db, dtemb, sub, B, s, act_done));
}

int adaln_site_fwd(const adaln_bf16* x, const adaln_bf16* residual, const adaln_bf16* shift, const adaln_bf16* scale,
                   const adaln_bf16* gate, int64_t mod_ld, adaln_bf16* h, adaln_bf16* out, float* mean, float* rstd,
                   int64_t B, int64_t S, int64_t D, float eps, void* stream) {
  const bool res = residual != nullptr;
  if (!x || !shift || !scale || !out || !mean || !rstd || (res && (!gate || !h))) return ADALN_ERR_NULL;
  if (!batch_ok(B) || !seq_ok(S) || D != kD || mod_ld < kD || mod_ld % 8 != 0) return ADALN_ERR_SHAPE;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return ADALN_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(shift) || !aligned16(scale) || !aligned16(out) || !aligned16(mean) ||
      !aligned16(rstd) || (res && (!aligned16(residual) || !aligned16(gate) || !aligned16(h))))
    return ADALN_ERR_ALIGN;
  const size_t rows = static_cast<size_t>(B * S);
  const size_t vspan = view_span(B, mod_ld, 2);
  std::vector<Range> outs = {{out, rows * kD * 2}, {mean, rows * 4}, {rstd, rows * 4}};
  std::vector<Range> ins = {{x, rows * kD * 2}, {shift, vspan}, {scale, vspan}};
  if (res) {
    outs.push_back({h, rows * kD * 2});
    ins.push_back({residual, rows * kD * 2});
    ins.push_back({gate, vspan});
  }
  if (int rc = check_overlap(outs, ins)) return rc;
  if (int rc = check_device(stream)) return rc;
  (void)hipGetLastError();
  const adaln::ModView mv{shift, scale, res ? gate : nullptr, mod_ld};
  return launched(adaln::launch_site_fwd(x, residual, mv, res ? h : nullptr, out, mean, rstd, B, S, eps,
                                         as_stream(stream)));
}

int adaln_residual_fwd(const adaln_bf16* x, const adaln_bf16* residual, const adaln_bf16* mod, adaln_bf16* h,
                       adaln_bf16* out, float* mean, float* rstd, int64_t B, int64_t S, int64_t D, float eps,
                       void* stream) {
  if (!x || !residual || !mod || !h || !out || !mean || !rstd) return ADALN_ERR_NULL;
  if (D != kD) return ADALN_ERR_SHAPE;
  return adaln_site_fwd(x, residual, mod, mod + kD, mod + 2 * kD, 3 * kD, h, out, mean, rstd, B, S, D, eps, stream);
}

int adaln_site_bwd(const adaln_bf16* g_out, const adaln_bf16* g_h, const adaln_bf16* x, const adaln_bf16* h,
                   const float* mean, const float* rstd, const adaln_bf16* scale, const adaln_bf16* gate,
                   int64_t mod_ld, adaln_bf16* d_residual, adaln_bf16* dx, float* d_shift, float* d_scale,
                   float* d_gate, int64_t dmod_ld, void* ws, size_t ws_bytes, int64_t B, int64_t S, int64_t D,
                   void* stream) {
  const bool res = g_h != nullptr;
  if (!g_out || !x || !mean || !rstd || !scale || !dx || !d_shift || !d_scale || !ws ||
      (res && (!h || !gate || !d_residual || !d_gate)))
    return ADALN_ERR_NULL;
  if (!batch_ok(B) || !seq_ok(S) || D != kD || mod_ld < kD || mod_ld % 8 != 0 || dmod_ld < kD || dmod_ld % 8 != 0)
    return ADALN_ERR_SHAPE;
  if (!aligned16(g_out) || !aligned16(x) || !aligned16(mean) || !aligned16(rstd) || !aligned16(scale) ||
      !aligned16(dx) || !aligned16(d_shift) || !aligned16(d_scale) || !aligned16(ws) ||
      (res && (!aligned16(g_h) || !aligned16(h) || !aligned16(gate) || !aligned16(d_residual) || !aligned16(d_gate))))
    return ADALN_ERR_ALIGN;
  const int64_t nseg = res ? 3 : 2;
  const size_t need = ws_pairs(B, S, nseg * kD);
  if (ws_bytes < need) return ADALN_ERR_WORKSPACE;
  const size_t rows = static_cast<size_t>(B * S);
  const size_t vspan = view_span(B, mod_ld, 2), dspan = view_span(B, dmod_ld, 4);
  std::vector<Range> outs = {{dx, rows * kD * 2}, {ws, need}};
  std::vector<Range> ins = {{g_out, rows * kD * 2}, {x, rows * kD * 2}, {mean, rows * 4}, {rstd, rows * 4},
                            {scale, vspan}};
  std::vector<float*> dviews = {d_shift, d_scale};
  if (res) {
    outs.push_back({d_residual, rows * kD * 2});
    ins.push_back({g_h, rows * kD * 2});
    ins.push_back({h, rows * kD * 2});
    ins.push_back({gate, vspan});
    dviews.push_back(d_gate);
  }
  if (int rc = check_overlap(outs, ins)) return rc;
  // the gradient views: against every dense range as spans, against each other row by row
  for (size_t i = 0; i < dviews.size(); ++i) {
    const Range vi{dviews[i], dspan};
    for (const Range& r : outs)
      if (overlaps(vi, r)) return ADALN_ERR_OVERLAP;
    for (const Range& r : ins)
      if (overlaps(vi, r)) return ADALN_ERR_OVERLAP;
    for (size_t j = i + 1; j < dviews.size(); ++j)
      if (views_overlap(dviews[i], dviews[j], kD * 4, dmod_ld * 4, B)) return ADALN_ERR_OVERLAP;
  }
  if (int rc = check_device(stream)) return rc;
  (void)hipGetLastError();
  const hipStream_t s = as_stream(stream);
  float* part = static_cast<float*>(ws);
  const adaln::ModView mv{nullptr, scale, res ? gate : nullptr, mod_ld};
  // one tile per sample (S <= 32): the tile blocks write the roots into the views, no fold
  const bool one_tile = S <= kTile;
  if (int rc = launched(adaln::launch_site_bwd(g_out, g_h, x, res ? h : x, mean, rstd, mv, res ? d_residual : nullptr,
                                               dx, part, B, S, s, one_tile ? d_shift : nullptr,
                                               one_tile ? d_scale : nullptr, (one_tile && res) ? d_gate : nullptr,
                                               dmod_ld)))
    return rc;
  if (one_tile) return ADALN_OK;
  return launched(adaln::launch_tree_fold_views(part, d_shift, d_scale, res ? d_gate : nullptr, dmod_ld, B,
                                                ceil_div(S, kTile), nseg, s));
}

int adaln_residual_bwd(const adaln_bf16* g_out, const adaln_bf16* g_h, const adaln_bf16* x, const adaln_bf16* h,
                       const float* mean, const float* rstd, const adaln_bf16* mod, adaln_bf16* d_residual,
                       adaln_bf16* dx, float* d_mod, void* ws, size_t ws_bytes, int64_t B, int64_t S, int64_t D,
                       void* stream) {
  if (!g_out || !g_h || !x || !h || !mean || !rstd || !mod || !d_residual || !dx || !d_mod || !ws)
    return ADALN_ERR_NULL;
  if (D != kD) return ADALN_ERR_SHAPE;
  return adaln_site_bwd(g_out, g_h, x, h, mean, rstd, mod + kD, mod + 2 * kD, 3 * kD, d_residual, dx, d_mod,
                        d_mod + kD, d_mod + 2 * kD, 3 * kD, ws, ws_bytes, B, S, D, stream);
}

int adaln_proj_out_fwd(const adaln_bf16* out, const adaln_bf16* W, const adaln_bf16* bias, adaln_bf16* latent,
                       void* ws, size_t ws_bytes, int64_t T, int64_t K, int64_t O, void* stream) {
  if (!out || !W || !bias || !latent || !ws) return ADALN_ERR_NULL;
  if (!tokens_ok(T) || K != kD || O != kProjOutO) return ADALN_ERR_SHAPE;
  if (!aligned16(out) || !aligned16(W) || !aligned16(bias) || !aligned16(latent) || !aligned16(ws))
    return ADALN_ERR_ALIGN;
  const size_t need = ws_proj_out_fwd(T);
  if (ws_bytes < need) return ADALN_ERR_WORKSPACE;
  if (int rc = check_overlap({{latent, static_cast<size_t>(T * kProjOutO * 2)}, {ws, need}},
                             {{out, static_cast<size_t>(T * kD * 2)}, {W, static_cast<size_t>(kProjOutO * kD * 2)},
                              {bias, static_cast<size_t>(kProjOutO * 2)}}))
    return rc;
  if (int rc = check_device(stream)) return rc;
  (void)hipGetLastError();
  return launched(adaln::launch_proj_out_fwd(out, W, bias, latent, T, as_stream(stream)));
}

int adaln_proj_out_bwd(const adaln_bf16* d_lat, const adaln_bf16* out, const adaln_bf16* W, adaln_bf16* d_out,
                       adaln_bf16* dW, adaln_bf16* db, void* ws, size_t ws_bytes, int64_t T, int64_t K, int64_t O,
                       void* stream) {
  if (!d_lat || !out || !W || !d_out || !dW || !db || !ws) return ADALN_ERR_NULL;
  if (!tokens_ok(T) || K != kD || O != kProjOutO) return ADALN_ERR_SHAPE;
  if (!aligned16(d_lat) || !aligned16(out) || !aligned16(W) || !aligned16(d_out) || !aligned16(dW) ||
      !aligned16(db) || !aligned16(ws))
    return ADALN_ERR_ALIGN;
  const size_t need = ws_proj_out(T);
  if (ws_bytes < need) return ADALN_ERR_WORKSPACE;
  if (int rc = check_overlap(
          {{d_out, static_cast<size_t>(T * kD * 2)}, {dW, static_cast<size_t>(kProjOutO * kD * 2)},
           {db, static_cast<size_t>(kProjOutO * 2)}, {ws, need}},
          {{d_lat, static_cast<size_t>(T * kProjOutO * 2)}, {out, static_cast<size_t>(T * kD * 2)},
           {W, static_cast<size_t>(kProjOutO * kD * 2)}}))
    return rc;
  if (int rc = check_device(stream)) return rc;
  (void)hipGetLastError();
  double* part = static_cast<double*>(ws);
  double* part_db = reinterpret_cast<double*>(static_cast<unsigned char*>(ws) + ws_proj_out_db_offset(T));
  return launched(adaln::launch_proj_out_bwd(d_lat, out, W, d_out, dW, db, part, part_db, T, as_stream(stream)));
}

int adaln_fwd_proj_out(const adaln_bf16* temb, const adaln_bf16* W, const adaln_bf16* bias, const adaln_bf16* x,
                       const adaln_bf16* Wp, const adaln_bf16* bp, adaln_bf16* emb, adaln_bf16* latent, float* mean,
                       float* rstd, void* ws, size_t ws_bytes, int64_t B, int64_t S, int64_t D, int64_t O, float eps,
                       void* stream) {
  if (!temb || !W || !bias || !x || !Wp || !bp || !emb || !latent || !mean || !rstd || !ws) return ADALN_ERR_NULL;
  if (!batch_ok(B) || !seq_ok(S) || !tokens_ok(B * S) || D != kD || O != kProjOutO) return ADALN_ERR_SHAPE;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return ADALN_ERR_SHAPE;
  if (!aligned16(temb) || !aligned16(W) || !aligned16(bias) || !aligned16(x) || !aligned16(Wp) || !aligned16(bp) ||
      !aligned16(emb) || !aligned16(latent) || !aligned16(mean) || !aligned16(rstd) || !aligned16(ws))
    return ADALN_ERR_ALIGN;
  const size_t need = ws_fwd_proj_out(B, S);
  if (ws_bytes < need) return ADALN_ERR_WORKSPACE;
  const size_t rows = static_cast<size_t>(B * S);
  if (int rc = check_overlap({{emb, static_cast<size_t>(B * kN * 2)}, {latent, rows * kProjOutO * 2},
                              {mean, rows * 4}, {rstd, rows * 4}, {ws, need}},
                             {{temb, static_cast<size_t>(B * kD * 2)}, {W, static_cast<size_t>(kN * kD * 2)},
                              {bias, static_cast<size_t>(kN * 2)}, {x, rows * kD * 2},
                              {Wp, static_cast<size_t>(kProjOutO * kD * 2)}, {bp, static_cast<size_t>(kProjOutO * 2)}}))
    return rc;
  if (int rc = check_device(stream)) return rc;
  (void)hipGetLastError();
  const hipStream_t s = as_stream(stream);
  uint16_t* a = static_cast<uint16_t*>(ws);
  if (int rc = launched(adaln::launch_fwd_stats(temb, W, bias, x, emb, mean, rstd, a, B, S, eps, s))) return rc;
  return launched(adaln::launch_proj_out_fwd_fused(x, emb, mean, rstd, Wp, bp, latent, B, S, s));
}

int adaln_selftest(void) {
  if (int rc = check_device(nullptr)) return rc;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ADALN_ERR_DEVICE;
  int v = g_probe_verdict[dev].load(std::memory_order_acquire);
  if (v == 0) {
    const int fails = run_probe();
    g_probe_failures[dev].store(fails < 0 ? 1 : fails, std::memory_order_relaxed);
    v = fails == 0 ? 1 : 2;
    g_probe_verdict[dev].store(v, std::memory_order_release);
  }
  return v == 1 ? ADALN_OK : g_probe_failures[dev].load(std::memory_order_relaxed);
}

}  // extern "C"
