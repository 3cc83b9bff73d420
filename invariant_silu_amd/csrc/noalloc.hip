// adaln_norm_mod_bwd_noalloc: the LayerNorm + modulation backward with the
// token-sum tree for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
// It runs adaln_norm_mod_bwd's kernels, unchanged, with the workspace (the
// tree's level-0 pairs) taken from a fixed file-scope device array instead of
// a caller buffer.
//
// The array is ADALN_NOALLOC_SCRATCH_BYTES (64 MiB) long; every GPU the library runs on holds its
// own copy until the process ends.  Its device address on the current device
// comes from hipGetSymbolAddress, asked once per device on the first call
// there and kept; host code never passes the array's name itself (in host
// code that name is a stand-in, not a device address).  Nothing in the
// workspace has to start at zero: every byte the kernels read was written
// earlier in the same call.  All calls on one GPU share that GPU's array, so
// calls that overlap in time on one GPU (different streams, or different
// host threads) race on it.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/adaln.h"

namespace {

constexpr size_t kScratchBytes = ADALN_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of this device's copy of `scratch`, or nullptr.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (p == nullptr) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[dev].store(q, std::memory_order_release);
    p = q;
  }
  return p;
}

}  // namespace

extern "C" {

int adaln_norm_mod_bwd_noalloc(const adaln_bf16* gout, const adaln_bf16* x, const float* mean, const float* rstd,
                               const adaln_bf16* emb, adaln_bf16* dx, float* d_emb, int64_t B, int64_t S, int64_t D,
                               void* stream) {
  const size_t need = adaln_workspace_bytes(ADALN_OP_NORM_MOD_BWD, B, S, D);
  if (need == 0) return ADALN_ERR_SHAPE;
  if (need > kScratchBytes) return ADALN_ERR_SCRATCH;
  void* ws = scratch_on_current_device();
  if (ws == nullptr) return ADALN_ERR_DEVICE;
  return adaln_norm_mod_bwd(gout, x, mean, rstd, emb, dx, d_emb, ws, kScratchBytes, B, S, D, stream);
}

}  // extern "C"
