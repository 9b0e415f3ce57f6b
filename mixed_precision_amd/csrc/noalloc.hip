// Attention entry point that allocates nothing, for callers that cannot call
// hipMalloc (code under graph capture, tight serving loops, harnesses that
// forbid allocation): the varlen/GQA work list the fused kernel reads lives in
// a file-scope device array instead of a caller-supplied workspace.
//
// The array (kScratchBytes) exists once per GPU the library runs on and stays
// until the process ends.  Its device address is taken once per device, with
// that device current, on the entry point's first call there; host code uses
// that address, never the array's name (which on the host is only a stand-in).
// Every call on a GPU shares the GPU's array: each call rewrites the whole work
// list before the attention kernel reads it (nothing needs clearing), and
// calls that overlap on one GPU (other streams, other threads) race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.hpp"
#include "tilemix.h"

namespace tilemix {
namespace {

constexpr size_t kScratchBytes = (size_t)TILEMIX_NOALLOC_WORKSPACE_BYTES;
__device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 256;
std::mutex g_mu;
void* g_scratch[kMaxDevices];   // device address of `scratch` per device, once taken

// The array's address on the current device (taken on first use), or nullptr
// with the HIP error in *err.
void* scratch_for_current_device(hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    *err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}

}  // namespace
}  // namespace tilemix

using namespace tilemix;

extern "C" int32_t tilemix_attn_prefill_noalloc(const tilemix_attn_params* params,
                                                const tilemix_attn_tensors* tensors, void* stream) {
  // host-side checks first: no HIP call is made for an invalid or oversized call
  int32_t st = validate_attn_call(params, tensors);
  if (st != TILEMIX_OK) return st;
  size_t need = 0;
  st = tilemix_attn_workspace_size(params, &need);
  if (st != TILEMIX_OK) return st;
  if (need > kScratchBytes) {
    char msg[256];
    snprintf(msg, sizeof(msg),
             "the work list of this call needs %zu bytes, above the %zu bytes of the no-allocation entry point; "
             "use tilemix_attn_prefill with a workspace",
             need, kScratchBytes);
    return set_last_error(TILEMIX_ERR_WORKSPACE, msg);
  }
  hipError_t e = hipSuccess;
  void* ws = scratch_for_current_device(&e);
  if (!ws) {
    char msg[256];
    snprintf(msg, sizeof(msg), "no-allocation work list: %s", hipGetErrorString(e));
    return set_last_error(TILEMIX_ERR_HIP, msg);
  }
  return tilemix_attn_prefill(params, tensors, ws, kScratchBytes, stream);
}
