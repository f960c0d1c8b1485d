// msgla_forward_noalloc: the layer forward for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc).  It is msgla_forward with its workspace taken from a
// device array this library owns, `scratch`, of MSGLA_NOALLOC_WORKSPACE_BYTES
// on every GPU the library runs on (held until the process ends).
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device, with that device current,
// with hipGetSymbolAddress, and only that address is ever handed to kernels.
// Every call on one GPU shares that GPU's array, so calls that overlap on one
// GPU (several streams, several threads) race; serialise them.  The forward
// needs nothing in its workspace to start at zero, so nothing is cleared.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/msgla.h"

static __device__ __align__(256) char scratch[MSGLA_NOALLOC_WORKSPACE_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_lock;
void* g_scratch[MAX_DEVICES] = {};  // device address of `scratch` per device, once looked up

// The current device's copy of `scratch` (nullptr if the lookup fails).
void* scratch_of_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
  std::lock_guard<std::mutex> guard(g_lock);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" msgla_status msgla_forward_noalloc(const msgla_config* cfg, const void* packed,
                                              const void* x, const uint8_t* mask, int64_t B,
                                              int64_t L, void* out, const void* state_in,
                                              void* state_out, void* stream) {
  if (msgla_status st = msgla_validate_config(cfg); st != MSGLA_OK) return st;
  if (!packed || !x || !out) return MSGLA_ERR_INVALID_ARG;
  const size_t need = msgla_workspace_bytes(cfg, B, L);
  if (need == 0) return MSGLA_ERR_INVALID_ARG;
  if (need > (size_t)MSGLA_NOALLOC_WORKSPACE_BYTES) return MSGLA_ERR_WORKSPACE;
  void* ws = scratch_of_current_device();
  if (!ws) return MSGLA_ERR_HIP;
  return msgla_forward(cfg, packed, x, mask, B, L, out, state_in, state_out, ws,
                       (size_t)MSGLA_NOALLOC_WORKSPACE_BYTES, stream);
}
