// The allocation-free variant of moe_layer_forward: the same launch sequence and
// kernels, with the layer workspace taken from a device-resident array this file
// defines (one copy per GPU the library runs on, held until the process ends) instead
// of a caller buffer.
#include <mutex>

#include "moe.h"
#include "moe_kernels.h"

// The scratch array.  In host code its name stands for a host-side shadow, not a
// device address: only the address hipGetSymbolAddress returns for the current device
// may be handed to kernels or copies.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device, NULL until set up

// The device address of the current device's scratch array, looked up once per device
// (with that device current) and cached.
moe_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_layer_forward_noalloc(const moe_layer_weights* w, const void* x, float* logits,
                                                void* out, int out_dtype, const moe_shape* s,
                                                moe_layer_aux* aux, void** stage_events, void* stream) {
  // Argument validation first, exactly as moe_layer_forward does it: with no workspace
  // the call returns before any launch, MOE_ERR_WORKSPACE when everything else is valid.
  moe_status rc = moe_layer_forward(w, x, logits, out, out_dtype, s, aux, stage_events, nullptr, 0, stream);
  if (rc != MOE_ERR_WORKSPACE) return rc;
  const size_t need = moe_workspace_bytes(s, MOE_CALL_LAYER);
  if (need == 0 || need > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  rc = scratch_of_current_device(&ws);
  if (rc != MOE_OK) return rc;
  // No part of the layer workspace has to start at zero (the tile-claim counters are
  // cleared by the kernel that writes the tile tables, inside the same call, and the
  // decode-scale router's hand-over word counts only when it holds the call's own tag),
  // so the previous call's contents need no clearing.
  return moe_layer_forward(w, x, logits, out, out_dtype, s, aux, stage_events, ws, MOE_NOALLOC_SCRATCH_BYTES,
                           stream);
}
