// hybrid_attn_fwd_noalloc: the forward for callers that cannot allocate
// device memory (code under HIP graph capture, serving loops, harnesses that
// forbid allocation). Its scratch is one file-scope device array per GPU,
// fixed at HWA_NOALLOC_SCRATCH_BYTES; the call runs the same kernels as
// hybrid_attn_fwd with that array as the workspace and never calls
// hipMalloc, hipFree or any allocating routine.

#include <string.h>

#include <mutex>

#include "hwa_internal.h"

namespace {

// the scratch array; in host code this name only stands for the symbol: its
// device address is taken with hipGetSymbolAddress, once per device
static __device__ __align__(256) unsigned char scratch[HWA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];  // device address of `scratch` on each device, or null

// Device address of this GPU's copy of the scratch array (the current device
// is the one the caller's stream belongs to); null on a HIP error.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" hwa_status hybrid_attn_fwd_noalloc(
    const void* q, const void* k, const void* v, const float* beta, const float* alpha,
    const void* gate, const float* text_state, int32_t frames, int32_t tokens_per_frame,
    int32_t chunk, int32_t radius, int32_t rule, void* out, hipStream_t stream,
    const hwa_params* p) {
  if (!p || p->struct_size < offsetof(hwa_params, softmax_lse)) return HWA_ERR_INVALID_ARG;
  // the caller's struct may be an older, shorter one: copy only what it holds
  hwa_params pc;
  memset(&pc, 0, sizeof(pc));
  memcpy(&pc, p, p->struct_size < sizeof(pc) ? p->struct_size : sizeof(pc));
  // every argument check of the forward first, with no workspace: it returns
  // the first bad argument's code, or HWA_ERR_WORKSPACE when only the
  // workspace is missing (it never enqueues anything without one)
  pc.workspace = nullptr;
  pc.workspace_bytes = 0;
  const hwa_status s = hybrid_attn_fwd(q, k, v, beta, alpha, gate, text_state, frames,
                                       tokens_per_frame, chunk, radius, rule, out, stream, &pc);
  if (s != HWA_ERR_WORKSPACE) return s;
  const size_t need = hwa_workspace_bytes(frames, tokens_per_frame, chunk, p);
  if (need > HWA_NOALLOC_SCRATCH_BYTES) return HWA_ERR_WORKSPACE;
  void* ws = scratch_ptr();
  if (!ws) return HWA_ERR_HIP;
  pc.workspace = ws;
  pc.workspace_bytes = HWA_NOALLOC_SCRATCH_BYTES;
  return hybrid_attn_fwd(q, k, v, beta, alpha, gate, text_state, frames, tokens_per_frame,
                         chunk, radius, rule, out, stream, &pc);
}
