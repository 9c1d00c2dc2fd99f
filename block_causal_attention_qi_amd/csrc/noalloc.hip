// The allocation-free DiT step (include/qi.h, qi_dit_step_noalloc): the
// workspace of qi_dit_step taken from a file-scope device array instead of a
// caller buffer.  The array lives in this translation unit's own code object,
// which only a process that calls this entry point has to load (and fill)
// on its GPU.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/qi.h"

namespace {

// One copy per GPU, held from the code object's load until the process ends.
// In host code `scratch` names a host-side stand-in, never the device memory:
// its device address is looked up once per device with hipGetSymbolAddress
// (with that device current) and only that address is handed to kernels.
static __device__ __align__(256) char scratch[QI_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
struct ScratchAddr {
  std::mutex mu;
  void *ptr[kMaxDevices] = {};
};
ScratchAddr g_scratch;

// Device address of the current device's scratch array.
qi_status scratch_address(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return QI_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return QI_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> g(g_scratch.mu);
  if (!g_scratch.ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return QI_ERR_HIP;
    g_scratch.ptr[dev] = p;
  }
  *out = g_scratch.ptr[dev];
  return QI_OK;
}

}  // namespace

extern "C" qi_status qi_dit_step_noalloc(const qi_dims *d, const qi_model_w *w, int32_t L, int32_t N,
                                         const float *img_tokens, const float *txt_feats, float timestep,
                                         const float *txt_cos, const float *txt_sin, const float *img_cos,
                                         const float *img_sin, const qi_kv_cache *cache, float *vel,
                                         void *stream) {
  if (!d) return QI_ERR_NULL;
  // the size check comes first: nothing is looked up or enqueued for a
  // request the scratch cannot hold
  const size_t need = qi_workspace_bytes(d, L, N);
  if (need == 0)  // invalid dims or sizes: qi_dit_step reports which, before it touches anything
    return qi_dit_step(d, w, L, N, img_tokens, txt_feats, timestep, txt_cos, txt_sin, img_cos, img_sin, cache,
                       vel, nullptr, 0, stream);
  if (need > (size_t)QI_NOALLOC_SCRATCH_BYTES) return QI_ERR_WORKSPACE;
  void *ws = nullptr;
  const qi_status st = scratch_address(&ws);
  if (st != QI_OK) return st;
  return qi_dit_step(d, w, L, N, img_tokens, txt_feats, timestep, txt_cos, txt_sin, img_cos, img_sin, cache, vel,
                     ws, QI_NOALLOC_SCRATCH_BYTES, stream);
}
