// efla_fwd_chunked_noalloc: the chunked forward for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc). It is efla_fwd_chunked with the
// time-segmented path's workspace taken from a fixed device array of this
// library instead of from the caller.
//
// `scratch` below is a file-scope device array. In host code its name is a
// host-side stand-in, not a device address, so it is never passed to a
// kernel or a copy: once per device, with that device current, its device
// address is looked up with hipGetSymbolAddress and kept in `g_scratch`, and
// only that address is used. Every call on one GPU shares that GPU's array.
// The kernels write every scratch value before they read it (segment maps,
// then start states), so nothing needs clearing between calls; calls that
// overlap on one GPU (several streams, or several host threads) race on it.

#include <hip/hip_runtime.h>

#include <mutex>

#include "efla.h"

namespace {

static __device__ __align__(256) unsigned char scratch[EFLA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_scratch[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up on the first
// call per device; nullptr if the runtime reports an error.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> g(g_lock);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" efla_status efla_fwd_chunked_noalloc(const void* q, const void* k, const void* v,
                                                const void* beta, const float* s0, void* o,
                                                float* s_final, int B, int H, int T, int d_k,
                                                int d_v, int chunk, efla_coef coef, efla_dtype dt,
                                                void* stream) {
  // 0 for a one-pass launch and for arguments the forward rejects (it then
  // reports them below, in its own order)
  const size_t need = efla_fwd_chunked_workspace_bytes(B, H, T, d_k, d_v, chunk, dt);
  if (need > (size_t)EFLA_NOALLOC_SCRATCH_BYTES) return EFLA_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  if (need > 0 && q && k && v && beta && o) {
    ws = scratch_on_current_device();
    if (ws == nullptr) return EFLA_ERR_HIP;
  }
  return efla_fwd_chunked(q, k, v, beta, s0, o, s_final, ws, ws ? need : 0, B, H, T, d_k, d_v, chunk,
                          coef, dt, stream);
}
