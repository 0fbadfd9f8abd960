// Allocation-free forward (graph_attn_fwd_noalloc): the forward of graph_attn_fwd with its
// hub-chunk partial states in a fixed scratch array of the library's device code instead
// of a caller workspace, for callers that cannot allocate (code under HIP graph capture,
// serving loops, harnesses that forbid allocation). The kernels are the forward's own.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ga_internal.h"

namespace {

constexpr size_t kScratchBytes = GA_FWD_NOALLOC_SCRATCH_BYTES;

// One copy per GPU, at a per-GPU address, allocated when the code object is loaded on
// that GPU and held until the process ends. Host code never passes this name to a
// kernel: in host code it is a stand-in, not a device address; the device address comes
// from hipGetSymbolAddress, once per device.
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 256;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's scratch, looked up on the first call on that
// device (with it current) and kept.
ga_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return GA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return GA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return GA_ERR_HIP;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return GA_OK;
}

}  // namespace

extern "C" ga_status graph_attn_fwd_noalloc(const ga_plan* p, ga_score score, ga_dtype dtype,
                                            int32_t heads, int32_t dim, float scale,
                                            float neg_slope, const void* a, const void* b,
                                            const void* v, void* out, float* lse, void* stream) {
  size_t need = 0;
  ga_status s = ga::fwd_check(p, score, dtype, heads, dim, a, b, v, out, lse, &need);
  if (s != GA_OK) return s;
  if (need > kScratchBytes) return GA_ERR_TOO_LARGE;
  if (!p->uploaded) return GA_ERR_NOT_READY;
  if (p->n == 0) return GA_OK;
  if ((s = ga::plan_device_check(p)) != GA_OK) return s;
  void* ws = nullptr;
  if ((s = scratch_of_current_device(&ws)) != GA_OK) return s;
  return ga::fwd_enqueue(p, score, dtype, heads, dim, scale, neg_slope, a, b, v, out, lse, ws,
                         stream);
}
