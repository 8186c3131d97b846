// noalloc.hip -- kvc_decode_attn_noalloc: one decode step whose split partials live in a file-scope device array,
// for callers that cannot allocate.  The kernels are those of kvc_decode_attn; only the workspace differs.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kvc_common.hpp"

namespace kvc {
namespace {

// The scratch array, one copy per GPU the library runs on (held until the process ends).  Host code never uses
// its name as an address: the device address of each GPU's copy comes from hipGetSymbolAddress.
__device__ __align__(256) unsigned char scratch[KVC_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};  // device address of scratch on each device, set on the device's first call

// This device's copy of scratch (the current device; looked up once per device).
kvc_status scratch_ptr(void** p) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return KVC_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void* q = nullptr;
    e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    if (!q) return KVC_ERR_HIP;
    g_scratch[dev] = q;
  }
  *p = g_scratch[dev];
  return KVC_OK;
}

}  // namespace
}  // namespace kvc

using namespace kvc;

extern "C" kvc_status kvc_decode_attn_noalloc(const kvc_layout* layout, const kvc_cache* cache,
                                              const kvc_decode_in* in, float* out, void* stream) {
  if (!in) return KVC_ERR_INVALID_ARG;
  size_t need = 0;
  const kvc_status s = kvc_decode_workspace_bytes(layout, in->B, in->max_T, in->num_splits, &need);
  if (s) return s;
  if (need > (size_t)KVC_NOALLOC_SCRATCH_BYTES) return KVC_ERR_SCRATCH;  // before any device call
  void* ws = nullptr;
  const kvc_status p = scratch_ptr(&ws);
  if (p) return p;
  // Every partial the kernels read is written by the same call, so nothing in the array needs clearing.
  return kvc_decode_attn(layout, cache, in, out, ws, (size_t)KVC_NOALLOC_SCRATCH_BYTES, stream);
}
