// wildcat_decode_noalloc: generation over the compressed cache with no
// device allocation and no caller workspace.  Its scratch is a file-scope
// device array (one per GPU, held until the process ends); the first call on
// a device looks up that device's address of the array once and every call
// hands the address to wildcat_decode as its workspace, so the kernels are
// the same.  The decode kernels write every scratch byte they read before
// reading it, so nothing needs clearing between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/wildcat.h"

namespace {

static __device__ __align__(256) unsigned char scratch[WILDCAT_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up once per
// device); nullptr if the lookup fails.
void* scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" wildcat_status wildcat_decode_noalloc(const wildcat_q_desc* desc, const void* Q, const void* K_S,
                                                 const float* X, const float* vmin, const float* vmax,
                                                 const void* K_new, const void* V_new, float* O,
                                                 hipStream_t stream) {
  const size_t need = wildcat_decode_workspace_bytes(desc);
  if (need == 0) return desc == nullptr ? WILDCAT_ERR_ARG : WILDCAT_ERR_SHAPE;   // invalid descriptor
  if (need > (size_t)WILDCAT_NOALLOC_SCRATCH_BYTES) return WILDCAT_ERR_SCRATCH;
  void* ws = scratch_ptr();
  if (ws == nullptr) return WILDCAT_ERR_HIP;
  return wildcat_decode(desc, Q, K_S, X, vmin, vmax, K_new, V_new, O, ws, (size_t)WILDCAT_NOALLOC_SCRATCH_BYTES,
                        stream);
}
