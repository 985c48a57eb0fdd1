// gdn_chunk_fwd_noalloc: the chunked forward pass with its workspace in a fixed
// device array owned by the library, for callers that cannot allocate device
// memory themselves (code under HIP graph capture, serving loops that forbid
// allocation).  The kernels are those of gdn_chunk_fwd; only the workspace
// differs.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gdn.h"
#include "gdn_internal.h"

namespace {

// The forward's workspace: per chunk and head the T diag(beta) fragments, the
// causal score and the decays, and the segment-split buffers.  Each device that
// runs the entry point holds one copy until the process ends.
static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices] = {};  // device address of `scratch`, per device

// The device address of `scratch` on the current device, looked up once per
// device.  (In host code `scratch` names a host-side stand-in, not device
// memory: only this address may reach a kernel.)
gdn_status scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GDN_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return GDN_ERR_HIP;
    }
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return GDN_OK;
}

}  // namespace

extern "C" gdn_status gdn_chunk_fwd_noalloc(const gdn_problem* p, const void* q, const void* k, const void* v,
                                            const float* g, const float* beta, const float* S0, void* o,
                                            float* S_final, void* stream) {
  size_t need = 0;
  gdn_status st = gdn::check_chunk_fwd(p, q, k, v, g, beta, S0, o, S_final, &need);
  if (st != GDN_OK) return st;
  if (need > GDN_NOALLOC_SCRATCH_BYTES) return GDN_ERR_SCRATCH;
  void* ws = nullptr;
  if (need) {
    st = scratch_on_current_device(&ws);
    if (st != GDN_OK) return st;
  }
  return gdn_chunk_fwd(p, q, k, v, g, beta, S0, o, S_final, ws, need, stream);
}
