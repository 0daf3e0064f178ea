// ia_noalloc.hip — ia_prefill_fwd_noalloc: the prefill with its workspace in a fixed device
// array of the library, for callers that cannot allocate device memory.
#include "ia.h"

#include <hip/hip_runtime.h>

#include <mutex>

namespace ia {
ia_status prefill_on_workspace(const ia_desc* d, const void* q, const void* k, const void* v,
                               const void* lambda, const void* beta, ia_state* st, void* o,
                               void* workspace, size_t ws_bytes, void* stream);
ia_status status_of(hipError_t e);
}

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;   // IA_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == IA_NOALLOC_SCRATCH_BYTES, "header and library agree");

// The workspace of ia_prefill_fwd_noalloc: one copy per device, alive until the process ends.
// Host code never uses this name as an address (on the host it is a stand-in); it uses the
// device address the runtime reports for the current device, kept in g_scratch.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_lock;
void* g_scratch[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per device.
hipError_t scratch_on_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_lock);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

ia_status ia_prefill_fwd_noalloc(const ia_desc* desc, const void* q, const void* k,
                                 const void* v, const void* lambda, const void* beta,
                                 ia_state* st, void* o, void* stream) {
  if (ia_prefill_workspace_bytes(desc) > kScratchBytes) return IA_ERR_WORKSPACE;
  void* ws = nullptr;
  const hipError_t e = scratch_on_current_device(&ws);
  if (e != hipSuccess) return ia::status_of(e);
  return ia::prefill_on_workspace(desc, q, k, v, lambda, beta, st, o, ws, kScratchBytes, stream);
}

}  // extern "C"
