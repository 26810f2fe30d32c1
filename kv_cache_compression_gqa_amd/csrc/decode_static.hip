// kvc_decode_attn_static: kvc_decode_attn with its scratch (split-K partials, window exp-sums, the step's tail
// length) in a static device array of the library instead of a caller workspace, for callers that cannot allocate
// device memory. The array is looked up once per device (hipGetSymbolAddress with that device current) and its
// address is what every launch receives; the array's own name is never passed to a kernel.
#include <mutex>

#include "kvc_internal.h"

namespace kvc {
namespace {

// each GPU the library runs on holds its own copy until the process ends
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// address of this device's copy of the array (nullptr if the lookup fails)
void* scratch_on_current_device() {
  int dev = -1;
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

int decode_static(const kvc_cache& c, const kvc_decode_args& a, hipStream_t s) {
  if (decode_workspace_bytes(c, a) > kStaticScratchBytes) return KVC_E_WORKSPACE;
  void* ws = scratch_on_current_device();
  if (ws == nullptr) return KVC_E_HIP;
  return launch_decode(c, a, ws, s) == hipSuccess ? KVC_OK : KVC_E_HIP;
}

}  // namespace kvc
