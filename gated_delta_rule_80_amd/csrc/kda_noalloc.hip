// kda_prefill_static: kda_prefill with its workspace in a static device array,
// for callers that cannot allocate device memory.  See include/kda.h.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kda.h"
#include "kda_launch.h"

namespace {

// The workspace of kda_prefill_static.  Each GPU the library runs on holds its
// own copy at its own address.  In host code the name is only a stand-in for
// the symbol: host code uses the device address that hipGetSymbolAddress gives
// for the current device, never the name itself.
__device__ __align__(256) char scratch[KDA_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device, once looked up

// The address of the current device's array, looked up on the first call there.
kda_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KDA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return KDA_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return KDA_OK;
}

}  // namespace

extern "C" kda_status kda_prefill_static(const kda_prefill_args* a, void* stream) {
  if (kda_status e = kda_validate_prefill(a); e != KDA_OK) return e;
  void* ws = nullptr;
  if (kda_status e = scratch_address(&ws); e != KDA_OK) return e;
  return kda::prefill_in_workspace(a, ws, KDA_STATIC_SCRATCH_BYTES, static_cast<hipStream_t>(stream));
}
