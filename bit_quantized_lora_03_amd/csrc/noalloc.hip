// The allocation-free forward pass: qlora_linear_fwd with its workspace in a
// file-scope device array that the library holds, for callers that cannot
// allocate device memory.  The kernels are the forward's own; only where the
// workspace lives differs.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "../../include/qlora.h"
#include "launch.h"

namespace {

// One copy per GPU, created when this code object is loaded on that GPU and
// held until the process ends.  Host code never uses this name as an
// address: the device address of each GPU's copy comes from
// hipGetSymbolAddress (scratch_on_current_device).
static __device__ __align__(256) uint8_t scratch[QLORA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices] = {};  // device address of scratch, per device

// The current device's copy of `scratch`, looked up once per device with
// that device current.
void* scratch_on_current_device(int* status) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *status = QLORA_EHIP;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      *status = QLORA_EHIP;
      return nullptr;
    }
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}

// Workspace source of the forward: rejects needs beyond the buffer before
// any HIP call.  No kernel of the forward reads workspace it has not
// written in the same call, so nothing is cleared.
void* scratch_source(size_t need, int* status) {
  if (need > QLORA_NOALLOC_SCRATCH_BYTES) {
    *status = QLORA_ESCRATCH;
    return nullptr;
  }
  return scratch_on_current_device(status);
}

}  // namespace

extern "C" int qlora_linear_fwd_noalloc(const qlora_nf4_weight* w, const uint16_t* x,
                                        int64_t M, const uint16_t* A, const uint16_t* B,
                                        int32_t r, float alpha, uint16_t* y, void* stream) {
  try {
    return qlora::linear_fwd_sourced(w, x, M, A, B, r, alpha, y, scratch_source, stream);
  } catch (...) {
    return QLORA_EHIP;
  }
}
