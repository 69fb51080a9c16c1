// Fixed device scratch for the allocation-free entry point.
//
// zebra_linear_attn_noalloc runs the linear-attention kernels with their
// partial states and folded state in this file-scope device array instead of
// a caller workspace, so a caller that cannot allocate (code under HIP graph
// capture, a serving loop that forbids hipMalloc) needs only its inputs and
// outputs. Each GPU the library runs on holds its own copy of the array until
// the process ends. Host code never passes the array's name to a kernel: on
// the host it is a stand-in, not a device address. Its device address is
// taken once per device with hipGetSymbolAddress, with that device current,
// and kept in a per-device table.
#include <mutex>

#include "common.h"

namespace zebra {

namespace {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

std::mutex g_mutex;
void* g_ptr[kMaxDevices] = {};

}  // namespace

// The current device's copy of the scratch array (its device address), taken
// on the first call per device; nullptr and the HIP error otherwise.
hipError_t noalloc_scratch(void** out) {
  *out = nullptr;
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace zebra
