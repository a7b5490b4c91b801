// Device scratch of moe_layer_forward_noalloc: the per-call regions (staged
// rows and routes, compaction, FC1 output, FC2 rows, tile list, header) of
// one call live in this file-scope array instead of a caller workspace, for
// callers that cannot allocate device memory.  Each device the library runs
// on holds its own copy until the process ends.
//
// In host code `scratch` names a host-side stand-in, not a device address:
// the device address is looked up once per device with
// hipGetSymbolAddress, on that device, and only that pointer is ever passed
// to kernels or copies.
#include <hip/hip_runtime.h>

#include <mutex>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;  // 64 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices];

}  // namespace

int noalloc_scratch(uint8_t** base, size_t* bytes) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return -1;
    g_ptr[dev] = p;
  }
  *base = static_cast<uint8_t*>(g_ptr[dev]);
  *bytes = kScratchBytes;
  return 0;
}

}  // namespace moe
