// The static scratch of sparse_mla_fwd_noalloc, the forward for callers that
// cannot allocate device memory, and its per-device address.
//
// The array stands in for the caller-provided workspace of sparse_mla_fwd
// (per-row tile counts, the longest-first row order, split partials).  Each
// device the library runs on holds its own copy until the process ends.  In
// host code the array's name is not a device address: its address on a
// device comes from hipGetSymbolAddress, looked up once per device with that
// device current, and only that address is handed to the kernels.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "smla.h"
#include "smla_internal.h"

namespace smla {

static __device__ __attribute__((aligned(256))) uint8_t scratch[SMLA_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};
}  // namespace

hipError_t noalloc_scratch(int dev, void** out) {
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace smla
