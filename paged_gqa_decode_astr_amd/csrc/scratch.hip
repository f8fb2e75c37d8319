// Library-owned device scratch for the allocation-free decode entry point
// (astr_paged_decode_noalloc): the split kernel's partials (o_part, ml_part)
// live in a file-scope device array instead of a caller workspace, for
// callers that cannot allocate device memory at call time.
//
// Each GPU the library runs on holds its own copy of the array from the first
// call on that device until the process ends.  In host code the array's name
// only stands in for the symbol; its device address comes from
// hipGetSymbolAddress, taken once per device (with that device current) and
// cached here.  Every allocation-free call on a device shares that device's
// copy, so calls that overlap on one GPU (e.g. on two streams) race.  The
// partials need no clearing: every slot the combine kernel reads is written
// by the split kernel of the same call.
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "astr_attn.h"
#include "launch.hpp"

namespace astr {

static __device__ __align__(256) unsigned char scratch[ASTR_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;   // per device id: device address of that device's `scratch`
}  // namespace

hipError_t scratch_buffer(void** out, size_t* bytes) {
  *out = nullptr;
  *bytes = 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  *bytes = ASTR_NOALLOC_SCRATCH_BYTES;
  return hipSuccess;
}

}  // namespace astr
