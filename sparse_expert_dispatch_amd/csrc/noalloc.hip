// Library-owned workspace of moe_expert_ffn_packed_noalloc, the packed
// expert FFN for callers that cannot allocate device memory (code under
// graph capture, tight serving loops, harnesses that forbid allocation).
//
// The workspace (the hidden activation H and the grouped GEMMs' tile
// counters) is a file-scope device array, so every GPU the library runs on
// holds its own copy from module load until the process ends.  In host code
// the array's name is only a stand-in: the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current,
// and that address is what the kernels receive, like any workspace pointer.
// Every call on a GPU shares that GPU's array, so calls that overlap on one
// GPU race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/moe_dispatch.h"
#include "kernels.hpp"

namespace moe {

static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace moe
