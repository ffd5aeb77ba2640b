// Library-owned device scratch for the allocation-free PDDP entry point
// (mcs_pddp_group_noalloc): a file-scope device array, so a call needs no
// hipMalloc. Each GPU the library runs on holds its own copy, at its own
// address, from the module's load until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device with hipGetSymbolAddress (with
// that device current) and kept; only that address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "mcs_internal.hpp"

namespace {

static __device__ __align__(256) unsigned char scratch[mcs::kScratchBytes];

std::mutex g_mu;
std::vector<void *> g_addr;  // per device ordinal; nullptr until looked up

}  // namespace

namespace mcs {

hipError_t scratch_address(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if ((size_t)dev >= g_addr.size()) g_addr.resize((size_t)dev + 1, nullptr);
  if (!g_addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_addr[dev] = p;
  }
  *out = g_addr[dev];
  return hipSuccess;
}

}  // namespace mcs
