// The static device array behind emu_allreduce_noalloc: the entry point for
// callers that cannot allocate device memory keeps its tables (fused tiles
// and order rows, stepwise tasks, loop blocks and tree records) and its LL
// status word here instead of in buffers the library allocates.
//
// Each device holds its own copy of the array from module load until the
// process ends.  In host code `scratch` is only a stand-in for the symbol:
// the device address of a device's copy comes from hipGetSymbolAddress,
// looked up once per device with that device current, and only that
// address is ever handed to kernels or copies.
#include <hip/hip_runtime.h>

#include <map>

#include "common.h"

namespace emu {

constexpr size_t kScratchBytes = (size_t)4 << 20;
static_assert(kScratchBytes == EMU_NOALLOC_SCRATCH_BYTES, "scratch size as declared in the header");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

size_t scratch_bytes() { return kScratchBytes; }

// Never destroyed (the library's state outlives the exit-time destructors).
static std::map<int, void*>& scratch_addrs = *new std::map<int, void*>();

// The address of `dev`'s copy of the array; `dev` must be the current
// device.  With create == false, only an address looked up before is
// reported (nullptr otherwise) and the runtime is not called.
hipError_t scratch_address(int dev, bool create, void** out) {
  *out = nullptr;
  auto it = scratch_addrs.find(dev);
  if (it != scratch_addrs.end()) {
    *out = it->second;
    return hipSuccess;
  }
  if (!create) return hipSuccess;
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (!p) return hipErrorInvalidSymbol;
  scratch_addrs[dev] = p;
  *out = p;
  return hipSuccess;
}

}  // namespace emu
