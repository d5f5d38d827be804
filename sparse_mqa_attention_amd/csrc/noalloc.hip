// The whole step without a caller workspace, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid allocation): its
// scratch is a fixed array of this library, one per device.
#include "dsa_internal.h"

namespace dsa {

// Scratch of dsa_sparse_attn_step_noalloc: the workspace header (rendezvous counters, zero when
// the code object loads and left zero by every call) followed by the decode kernels' P and stats
// or the general kernel's split partials.
constexpr size_t kScratchBytes = DSA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes >= kWsHeaderBytes, "the scratch holds at least the workspace header");
static_assert(DSA_WORKSPACE_HEADER_BYTES == kWsHeaderBytes, "the header size the ABI states");

__device__ __align__(256) unsigned char scratch[kScratchBytes];

// Called by dsa_init with `dev` current: the array's device address on this device (host code
// must not pass the array's own name to a kernel, it is a host-side stand-in).
int scratch_device_init(int dev, DeviceState& ds) {
  void* ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || ptr == nullptr)
    return fail(DSA_ERR_HIP, "dsa_init: scratch address on device %d: %s", dev, hipGetErrorString(e));
  ds.scratch = ptr;
  return DSA_OK;
}

size_t scratch_bytes() { return kScratchBytes; }

}  // namespace dsa
