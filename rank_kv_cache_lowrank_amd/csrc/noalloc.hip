// Device scratch of the allocation-free decode entry point (lowrank_attn_decode_noalloc).
//
// Callers that cannot allocate device memory (code under graph capture, tight serving loops,
// harnesses that forbid hipMalloc) decode through a workspace that lives in this file-scope device
// array instead of one they pass in. The array is part of the library's code object: every GPU the
// library runs on holds its own copy, at its own address, from the first use until the process
// ends. Calls on one GPU share it and the contents persist from call to call; the decode kernels
// need no part of it cleared (their partials and flags are written before they are read within a
// call), and two calls that overlap on one GPU race on it.
#include <mutex>

#include "internal.h"

namespace lr {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

// The device address of this GPU's scratch array, looked up once per device with that device
// current. In host code `scratch` names a host-side stand-in, never the device memory: only the
// address returned here may reach a kernel.
hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr || ((uintptr_t)p & 255u) != 0) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace lr
