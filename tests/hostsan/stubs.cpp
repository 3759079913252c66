// Host-only stand-ins for the kernel launchers and the few HIP runtime calls of the C ABI layer, so
// that abi.cpp and plans.cpp can be built and exercised under the address and undefined-behaviour
// sanitizers on a machine without a GPU: every launcher accepts its arguments and launches
// nothing, and the runtime reports one device with 256 compute units.
#include "internal.h"

extern "C" {
hipError_t hipGetDevice(int* device) {
  *device = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t, int) {
  *value = 256;
  return hipSuccess;
}
const char* hipGetErrorString(hipError_t) { return "stub"; }
}

namespace lr {
hipError_t launch_decode(const DecodePlan&, const lr_layer_cache*, const void*, void*, int, void*, hipStream_t,
                         hipEvent_t, hipEvent_t, const void*, const void*, const void*, const void*) {
  return hipSuccess;
}
hipError_t launch_decode_step(const AppendPlan&, const DecodePlan&, const lr_layer_cache*, const void*, const void*,
                              const void*, void*, int, void*, hipStream_t, hipEvent_t, hipEvent_t) {
  return hipSuccess;
}
hipError_t launch_append(const AppendPlan&, const lr_layer_cache*, const void*, const void*, float*, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_store(const AppendPlan&, const lr_layer_cache*, int64_t, int64_t, const float*, const float*,
                        hipStream_t) {
  return hipSuccess;
}
hipError_t launch_dequant(const AppendPlan&, const lr_layer_cache*, int64_t, float*, float*, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_rebase(const RebasePlan&, const lr_layer_cache*, const lr_layer_cache*, const void*, const void*,
                         hipStream_t) {
  return hipSuccess;
}
hipError_t launch_sens_svd(const void*, const float*, int, int, int, int, int, void*, int, float*, void*,
                           hipStream_t) {
  return hipSuccess;
}
hipError_t launch_rank_allocate(const float*, int, int, long long, int, int, int, int32_t*, void*, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_basis_update(const void*, int, const float*, int, const void*, int, int, int, int, void*, float*,
                               void*, void*, hipStream_t) {
  return hipSuccess;
}
hipError_t noalloc_scratch(void** ptr) {
  static unsigned char host_stand_in[256];
  *ptr = host_stand_in;
  return hipSuccess;
}
}  // namespace lr
