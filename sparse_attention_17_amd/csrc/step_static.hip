// The decode step with its scratch in a static device array instead of a
// caller-provided workspace, for callers that cannot allocate device memory
// (code under HIP graph capture, serving loops that forbid allocation).
// Each device holds one array of CSA_STEP_SCRATCH_BYTES for the life of the
// process; every call on a device uses that device's array, so calls that
// overlap on one device race.  The step's kernels write every scratch word
// they later read within the same call, so nothing needs clearing.
#include "csa_mi355x.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"

namespace {

static __device__ __align__(256) unsigned char scratch[CSA_STEP_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

// The device address of this device's array: the array's name is only a
// host-side stand-in, so its address is looked up once per device, with that
// device current.
hipError_t scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
  });
  *out = g_ptr[dev];
  return g_err[dev];
}

}  // namespace

extern "C" csa_status_t csa_hybrid_decode_step_static(const csa_decode_step_t* step, void* stream) {
  if (step == nullptr) return csa::set_error(CSA_INVALID_ARGUMENT, "step must not be NULL");
  const size_t need = csa_hybrid_decode_step_workspace(step);
  if (need > (size_t)CSA_STEP_SCRATCH_BYTES)
    return csa::set_error(CSA_WORKSPACE_TOO_SMALL,
                          "the step needs %zu bytes of scratch; the static array holds %zu",
                          need, (size_t)CSA_STEP_SCRATCH_BYTES);
  void* ptr = nullptr;
  const hipError_t e = scratch_ptr(&ptr);
  if (e != hipSuccess || ptr == nullptr)
    return csa::set_error(CSA_DEVICE_ERROR, "locating the static scratch array: %s", hipGetErrorString(e));
  return csa_hybrid_decode_step(step, ptr, (size_t)CSA_STEP_SCRATCH_BYTES, stream);
}
