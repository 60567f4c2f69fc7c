// Host-only stand-ins for the kernel launchers, so that the C-ABI's
// validation layer (api.cpp) links into a sanitizer build without device
// code.  Every case the driver runs must be rejected before any launch: a
// call here records itself and fails.
#include <hip/hip_runtime_api.h>

#include "geom.hpp"

int g_stub_calls = 0;

namespace sinkattn {
hipError_t launch_forward(const Geom&, int, const FwdLaunch&, const Workspace&, hipStream_t) {
  ++g_stub_calls;
  return hipErrorInvalidValue;
}
hipError_t launch_backward(const Geom&, int, const BwdLaunch&, const Workspace&, hipStream_t) {
  ++g_stub_calls;
  return hipErrorInvalidValue;
}
hipError_t launch_block_diameters(const Geom&, int, const void*, const void*, int, float*, float*, hipStream_t) {
  ++g_stub_calls;
  return hipErrorInvalidValue;
}
hipError_t launch_certificate(const Geom&, int, const BwdLaunch&, int, const Workspace&, float*, float*, double*,
                              hipStream_t) {
  ++g_stub_calls;
  return hipErrorInvalidValue;
}
hipError_t launch_peak_probes(double*, double*, double*, hipStream_t) {
  ++g_stub_calls;
  return hipErrorInvalidValue;
}
hipError_t launch_lds_probe(int, int, double*, hipStream_t) {
  ++g_stub_calls;
  return hipErrorInvalidValue;
}
}  // namespace sinkattn
