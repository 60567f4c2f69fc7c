// Forward pass that allocates nothing: for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid allocation).  Same computation and kernels as sinkattn_forward;
// the workspace is a file-scope device array of fixed size instead of a
// caller buffer.  Each GPU the library runs on holds its own copy of the
// array until the process ends; every call on that GPU reuses it, so calls
// that overlap in time on one GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "abi_internal.hpp"
#include "geom.hpp"

namespace sinkattn {

hipError_t launch_forward(const Geom& g, int dtype, const FwdLaunch& f, const Workspace& w, hipStream_t st);

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;  // 64 MiB per GPU
static_assert(kScratchBytes == SINKATTN_NOALLOC_SCRATCH_BYTES, "header and library agree on the scratch size");

__device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`, resolved once per
// device (the array's name is a host-side stand-in, not a device address).
hipError_t scratch_for_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace
}  // namespace sinkattn

using namespace sinkattn;

extern "C" int sinkattn_forward_noalloc(const void* Q, const void* K, const void* V, int W, int T, int R,
                                        const float* a, const float* b, const sinkattn_shape* s, float* O, float* u,
                                        float* v, hipStream_t stream) {
  if (!Q || !K || !V || !a || !b || !O || !u || !v) return SINKATTN_EINVAL;
  if (T < 0 || R < 0) return SINKATTN_EINVAL;
  Geom g;
  int st = make_geom(s, W, &g);
  if (st != SINKATTN_OK) return st;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return SINKATTN_EINVAL;
  const size_t need = carve(nullptr, g, R).floats * sizeof(float);
  if (need > kScratchBytes) return SINKATTN_ESCRATCH;
  void* ws = nullptr;
  st = hip_status(scratch_for_current_device(&ws));
  if (st != SINKATTN_OK) return st;
  // the kernels clear every counter and buffer they need (progress counters
  // by a fill kernel); what the previous call left in the scratch is not read
  const Workspace w = carve(static_cast<float*>(ws), g, R);
  FwdLaunch f{Q, K, V, a, b, O, u, v, T, R};
  int flags = 0;
  if (debug_checks()) f.debug_flags = &flags;
  return forward_status(launch_forward(g, s->dtype, f, w, stream), flags);
}
