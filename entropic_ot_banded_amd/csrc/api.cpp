// C-ABI of the banded Sinkhorn attention library: argument validation, band
// geometry, workspace layout and the stream-ordered launch sequence.  Every
// check here runs on the host before anything is enqueued, so a bad call
// returns a status code without touching the device.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdlib>
#include <cstdint>
#include <map>
#include <mutex>
#include <vector>

#include "../../include/sinkattn.h"
#include "abi_internal.hpp"
#include "geom.hpp"

namespace sinkattn {

hipError_t launch_forward(const Geom& g, int dtype, const FwdLaunch& f, const Workspace& w, hipStream_t st);
hipError_t launch_backward(const Geom& g, int dtype, const BwdLaunch& f, const Workspace& w, hipStream_t st);
hipError_t launch_block_diameters(const Geom& g, int dtype, const void* Q, const void* K, int Bd, float* delta,
                                  float* kappa, hipStream_t st);
hipError_t launch_certificate(const Geom& g, int dtype, const BwdLaunch& base, int R_max, const Workspace& w,
                              float* dQs, float* dKs, double* eta, hipStream_t st);
hipError_t launch_peak_probes(double* mfma_flops, double* exps, double* clock_hz, hipStream_t st);
hipError_t launch_lds_probe(int row_stride, int swizzle, double* cycles_per_read, hipStream_t st);

namespace {

constexpr int kMaxTailBackward = 8;

bool dtype_d_supported(int dtype, int d) {
  if (dtype == SINKATTN_F32) return d == 16 || d == 32 || d == 64;
  if (dtype == SINKATTN_BF16) return d == 32 || d == 64 || d == 128;
  return false;
}

}  // namespace

// Validate the shape descriptor; fill the band geometry for band width W.
int make_geom(const sinkattn_shape* s, int W, Geom* g) {
  if (!s) return SINKATTN_EINVAL;
  if (s->B < 1 || s->H < 1 || s->L < 1 || s->d < 1) return SINKATTN_EINVAL;
  if (s->dtype != SINKATTN_F32 && s->dtype != SINKATTN_BF16) return SINKATTN_EINVAL;
  if (W < 1) return SINKATTN_EINVAL;
  if (s->dustbin && !s->lengths) return SINKATTN_EINVAL;  // dustbin index n_b needs n_b < L
  const long long bhl = (long long)s->B * s->H * s->L;
  if (bhl * s->d > (long long)INT_MAX * 4 || bhl > INT_MAX) return SINKATTN_EUNSUPPORTED;
  // per-(b, h) kernels index B H on the grid's y dimension (at most 65535)
  if ((long long)s->B * s->H > 65535) return SINKATTN_EUNSUPPORTED;
  // row offsets within one (b, h) slice of Q, K, V, dO are 32-bit
  const long long esize = s->dtype == SINKATTN_BF16 ? 2 : 4;
  if ((long long)s->L * s->d * esize > INT_MAX) return SINKATTN_EUNSUPPORTED;
  if (!dtype_d_supported(s->dtype, s->d)) return SINKATTN_EUNSUPPORTED;
  Geom x{};
  x.B = s->B;
  x.H = s->H;
  x.L = s->L;
  x.d = s->d;
  int h1 = W / 2, h2 = (W + 1) / 2 - 1;
  // offsets beyond L - 1 never occur: clamp (keeps W >= 2L - 1 cheap)
  if (h1 > s->L - 1) h1 = s->L - 1;
  if (h2 > s->L - 1) h2 = s->L - 1;
  x.h1 = h1;
  x.h2 = h2;
  x.TL = (h1 + 15) / 16;
  x.TR = (15 + h2) / 16;
  x.NT = x.TL + x.TR + 1;
  x.TLc = (h2 + 15) / 16;
  x.TRc = (15 + h1) / 16;
  x.NTc = x.TLc + x.TRc + 1;
  // the band must fit the compiled tile counts (checked before the per-tile
  // bit mask below is formed)
  if (x.NT > kMaxTiles || x.NTc > kMaxTiles) return SINKATTN_EUNSUPPORTED;
  // round the row-sweep tile count up to a compiled instance (3, 5, 9, 17)
  {
    const int inst[4] = {3, 5, 9, kMaxTiles};
    for (int k = 0; k < 4; ++k)
      if (x.NT <= inst[k]) {
        x.TR += inst[k] - x.NT;
        x.NT = inst[k];
        break;
      }
  }
  // tile t holds offsets [16 (t - TL) - 15, 16 (t - TL) + 15]: interior when
  // that range lies inside [-h1, h2]
  {
    auto fdiv = [](int a, int b) { return a >= 0 ? a / b : -((-a + b - 1) / b); };
    x.tin_lo = x.TL - fdiv(h1 - 15, 16);
    x.tin_hi = x.TL + fdiv(h2 - 15, 16);
    x.edge_mask = 0u;
    for (int t = 0; t < x.NT; ++t)
      if (t < x.tin_lo || t > x.tin_hi) x.edge_mask |= 1u << t;
  }
  // per-(b, h) slices are addressed with 32-bit byte offsets
  if ((long long)s->L * s->d * (s->dtype == SINKATTN_BF16 ? 2 : 4) >= (1ll << 31)) return SINKATTN_EUNSUPPORTED;
  x.nblk = (s->L + kBlockRows - 1) / kBlockRows;
  x.NWC = 16 * (x.TL + x.TR + kWaves);
  // Segments: a workgroup sweeps SB consecutive blocks so the K window slides
  // (128 new rows per block) instead of being re-read; aim at one workgroup
  // per CU.
  {
    const long long total = (long long)s->B * s->H * x.nblk;
    long long sb = (total + kTargetGroups - 1) / kTargetGroups;
    if (sb < 1) sb = 1;
    if (sb > x.nblk) sb = x.nblk;
    x.SB = (int)sb;
  }
  x.nseg = (x.nblk + x.SB - 1) / x.SB;
  x.SW = x.SB * kBlockRows + 16 * (x.TL + x.TR);
  x.dustbin = s->dustbin ? 1 : 0;
  x.lengths = s->lengths;
  x.inv_sqrt_d = 1.0f / std::sqrt((float)s->d);
  x.scale2 = 1.4426950408889634f * x.inv_sqrt_d;
  *g = x;
  return SINKATTN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

namespace {
// Diagnostic launch timing: a reusable pool of events, used in pairs.
struct TimingState {
  bool on = false;
  std::vector<hipEvent_t> pool;
  std::vector<int> launches;  // per bracket (start/end event pair)
  size_t used = 0;            // events recorded since the last collect
  bool failed = false;
};
TimingState& timing() {
  static TimingState t;
  return t;
}

}  // namespace

namespace {
struct AttrKey {
  int dev;
  const void* kernel;
  size_t lds;
  int threads;
  bool operator<(const AttrKey& o) const {
    if (dev != o.dev) return dev < o.dev;
    if (kernel != o.kernel) return kernel < o.kernel;
    if (lds != o.lds) return lds < o.lds;
    return threads < o.threads;
  }
};
std::mutex g_attr_mu;
std::map<AttrKey, size_t> g_lds_set;       // (dev, kernel) -> largest limit set
std::map<AttrKey, long long> g_coop;       // (dev, kernel, lds, threads) -> resident groups
}  // namespace

hipError_t ensure_lds(const void* kernel, size_t lds) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_attr_mu);
  const AttrKey k{dev, kernel, 0, 0};
  auto it = g_lds_set.find(k);
  if (it != g_lds_set.end() && it->second >= lds) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e == hipSuccess) g_lds_set[k] = lds;
  return e;
}

hipError_t coop_groups(const void* kernel, int threads, size_t lds, long long* groups) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_attr_mu);
  const AttrKey k{dev, kernel, lds, threads};
  auto it = g_coop.find(k);
  if (it != g_coop.end()) {
    *groups = it->second;
    return hipSuccess;
  }
  int coop = 0, cus = 0, per = 0;
  e = hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, threads, lds);
  if (e != hipSuccess) return e;
  *groups = coop ? (long long)per * cus : 0;
  g_coop[k] = *groups;
  return hipSuccess;
}

bool timing_enabled() { return timing().on; }

void timing_mark(hipStream_t st, bool end, int launches) {
  TimingState& t = timing();
  if (end) t.launches.push_back(launches);  // events alternate start, end
  if (t.used == t.pool.size()) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) {
      t.failed = true;
      return;
    }
    t.pool.push_back(e);
  }
  if (hipEventRecord(t.pool[t.used], st) != hipSuccess) t.failed = true;
  ++t.used;
}
}  // namespace sinkattn

using namespace sinkattn;

namespace {
// the HIP error behind the calling thread's last SINKATTN_EHIP status
thread_local hipError_t g_last_hip = hipSuccess;
}  // namespace

namespace sinkattn {
int hip_status(hipError_t e) {
  if (e == hipSuccess) return SINKATTN_OK;
  g_last_hip = e;
  return SINKATTN_EHIP;
}

// SINKATTN_DEBUG set to anything but "" or "0": the forward entry points
// check their results (read at every call)
bool debug_checks() {
  const char* e = std::getenv("SINKATTN_DEBUG");
  return e && e[0] && !(e[0] == '0' && e[1] == 0);
}

// status of a forward launch, with the debug check's findings
int forward_status(hipError_t e, int flags) {
  if (e == hipErrorInvalidConfiguration) return SINKATTN_EUNSUPPORTED;
  if (e != hipSuccess) return hip_status(e);
  if (flags & 2) return SINKATTN_ESTALL;
  if (flags & 1) return SINKATTN_ENONFINITE;
  return SINKATTN_OK;
}
}  // namespace sinkattn

extern "C" {

const char* sinkattn_last_hip_error(void) { return hipGetErrorName(g_last_hip); }

int sinkattn_version(void) { return 10100; }  // 1.1.0: sinkattn_measure_lds

const char* sinkattn_status_string(int status) {
  switch (status) {
    case SINKATTN_OK: return "ok";
    case SINKATTN_EINVAL: return "invalid argument";
    case SINKATTN_EUNSUPPORTED: return "unsupported configuration (outside the built kernels' envelope)";
    case SINKATTN_EHIP: return "HIP runtime or launch error";
    case SINKATTN_EWORKSPACE: return "workspace too small";
    case SINKATTN_ENONFINITE: return "non-finite potentials on active tokens (SINKATTN_DEBUG check)";
    case SINKATTN_ESTALL: return "a neighbour wait of the persistent step launch gave up: results invalid";
    case SINKATTN_ESCRATCH: return "the call needs more device memory than the static scratch of sinkattn_forward_noalloc";
    default: return "unknown status";
  }
}

int sinkattn_timing_enable(int on) {
  TimingState& t = timing();
  int status = SINKATTN_OK;
  if (!on) {
    // release the event pool: no HIP object of the library outlives the
    // timing session (events still pending are released once they complete)
    for (hipEvent_t e : t.pool) {
      const hipError_t r = hipEventDestroy(e);
      if (r != hipSuccess && status == SINKATTN_OK) status = hip_status(r);
    }
    t.pool.clear();
  }
  t.on = on != 0;
  t.used = 0;
  t.launches.clear();
  t.failed = false;
  return status;
}

int sinkattn_timing_collect(double* total_ms, long long* launches) {
  if (!total_ms || !launches) return SINKATTN_EINVAL;
  TimingState& t = timing();
  double sum = 0.0;
  long long count = 0;
  int status = t.failed ? SINKATTN_EHIP : SINKATTN_OK;
  for (size_t k = 0; k + 1 < t.used; k += 2) {
    hipError_t e = hipEventSynchronize(t.pool[k + 1]);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, t.pool[k], t.pool[k + 1]);
    if (e != hipSuccess) {
      status = hip_status(e);
      break;
    }
    sum += ms;
    count += k / 2 < t.launches.size() ? t.launches[k / 2] : 1;
  }
  *total_ms = sum;
  *launches = count;
  t.used = 0;
  t.launches.clear();
  t.failed = false;
  return status;
}

size_t sinkattn_workspace_bytes(const sinkattn_shape* s, int W, int R) {
  Geom g;
  if (R < 0 || make_geom(s, W, &g) != SINKATTN_OK) return 0;
  return carve(nullptr, g, R).floats * sizeof(float);
}

size_t sinkattn_tail_offset(const sinkattn_shape* s, int R, int r, int is_v) {
  if (!s || R < 0 || r < 0 || r > R || s->B < 1 || s->H < 1 || s->L < 1) return (size_t)-1;
  const size_t BHL = (size_t)s->B * s->H * s->L;
  const size_t u_block = align64(2 * (size_t)(R + 1) * BHL) * sizeof(float);  // fp64 slots
  return (is_v ? u_block : 0) + (size_t)r * BHL * sizeof(double);
}

int sinkattn_forward(const void* Q, const void* K, const void* V, int W, int T, int R, const float* a,
                     const float* b, const sinkattn_shape* s, float* O, float* u, float* v, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
  if (!Q || !K || !V || !a || !b || !O || !u || !v || !workspace) return SINKATTN_EINVAL;
  if (T < 0 || R < 0) return SINKATTN_EINVAL;
  Geom g;
  int st = make_geom(s, W, &g);
  if (st != SINKATTN_OK) return st;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(workspace))
    return SINKATTN_EINVAL;
  Workspace w = carve(static_cast<float*>(workspace), g, R);
  if (workspace_bytes < w.floats * sizeof(float)) return SINKATTN_EWORKSPACE;
  FwdLaunch f{Q, K, V, a, b, O, u, v, T, R};
  int flags = 0;
  if (debug_checks()) f.debug_flags = &flags;
  return forward_status(launch_forward(g, s->dtype, f, w, stream), flags);
}

int sinkattn_forward_converge(const void* Q, const void* K, const void* V, int W, int T_max, int R,
                              const float* a, const float* b, const sinkattn_shape* s, double tol,
                              int check_every, float* O, float* u, float* v, void* workspace,
                              size_t workspace_bytes, int* T_used, double* err_last, hipStream_t stream) {
  if (!Q || !K || !V || !a || !b || !O || !u || !v || !workspace || !T_used) return SINKATTN_EINVAL;
  if (T_max < 0 || R < 1 || check_every < 1 || !(tol >= 0.0)) return SINKATTN_EINVAL;
  Geom g;
  int st = make_geom(s, W, &g);
  if (st != SINKATTN_OK) return st;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(workspace))
    return SINKATTN_EINVAL;
  Workspace w = carve(static_cast<float*>(workspace), g, R);
  if (workspace_bytes < w.floats * sizeof(float)) return SINKATTN_EWORKSPACE;
  FwdLaunch f{Q, K, V, a, b, O, u, v, T_max, R};
  f.stop.every = check_every;
  f.stop.tol = tol;
  f.stop.T_used = T_used;
  f.stop.err_last = err_last;
  int flags = 0;
  if (debug_checks()) f.debug_flags = &flags;
  return forward_status(launch_forward(g, s->dtype, f, w, stream), flags);
}

int sinkattn_backward(const void* Q, const void* K, const void* V, int W, int T, int R, const float* a,
                      const float* b, const sinkattn_shape* s, const float* O, const void* dO, void* workspace,
                      size_t workspace_bytes, float* dQ, float* dK, float* dV, float* vbar0,
                      hipStream_t stream) {
  if (!Q || !K || !V || !a || !b || !O || !dO || !workspace || !dQ || !dK || !dV) return SINKATTN_EINVAL;
  if (T < 0 || R < 0) return SINKATTN_EINVAL;
  if (R > kMaxTailBackward) return SINKATTN_EUNSUPPORTED;
  Geom g;
  int st = make_geom(s, W, &g);
  if (st != SINKATTN_OK) return st;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(dO) || !aligned16(dQ) ||
      !aligned16(dK) || !aligned16(dV) || !aligned16(workspace))
    return SINKATTN_EINVAL;
  Workspace w = carve(static_cast<float*>(workspace), g, R);
  if (workspace_bytes < w.floats * sizeof(float)) return SINKATTN_EWORKSPACE;
  BwdLaunch f{Q, K, V, dO, O, a, b, dQ, dK, dV, vbar0, T, R};
  hipError_t e = launch_backward(g, s->dtype, f, w, stream);
  if (e == hipErrorInvalidConfiguration) return SINKATTN_EUNSUPPORTED;
  return hip_status(e);
}

int sinkattn_tail_certificate(const void* Q, const void* K, const void* V, int W, int T, int R_max, const float* a,
                              const float* b, const sinkattn_shape* s, const float* O, const void* dO,
                              void* workspace, size_t workspace_bytes, float* dQ, float* dK, float* dV,
                              float* dQ_scratch, float* dK_scratch, double* eta, double tau, int* R_selected,
                              hipStream_t stream) {
  if (!Q || !K || !V || !a || !b || !O || !dO || !workspace || !dQ || !dK || !dV || !dQ_scratch ||
      !dK_scratch || !eta)
    return SINKATTN_EINVAL;
  if (T < 0 || R_max < 1 || !(tau >= 0.0)) return SINKATTN_EINVAL;
  if (R_max > kMaxTailBackward || R_max > kMaxCertR) return SINKATTN_EUNSUPPORTED;
  Geom g;
  int st = make_geom(s, W, &g);
  if (st != SINKATTN_OK) return st;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(dO) || !aligned16(dQ) ||
      !aligned16(dK) || !aligned16(dV) || !aligned16(dQ_scratch) || !aligned16(dK_scratch) || !aligned16(workspace))
    return SINKATTN_EINVAL;
  Workspace w = carve(static_cast<float*>(workspace), g, R_max);
  if (workspace_bytes < w.floats * sizeof(float)) return SINKATTN_EWORKSPACE;
  BwdLaunch f{Q, K, V, dO, O, a, b, dQ, dK, dV, nullptr, T, R_max};
  hipError_t e = launch_certificate(g, s->dtype, f, R_max, w, dQ_scratch, dK_scratch, eta, stream);
  if (e == hipErrorInvalidConfiguration) return SINKATTN_EUNSUPPORTED;
  if (e != hipSuccess) return hip_status(e);
  if (R_selected) {
    // the smallest depth whose residual is below tau; the deepest when none is
    int sel = R_max;
    for (int r = 0; r <= R_max; ++r)
      if (eta[r] < tau) {
        sel = r;
        break;
      }
    *R_selected = sel;
  }
  return SINKATTN_OK;
}

int sinkattn_block_contraction(const void* Q, const void* K, int W, const sinkattn_shape* s, int block,
                               float* delta, float* kappa, hipStream_t stream) {
  if (!Q || !K || !delta) return SINKATTN_EINVAL;
  Geom g;
  int st = make_geom(s, W, &g);
  if (st != SINKATTN_OK) return st;
  // the block must lie wholly inside the band (a strictly positive kernel)
  const int inside = (g.h1 < g.h2 ? g.h1 : g.h2) + 1;
  if (block < 1 || block > 128 || block > inside) return SINKATTN_EINVAL;
  hipError_t e = launch_block_diameters(g, s->dtype, Q, K, block, delta, kappa, stream);
  if (e == hipErrorInvalidConfiguration) return SINKATTN_EUNSUPPORTED;
  return hip_status(e);
}

int sinkattn_measure_peaks(double* mfma_bf16_flops, double* exp_per_s, double* clock_hz, hipStream_t stream) {
  if (!mfma_bf16_flops || !exp_per_s) return SINKATTN_EINVAL;
  return hip_status(launch_peak_probes(mfma_bf16_flops, exp_per_s, clock_hz, stream));
}

int sinkattn_measure_lds(int row_stride, int swizzle, double* cycles_per_read, hipStream_t stream) {
  if (!cycles_per_read) return SINKATTN_EINVAL;
  const bool ok = swizzle ? (swizzle == 1 && row_stride == 256)
                          : (row_stride >= 256 && row_stride <= 320 && row_stride % 16 == 0);
  if (!ok) return SINKATTN_EINVAL;
  return hip_status(launch_lds_probe(row_stride, swizzle, cycles_per_read, stream));
}

}  // extern "C"
