// Band geometry and workspace layout shared by the host launchers and the
// kernels.  A "strip" is 16 consecutive rows (or columns); a "block" is the
// 8 strips (128 rows) one workgroup of 8 waves handles.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sinkattn {

constexpr int kStrip = 16;          // rows per strip = MFMA tile edge
constexpr int kWaves = 8;           // waves per workgroup in the row sweeps
constexpr int kBlockRows = kStrip * kWaves;  // 128
constexpr int kMaxTiles = 17;       // register-resident column tiles per strip
constexpr int kBwdWaves = 4;        // waves per workgroup in the backward sweeps
constexpr int kBwdBlock = kStrip * kBwdWaves;  // 64
constexpr int kTargetGroups = 256;  // one segment workgroup per CU of an MI355X

struct Geom {
  int B, H, L, d;
  int h1, h2;      // band offsets j - i in [-h1, h2] (clamped to L - 1)
  int TL, TR;      // column tiles left/right of a row strip's own tile
  int NT;          // tiles per row strip = TL + TR + 1 (a compiled instance size;
                   // TR is extended so, the surplus tiles lie outside the band)
  int tin_lo, tin_hi;  // strip tiles [tin_lo, tin_hi] lie entirely inside the band
  unsigned edge_mask;  // bit t set: strip tile t (t < NT) crosses a band edge
  int TLc, TRc;    // row tiles above/below a column strip's own tile
  int NTc;         // tiles per column strip = TLc + TRc + 1
  int nblk;        // 128-row blocks per sequence
  int NWC;         // window columns of a 128-row block = 16 * (TL + TR + 8)
  int SB;          // blocks per segment (one workgroup sweeps a segment)
  int nseg;        // segments per sequence = ceil(nblk / SB)
  int SW;          // window columns of a segment = SB * 128 + 16 * (TL + TR)
  int dustbin;
  const int* lengths;  // device int32[B] or nullptr
  float scale2;    // log2(e) / sqrt(d): scores in log2 units
  float inv_sqrt_d;
};

__host__ __device__ inline int ceil_div_pos(int a, int b) { return (a + b - 1) / b; }

// Real-token count of sequence bb, clamped so that every index stays in range.
__device__ inline int real_len(const Geom& g, int bb) {
  int cap = g.L - (g.dustbin ? 1 : 0);
  int n = g.lengths ? g.lengths[bb] : cap;
  n = n < 0 ? 0 : n;
  return n > cap ? cap : n;
}

// Workspace carve-up.  Potentials (the Sinkhorn state) are fp64 in log2
// units; partial sums and backward vectors are fp32.  Sizes in floats.
struct Workspace {
  double* tail_u;  // [R+1][BHL] u^(0..R)
  double* tail_v;  // [R+1][BHL] v^(0..R)
  double* ubuf;    // [2][BHL] u^(t) by step parity (slot t & 1)
  double* vbuf;    // [2][BHL] ping-pong v
  double* dstate;  // [BH][4]  dustbin (u, v, row shift, h)
  float* part;     // [2][BH][nseg][SW] column partial sums
  float* partd;    // [2][BH][nseg]     dustbin-column partial sums
  float* sdr;      // [BHL] dustbin row scores (log2 units)
  float* sdc;      // [BHL] dustbin column scores (log2 units)
  float* bw;       // backward vectors [(3R + 8) * BHL]
  double* err;     // [BH] base convergence check (row-marginal L1 error)
  double* red;     // [kRedParts][2] + [kMaxCertR + 1][4] norm reductions of the tail certificate
  int* prog;       // [2 * BH * nseg + 2] persistent step kernel: per-segment head and done steps, then an
                   // error flag (a neighbour wait gave up) and the debug check's non-finite count
  float* dpart;    // [BH][ceil(L / 256)][d] dustbin row / column sums per chunk of 256 tokens (dustbin only)
  size_t floats;
};

inline size_t align64(size_t n) { return (n + 63) & ~size_t(63); }

constexpr int kRedParts = 1024;  // workgroups of the certificate's norm reduction
constexpr int kMaxCertR = 8;     // deepest tail the certificate compares against

inline Workspace carve(float* base, const Geom& g, int R) {
  const size_t BHL = (size_t)g.B * g.H * g.L;
  const size_t BH = (size_t)g.B * g.H;
  Workspace w{};
  size_t off = 0;
  auto take = [&](size_t n) { float* p = base ? base + off : nullptr; off += align64(n); return p; };
  auto take_d = [&](size_t n) { return reinterpret_cast<double*>(take(2 * n)); };
  w.tail_u = take_d((size_t)(R + 1) * BHL);
  w.tail_v = take_d((size_t)(R + 1) * BHL);
  w.ubuf = take_d(2 * BHL);
  w.vbuf = take_d(2 * BHL);
  w.dstate = take_d(4 * BH);
  w.part = take(2 * BH * (size_t)g.nseg * g.SW);
  w.partd = take(2 * BH * (size_t)g.nseg);
  w.sdr = take(BHL);
  w.sdc = take(BHL);
  w.bw = take((size_t)(3 * R + 8) * BHL);
  w.err = take_d(BH);
  w.red = take_d(2 * kRedParts + 4 * (kMaxCertR + 1));
  w.prog = reinterpret_cast<int*>(take(2 * BH * (size_t)g.nseg + 2));
  w.dpart = take(g.dustbin ? BH * (size_t)((g.L + 255) / 256) * g.d : 0);
  w.floats = off;
  return w;
}

// Launch attributes, cached per (device, kernel) on the host so that a call
// pays no attribute or occupancy query after the first one.
// ensure_lds: raise the kernel's dynamic LDS limit to at least `lds` bytes
// (hipFuncSetAttribute, once per kernel, device and larger size).
// coop_groups: how many workgroups of `threads` threads and `lds` bytes can be
// resident at once on the current device (occupancy x CUs), 0 when it
// cannot launch cooperatively.
hipError_t ensure_lds(const void* kernel, size_t lds);
hipError_t coop_groups(const void* kernel, int threads, size_t lds, long long* groups);

// Launch timing of the fused step kernel (diagnostic; see
// sinkattn_timing_enable).  timing_mark records the start (end = false) or
// end (end = true) event of a bracket on `st` covering `launches` step-kernel
// launches (counted at the end mark); no-op when disabled.
bool timing_enabled();
void timing_mark(hipStream_t st, bool end, int launches = 1);

// Early stop of the stopped base (see sinkattn_forward_converge): check
// every `every` steps (0 = fixed T); the base length used goes to *T_used.
struct BaseStop {
  int every;
  double tol;
  int* T_used;       // host pointer
  double* err_last;  // host pointer, optional: largest per-(b, h) error at the last check
};

// Arguments of the host launchers (device pointers).
struct FwdLaunch {
  const void* Q;
  const void* K;
  const void* V;
  const float* a;
  const float* b;
  float* O;
  float* u;
  float* v;
  int T, R;      // T: base steps (the maximum when stop.every > 0)
  BaseStop stop; // zero-initialised: fixed T
  int* debug_flags;  // host int, or nullptr: when set, the launcher waits for the
                     // stream and reports bit 0 (non-finite u^(0), v^(0), u or v on
                     // an active token) and bit 1 (a neighbour wait gave up)
};

struct BwdLaunch {
  const void* Q;
  const void* K;
  const void* V;
  const void* dO;
  const float* O;
  const float* a;
  const float* b;
  float* dQ;
  float* dK;
  float* dV;
  float* vbar0;
  int T, R;
  int slot0;  // tail-stack slot of this pass's u^(0), v^(0): R_fwd - R when the
              // forward kept a deeper tail R_fwd (0 otherwise)
  int grad_only;  // nonzero: only dQ and dK, from the adjoint vectors that a full
                  // pass of depth R_vec (>= R, same forward) left in the workspace
  int R_vec;
};

}  // namespace sinkattn
