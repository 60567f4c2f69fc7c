// Forward pass of banded, balanced, log-domain Sinkhorn attention on gfx950.
//
// "Blockwise Differentiable Sinkhorn Attention", section 2.1: T stopped base
// steps and R tail steps of balanced Sinkhorn on the band Omega with
// S = Q K^T / sqrt(d), then O = P V.  Section 2.3: the dustbin row/column is
// active against every active token.
//
// One launch of iter_kernel performs one full Sinkhorn step t (row update
// u^(t) = U(v^(t-1)) and everything the column update v^(t) = V(u^(t)) needs)
// from a single evaluation of the band score tiles:
//   e_ij  = exp(S_ij + v^(t-1)_j - c_i)          (one exp per band entry)
//   rho_i = sum_j e_ij,  u^(t)_i = log a_i - log rho_i - c_i
//   gamma_j (partial) = sum_i e_ij * (a_i / rho_i) = sum_i P^(t,t-1)_ij
// because exp(S_ij + u^(t)_i) = e_ij * a_i / rho_i * exp(-v^(t-1)_j): the
// column log-sum-exp of the column update is a weighted sum of the same
// exponentials, so each step costs one score tile and one exp per entry.
// The per-block column partial sums are finished (v^(t) = v^(t-1) + log b -
// log gamma) at the start of the next launch, in a fixed block order.  Any
// per-row shift c_i cancels both in u^(t) and in a_i / rho_i.
//
// Shifts: c_i is a per-block constant, the value of v^(t-1) at a reference
// column of the block (entries are then exp(S_ij + v_j - v_ref), close to 1
// for a converging iteration); if a row sum leaves [2^-120, 2^120] the strip
// is recomputed with the exact per-row maximum.  The first step (u = v = 0)
// always uses the exact maximum.
//
// Precision: the Sinkhorn state (every potential the kernels keep: latest u,
// ping-pong v, tail stack, dustbin state) is fp64 in log2 units; per-row and
// per-column logs are taken in fp64.  Per-entry work (scores, exp, sums) is
// fp32.  Rounding the state to fp32 each step would bias the neutral gauge
// direction (u + c, v - c) by about one ulp of |log b| per step.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <type_traits>
#include <vector>

#include "common.hpp"
#include "geom.hpp"

namespace sinkattn {

struct IterArgs {
  const void* Q;
  const void* K;
  const float* a;
  const float* b;
  const double* v_prev2;  // v^(t-2), nullptr => zeros
  const float* part_in;   // column partials of step t-1, nullptr => v^(t-1) = 0
  double* v_out;          // v^(t-1), owners write (nullptr when part_in is nullptr)
  double* v_tail;         // optional copy of v^(t-1)
  double* u_out;          // u^(t), owners write
  const double* u_prev;   // u^(t-1) (exact column updates), nullptr when t == 1
  double* u_tail;         // optional copy of u^(t)
  float* part_out;        // [BH][nseg][SW] column partials of step t
  float* partd_out;       // [BH][nseg] dustbin-column partials of step t
  const double* dstate;   // dustbin state after step t-1 (nullptr => zeros)
  const float* sdr;       // dustbin row scores [BHL], log2 units
  const float* sdc;       // dustbin column scores [BHL], log2 units
  int first;              // 1 => step 1: v^(0) = 0 and exact row maxima
  int padded_grid;
};

// One 256-byte row by LDS DMA (a dword per lane): bytes gb + 256 r + 4 lane
// to lds_row + 4 lane.  The instruction's immediate offset (256 r here) is
// added to both the global and the LDS address and must be a compile-time
// constant, hence one case per row r in [0, 16).
__device__ __forceinline__ void dma_row256(const char* gb, char* lds_row, int r) {
  char* l = lds_row - 256 * r;
  switch (r) {
    case 0: __builtin_amdgcn_global_load_lds(gb, l, 4, 0, 0); break;
    case 1: __builtin_amdgcn_global_load_lds(gb, l, 4, 256, 0); break;
    case 2: __builtin_amdgcn_global_load_lds(gb, l, 4, 512, 0); break;
    case 3: __builtin_amdgcn_global_load_lds(gb, l, 4, 768, 0); break;
    case 4: __builtin_amdgcn_global_load_lds(gb, l, 4, 1024, 0); break;
    case 5: __builtin_amdgcn_global_load_lds(gb, l, 4, 1280, 0); break;
    case 6: __builtin_amdgcn_global_load_lds(gb, l, 4, 1536, 0); break;
    case 7: __builtin_amdgcn_global_load_lds(gb, l, 4, 1792, 0); break;
    case 8: __builtin_amdgcn_global_load_lds(gb, l, 4, 2048, 0); break;
    case 9: __builtin_amdgcn_global_load_lds(gb, l, 4, 2304, 0); break;
    case 10: __builtin_amdgcn_global_load_lds(gb, l, 4, 2560, 0); break;
    case 11: __builtin_amdgcn_global_load_lds(gb, l, 4, 2816, 0); break;
    case 12: __builtin_amdgcn_global_load_lds(gb, l, 4, 3072, 0); break;
    case 13: __builtin_amdgcn_global_load_lds(gb, l, 4, 3328, 0); break;
    case 14: __builtin_amdgcn_global_load_lds(gb, l, 4, 3584, 0); break;
    case 15: __builtin_amdgcn_global_load_lds(gb, l, 4, 3840, 0); break;
    default: break;
  }
}

// floor(a / b) for b > 0 and any sign of a.
__device__ __forceinline__ int floor_div(int a, int b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }

// Ring slot of a global 16-row tile inside a window of NWT tiles.  Windows of
// consecutive blocks differ by 8 tiles; the tile that enters takes the slot
// of the tile that leaves.
__device__ __forceinline__ int ring_tile(int tg, int NWT) {
  const int m = tg % NWT;
  return m < 0 ? m + NWT : m;
}

// Inputs of the column finish for one band column j, gathered early so the
// loads overlap compute.  Partial sums of step t-1 come from the (at most
// kMaxSeg) segments whose windows contain j, summed in increasing order.
constexpr int kMaxSeg = 3;
struct VIn {
  double vprev;
  float b;
  float part[kMaxSeg];
  float sdr;       // dustbin-row score s_(delta j) (0 without a dustbin)
  unsigned valid;  // bit k < kMaxSeg: part[k] comes from a segment window
                   // holding j; bit kMaxSeg: vprev holds v^(t-2) (else 0)
};

// Dustbin state of the previous step that the column finish needs: launch
// constants of one (b, h).
struct DustC {
  int on;
  double m;   // shift M of the previous step's dustbin row
  float h;    // a_delta / rho_delta of that row (relative to M)
};

__device__ __forceinline__ DustC load_dust(const Geom& g, int bh, const double* dstate) {
  DustC c{0, 0.0, 0.f};
  if (g.dustbin && dstate) {
    c.on = 1;
    c.m = dstate[4 * bh + 2];
    c.h = (float)dstate[4 * bh + 3];
  }
  return c;
}

// Loads and stores of the values other workgroups of the same launch read
// (column partials, published v): device-scope when COH (the persistent step
// kernel, whose steps run in one launch: no cache may serve a stale copy),
// plain otherwise.
// (COH accesses name the global address space explicitly: their pointers
// may have been read from LDS, and flat accesses would also count against
// the LDS wait counter, forcing full waits on the LDS reads around them.)
template <typename X>
__device__ __forceinline__ __attribute__((address_space(1))) X* gmem(X* p) {
  return (__attribute__((address_space(1))) X*)p;
}
template <bool COH, typename X>
__device__ __forceinline__ X ld_shared(const X* p) {
  if constexpr (COH) return __hip_atomic_load(gmem(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else return *p;
}
template <bool COH, typename X>
__device__ __forceinline__ void st_shared(X* p, X v) {
  if constexpr (COH) __hip_atomic_store(gmem(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}

// Loads only (no arithmetic on the loaded values), so that issuing it does
// not make the wave wait for the data.  Column j lies in the windows of the
// segments [slo, shi].
template <bool COH = false>
// own_seg >= 0: that segment's partial is `own` (the caller holds it) instead
// of being loaded.
__device__ __forceinline__ VIn gather_v_range(const Geom& g, int bh, int n, int j, int slo, int shi,
                                              const double* v_prev2, const float* part_in, const float* b,
                                              int bb, const float* sdr, int own_seg = -1, float own = 0.f) {
  const size_t L = g.L;
  const int segw = g.SB * kBlockRows;
  VIn r;
  r.vprev = v_prev2 ? ld_shared<COH>(v_prev2 + bh * L + j) : 0.0;
  r.b = b[(size_t)bb * L + j];
#pragma unroll
  for (int k = 0; k < kMaxSeg; ++k) {
    const int sg = slo + k;
    r.part[k] = 0.f;
    if (sg <= shi && sg * segw < n)  // segments without real rows wrote nothing
      r.part[k] = sg == own_seg ? own
                                : ld_shared<COH>(part_in + ((size_t)bh * g.nseg + sg) * g.SW + (j - (sg * segw - 16 * g.TL)));
  }
  r.sdr = g.dustbin ? sdr[bh * L + j] : 0.f;
  r.valid = (2u << kMaxSeg) - 1;
  return r;
}

// Same inputs, every load issued unconditionally from an address clamped into
// its buffer (j in [0, L)); `valid` marks the partials that count.  No
// branch and no register written before the loads, so a wave issuing them
// in the middle of other work never waits for earlier loads.
template <bool COH = false>
__device__ __forceinline__ VIn gather_v_clamped(const Geom& g, int bh, int n, int j, int slo, int shi,
                                                const double* v_prev2, const float* part_in, const float* b,
                                                int bb, const float* sdr) {
  const size_t L = g.L;
  const int segw = g.SB * kBlockRows;
  VIn r;
  // v^(t-2) = 0 when v_prev2 is null: load from `b` instead (any readable
  // address; the finish ignores it), so no branch sits before the loads
  // (per-(b, h) base pointers with unsigned 32-bit lane offsets: j >= 0)
  const uint32_t ju = (uint32_t)j;
  const double* vp = v_prev2 ? v_prev2 + bh * L : reinterpret_cast<const double*>(b);
  r.vprev = ld_shared<COH>(vp + (v_prev2 ? ju : 0u));
  r.b = (b + (size_t)bb * L)[ju];
  r.valid = v_prev2 ? 1u << kMaxSeg : 0u;
  const float* pb = part_in + (size_t)bh * g.nseg * g.SW;
#pragma unroll
  for (int k = 0; k < kMaxSeg; ++k) {
    const int sg = slo + k;
    const bool ok = sg <= shi && sg * segw < n;
    const int sgc = sg < g.nseg ? sg : g.nseg - 1;
    int off = j - (sgc * segw - 16 * g.TL);
    off = off < 0 ? 0 : (off >= g.SW ? g.SW - 1 : off);
    r.part[k] = ld_shared<COH>(pb + (uint32_t)(sgc * g.SW + off));
    r.valid |= (ok ? 1u : 0u) << k;
  }
  r.sdr = (sdr + bh * L)[ju];  // always allocated; used only with a dustbin
  return r;
}

// Segment s's window covers columns [s segw - 16 TL, s segw - 16 TL + SW).
__device__ __forceinline__ void window_segments(const Geom& g, int j, int& slo, int& shi) {
  const int segw = g.SB * kBlockRows;
  const int x = j + 16 * g.TL;
  shi = x / segw;
  shi = shi > g.nseg - 1 ? g.nseg - 1 : shi;
  slo = floor_div(x - g.SW, segw) + 1;
  slo = slo < 0 ? 0 : slo;
}

template <bool COH = false>
__device__ __forceinline__ VIn gather_v(const Geom& g, int bh, int n, int j, const double* v_prev2,
                                        const float* part_in, const float* b, int bb, const float* sdr,
                                        int own_seg = -1, float own = 0.f) {
  int slo, shi;
  window_segments(g, j, slo, shi);
  return gather_v_range<COH>(g, bh, n, j, slo, shi, v_prev2, part_in, b, bb, sdr, own_seg, own);
}

// v^(t-1)_j = v^(t-2)_j + log2(b_j / gamma_j), gamma_j = sum_i P^(t-1,t-2)_ij
// (log2 units, fp64 state; the log of a ratio near 1 is taken in fp32).  The
// dustbin row adds its entry of P^(t-1,t-2), exp2(s_(delta j) + v^(t-2)_j - M)
// times a_delta / rho_delta.
// *ok reports whether gamma_j lies in [2^-120, 2^120]; outside that range
// the result is not usable (see finish_checked).
__device__ __forceinline__ double finish_from(const VIn& r, const DustC& dc, bool* ok = nullptr) {
  const double vprev = ((r.valid >> kMaxSeg) & 1u) ? r.vprev : 0.0;
  float gam = 0.f;
#pragma unroll
  for (int k = 0; k < kMaxSeg; ++k) gam += ((r.valid >> k) & 1u) ? r.part[k] : 0.f;
  if (dc.on) gam += exp2_fast((float)((double)r.sdr + vprev - dc.m)) * dc.h;
  if (ok) *ok = gam >= 0x1p-120f && gam <= 0x1p120f;
  return vprev + log2_split(r.b * __builtin_amdgcn_rcpf(gam));
}

// Exact column update of band column j (log2 units, fp64 state):
//   v_j = log2 b_j - log2 sum_{i in Omega^j} 2^(S2_ij + u_i)
// with S2_ij = q_i . k_j log2(e) / sqrt(d) recomputed from Q and K, u the
// row potentials the column update follows (the same step's), and the
// dustbin row (score sdr_j, potential u_n) when there is one.  The finish
// takes it when the row pass's weighted column sum gamma_j leaves
// [2^-120, 2^120]: scores spread so wide that the column's entries underflow
// against their rows' shifts (the column-side counterpart of the row pass's
// exact-maximum fallback).  One thread, a plain loop over the column's rows:
// fp32 scores, an fp64 running maximum, and the sum of 2^(x_i - max) in fp32
// (its terms are at most 1), rescaled whenever the maximum grows.  Slow, and
// reached only for extreme inputs.
template <typename T, bool COH>
__device__ double exact_column_v(const Geom& g, int bh, int n, int j, const char* Qb, const char* Kb,
                                 const double* u, float bj, float sdr_j) {
  const int D = g.d;
  const size_t L = g.L;
  const T* kj = reinterpret_cast<const T*>(Kb) + (size_t)j * D;
  int i0 = j - g.h2, i1 = j + g.h1;
  i0 = i0 < 0 ? 0 : i0;
  i1 = i1 > n - 1 ? n - 1 : i1;
  double m = -__builtin_inf();
  float s = 0.f;
  auto add = [&](double x) {
    if (x > m) {
      s = s * exp2_fast((float)(m - x)) + 1.f;
      m = x;
    } else {
      s += exp2_fast((float)(x - m));
    }
  };
  for (int i = i0; i <= i1; ++i) {
    const T* qi = reinterpret_cast<const T*>(Qb) + (size_t)i * D;
    float acc = 0.f;
    for (int c = 0; c < D; ++c) acc = __builtin_fmaf(Elt<T>::load(qi, c), Elt<T>::load(kj, c), acc);
    add((double)(acc * g.scale2) + ld_shared<COH>(u + bh * L + i));
  }
  if (g.dustbin) add((double)sdr_j + ld_shared<COH>(u + bh * L + n));
  return log2_split(bj) - m - log2_split(s);
}

// v^(t-1)_j from the gathered inputs, or from its exact column log-sum-exp
// when gamma_j is out of range (u_prev: u^(t-1); Qb, Kb: the (b, h) slices).
template <typename T, bool COH>
__device__ __forceinline__ double finish_checked(const Geom& g, const VIn& r, const DustC& dc, int bh, int n, int j,
                                                 const char* Qb, const char* Kb, const double* u_prev) {
  bool ok;
  const double v = finish_from(r, dc, &ok);
  if (ok || !u_prev) return v;
  return exact_column_v<T, COH>(g, bh, n, j, Qb, Kb, u_prev, r.b, r.sdr);
}

template <typename T>
__device__ __forceinline__ double finish_v(const Geom& g, int bh, int n, int j, const double* v_prev2,
                                           const float* part_in, const float* b, int bb,
                                           const double* dstate, const float* sdr, const void* Q, const void* K,
                                           const double* u) {
  const size_t slice = (size_t)bh * g.L * g.d * sizeof(T);
  return finish_checked<T, false>(g, gather_v(g, bh, n, j, v_prev2, part_in, b, bb, sdr), load_dust(g, bh, dstate),
                                  bh, n, j, reinterpret_cast<const char*>(Q) + slice,
                                  reinterpret_cast<const char*>(K) + slice, u);
}

// Steps t_begin .. t_end of one persistent launch (see iter_kernel): the
// buffers each step reads and writes follow from t, as in the host's launch
// loop.  Per segment (index bh * nseg + seg), head is the last step whose
// starting-end boundary partials it has written and done the last step it
// has finished; *err is set if a neighbour wait gave up (then the results
// are invalid).
struct StepPlan {
  float* part;       // [2][part_slot] column partials (by step parity)
  double* vbuf;      // [2][BHL] v ping-pong
  double* ubuf;      // [2][BHL] u^(t) in slot t & 1
  double* tail_u;    // [R + 1][BHL]
  double* tail_v;    // [R + 1][BHL]
  size_t part_slot, BHL;
  int T;             // stopped-base steps
  int t_begin, t_end;
  int* head;  // [BH * nseg] last step whose start-side boundary region a segment has written
  int* done;  // [BH * nseg] last step a segment has finished
  int* err;
  int max_spins;  // bound of one neighbour wait
  int wait_bias;  // added to every awaited count: 0, or (failure-path testing) a value no count reaches
};

__device__ __forceinline__ IterArgs step_args(const IterArgs& base, const StepPlan& q, int t) {
  IterArgs a = base;
  a.first = t == 1;
  a.part_in = t == 1 ? nullptr : q.part + (size_t)((t - 1) & 1) * q.part_slot;
  a.v_prev2 = t <= 2 ? nullptr : q.vbuf + (size_t)((t - 2) & 1) * q.BHL;
  a.v_out = t == 1 ? nullptr : q.vbuf + (size_t)((t - 1) & 1) * q.BHL;
  a.v_tail = (t >= 2 && t - 1 >= q.T) ? q.tail_v + (size_t)(t - 1 - q.T) * q.BHL : nullptr;
  a.u_out = q.ubuf + (size_t)(t & 1) * q.BHL;
  a.u_prev = t >= 2 ? q.ubuf + (size_t)((t - 1) & 1) * q.BHL : nullptr;
  a.u_tail = t >= q.T ? q.tail_u + (size_t)(t - q.T) * q.BHL : nullptr;
  a.part_out = q.part + (size_t)(t & 1) * q.part_slot;
  a.partd_out = nullptr;
  a.dstate = nullptr;
  return a;
}

constexpr int kMaxSpins = 1 << 20;  // bound of a neighbour wait (each spin sleeps ~256 cycles)
// Failure-path testing (SINKATTN_DEBUG_STALL set): every neighbour wait is
// made unsatisfiable and gives up after a few spins, so the launch still
// runs to its end and the give-up is reported.
constexpr int kStallTestSpins = 4;
constexpr int kStallTestBias = 1 << 30;

// One launch = one Sinkhorn step over every (b, h).  A workgroup sweeps a
// segment of SB consecutive 128-row blocks of one sequence:
//  * the K window of a block (NWT tiles of 16 rows) lives in an LDS ring of
//    NWT + 8 tiles that slides by 8 tiles per block; w_j = v^(t-1)_j - vref
//    of each ring column sits in a separate array (a tile's four lanes per
//    column read one word);
//  * each wave computes one 16-row strip per block; its column partials go
//    to a per-wave buffer (two buffers, alternating by block), and the fold of
//    block k-1's partials into the segment's column sums runs during block k,
//    off the barrier-to-barrier path; a column's sum is written once, when
//    the column leaves the window;
//  * the next block's K rows, Q strips, a_i and column-finish inputs are
//    loaded while the current block computes (the strip issues no other
//    global loads, so those loads stay in flight); its 8 new K tiles go to
//    the ring's 8 spare slots, which no strip of the current block reads, so
//    one barrier per block suffices.  256-byte rows are copied by LDS DMA
//    straight into their ring rows (no registers, no store phase); other row
//    sizes pass through registers and are stored when a wave's strip is done.
// NT (tiles per strip) and the ring size are compile-time; tiles that cross
// the band edge (a host-computed bit mask) or strips with non-real rows are
// masked per entry.
//
// PERS: one launch runs the steps of a StepPlan (no dustbin).  Sweeps
// alternate direction, so the ring at the end of a step already holds the
// window the next step starts with, instead of a new launch reloading it.
// Every segment sweeps in the same direction in a step, so the neighbour at
// the end where a sweep finishes began its own sweep at that shared boundary
// and wrote the partials (and published the v) the next window needs in its
// first blocks: at a turn a workgroup waits only for that neighbour's head
// count, then finishes v for its window.  The far neighbour's finished step
// is awaited later in the sweep, before the first block whose entering
// columns reach its window; both conditions also keep a segment from
// overwriting step-parity buffers a neighbour still reads.  This covers every
// segment whose partials a window column needs only when a segment spans at
// least the band's 16 (TL + TR) columns (then the windows of segments two
// apart are disjoint); the host launches this instance only then.  All
// workgroups must be resident (cooperative launch).
template <typename T, int D, int NT, bool PERS, bool FE = false>
__global__ __launch_bounds__(512) void iter_kernel(Geom g, IterArgs p0, StepPlan q) {
  constexpr int RB = D * Elt<T>::kBytes;  // bytes per Q/K row
  constexpr int NCH = RB / 64;             // 16-byte lane chunks per row
  // LDS row: K row + 16 bytes, which spreads the operand reads of 16
  // consecutive rows over the banks (gfx950 still counts 4 conflict cycles per
  // 128-bit read; a conflict-free XOR layout, which needs per-chunk lane
  // offsets, measured slower: the tile loop is bound by its VALU issue)
  constexpr int RS = RB + 16;
  constexpr int TILEB = 16 * RS;           // bytes per ring tile
  constexpr int PER_ROW = RB / 16;         // 16-byte chunks per row
  constexpr int NEWLD = (kBlockRows * PER_ROW + 511) / 512;  // chunks per thread per block
  // 256-byte rows: the next block's K rows go straight from memory into
  // their ring rows (LDS DMA, one row per instruction, a dword per lane)
  constexpr bool KDMA = RB == 256;
  constexpr int NWT = NT + kWaves - 1;     // window tiles of one block
  constexpr int NWC = NWT * 16;
  constexpr int RING = NWT + 8;            // ring tiles: the window + the next block's 8 new tiles
  constexpr int NRC = RING * 16;           // ring columns
  constexpr int CBW = NT * 16;             // per-wave partials: one per strip column
  constexpr int kThreads = 512;            // launch size (a constant: reading blockDim.x is a memory load)
  static_assert(kBlockRows * PER_ROW == NEWLD * kThreads, "whole 16-byte chunks per thread");
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const IterArgs& p = p0;  // step-independent arguments
  const bool dust = !PERS && g.dustbin;  // (the persistent instance runs without a dustbin)
  int t = PERS ? q.t_begin : 0;  // step (PERS)
  // The step's buffers: from the arguments, or (PERS) from a copy in LDS
  // that thread 0 derives from t at each step (LDS reads cannot move across
  // the block barriers, so nothing per step stays live in registers across
  // the sweep).
  struct StepPtrs {
    const float* part_in;
    const double* v_prev2;
    double* v_out;
    double* v_tail;
    double* u_tail;
    double* u_out;
    const double* u_prev;
    float* part_out;
    int first;
  };
  __shared__ StepPtrs sptr;
  auto set_step = [&]() {
    if (threadIdx.x == 0) {
      const IterArgs a = step_args(p0, q, t);
      sptr.part_in = a.part_in;
      sptr.v_prev2 = a.v_prev2;
      sptr.v_out = a.v_out;
      sptr.v_tail = a.v_tail;
      sptr.u_tail = a.u_tail;
      sptr.u_out = a.u_out;
      sptr.u_prev = a.u_prev;
      sptr.part_out = a.part_out;
      sptr.first = a.first;
    }
  };
  auto s_part_in = [&]() -> const float* {
    if constexpr (PERS) return sptr.part_in;
    else return p0.part_in;
  };
  auto s_v_prev2 = [&]() -> const double* {
    if constexpr (PERS) return sptr.v_prev2;
    else return p0.v_prev2;
  };
  auto s_v_out = [&]() -> double* {
    if constexpr (PERS) return sptr.v_out;
    else return p0.v_out;
  };
  auto s_v_tail = [&]() -> double* {
    if constexpr (PERS) return sptr.v_tail;
    else return p0.v_tail;
  };
  auto s_u_out = [&]() -> double* {
    if constexpr (PERS) return sptr.u_out;
    else return p0.u_out;
  };
  auto s_u_prev = [&]() -> const double* {
    if constexpr (PERS) return sptr.u_prev;
    else return p0.u_prev;
  };
  auto s_u_tail = [&]() -> double* {
    if constexpr (PERS) return sptr.u_tail;
    else return p0.u_tail;
  };
  auto s_part_out = [&]() -> float* {
    if constexpr (PERS) return sptr.part_out;
    else return p0.part_out;
  };
  auto s_first = [&]() -> bool {
    if constexpr (PERS) return sptr.first != 0;
    else return p0.first != 0;
  };

  const int nbh = g.B * g.H;
  const int logical = xcd_remap(blockIdx.x, p.padded_grid);
  if (logical >= nbh * g.nseg) return;
  const int bh = logical / g.nseg;
  const int seg = logical - bh * g.nseg;
  const int bb = bh / g.H;
  const int n = real_len(g, bb);
  const int b0 = seg * g.SB;
  if (b0 * kBlockRows >= n) return;
  int kend = b0 + g.SB;
  if (kend > g.nblk) kend = g.nblk;
  {
    const int kreal = (n + kBlockRows - 1) / kBlockRows;  // blocks holding real rows
    if (kend > kreal) kend = kreal;
  }

  const size_t L = g.L;
  const int seg_r0 = b0 * kBlockRows;
  const int seg_r1 = seg_r0 + g.SB * kBlockRows;  // owned columns [seg_r0, seg_r1)
  const int cs = seg_r0 - 16 * g.TL;              // first column of the segment window
  char* kw = smem;                                                     // [NRC][RS] K ring
  float* wv = reinterpret_cast<float*>(smem + (size_t)NRC * RS);      // [NRC] w_j = v_j - vref
  float* colsum = wv + NRC;                                            // [NRC] segment sums
  float* colbuf = colsum + NRC;                                        // [2][8][CBW] partials
  float* misc = colbuf + 2 * kWaves * CBW;                             // [2][8] dustbin partials

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  // the entering columns of a block (finish inputs, v, w) belong to the
  // first two waves
  const int ec = tid < kBlockRows ? tid : -1;  // entering column, valid when >= 0
  const char* Kb = reinterpret_cast<const char*>(p.K) + (size_t)bh * L * RB;
  const char* Qb = reinterpret_cast<const char*>(p.Q) + (size_t)bh * L * RB;
  const DustC dc = load_dust(g, bh, p.dstate);
  const double vd = (dust && p.dstate) ? p.dstate[4 * bh + 1] : 0.0;  // v^(t-1)_delta

  // shift reference: v^(t-2) at the segment's first column (any value near
  // the window's potentials keeps the entries in range)
  if constexpr (PERS) {
    set_step();
    __syncthreads();
  }
  double vref = s_v_prev2() ? ld_shared<PERS>(s_v_prev2() + bh * L + seg_r0) : 0.0;

  auto publish_v = [&](int j, double vj) {
    if (s_v_out() && j >= seg_r0 && j < seg_r1) {
      st_shared<PERS>(s_v_out() + bh * L + j, vj);
      if (s_v_tail()) gmem(s_v_tail())[bh * L + j] = vj;
    }
  };
  auto wrap = [](int x) { return x >= RING ? x - RING : x; };  // x in [0, 2 RING)
  // w of ring column c (the four lanes of a tile column read one word)
  auto put_w = [&](int c, float w) { wv[c] = w; };

  // prologue: window of block b0 in ring slots 0 .. NWT-1.  All loads are
  // issued before any is used (one memory round trip, not one per row group).
  {
    static_assert(NWC <= kThreads, "one window column per thread");
    constexpr int PRO = (NWC * PER_ROW + kThreads - 1) / kThreads;
    const int jw = (b0 * 8 - g.TL) * 16;
    u4 kv[PRO];
#pragma unroll
    for (int e = 0; e < PRO; ++e) {
      const int idx = tid + e * kThreads;
      kv[e] = (u4){0u, 0u, 0u, 0u};
      if (idx < NWC * PER_ROW) {
        const int j = jw + idx / PER_ROW;
        if (j >= 0 && j < n) kv[e] = ld16(Kb + (size_t)j * RB + (idx % PER_ROW) * 16);
      }
    }
    const int jc = jw + tid;
    const bool colok = tid < NWC && jc >= 0 && jc < n;
    VIn pin;
    if (colok && s_part_in()) pin = gather_v<PERS>(g, bh, n, jc, s_v_prev2(), s_part_in(), p.b, bb, p.sdr);
    if (tid < NWC) {
      float w = kNegInf;
      if (colok) {
        const double vj = s_part_in() ? finish_checked<T, PERS>(g, pin, dc, bh, n, jc, Qb, Kb, s_u_prev()) : 0.0;
        publish_v(jc, vj);
        w = (float)(vj - vref);
      }
      put_w(tid, w);
    }
    for (int c = tid; c < NRC; c += kThreads) colsum[c] = 0.f;
#pragma unroll
    for (int e = 0; e < PRO; ++e) {
      const int idx = tid + e * kThreads;
      if (idx < NWC * PER_ROW) st16(kw + (size_t)(idx / PER_ROW) * RS + (idx % PER_ROW) * 16, kv[e]);
    }
  }
  float dust_acc = 0.f;  // dustbin-column partial of the segment (thread kBlockRows)

  // Per-block inputs of the wave's strip, fetched one block ahead: the Q
  // strip (MFMA B operand) and, for the lane's four rows, a_i and the
  // dustbin-column score.
  struct RowIn {
    u4 q[NCH];
    float a[4];
    float sd[4];
  };
  // Loads are unconditional from row indices clamped into [0, L): rows past
  // the sequence only feed entries that the strip masks (rowok).
  const float* a_b = p.a + (size_t)bb * L;   // per-sequence / per-(b, h) bases
  const float* sdc_bh = p.sdc + (size_t)bh * L;
  auto load_q_chunk = [&](int k, int c, RowIn& ri) {
    const int qi = min(k * kBlockRows + wave * 16 + lr, (int)L - 1);
    ri.q[c] = ld16(Qb + (uint32_t)(qi * RB + c * 64 + lg * 16));
  };
  auto load_row_scalars = [&](int k, RowIn& ri) {
    const int ib = k * kBlockRows + wave * 16 + 4 * lg;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t i = (uint32_t)min(ib + r, (int)L - 1);
      ri.a[r] = a_b[i];
      if constexpr (!PERS) ri.sd[r] = sdc_bh[i];  // always allocated; used only with a dustbin
    }
  };
  RowIn cur;
#pragma unroll
  for (int c = 0; c < NCH; ++c) load_q_chunk(b0, c, cur);
  load_row_scalars(b0, cur);
  // drain the prologue's loads here, so the loop header carries no pending
  // load (otherwise the first MFMA of every strip waits on all loads in flight)
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // Fold block kf's per-wave partials (buffer bf; its window starts at ring
  // slot rbf) into the segment sums in wave order; write out the columns
  // that leave the window after block kf (all of them when `last`).
  // Threads kBlockRows .. kBlockRows + nthr - 1 take the window columns in
  // turn (the first two waves handle the entering columns instead, which
  // balances the work ahead of the block barrier).
  static_assert(NWC <= kThreads - kBlockRows, "one window column per folding thread");
  int dir = 1;  // sweep direction of the current step (always forward unless PERS)
  auto fold = [&](int kf, int bf, int rbf, bool last, bool fwd, int nthr) {
    const int wc0 = tid - kBlockRows;
    if (wc0 < 0 || wc0 >= nthr) return;
    float* const pout = s_part_out() + ((size_t)bh * g.nseg + seg) * g.SW - cs;  // indexed by column
    for (int wc = wc0; wc < NWC; wc += nthr) {
      const int off = wc >> 4;                         // tile offset within block kf's window
      const int c = wrap(rbf + off) * 16 + (wc & 15);  // its ring column
      // the column's reads are all issued before any is summed (one LDS
      // round trip per column)
      float xs[kWaves];
#pragma unroll
      for (int w = 0; w < kWaves; ++w) xs[w] = colbuf[(bf * kWaves + w) * CBW + (off - w) * 16 + (wc & 15)];
      float s = colsum[c];
      __builtin_amdgcn_sched_group_barrier(0x100, kWaves + 1, 0);  // the LDS reads first
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        // the tile's index in wave w's strip; the read address stays inside
        // the buffers for every off and w (lt in [-7, NWT)), so it is affine
        // in w and unselected values are discarded
        const int lt = off - w;
        const bool wrote = lt >= 0 && lt < NT && kf * kBlockRows + 16 * w < n;
        s += wrote ? xs[w] : 0.f;
      }
      // columns leave at the low end of the window in a forward sweep, at
      // the high end in a backward one
      if ((fwd ? off < 8 : off >= NWT - 8) || last) {
        const int j = (kf * 8 - g.TL + off) * 16 + (wc & 15);
        st_shared<PERS>(pout + j, s);
        // a sweep's last fold leaves its sums in place: the next step's
        // window (this one) takes the segment's own partials from here
        if (!last) s = 0.f;
      }
      colsum[c] = s;
    }
    if (dust && tid == kBlockRows) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w)
        if (kf * kBlockRows + 16 * w < n) dust_acc += misc[bf * kWaves + w];
    }
  };

  const char* lane_k = kw + lr * RS + lg * 16;  // lane's operand bytes in ring row lr
  // Additive band masks of the strip's first and last tiles (0 inside the
  // band, -inf outside, full rows): when those are the only tiles crossing a
  // band edge, a full strip masks them with four adds instead of the
  // per-entry offset test.
  float mb0[4], mb1[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int o0 = -g.TL * 16 + lr - 4 * lg - r;
    const int o1 = (NT - 1 - g.TL) * 16 + lr - 4 * lg - r;
    mb0[r] = (o0 >= -g.h1 && o0 <= g.h2) ? 0.f : kNegInf;
    mb1[r] = (o1 >= -g.h1 && o1 <= g.h2) ? 0.f : kNegInf;
  }
  const bool ends_only = (g.edge_mask & ~(1u | (1u << (NT - 1)))) == 0u;
  const float* lane_wv = wv + lr;               // w of the lane's tile column
  int jpend = -1;                               // entering column whose v is not yet stored
  double vpend = 0.0;
  auto flush_pending = [&]() {
    if (jpend >= 0) publish_v(jpend, vpend);
    jpend = -1;
  };
  int rb = 0;                                   // ring slot of block k's first window tile
  int rbp = 0;                                  // same for the previous block
  const int nbs = kend - b0;                    // blocks in the segment
  // Persistent instance: neighbour handshakes.  A sweep writes the partials
  // of the columns it shares with the neighbour at its starting end within
  // its first nb_region blocks (their folds run one block later), and it
  // needs the far neighbour's previous step only from sweep index bi_far on
  // (the first block whose entering columns reach that neighbour's window).
  const int nb_region = (g.TL + g.TR + 7) / 8;
  const int bi_head = nb_region + 1;  // head(t) is published at the start of this block
  const int bi_far = nbs - 1 - nb_region;
  const int me = bh * g.nseg + seg;
  const bool has_l = seg > 0;
  const bool has_r = seg + 1 < g.nseg && (seg + 1) * g.SB * kBlockRows < n;
  // tid 0: wait until cnt_a[ia] >= va (when use_a) and cnt_b[ib] >= vb (when
  // use_b), with a bounded spin that flags an error instead of hanging
  auto wait_for = [&](const int* cnt_a, int ia, bool use_a, int va, const int* cnt_b, int ib, bool use_b, int vb) {
    int spins = 0;
    va += q.wait_bias;
    vb += q.wait_bias;
    while ((use_a && ld_shared<true>(cnt_a + ia) < va) || (use_b && ld_shared<true>(cnt_b + ib) < vb)) {
      if (++spins > q.max_spins) {
        st_shared<true>(q.err, 1);
        break;
      }
      __builtin_amdgcn_s_sleep(4);
    }
  };
  // One sweep over the segment's blocks (DIR = +1 forward, -1 backward: a
  // compile-time direction, so each instantiation keeps one set of indices).
  auto sweep = [&](auto dirc) {
    constexpr int DIR = decltype(dirc)::value;
  for (int bi = 0; bi < nbs; ++bi) {
    const int k = DIR > 0 ? b0 + bi : kend - 1 - bi;
    const int buf = bi & 1;
    const bool more = bi + 1 < nbs;
    // the starting-end boundary partials of step t are out (their stores
    // drained before the last barrier)
    if constexpr (PERS)
      if (bi == bi_head && tid == 0) st_shared<true>(q.head + me, t);
    // ---- prefetch for block k + 1 (8 new K tiles, Q strips, a_i, column-
    // finish inputs) in NPF slices, one issued per tile of the strip's first
    // tiles: a wave issuing them all at once stalls on the CU's memory pipe.
    // The loads are unconditional (clamped addresses) so that no register
    // write on an untaken path makes the compiler wait for them early.
    // first row/column of the 8 tiles entering with the next block (the
    // top of its window in a forward sweep, the bottom in a backward one)
    const int jn0 = DIR > 0 ? ((k + 1) * 8 + g.TR) * 16 : ((k - 1) * 8 - g.TL) * 16;
    // block whose inputs the slices load: the next one, or k itself in the
    // last block (nothing is used there; its rows are cached, so no extra
    // HBM traffic)
    const int kn = more ? k + DIR : k;
    const int jp0 = DIR > 0 ? (kn * 8 + g.TR) * 16 : (kn * 8 - g.TL) * 16;
    u4 knew[KDMA ? 1 : NEWLD];
    VIn vin;
    RowIn nxt;
    constexpr int NPF = NEWLD + NCH + 2;
    // (issued in the segment's last block too, where nothing uses the values:
    // every address is clamped into its buffer)
    auto prefetch = [&](int part) {
      if (part < NEWLD) {
        if constexpr (KDMA) {
          // wave w fills new tile w (ring slot rb + NWT + w), 16 / NEWLD rows
          // per slice.  Rows outside the sequence are loaded from the
          // nearest real row: their columns carry w = -inf, so every entry
          // they feed is exactly zero.  Nothing is loaded in the segment's
          // last block (a DMA still in flight when the workgroup ends could
          // land in another workgroup's LDS).
          if (more) {
            const int slot = wrap(rb + NWT + wave);
            const int jb = jp0 + wave * 16;
            if (jb >= 0 && jb + 15 < n) {
              // all 16 rows real: one lane address for the tile, the row in
              // the immediate offset (no per-row address arithmetic)
              const char* gb = Kb + (uint32_t)(jb * RB + lane * 4);
#pragma unroll
              for (int i = 0; i < 16 / NEWLD; ++i) {
                const int r = (16 / NEWLD) * part + i;
                dma_row256(gb, kw + (slot * 16 + r) * RS, r);
              }
            } else {
#pragma unroll
              for (int i = 0; i < 16 / NEWLD; ++i) {
                const int r = (16 / NEWLD) * part + i;
                int j = jb + r;
                j = j < 0 ? 0 : (j >= n ? n - 1 : j);
                __builtin_amdgcn_global_load_lds(Kb + (uint32_t)(j * RB + lane * 4), kw + (slot * 16 + r) * RS, 4, 0, 0);
              }
            }
          }
        } else {
          // rows past the sequence are zeroed when stored to LDS
          // (a per-(b, h) base pointer plus a 32-bit lane offset: the load
          // takes the scalar base DIRectly, no 64-bit address arithmetic)
          const int idx = tid + part * kThreads;
          int j = min(jp0 + idx / PER_ROW, (int)L - 1);
          if constexpr (PERS) j = max(j, 0);
          knew[part] = ld16(Kb + (uint32_t)(j * RB + (idx % PER_ROW) * 16));
        }
      } else if (part < NEWLD + NCH) {
        load_q_chunk(kn, part - NEWLD, nxt);
      } else if (part == NEWLD + NCH) {
        load_row_scalars(kn, nxt);
      } else if (ec >= 0 && s_part_in()) {
        // j + 16 TL = (k + 1) 128 + 16 (TL + TR) + ec with ec < 128, so the
        // first segment window holding j is (k + 1) / SB and the last is at
        // most two further (16 (TL + TR) <= 256 <= 2 segw)
        int j = jp0 + ec;
        int slo, shi;
        if constexpr (PERS) {
          // the segment windows holding j (as window_segments): the 128
          // entering columns are consecutive and a segment spans at least
          // 128, so each bound is the block's first column's plus 0 or 1
          // (one block-uniform division per bound instead of two per lane)
          const int segw = g.SB * kBlockRows;
          const int xb = jp0 + 16 * g.TL;  // >= 0
          const int h0 = xb / segw;
          const int l0 = floor_div(xb - g.SW, segw);
          const int x = xb + ec;
          shi = h0 + (x >= (h0 + 1) * segw ? 1 : 0);
          shi = shi > g.nseg - 1 ? g.nseg - 1 : shi;
          slo = l0 + 1 + (x - g.SW >= (l0 + 1) * segw ? 1 : 0);
          slo = slo < 0 ? 0 : slo;
          j = j < 0 ? 0 : j;
        } else {
          const int segw = g.SB * kBlockRows;
          slo = kn / g.SB;
          const int x = j + 16 * g.TL;
          shi = slo + (x >= (slo + 1) * segw ? 1 : 0) + (x >= (slo + 2) * segw ? 1 : 0);
          shi = shi > g.nseg - 1 ? g.nseg - 1 : shi;
        }
        j = j < (int)L ? j : (int)L - 1;  // columns outside the sequence are not used
        vin = gather_v_clamped<PERS>(g, bh, n, j, slo, shi, s_v_prev2(), s_part_in(), p.b, bb, p.sdr);
      }
    };

    // ---- block k: one 16-row strip per wave (all strip values wave-uniform)
    const int i0 = k * kBlockRows + wave * 16;
    if (i0 < n) {
      // Store the entering columns' v from the previous block now, a whole
      // strip before the next loop top (the first two waves hold them).
      flush_pending();
      const int sw = wrap(rb + wave);  // ring slot of strip tile t = 0
      const bool partial = i0 + 16 > n;
      bool rowok[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) rowok[r] = i0 + 4 * lg + r < n;
      // dustbin column exponent for the lane's rows, relative to vref
      float xd[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
      if (dust) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (rowok[r]) xd[r] = (float)((double)cur.sd[r] + vd - vref);
      }
      // Band geometry pinned inside the block loop: the empty asm keeps the
      // compiler from precomputing every tile's lane masks up front (which
      // exhausts the scalar registers); recomputing them is a few ops.
      int TLs = g.TL, h1s = g.h1, h2s = g.h2;
      unsigned emask = partial ? 0xffffffffu : g.edge_mask;  // bit t: tile t needs masking
      asm volatile("" : "+s"(TLs), "+s"(h1s), "+s"(h2s), "+s"(emask));
      auto masked = [&](int t, float (&x)[4]) {
        int dl = lr - 4 * lg;
        asm volatile("" : "+v"(dl));
        const int obase = (t - TLs) * 16 + dl;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int o = obase - r;
          const bool ok = o >= -h1s && o <= h2s && rowok[r];
          x[r] = ok ? x[r] : kNegInf;
        }
      };
      // the band mask of tile t (emask bit t set)
      const bool fast_ends = ends_only && !partial;
      auto mask_tile = [&](int t, float (&x)[4]) {
        if ((t == 0 || t == NT - 1) && fast_ends) {
#pragma unroll
          for (int r = 0; r < 4; ++r) x[r] += t == 0 ? mb0[r] : mb1[r];
        } else {
          masked(t, x);
        }
      };
      auto read_tile = [&](int t, u4 (&kb)[NCH], float& w) {
        const int sl = wrap(sw + t);
        const char* src = lane_k + sl * TILEB;
#pragma unroll
        for (int c = 0; c < NCH; ++c) kb[c] = ld16(src + c * 64);
        w = lane_wv[sl * 16];
      };
      auto mma_tile = [&](const u4 (&kb)[NCH]) {
        f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NCH; ++c) acc = Elt<T>::mma_chunk(acc, cur.q[c], kb[c]);
        return acc;
      };

      float e[NT][4];
      float shift[4] = {0.f, 0.f, 0.f, 0.f};
      float rs[4] = {0.f, 0.f, 0.f, 0.f};
      float ed[4] = {0.f, 0.f, 0.f, 0.f};
      // The fast pass runs except on the first step, which goes straight to
      // the exact row maxima below (and issues the prefetch slices itself);
      // when a fast row sum leaves the safe range the strip is recomputed
      // there as well.
      bool need_safe = s_first() != 0;
      if (!need_safe) {
        // fast path: shift vref only; pipelined MFMA / exp.  FE instance (the
        // host launches it when the band's only edge-crossing strip tiles
        // are the first and last): those two take the additive band masks
        // and no tile has a branch, so each tile's work is one scheduling
        // region; rows past the sequence are not masked in the loop, their
        // entries are zeroed after it (every real row's arithmetic is the
        // other instance's; both loops in one instance exhaust the registers)
        auto tile_loop = [&](auto fec) {
          constexpr bool kFE = decltype(fec)::value;
          auto consume = [&](int t, const f4& acc, float w) {
            float x[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) x[r] = __builtin_fmaf(acc[r], g.scale2, w);
            if constexpr (kFE) {
              if (t == 0 || t == NT - 1) {
#pragma unroll
                for (int r = 0; r < 4; ++r) x[r] += t == 0 ? mb0[r] : mb1[r];
              }
            } else {
              if ((emask >> t) & 1u) mask_tile(t, x);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              e[t][r] = exp2_fast(x[r]);
              rs[r] += e[t][r];
            }
            // pin the sums here: otherwise the exps sink below the tile loop
            asm volatile("" : "+v"(rs[0]), "+v"(rs[1]), "+v"(rs[2]), "+v"(rs[3]));
          };
          u4 kbA[NCH], kbB[NCH];
          float wA, wB;
          read_tile(0, kbA, wA);
          f4 accP = {0.f, 0.f, 0.f, 0.f};
          float wP = 0.f;
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            if (t < NPF) {
              asm volatile("" ::: "memory");  // keep slice t at tile t (no hoisting)
              prefetch(t);
            }
            if (t & 1) {
              if (t + 1 < NT) read_tile(t + 1, kbA, wA);
              const f4 acc = mma_tile(kbB);
              if (t > 0) consume(t - 1, accP, wP);
              accP = acc;
              wP = wB;
            } else {
              if (t + 1 < NT) read_tile(t + 1, kbB, wB);
              const f4 acc = mma_tile(kbA);
              if (t > 0) consume(t - 1, accP, wP);
              accP = acc;
              wP = wA;
            }
            // tile t-1's exp/sum work stays in this iteration, interleaved with
            // tile t's MFMAs and tile t+1's LDS reads (with every exp after the
            // loop, the LDS/MFMA and VALU phases of all waves run one after
            // the other)
            __builtin_amdgcn_sched_barrier(0);
          }
          consume(NT - 1, accP, wP);
        };
        if constexpr (FE) {
          tile_loop(std::true_type{});
          if (partial) {
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
#pragma unroll
              for (int r = 0; r < 4; ++r) e[tt][r] = rowok[r] ? e[tt][r] : 0.f;
          }
        } else {
          tile_loop(std::false_type{});
        }
#pragma unroll
        for (int q = NT; q < NPF; ++q) prefetch(q);
        // every row sum in [2^-120, 2^120] (and not NaN): its bits minus
        // those of 2^-120, as unsigned, stay at most the span's (rows past
        // the sequence count as 1)
        constexpr uint32_t kLoBits = 0x03800000u, kSpan = 0x7b800000u - 0x03800000u;
        uint32_t worst = 0u;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          rs[r] = row16_sum(rs[r]);
          if (dust) {
            ed[r] = exp2_fast(xd[r]);
            rs[r] += ed[r];
          }
          float x = rs[r];
          if (partial) x = rowok[r] ? x : 1.f;
          const uint32_t d = __float_as_uint(x) - kLoBits;
          worst = worst > d ? worst : d;
        }
        need_safe = __any(worst > kSpan);
      } else {
#pragma unroll
        for (int q = 0; q < NPF; ++q) prefetch(q);
      }
      if (need_safe) {
        // exact per-row maxima (first step, or entries out of range)
        float m[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          u4 kb[NCH];
          float w;
          read_tile(t, kb, w);
          const f4 acc = mma_tile(kb);
#pragma unroll
          for (int r = 0; r < 4; ++r) e[t][r] = __builtin_fmaf(acc[r], g.scale2, w);
          if ((emask >> t) & 1u) mask_tile(t, e[t]);
#pragma unroll
          for (int r = 0; r < 4; ++r) m[r] = fmaxf(m[r], e[t][r]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          m[r] = row16_max(m[r]);
          if (dust) m[r] = fmaxf(m[r], xd[r]);
          if (!(m[r] > kNegInf)) m[r] = 0.f;  // inactive row
          shift[r] = m[r];
          rs[r] = 0.f;
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            e[t][r] = exp2_fast(e[t][r] - shift[r]);
            rs[r] += e[t][r];
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          rs[r] = row16_sum(rs[r]);
          ed[r] = dust ? exp2_fast(xd[r] - shift[r]) : 0.f;
          rs[r] += ed[r];
        }
      }

      // the DMA rows of the next block are complete before this wave's
      // stores below (waiting at the barrier would also wait for those)
      if constexpr (KDMA) __builtin_amdgcn_s_waitcnt(kVmcnt0);
      // row weights h_i = a_i / rho_i (rho_i lies in [2^-120, 2^120] here)
      float h[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) h[r] = rowok[r] ? cur.a[r] * __builtin_amdgcn_rcpf(rs[r]) : 0.f;
      // u^(t)_i = log2(a_i / rho_i) - c_i - vref (fp64 state), by lane lr = r
      {
        const int rsel = lr & 3;
        // a_i as opaque registers: selected straight from the array, the
        // compiler turns the choice into a run-time index and moves the array
        // to scratch memory (a store and a dependent load in every block)
        float ar[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          ar[r] = cur.a[r];
          asm volatile("" : "+v"(ar[r]));
        }
        float rsv = rs[0], av = ar[0], shv = shift[0];
        bool okv = rowok[0];
#pragma unroll
        for (int r = 1; r < 4; ++r) {
          const bool pick = rsel == r;
          rsv = pick ? rs[r] : rsv;
          av = pick ? ar[r] : av;
          shv = pick ? shift[r] : shv;
          okv = pick ? rowok[r] : okv;
        }
        if (lr < 4 && okv) {
          const int i = i0 + 4 * lg + rsel;
          const double u = log2_split(av * __builtin_amdgcn_rcpf(rsv)) - (double)shv - vref;
          // device scope in the persistent launch: an exact column update of
          // another workgroup may read it in the next step
          st_shared<PERS>(s_u_out() + bh * L + i, u);
          if (s_u_tail()) gmem(s_u_tail())[bh * L + i] = u;
        }
      }
      // column partials of this strip, sum_i e_ij h_i, reduced over the four
      // lane rows four tiles at a time (row g ends with tile t + g's sums)
      float* cb = colbuf + (buf * kWaves + wave) * CBW;  // indexed by strip column
      auto colp = [&](int t) {
        float cp = e[t][0] * h[0];
        cp = __builtin_fmaf(e[t][1], h[1], cp);
        cp = __builtin_fmaf(e[t][2], h[2], cp);
        return __builtin_fmaf(e[t][3], h[3], cp);
      };
#pragma unroll
      for (int t = 0; t + 3 < NT; t += 4) {
        const float s4 = cross_row_sum4(colp(t), colp(t + 1), colp(t + 2), colp(t + 3));
        cb[(t + lg) * 16 + lr] = s4;
      }
#pragma unroll
      for (int t = NT & ~3; t < NT; ++t) {
        const float s1 = cross_row_sum(colp(t));
        if (lg == 0) cb[t * 16 + lr] = s1;
      }
      if (dust) {
        float dp = 0.f;
        if (lr == 0) {
#pragma unroll
          for (int r = 0; r < 4; ++r) dp = __builtin_fmaf(ed[r], h[r], dp);
        }
        dp = wave_sum(dp);
        if (lane == 0) misc[buf * kWaves + wave] = dp;
      }
    } else {
      // No real rows for this wave: the sequence's partial last block, which
      // a backward sweep (persistent instance) visits first.  The wave still
      // loads its share of the next block's inputs.
      flush_pending();
#pragma unroll
      for (int q = 0; q < NPF; ++q) prefetch(q);
      if constexpr (KDMA) __builtin_amdgcn_s_waitcnt(kVmcnt0);
    }

    // ---- partials of the previous block into the segment sums (waves 2
    // and 3, which finish their strips first; block k + 1 overwrites that
    // buffer only after the barrier)
    if (bi > 0 && (wave == 2 || wave == 3)) fold(k - DIR, buf ^ 1, rbp, false, DIR > 0, 2 * 64);
    // the region's last fold: its stores complete before the barrier, and so
    // do every wave's u stores of the region's rows (a neighbour's exact
    // column update may read them once head(t) is out)
    if constexpr (PERS)
      if (bi == bi_head - 1) __builtin_amdgcn_s_waitcnt(kVmcnt0);

    // ---- v^(t-1) of the columns entering with block k + 1 (written to
    // memory during the next strip: a store still in flight at the loop top
    // would make the next block's first loads wait for it)
    float wnew = kNegInf;
    if (more && ec >= 0) {
      const int j = jn0 + ec;
      if (j >= 0 && j < n) {
        const double vj = s_part_in() ? finish_checked<T, PERS>(g, vin, dc, bh, n, j, Qb, Kb, s_u_prev()) : 0.0;
        jpend = j;
        vpend = vj;
        wnew = (float)(vj - vref);
      }
    }
    if (more) {
      // ---- the new tiles take ring slots rb + NWT .. rb + NWT + 7, which no
      // strip of block k reads (block k - 1's first tiles left them), so each
      // wave stores its share as soon as its own strip is done: one barrier
      // per block
#pragma unroll
      for (int e = 0; e < (KDMA ? 0 : NEWLD); ++e) {
        const int idx = tid + e * 512;
        const int row = idx / PER_ROW;
        const int j = jn0 + row;
        const bool jok = PERS ? (j >= 0 && j < n) : j < n;
        const u4 val = jok ? knew[e] : (u4){0u, 0u, 0u, 0u};
        st16(kw + (size_t)(wrap(rb + NWT + (row >> 4)) * 16 + (row & 15)) * RS + (idx % PER_ROW) * 16, val);
      }
      if (ec >= 0) put_w(wrap(rb + NWT + (ec >> 4)) * 16 + (ec & 15), wnew);
    }
    if constexpr (PERS) {
      // the far neighbour must have finished step t - 1 before the next block
      // gathers columns of its window (and before this sweep overwrites the
      // step t - 1 partials and v^(t-2) it read); the barrier below orders it
      if (tid == 0 && bi == bi_far - 1 && t > q.t_begin) {
        const bool far_r = DIR < 0;  // a backward sweep ends at the left neighbour
        wait_for(q.done, far_r ? me + 1 : me - 1, far_r ? has_r : has_l, t - 1, q.done, 0, false, 0);
      }
    }
    __syncthreads();
    if (more) {
      cur = nxt;
      rbp = rb;
      rb = wrap(rb + (DIR > 0 ? 8 : NWT));  // NWT = -8 modulo the ring
    }
  }
    flush_pending();
    // the last block's partials; every column still in the window leaves
    fold(DIR > 0 ? kend - 1 : b0, (nbs - 1) & 1, rb, true, DIR > 0, kThreads - kBlockRows);
  };
  for (;;) {
  if constexpr (PERS) {
    if (dir > 0) sweep(std::integral_constant<int, 1>{});
    else sweep(std::integral_constant<int, -1>{});
  } else {
    sweep(std::integral_constant<int, 1>{});
  }
  if constexpr (!PERS) {
    break;
  } else {
    if (t == q.t_end) break;
    // ---- next step: wait for the neighbour at this end, then finish v^(t)
    // for the window the new sweep starts with (its K rows are in the ring).
    // A segment of more than a few blocks publishes done(t) only at the end
    // of the turn: its own partials of the window come from LDS, so the last
    // fold's stores drain while the turn runs.  A short one (which may need
    // the far neighbour now) publishes first, so that no two turns wait on
    // each other.
    const bool short_seg = bi_far < 1 || bi_head >= nbs;
    if (short_seg) __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const bool right = dir > 0;  // this sweep ended at the right neighbour
    ++t;
    dir = -dir;
    if (tid == 0) {
      if (short_seg) {
        st_shared<true>(q.done + me, t - 1);
        if (bi_head >= nbs) st_shared<true>(q.head + me, t - 1);
      }
      // The next sweep starts at this end: the neighbour there must have
      // written its starting-end region of step t - 1 (its sweep began at the
      // shared boundary).  Its first poll is issued ahead of set_step.
      const bool has_e = right ? has_r : has_l;
      const int e_idx = right ? me + 1 : me - 1;
      const int e0 = has_e ? ld_shared<true>(q.head + e_idx) : t;
      set_step();  // nothing reads the step's pointers until the barrier below
      const bool far_now = bi_far < 1;
      if (e0 < t - 1 || far_now)
        wait_for(q.head, e_idx, has_e, t - 1, q.done, right ? me - 1 : me + 1, far_now && (right ? has_l : has_r),
                 t - 1);
    }
    // every wave's u^(t-1) stores have completed (they drained during the
    // neighbour wait): the window's exact column updates may read them
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    __syncthreads();
    vref = s_v_prev2() ? ld_shared<true>(s_v_prev2() + bh * L + seg_r0) : 0.0;
    {
      const int kc = dir > 0 ? b0 : kend - 1;  // the block the new sweep starts at
      const int jc = (kc * 8 - g.TL) * 16 + tid;
      const bool colok = tid < NWC && jc >= 0 && jc < n;
      const int c = wrap(rb + (tid >> 4)) * 16 + (tid & 15);  // its ring column
      float own = 0.f;
      if (tid < NWC) {
        own = colsum[c];  // this segment's partial (the last fold's sum)
        colsum[c] = 0.f;
      }
      VIn pin;
      if (colok && s_part_in()) pin = gather_v<true>(g, bh, n, jc, s_v_prev2(), s_part_in(), p.b, bb, p.sdr, seg, own);
      if (tid < NWC) {
        float w = kNegInf;
        if (colok) {
          const double vj = s_part_in() ? finish_checked<T, true>(g, pin, dc, bh, n, jc, Qb, Kb, s_u_prev()) : 0.0;
          publish_v(jc, vj);
          w = (float)(vj - vref);
        }
        put_w(c, w);
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (!short_seg && tid == 0) {
        st_shared<true>(q.done + me, t - 1);  // every store of step t - 1 has drained
      }
    }
  }
  }
  if (dust && tid == kBlockRows) p.partd_out[(size_t)bh * g.nseg + seg] = dust_acc;
}

// ---------------------------------------------------------------------------
// Dustbin step (section 2.3; potentials fp64 in log2 units): after the band
// step t, finish the dustbin row (u_delta^(t), an exact log-sum-exp over
// every active column with v^(t-1)) and the dustbin column (v_delta^(t) from
// the band blocks' partial sums plus the corner).  One workgroup per (b, h).
// dstate layout: [u_delta, v_delta, row shift, h_delta = a / rho].
// ---------------------------------------------------------------------------
struct DustArgs {
  const float* a;
  const float* b;
  const double* v_cur;  // v^(t-1) on real tokens (nullptr => zeros)
  const float* partd;   // [BH][nseg] dustbin-column partials of step t
  double* dstate;       // in: state after t-1 (ignored when first); out: after t
  const float* sdr;
  const float* sdc;     // dustbin column scores (exact column update)
  double* u_tail;       // optional: u^(t) slot
  double* v_tail;       // optional: v^(t) slot
  double* u_out;        // latest-u buffer (dustbin entry)
  double* v_prev_tail;  // optional: copy of v^(t-1)_delta (the state this step starts from)
  int first;
};

__global__ __launch_bounds__(256) void dustbin_step(Geom g, DustArgs p) {
  const int bh = blockIdx.x;
  const int bb = bh / g.H;
  const int n = real_len(g, bb);
  const size_t L = g.L;
  const int tid = threadIdx.x;
  __shared__ double redd[256];
  __shared__ float red[256];
  const double vd_prev = p.first ? 0.0 : p.dstate[4 * bh + 1];
  if (p.v_prev_tail && tid == 0) p.v_prev_tail[bh * L + n] = vd_prev;
  const float* srow = p.sdr + bh * L;
  // x_j = S_delta,j + v_j (log2) over active j; the corner uses v_delta.
  // One pass: each thread keeps a running maximum m and the sum s of
  // 2^(x - m) (rescaled when m grows), and the pairs merge in a tree.
  double m = -__builtin_inf();
  float acc = 0.f;
  for (int j = tid; j <= n; j += blockDim.x) {
    const double vj = (j == n) ? vd_prev : (p.v_cur ? p.v_cur[bh * L + j] : 0.0);
    const double x = (double)srow[j] + vj;
    if (x > m) {
      acc = acc * exp2_fast((float)(m - x)) + 1.f;
      m = x;
    } else {
      acc += exp2_fast((float)(x - m));
    }
  }
  redd[tid] = m;
  red[tid] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) {
      const double m1 = redd[tid], m2 = redd[tid + s];
      const double mm = fmax(m1, m2);
      // an empty side (m = -inf) contributes nothing
      const float a1 = m1 == -__builtin_inf() ? 0.f : red[tid] * exp2_fast((float)(m1 - mm));
      const float a2 = m2 == -__builtin_inf() ? 0.f : red[tid + s] * exp2_fast((float)(m2 - mm));
      redd[tid] = mm;
      red[tid] = a1 + a2;
    }
    __syncthreads();
  }
  const double M = redd[0];
  __shared__ double sh_ud;
  __shared__ int sh_exact;
  const float bd = p.b[(size_t)bb * L + n];
  double vd = 0.0;
  if (tid == 0) {
    const float rho = red[0];
    const float ad = p.a[(size_t)bb * L + n];
    const double ud = log2((double)ad) - log2((double)rho) - M;
    const float hd = ad / rho;
    float gam = 0.f;
    for (int sg = 0; sg < g.nseg && sg * g.SB * kBlockRows < n; ++sg) gam += p.partd[(size_t)bh * g.nseg + sg];
    gam += exp2_fast((float)((double)srow[n] + vd_prev - M)) * hd;  // corner of P^(t,t-1)
    vd = vd_prev + log2((double)bd) - log2((double)gam);
    sh_ud = ud;
    sh_exact = !(gam >= 0x1p-120f && gam <= 0x1p120f);
  }
  __syncthreads();
  if (sh_exact) {
    // gamma out of range: the exact column log-sum-exp of the dustbin column,
    // log2 sum_i 2^(S2_i,delta + u^(t)_i) over the real rows and the corner
    const double ud = sh_ud;
    const float* scol = p.sdc + bh * L;
    double mx = -__builtin_inf();
    for (int i = tid; i < n; i += blockDim.x) mx = fmax(mx, (double)scol[i] + p.u_out[bh * L + i]);
    redd[tid] = mx;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
      if (tid < s) redd[tid] = fmax(redd[tid], redd[tid + s]);
      __syncthreads();
    }
    const double Mc = fmax(redd[0], (double)srow[n] + ud);
    __syncthreads();
    double sc = 0.0;
    for (int i = tid; i < n; i += blockDim.x) sc += exp2((double)scol[i] + p.u_out[bh * L + i] - Mc);
    redd[tid] = sc;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
      if (tid < s) redd[tid] += redd[tid + s];
      __syncthreads();
    }
    if (tid == 0) vd = log2((double)bd) - Mc - log2(redd[0] + exp2((double)srow[n] + ud - Mc));
  }
  if (tid == 0) {
    const double ud = sh_ud;
    const float rho = red[0];
    const float hd = p.a[(size_t)bb * L + n] / rho;
    double* ds = p.dstate + 4 * bh;
    ds[0] = ud;
    ds[1] = vd;
    ds[2] = M;
    ds[3] = hd;
    if (p.u_tail) p.u_tail[bh * L + n] = ud;
    if (p.v_tail) p.v_tail[bh * L + n] = vd;
    p.u_out[bh * L + n] = ud;
  }
}

// Dustbin score vectors in log2 units: sdr_j = q_delta . k_j log2(e) / sqrt(d),
// sdc_i = q_i . k_delta log2(e) / sqrt(d).
template <typename T>
__global__ __launch_bounds__(256) void dustbin_scores(Geom g, const T* Q, const T* K, float* sdr, float* sdc) {
  const int bh = blockIdx.y;
  const int bb = bh / g.H;
  const int n = real_len(g, bb);
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j > n) return;
  const size_t L = g.L;
  const int d = g.d;
  const T* qd = Q + ((size_t)bh * L + n) * d;
  const T* kd = K + ((size_t)bh * L + n) * d;
  const T* qj = Q + ((size_t)bh * L + j) * d;
  const T* kj = K + ((size_t)bh * L + j) * d;
  float sr = 0.f, sc = 0.f;
  for (int c = 0; c < d; ++c) {
    sr = __builtin_fmaf(Elt<T>::load(qd, c), Elt<T>::load(kj, c), sr);
    sc = __builtin_fmaf(Elt<T>::load(qj, c), Elt<T>::load(kd, c), sc);
  }
  sdr[bh * L + j] = sr * g.scale2;
  sdc[bh * L + j] = sc * g.scale2;
}

// Zero start (T = 0): u^(0) = v^(0) = 0.
__global__ void zero_start(Geom g, double* tail_u0, double* tail_v0) {
  const int bh = blockIdx.y;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= g.L) return;
  const size_t o = (size_t)bh * g.L + i;
  tail_u0[o] = 0.0;
  tail_v0[o] = 0.0;
}

// Convergence check of the stopped base (section 2.1 runs the base until
// convergence or for a fixed number of steps).  After step t the plan
// P^(t,t) = exp(S + u^(t) (+) v^(t)) has exact column sums b, and its row sums
// are a_i 2^(u^(t)_i - u^(t+1)_i) (log2 units) with u^(t+1) = U(v^(t)), the
// row update of the next step.  So
//   e_t = sum_i |rowsum_i(P^(t,t)) - a_i| = sum_i a_i |2^(u^(t)_i - u^(t+1)_i) - 1|
// over the active rows (the dustbin row included), in fp64 and a fixed order.
// The step carrying the check left u^(t+1) in `unew` and u^(t) in its
// parity slot `uold`; this kernel also moves the potentials on: u^(t) to
// `uold_copy` (the stopped-base slot, should the check pass) and u^(t+1) to
// its parity slot `unext`.  One workgroup per (b, h).
__global__ __launch_bounds__(256) void base_check(Geom g, const float* a, const double* uold, double* unext,
                                                  const double* unew, double* uold_copy, double* err) {
  const int bh = blockIdx.x;
  const int bb = bh / g.H;
  const int n = real_len(g, bb);
  const size_t L = g.L;
  const int tid = threadIdx.x;
  const int last = g.dustbin ? n : n - 1;  // last active index
  __shared__ double red[256];
  double acc = 0.0;
  for (int i = tid; i <= last; i += 256) {
    const size_t o = (size_t)bh * L + i;
    const double uo = uold[o], un = unew[o];
    acc += (double)a[(size_t)bb * L + i] * fabs(expm1((uo - un) * 0.6931471805599453));
    uold_copy[o] = uo;
    unext[o] = un;
  }
  red[tid] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  if (tid == 0) err[bh] = red[0];
}

// ---------------------------------------------------------------------------
// Output epilogue: P = exp(S + u (+) v) on the band (plus the dustbin column
// for real rows), O = P V on MFMA.  The tile orientation here puts one query
// row per lane (score tile = K_tile Q_strip^T) so the plan tile is directly
// the A operand of P V.  bf16 inputs: P is split into hi + lo bf16 parts so
// the product keeps ~16 mantissa bits.  Also finishes v^(N) and writes u, v
// (natural log).
// ---------------------------------------------------------------------------
struct OutArgs {
  const void* Q;
  const void* K;
  const void* V;
  const float* a;
  const float* b;
  const double* v_prev2;  // v^(N-1), nullptr => zeros
  const float* part_in;   // partials of step N, nullptr => v^(N) = 0
  const double* u_in;     // u^(N) (latest-u buffer), nullptr => zeros
  const double* dstate;   // dustbin state after step N (nullptr if none / N == 0)
  const float* sdr;
  const float* sdc;
  float* O;
  float* u_out;
  float* v_out;
  double* v_tail;         // v^(N) (tail slot R)
  int padded_grid;
};

template <typename T, int D>
__global__ __launch_bounds__(512) void output_kernel(Geom g, OutArgs p) {
  constexpr int RB = D * Elt<T>::kBytes;
  constexpr int NCH = RB / 64;
  constexpr int EB = Elt<T>::kBytes;
  constexpr int ND = D / 16;  // 16-wide output column chunks
  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ double sh_vref;

  const int nbh = g.B * g.H;
  const int logical = xcd_remap(blockIdx.x, p.padded_grid);
  if (logical >= nbh * g.nblk) return;
  const int bh = logical / g.nblk;
  const int blk = logical - bh * g.nblk;
  const int bb = bh / g.H;
  const int n = real_len(g, bb);
  const int r0 = blk * kBlockRows;
  const size_t L = g.L;
  const int NWC = g.NWC;
  const int VTS = NWC + 8;  // padded V^T row (elements)
  const int tw0 = (r0 >> 4) - g.TL;
  const int tid = threadIdx.x;
  const double ln2 = 0.6931471805599453;

  // u outputs, filler rows of u, v and O for the owned range
  for (int c = tid; c < kBlockRows; c += blockDim.x) {
    const int i = r0 + c;
    if (i >= g.L) break;
    if (i >= n) {
      if (!(g.dustbin && i == n)) {
        p.u_out[bh * L + i] = kNegInf;
        p.v_out[bh * L + i] = kNegInf;
      }
    } else {
      p.u_out[bh * L + i] = p.u_in ? (float)(p.u_in[bh * L + i] * ln2) : 0.f;
    }
  }
  for (int idx = tid; idx < kBlockRows * D; idx += blockDim.x) {
    const int i = r0 + idx / D;
    if (i < g.L && i >= n && !(g.dustbin && i == n)) p.O[(bh * L + i) * D + idx % D] = 0.f;
  }
  if (r0 >= n) return;

  if (tid == 0)
    sh_vref = p.part_in ? finish_v<T>(g, bh, n, r0, p.v_prev2, p.part_in, p.b, bb, p.dstate, p.sdr, p.Q, p.K, p.u_in)
                        : 0.0;
  __syncthreads();
  const double vref = sh_vref;

  float* w2s = reinterpret_cast<float*>(smem);                       // [NWC]
  char* vt = smem + (size_t)NWC * 4;                                 // [D][VTS] elements
  for (int c = tid; c < NWC; c += blockDim.x) {
    const int j = tw0 * 16 + c;
    float w = kNegInf;
    if (j >= 0 && j < n) {
      double vj = 0.0;
      if (p.part_in) vj = finish_v<T>(g, bh, n, j, p.v_prev2, p.part_in, p.b, bb, p.dstate, p.sdr, p.Q, p.K, p.u_in);
      if (j >= r0 && j < r0 + kBlockRows) {
        p.v_out[bh * L + j] = (float)(vj * ln2);
        if (p.v_tail) p.v_tail[bh * L + j] = vj;
      }
      w = (float)(vj - vref);
    }
    w2s[c] = w;
  }
  {  // V window, transposed into LDS
    const char* Vb = reinterpret_cast<const char*>(p.V) + (size_t)bh * L * RB;
    const int per_row = RB / 16;
    for (int idx = tid; idx < NWC * per_row; idx += blockDim.x) {
      const int row = idx / per_row, c16 = idx - row * per_row;
      const int j = tw0 * 16 + row;
      u4 val = {0u, 0u, 0u, 0u};
      if (j >= 0 && j < n) val = ld16(Vb + (size_t)j * RB + c16 * 16);
      if (EB == 2) {
        const uint16_t* hv = reinterpret_cast<const uint16_t*>(&val);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          reinterpret_cast<uint16_t*>(vt)[(size_t)(c16 * 8 + e) * VTS + row] = hv[e];
      } else {
        const uint32_t* fv = reinterpret_cast<const uint32_t*>(&val);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          reinterpret_cast<uint32_t*>(vt)[(size_t)(c16 * 4 + e) * VTS + row] = fv[e];
      }
    }
  }
  __syncthreads();

  const int wave = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int i0 = r0 + wave * 16;
  if (i0 >= n) return;
  const int NT = g.NT;
  const int tg0 = tw0 + wave;
  int t_lo = -tg0;
  t_lo = t_lo < 0 ? 0 : t_lo;
  int t_hi = (n - 1) / 16 - tg0;
  t_hi = t_hi > NT - 1 ? NT - 1 : t_hi;

  // Q strip as the B operand (row i0 + lr), K tiles as the A operand.
  const char* Qb = reinterpret_cast<const char*>(p.Q) + (size_t)bh * L * RB;
  const char* Kb = reinterpret_cast<const char*>(p.K) + (size_t)bh * L * RB;
  const int qi = i0 + lr;
  const bool myrow = qi < n;
  u4 qb[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    qb[c] = (u4){0u, 0u, 0u, 0u};
    if (myrow) qb[c] = ld16(Qb + (size_t)qi * RB + c * 64 + lg * 16);
  }
  // u_i + v_ref (the window holds v_j - v_ref)
  const float ui2 = (float)(((myrow && p.u_in) ? p.u_in[bh * L + qi] : 0.0) + vref);

  f4 oacc[ND];
#pragma unroll
  for (int c = 0; c < ND; ++c) oacc[c] = (f4){0.f, 0.f, 0.f, 0.f};

  // plan tile t: lane holds P[i0 + lr][(tg0 + t) * 16 + 4 lg + r]
  auto plan_tile = [&](int t, float (&pt)[4]) {
    if (t >= NT || t < t_lo || t > t_hi) {
#pragma unroll
      for (int r = 0; r < 4; ++r) pt[r] = 0.f;
      return;
    }
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    const int jrow = (tg0 + t) * 16 + lr;  // A operand row (K), may be outside [0, n)
    const bool kin = jrow >= 0 && jrow < n;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      u4 ka = {0u, 0u, 0u, 0u};
      if (kin) ka = ld16(Kb + (size_t)jrow * RB + c * 64 + lg * 16);
      acc = Elt<T>::mma_chunk(acc, ka, qb[c]);
    }
    const int obase = (t - g.TL) * 16 + 4 * lg - lr;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int o = obase + r;
      const float w = w2s[(wave + t) * 16 + 4 * lg + r];
      float x = __builtin_fmaf(acc[r], g.scale2, w + ui2);
      x = (o >= -g.h1 && o <= g.h2 && myrow) ? x : kNegInf;
      pt[r] = exp2_fast(x);
    }
  };

  if constexpr (EB == 2) {
    for (int t = 0; t < NT; t += 2) {
      float p0[4], p1[4];
      plan_tile(t, p0);
      plan_tile(t + 1, p1);
      // split P into hi + lo bf16 operands, k slots 8 lg + (0..3 | 4..7)
      uint32_t hb[8], lb[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        hb[r] = float_to_bf16_bits(p0[r]);
        hb[4 + r] = float_to_bf16_bits(p1[r]);
        lb[r] = float_to_bf16_bits(p0[r] - bits_to_float(hb[r] << 16));
        lb[4 + r] = float_to_bf16_bits(p1[r] - bits_to_float(hb[4 + r] << 16));
      }
      const u4 hi = {hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16), hb[4] | (hb[5] << 16), hb[6] | (hb[7] << 16)};
      const u4 lo = {lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16), lb[4] | (lb[5] << 16), lb[6] | (lb[7] << 16)};
      const int c0 = (wave + t) * 16 + 4 * lg;  // window column of slot 0
#pragma unroll
      for (int dc = 0; dc < ND; ++dc) {
        const uint16_t* row = reinterpret_cast<const uint16_t*>(vt) + (size_t)(dc * 16 + lr) * VTS;
        const u2 x0 = *reinterpret_cast<const u2*>(row + c0);
        u2 x1 = {0u, 0u};
        if (t + 1 < NT) x1 = *reinterpret_cast<const u2*>(row + c0 + 16);
        const u4 vb = {x0.x, x0.y, x1.x, x1.y};
        oacc[dc] = Elt<bf16_t>::mma_chunk(oacc[dc], hi, vb);
        oacc[dc] = Elt<bf16_t>::mma_chunk(oacc[dc], lo, vb);
      }
    }
  } else {
    for (int t = 0; t < NT; ++t) {
      float pt[4];
      plan_tile(t, pt);
      const int c0 = (wave + t) * 16 + 4 * lg;
#pragma unroll
      for (int dc = 0; dc < ND; ++dc) {
        const float* row = reinterpret_cast<const float*>(vt) + (size_t)(dc * 16 + lr) * VTS;
        const f4 vb = *reinterpret_cast<const f4*>(row + c0);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          oacc[dc] = __builtin_amdgcn_mfma_f32_16x16x4f32(pt[r], vb[r], oacc[dc], 0, 0, 0);
      }
    }
  }
  // dustbin column term for real rows: P_i,delta V_delta
  float pd[4] = {0.f, 0.f, 0.f, 0.f};
  if (g.dustbin) {
    const double vd = p.dstate ? p.dstate[4 * bh + 1] : 0.0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = i0 + 4 * lg + r;
      if (i < n) {
        const double ui = p.u_in ? p.u_in[bh * L + i] : 0.0;
        pd[r] = exp2_fast((float)((double)p.sdc[bh * L + i] + ui + vd));
      }
    }
  }
  const T* Vbase = reinterpret_cast<const T*>(p.V) + ((size_t)bh * L + (g.dustbin ? n : 0)) * D;
#pragma unroll
  for (int dc = 0; dc < ND; ++dc) {
    const int col = dc * 16 + lr;
    const float vdel = g.dustbin ? Elt<T>::load(Vbase, col) : 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = i0 + 4 * lg + r;
      if (i < n) p.O[((size_t)bh * L + i) * D + col] = oacc[dc][r] + pd[r] * vdel;
    }
  }
}

// Output epilogue for bf16 with d >= 64: the same results as output_kernel,
// with the band tiles streamed through LDS as in the backward sweeps.  One
// workgroup of 8 waves per 128-row block; the block's NT + 7 window tiles of
// K (score side, MFMA A operand) and V (product side) pass through LDS two at
// a time, double-buffered; a wave keeps its 16-row Q strip and its O tile in
// registers.  P enters the P V product as hi + lo bf16 (4 + 4 k-slots per
// lane over the tile pair) against V rows read transposed from LDS.
template <int D>
__global__ __launch_bounds__(512) void output_sweep_kernel(Geom g, OutArgs p) {
  constexpr int RB = D * 2;
  constexpr int CPR = RB / 16;
  constexpr int NCH = RB / 64;
  constexpr int ND = D / 16;
  constexpr int TBYTES = 32 * RB;
  constexpr int kThreads = 512;
  static_assert(CPR >= 8, "the chunk swizzle needs 8 chunks per row");
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int nbh = g.B * g.H;
  const int logical = xcd_remap(blockIdx.x, p.padded_grid);
  if (logical >= nbh * g.nblk) return;
  const int bh = logical / g.nblk;
  const int blk = logical - bh * g.nblk;
  const int bb = bh / g.H;
  const int n = real_len(g, bb);
  const int r0 = blk * kBlockRows;
  const size_t L = g.L;
  const int tid = threadIdx.x;
  const double ln2 = 0.6931471805599453;

  // u outputs, filler rows of u, v and O for the owned range
  auto owned_rows = [&]() {
    for (int c = tid; c < kBlockRows; c += kThreads) {
      const int i = r0 + c;
      if (i >= g.L) break;
      if (i >= n) {
        if (!(g.dustbin && i == n)) {
          p.u_out[bh * L + i] = kNegInf;
          p.v_out[bh * L + i] = kNegInf;
        }
      } else {
        p.u_out[bh * L + i] = p.u_in ? (float)(p.u_in[bh * L + i] * ln2) : 0.f;
      }
    }
    for (int idx = tid; idx < kBlockRows * D; idx += kThreads) {
      const int i = r0 + idx / D;
      if (i < g.L && i >= n && !(g.dustbin && i == n)) p.O[(bh * L + i) * D + idx % D] = 0.f;
    }
  };
  if (r0 >= n) {
    owned_rows();
    return;
  }

  const int NT = g.NT;
  const int NW = NT + kWaves - 1;
  const int NP = (NW + 1) >> 1;
  const int NWC = 2 * NP * 16;
  const int tw0 = blk * 8 - g.TL;
  constexpr int NBUF = 4;                                          // pair buffers: three pairs in flight
  char* tbuf = smem;                                               // [NBUF][2 tensors][32 rows][RB]
  double* vjs = reinterpret_cast<double*>(smem + NBUF * 2 * TBYTES);  // [NWC] v_j of the window columns
  float* wv = reinterpret_cast<float*>(vjs + NWC);                 // [NWC] v_j - vref

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  // The set-up's loads (Q strip, u of the strip rows, the inputs of every
  // window column's v) are issued from clamped, always valid indices with no
  // branch before them, so they are all in flight together; results are
  // selected afterwards.
  const int i0 = r0 + wave * 16;
  const int si = i0 + lr;
  const bool sok = si < n;
  const int sic = sok ? si : n - 1;  // n >= 1: the block holds a real row
  const char* Qb = reinterpret_cast<const char*>(p.Q) + (size_t)bh * L * RB;
  u4 qs[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const u4 q = ld16(Qb + (size_t)sic * RB + c * 64 + lg * 16);
    qs[c] = sok ? q : (u4){0u, 0u, 0u, 0u};
  }
  const double ui_s = p.u_in ? p.u_in[bh * L + sic] : 0.0;

  // v of the window's columns: v^(N) from the last step's column partials
  // (zero when there was no step); the block's own columns are published
  const DustC dc = load_dust(g, bh, p.dstate);
  const size_t slice = (size_t)bh * L * RB;
  for (int c = tid; c < NWC; c += kThreads) {
    const int j = tw0 * 16 + c;
    const int jc = j < 0 ? 0 : (j < n ? j : n - 1);
    double vj = 0.0;
    if (p.part_in) {
      int slo, shi;
      window_segments(g, jc, slo, shi);
      vj = finish_checked<bf16_t, false>(g, gather_v_clamped(g, bh, n, jc, slo, shi, p.v_prev2, p.part_in, p.b, bb,
                                                             p.sdr),
                                         dc, bh, n, jc, reinterpret_cast<const char*>(p.Q) + slice,
                                         reinterpret_cast<const char*>(p.K) + slice, p.u_in);
    }
    if (j == jc && j >= r0 && j < r0 + kBlockRows) {
      p.v_out[bh * L + j] = (float)(vj * ln2);
      if (p.v_tail) p.v_tail[bh * L + j] = vj;
    }
    vjs[c] = vj;
  }
  owned_rows();
  __syncthreads();
  // the exponent split's reference: v of the block's first column (inside
  // the window, at position 16 TL)
  const double vref = vjs[16 * g.TL];
  for (int c = tid; c < NWC; c += kThreads) {
    const int j = tw0 * 16 + c;
    wv[c] = (j >= 0 && j < n) ? (float)(vjs[c] - vref) : kNegInf;
  }
  const float ui2 = sok ? (float)(ui_s + vref) : 0.f;

  const char* Kb = reinterpret_cast<const char*>(p.K) + (size_t)bh * L * RB;
  const char* Vb = reinterpret_cast<const char*>(p.V) + (size_t)bh * L * RB;
  // K and V tile pairs stream into LDS by DMA, three pairs ahead: wave w
  // fills bytes [w KB, (w + 1) KB) of each tensor's pair buffer, and the lane
  // at chunk position pc of its row loads logical chunk pc ^ f(row), leaving
  // the swizzled layout the reads expect.  Rows outside the sequence are
  // loaded from the nearest real row (their scores are masked to -inf, so
  // every product they enter is exactly zero).
  constexpr int RPW = 1024 / RB;  // rows per wave instruction
  const bool dma_wave = wave < 32 / RPW;
  const uint32_t lds_base = lds_addr(tbuf);
  auto issue_pair = [&](int pp) {
    if (dma_wave) {
      const int pos = lane * 16;
      const int r32 = wave * RPW + pos / RB;
      const int c = sw_chunk<CPR>((pos % RB) / 16, r32);
      int row = (tw0 + 2 * pp) * 16 + r32;
      row = row < 0 ? 0 : (row >= n ? n - 1 : row);
      const uint32_t dst = lds_base + (uint32_t)((pp % NBUF) * 2) * TBYTES + wave * 1024;
      const uint32_t off = (uint32_t)(row * RB + c * 16);
      lds_dma16(Kb, off, dst);
      lds_dma16(Vb, off, dst + TBYTES);
    }
  };
  // this wave's LDS reads done and its DMAs of the next pair landed (at most
  // `later` pairs after it in flight; the loop issues no other vector memory
  // operation), then the waves meet (a plain __syncthreads would wait for
  // every DMA in flight)
  auto pipe_barrier = [&](int later) {
    asm volatile("" ::: "memory");
    constexpr int kLgkm0 = 0x0070;  // lgkmcnt(0), expcnt left free; vmcnt in bits 3:0
    if (later >= 2) __builtin_amdgcn_s_waitcnt(kLgkm0 | 4);
    else if (later == 1) __builtin_amdgcn_s_waitcnt(kLgkm0 | 2);
    else __builtin_amdgcn_s_waitcnt(kLgkm0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  int offA[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) offA[c] = lr * RB + sw_chunk<CPR>(4 * c + lg, lr) * 16;
  int offB[ND];
  {
    const int row = 4 * lg + (lr >> 2);
#pragma unroll
    for (int ds = 0; ds < ND; ++ds) offB[ds] = row * RB + sw_chunk<CPR>(2 * ds + ((lr & 3) >> 1), row) * 16 + 8 * (lr & 1);
  }

  f4 oacc[ND];
#pragma unroll
  for (int ds = 0; ds < ND; ++ds) oacc[ds] = (f4){0.f, 0.f, 0.f, 0.f};

  for (int q = 0; q < 3 && q < NP; ++q) issue_pair(q);
  pipe_barrier((NP - 1 < 2) ? NP - 1 : 2);  // pair 0
  const bool wactive = i0 < n;
  for (int pp = 0; pp < NP; ++pp) {
    const int buf = pp % NBUF;
    // pair pp + 3 into the buffer pair pp - 1 used (every wave is past it)
    if (pp + 3 < NP) issue_pair(pp + 3);
    float val[2][4];
    bool any = false;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int wt = 2 * pp + tt;
      const int t = wt - wave;
      const int tg = tw0 + wt;
      const bool act = wactive && t >= 0 && t < NT && tg >= 0 && tg * 16 < n;
#pragma unroll
      for (int r = 0; r < 4; ++r) val[tt][r] = 0.f;
      if (act) {
        any = true;
        const char* tb0 = tbuf + (size_t)(buf * 2) * TBYTES + tt * 16 * RB;
        f4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          const u4 a = ld16(tb0 + offA[c]);
          sacc = Elt<bf16_t>::mma_chunk(sacc, a, qs[c]);
        }
        const int cw = wt * 16 + 4 * lg;
        const f4 w4 = *reinterpret_cast<const f4*>(wv + cw);
        // wave-uniform: every entry of the tile lies inside the band and
        // between real rows and columns, so no entry needs the mask
        const int olo = tg * 16 - i0 - 15;  // lowest j - i of the tile
        const bool inner = olo >= -g.h1 && olo + 30 <= g.h2 && i0 + 16 <= n && tg * 16 + 16 <= n;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int wj = tg * 16 + 4 * lg + r;
          const int o = wj - si;
          float x = __builtin_fmaf(sacc[r], g.scale2, w4[r] + ui2);
          if (!inner) x = (o >= -g.h1 && o <= g.h2 && sok && wj >= 0 && wj < n) ? x : kNegInf;
          val[tt][r] = exp2_fast(x);
        }
      }
    }
    if (any) {
      u4 hi, lo;
      split_hilo(val[0], val[1], hi, lo);
      const char* pb = tbuf + (size_t)(buf * 2 + 1) * TBYTES;
#pragma unroll
      for (int ds = 0; ds < ND; ++ds) {
        const int ob = offB[ds];
        const u2 b0 = ld_tr16(pb + ob);
        const u2 b1 = ld_tr16(pb + 16 * RB + ob);
        const u4 bv = {b0.x, b0.y, b1.x, b1.y};
        oacc[ds] = Elt<bf16_t>::mma_chunk(oacc[ds], hi, bv);
        oacc[ds] = Elt<bf16_t>::mma_chunk(oacc[ds], lo, bv);
      }
    }
    const int later = NP - 2 - pp;  // pairs issued after pair pp + 1
    pipe_barrier(later < 0 ? 0 : (later > 2 ? 2 : later));
  }
  if (!wactive) return;
  // dustbin column term for real rows: P_i,delta V_delta
  // (loads from clamped rows, all issued before the first store of O)
  float pd[4] = {0.f, 0.f, 0.f, 0.f};
  float vdel[ND];
#pragma unroll
  for (int ds = 0; ds < ND; ++ds) vdel[ds] = 0.f;
  if (g.dustbin) {
    const double vd = p.dstate ? p.dstate[4 * bh + 1] : 0.0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = i0 + 4 * lg + r;
      const int ic = i < n ? i : n - 1;
      const double ui = p.u_in ? p.u_in[bh * L + ic] : 0.0;
      const float e = exp2_fast((float)((double)p.sdc[bh * L + ic] + ui + vd));
      pd[r] = i < n ? e : 0.f;
    }
    const bf16_t* Vd = reinterpret_cast<const bf16_t*>(p.V) + ((size_t)bh * L + n) * D;
#pragma unroll
    for (int ds = 0; ds < ND; ++ds) vdel[ds] = Elt<bf16_t>::load(Vd, ds * 16 + lr);
  }
#pragma unroll
  for (int ds = 0; ds < ND; ++ds) {
    const int col = ds * 16 + lr;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = i0 + 4 * lg + r;
      if (i < n) p.O[((size_t)bh * L + i) * D + col] = oacc[ds][r] + pd[r] * vdel[ds];
    }
  }
}

// Dustbin row of the output: O_delta = sum_j P_delta,j V_j over active j,
// plus u, v of the dustbin (state fp64 log2 units, outputs natural).
// The columns go in chunks of 256, one workgroup per (chunk, (b, h)): each
// thread forms the plan entry of one column, then every output element sums
// the chunk's weighted V rows (256 / d threads per element, each taking every
// (256 / d)-th row) into `dpart`; dustbin_output_fin adds the chunks in a
// fixed order.
template <typename T>
__global__ __launch_bounds__(256) void dustbin_output_part(Geom g, const T* V, const double* v2_real,
                                                           const double* dstate, const float* sdr, float* dpart) {
  const int bh = blockIdx.y;
  const int chunk = blockIdx.x;
  const int n = real_len(g, bh / g.H);
  const size_t L = g.L;
  const int d = g.d;
  const int tid = threadIdx.x;
  const int j0 = chunk * 256;
  if (j0 > n) return;  // past the dustbin: the finish reads only the chunks up to it
  const double ud = dstate ? dstate[4 * bh + 0] : 0.0;
  const double vd = dstate ? dstate[4 * bh + 1] : 0.0;
  __shared__ float wch[256];
  __shared__ float red[256];
  const int tpc = 256 / d;  // d divides 256
  const int col = tid % d, part = tid / d;
  const int j = j0 + tid;
  float w = 0.f;
  if (j <= n) {
    const double vj = (j == n) ? vd : v2_real[bh * L + j];
    w = exp2_fast((float)((double)sdr[bh * L + j] + ud + vj));
  }
  wch[tid] = w;
  __syncthreads();
  const int cnt = n + 1 - j0 < 256 ? n + 1 - j0 : 256;
  float acc = 0.f;
  for (int k = part; k < cnt; k += tpc) acc = __builtin_fmaf(wch[k], Elt<T>::load(V, ((size_t)bh * L + j0 + k) * d + col), acc);
  red[tid] = acc;
  __syncthreads();
  if (part == 0) {
    float sum = 0.f;
    for (int k = 0; k < tpc; ++k) sum += red[col + k * d];
    dpart[((size_t)bh * gridDim.x + chunk) * d + col] = sum;
  }
}

__global__ __launch_bounds__(256) void dustbin_output_fin(Geom g, const double* dstate, const float* dpart, int nch,
                                                          float* O, float* u_out, float* v_out) {
  const int bh = blockIdx.x;
  const int n = real_len(g, bh / g.H);
  const size_t L = g.L;
  const int d = g.d;
  const int tid = threadIdx.x;
  const int used = (n + 1 + 255) / 256;
  const float* in = dpart + (size_t)bh * nch * d;
  for (int c = tid; c < d; c += 256) {
    float sum = 0.f;
    for (int k = 0; k < used; ++k) sum += in[(size_t)k * d + c];
    O[((size_t)bh * L + n) * d + c] = sum;
  }
  if (tid == 0) {
    const double ln2 = 0.6931471805599453;
    const double ud = dstate ? dstate[4 * bh + 0] : 0.0;
    const double vd = dstate ? dstate[4 * bh + 1] : 0.0;
    u_out[bh * L + n] = (float)(ud * ln2);
    v_out[bh * L + n] = (float)(vd * ln2);
  }
}

__global__ void fill_int(int* p, int n, int v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// A neighbour wait of the persistent step kernel gave up (results invalid):
// make that visible in the outputs.
__global__ void step_wait_failed(const int* err, float* O, float* u) {
  if (*err) {
    O[0] = __builtin_nanf("");
    u[0] = __builtin_nanf("");
  }
}

// Debug content check (SINKATTN_DEBUG): counts the non-finite values among the
// stopped base u^(0), v^(0) (fp64 tail slot 0) and the returned u, v on the
// active tokens of every (b, h).
__global__ void debug_scan(Geom g, const double* u0, const double* v0, const float* u, const float* v, int* count) {
  const int bh = blockIdx.y;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int n = real_len(g, bh / g.H) + (g.dustbin ? 1 : 0);
  if (i >= n) return;
  const size_t o = (size_t)bh * g.L + i;
  const bool bad = !isfinite(u0[o]) || !isfinite(v0[o]) || !isfinite(u[o]) || !isfinite(v[o]);
  if (bad) atomicAdd(count, 1);
}

// ---------------------------------------------------------------------------
// Host launcher for the whole forward pass.
// ---------------------------------------------------------------------------
static inline int padded8(int x) { return (x + 7) & ~7; }

template <typename T, int D>
static hipError_t forward_impl(const Geom& g, const FwdLaunch& f, const Workspace& w, hipStream_t st) {
  constexpr int RB = D * Elt<T>::kBytes;
  const int nbh = g.B * g.H;
  const size_t BHL = (size_t)nbh * g.L;
  const int grid = padded8(nbh * g.nblk);
  const int iter_grid = padded8(nbh * g.nseg);
  const int ring_cols = g.NWC + 8 * 16;  // window + the next block's 8 tiles
  const size_t iter_lds = (size_t)ring_cols * (RB + 16) + (size_t)ring_cols * 4 * 2 +
                          (size_t)2 * kWaves * g.NT * 16 * 4 + 2 * kWaves * 4 + 64;
  const size_t out_lds = (size_t)g.NWC * 4 + (size_t)D * (g.NWC + 8) * Elt<T>::kBytes + 64;
  hipError_t err;
  if (iter_lds > 160 * 1024 || out_lds > 160 * 1024) return hipErrorInvalidConfiguration;
  // compile-time tile count: the smallest instance covering the band
  const void* ik;
  const void* ikp;  // persistent instance
  // a band whose only edge-crossing strip tiles are the first and last takes
  // the persistent instance compiled for that case (FE)
  const bool ends_only = (g.edge_mask & ~(1u | (1u << (g.NT - 1)))) == 0u;
  auto pick = [&](auto ntc) {
    constexpr int N = decltype(ntc)::value;
    ik = reinterpret_cast<const void*>(iter_kernel<T, D, N, false>);
    ikp = ends_only ? reinterpret_cast<const void*>(iter_kernel<T, D, N, true, true>)
                    : reinterpret_cast<const void*>(iter_kernel<T, D, N, true, false>);
  };
  if (g.NT <= 3) pick(std::integral_constant<int, 3>{});
  else if (g.NT <= 5) pick(std::integral_constant<int, 5>{});
  else if (g.NT <= 9) pick(std::integral_constant<int, 9>{});
  else pick(std::integral_constant<int, kMaxTiles>{});
  err = ensure_lds(ik, iter_lds);
  if (err != hipSuccess) return err;
  err = ensure_lds(ikp, iter_lds);
  if (err != hipSuccess) return err;
  err = ensure_lds(reinterpret_cast<const void*>(output_kernel<T, D>), out_lds);
  if (err != hipSuccess) return err;

  if (g.dustbin) {
    dim3 sg((g.L + 255) / 256, nbh);
    hipLaunchKernelGGL(dustbin_scores<T>, sg, dim3(256), 0, st, g, reinterpret_cast<const T*>(f.Q),
                       reinterpret_cast<const T*>(f.K), w.sdr, w.sdc);
  }
  if (f.T == 0) {
    dim3 zg((g.L + 255) / 256, nbh);
    hipLaunchKernelGGL(zero_start, zg, dim3(256), 0, st, g, w.tail_u, w.tail_v);
  }
  const size_t part_slot = (size_t)nbh * g.nseg * g.SW;
  const bool stop_early = f.stop.every > 0;
  // Step t of a run whose base has T steps.  A checked step (t = c + 1 after
  // a check point c) writes u^(t) only to tail slot 1 and v^(t-1) to slot 0,
  // so that it is the first tail step if the check passes; base_check then
  // moves the latest-u buffer on.
  auto launch_step = [&](int t, int Tbase, bool check) {
    const int N = Tbase + f.R;
    IterArgs a{};
    a.Q = f.Q;
    a.K = f.K;
    a.a = f.a;
    a.b = f.b;
    a.first = (t == 1);
    a.part_in = (t == 1) ? nullptr : w.part + (size_t)((t - 1) & 1) * part_slot;
    a.v_prev2 = (t <= 2) ? nullptr : w.vbuf + (size_t)((t - 2) & 1) * BHL;
    a.v_out = (t == 1) ? nullptr : w.vbuf + (size_t)((t - 1) & 1) * BHL;
    a.v_tail = (t >= 2 && t - 1 >= Tbase) ? w.tail_v + (size_t)(t - 1 - Tbase) * BHL : nullptr;
    a.u_out = w.ubuf + (size_t)(t & 1) * BHL;
    a.u_prev = t >= 2 ? w.ubuf + (size_t)((t - 1) & 1) * BHL : nullptr;
    a.u_tail = (t >= Tbase) ? w.tail_u + (size_t)(t - Tbase) * BHL : nullptr;
    if (check) {
      a.v_tail = w.tail_v;
      a.u_out = w.tail_u + BHL;
      a.u_tail = nullptr;
    }
    a.part_out = w.part + (size_t)(t & 1) * part_slot;
    a.partd_out = w.partd + (size_t)(t & 1) * nbh * g.nseg;
    a.dstate = (g.dustbin && t > 1) ? w.dstate : nullptr;
    a.sdr = w.sdr;
    a.sdc = w.sdc;
    a.padded_grid = iter_grid;
    // timing brackets: the whole run of step launches, or each launch when
    // the dustbin kernel runs between them (not kept when the base may stop
    // early: the host waits at every check)
    const bool tm = timing_enabled() && !stop_early;
    if (tm && (g.dustbin || t == 1)) timing_mark(st, false);
    if (g.NT <= 3)
      hipLaunchKernelGGL((iter_kernel<T, D, 3, false>), dim3(iter_grid), dim3(512), iter_lds, st, g, a,
                         StepPlan{});
    else if (g.NT <= 5)
      hipLaunchKernelGGL((iter_kernel<T, D, 5, false>), dim3(iter_grid), dim3(512), iter_lds, st, g, a,
                         StepPlan{});
    else if (g.NT <= 9)
      hipLaunchKernelGGL((iter_kernel<T, D, 9, false>), dim3(iter_grid), dim3(512), iter_lds, st, g, a,
                         StepPlan{});
    else
      hipLaunchKernelGGL((iter_kernel<T, D, kMaxTiles, false>), dim3(iter_grid), dim3(512), iter_lds, st, g, a,
                         StepPlan{});
    if (tm && (g.dustbin || t == N)) timing_mark(st, true, g.dustbin ? 1 : N);
    if (g.dustbin) {
      DustArgs da{};
      da.a = f.a;
      da.b = f.b;
      da.v_cur = (t == 1) ? nullptr : a.v_out;
      da.partd = a.partd_out;
      da.dstate = w.dstate;
      da.sdr = w.sdr;
      da.sdc = w.sdc;
      da.u_tail = a.u_tail;
      da.v_tail = (t >= Tbase) ? w.tail_v + (size_t)(t - Tbase) * BHL : nullptr;
      da.u_out = a.u_out;
      if (check) {
        da.v_tail = w.tail_v + BHL;
        da.v_prev_tail = w.tail_v;
      }
      da.first = (t == 1);
      hipLaunchKernelGGL(dustbin_step, dim3(nbh), dim3(256), 0, st, g, da);
    }
  };
  // Base: T steps, or (early stop) up to T steps with a check of e_c (see
  // base_check) carried by step c + 1 for c = every, 2 every, ... while
  // c + 2 <= T.  The base ends at the first c with max over (b, h) of
  // e_c < tol; step c + 1 is then the first tail step.
  int Tb = f.T;
  int t = 1;
  const int N = f.T + f.R;
  // Every step in one cooperative launch of the persistent instance, when all
  // its workgroups fit on the device at once (no dustbin, no early stop; set
  // SINKATTN_STEP_LAUNCHES to launch once per step instead), and when a
  // segment is at least as wide as the band's tile span: the persistent
  // kernel synchronises a segment with its two neighbours only, and with
  // narrower segments the windows of segments two apart overlap, so a turn
  // would read partial sums of a segment it never waited for.
  bool persistent = false;
  if (N >= 2 && !g.dustbin && !stop_early && g.SB * kBlockRows >= 16 * (g.TL + g.TR) &&
      !std::getenv("SINKATTN_STEP_LAUNCHES")) {
    long long resident = 0;
    err = coop_groups(ikp, 512, iter_lds, &resident);
    if (err != hipSuccess) return err;
    if (resident >= iter_grid) {
      const int nprog = 2 * nbh * g.nseg + 2;  // counters, the error flag, the debug count
      hipLaunchKernelGGL(fill_int, dim3((nprog + 255) / 256), dim3(256), 0, st, w.prog, nprog, 0);
      IterArgs a{};
      a.Q = f.Q;
      a.K = f.K;
      a.a = f.a;
      a.b = f.b;
      a.sdr = w.sdr;
      a.sdc = w.sdc;
      a.padded_grid = iter_grid;
      const bool stall_test = std::getenv("SINKATTN_DEBUG_STALL") != nullptr;
      StepPlan q{w.part, w.vbuf, w.ubuf, w.tail_u, w.tail_v, part_slot, BHL, f.T, 1, N, w.prog,
                 w.prog + nbh * g.nseg, w.prog + 2 * nbh * g.nseg,
                 stall_test ? kStallTestSpins : kMaxSpins, stall_test ? kStallTestBias : 0};
      Geom gg = g;
      void* args[] = {&gg, &a, &q};
      if (timing_enabled()) timing_mark(st, false);
      err = hipLaunchCooperativeKernel(ikp, dim3(iter_grid), dim3(512), args, (unsigned)iter_lds, st);
      if (err == hipSuccess) {
        if (timing_enabled()) timing_mark(st, true, N);
        persistent = true;
        t = N + 1;
      } else if (err == hipErrorCooperativeLaunchTooLarge || err == hipErrorNotSupported) {
        // the device refused to make every workgroup resident at once (for
        // example while another process holds part of it): run the same
        // steps as one launch each instead (the progress counters reset
        // above are not used by those launches)
        (void)hipGetLastError();
        if (timing_enabled()) timing_mark(st, true, 0);
      } else {
        return err;
      }
    }
  }
  if (persistent) {
  } else if (stop_early) {
    std::vector<double> eh((size_t)nbh);
    for (; t <= f.T; ++t) {
      const int c = t - 1;
      const bool check = c >= 1 && c % f.stop.every == 0 && c + 2 <= f.T;
      launch_step(t, f.T, check);
      if (!check) continue;
      hipLaunchKernelGGL(base_check, dim3(nbh), dim3(256), 0, st, g, f.a, w.ubuf + (size_t)(c & 1) * BHL,
                         w.ubuf + (size_t)(t & 1) * BHL, w.tail_u + BHL, w.tail_u, w.err);
      err = hipMemcpyAsync(eh.data(), w.err, (size_t)nbh * sizeof(double), hipMemcpyDeviceToHost, st);
      if (err == hipSuccess) err = hipStreamSynchronize(st);
      if (err != hipSuccess) return err;
      double emax = 0.0;
      bool finite = true;
      for (double e : eh) {
        finite = finite && e == e;
        emax = e > emax ? e : emax;
      }
      if (f.stop.err_last) *f.stop.err_last = finite ? emax : NAN;
      if (finite && emax < f.stop.tol) {
        Tb = c;
        ++t;
        break;
      }
    }
  } else {
    for (; t <= f.T; ++t) launch_step(t, f.T, false);
  }
  for (; t <= Tb + f.R; ++t) launch_step(t, Tb, false);
  if (f.stop.T_used) *f.stop.T_used = Tb;
  const int Nrun = Tb + f.R;
  OutArgs o{};
  o.Q = f.Q;
  o.K = f.K;
  o.V = f.V;
  o.a = f.a;
  o.b = f.b;
  o.part_in = (Nrun == 0) ? nullptr : w.part + (size_t)(Nrun & 1) * part_slot;
  o.v_prev2 = (Nrun <= 1) ? nullptr : w.vbuf + (size_t)((Nrun - 1) & 1) * BHL;
  o.u_in = (Nrun == 0) ? nullptr : w.ubuf + (size_t)(Nrun & 1) * BHL;
  o.dstate = (g.dustbin && Nrun >= 1) ? w.dstate : nullptr;
  o.sdr = w.sdr;
  o.sdc = w.sdc;
  o.O = f.O;
  o.u_out = f.u;
  o.v_out = f.v;
  o.v_tail = w.tail_v + (size_t)f.R * BHL;
  o.padded_grid = grid;
  if constexpr (sizeof(T) == 2 && D >= 64) {
    const int NP = (g.NT + kWaves) / 2;
    const size_t sweep_lds = (size_t)8 * 32 * D * 2 + (size_t)2 * NP * 16 * 12 + 64;  // 4 pair buffers of K and V, vjs, wv
    err = ensure_lds(reinterpret_cast<const void*>(output_sweep_kernel<D>), sweep_lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((output_sweep_kernel<D>), dim3(grid), dim3(512), sweep_lds, st, g, o);
  } else {
    hipLaunchKernelGGL((output_kernel<T, D>), dim3(grid), dim3(512), out_lds, st, g, o);
  }
  if (persistent)
    hipLaunchKernelGGL(step_wait_failed, dim3(1), dim3(1), 0, st, w.prog + 2 * nbh * g.nseg, f.O, f.u);
  if (g.dustbin) {
    const int dch = (g.L + 255) / 256;
    hipLaunchKernelGGL(dustbin_output_part<T>, dim3(dch, nbh), dim3(256), 0, st, g, reinterpret_cast<const T*>(f.V),
                       w.tail_v + (size_t)f.R * BHL, o.dstate, w.sdr, w.dpart);
    hipLaunchKernelGGL(dustbin_output_fin, dim3(nbh), dim3(256), 0, st, g, o.dstate,
                       static_cast<const float*>(w.dpart), dch, f.O, f.u, f.v);
  }
  if (f.debug_flags) {
    // debug check: wait for the stream, then report a wait that gave up
    // (bit 1) and non-finite potentials (bit 0)
    int* cnt = w.prog + 2 * nbh * g.nseg;  // [error flag, non-finite count]
    if (!persistent) {
      hipLaunchKernelGGL(fill_int, dim3(1), dim3(64), 0, st, cnt, 2, 0);
    } else {
      hipLaunchKernelGGL(fill_int, dim3(1), dim3(64), 0, st, cnt + 1, 1, 0);
    }
    hipLaunchKernelGGL(debug_scan, dim3((g.L + 255) / 256, nbh), dim3(256), 0, st, g, w.tail_u, w.tail_v, f.u, f.v,
                       cnt + 1);
    int hv[2] = {0, 0};
    err = hipGetLastError();
    if (err == hipSuccess) err = hipMemcpyAsync(hv, cnt, sizeof(hv), hipMemcpyDeviceToHost, st);
    if (err == hipSuccess) err = hipStreamSynchronize(st);
    if (err != hipSuccess) return err;
    *f.debug_flags = (hv[0] ? 2 : 0) | (hv[1] ? 1 : 0);
  }
  return hipGetLastError();
}

hipError_t launch_forward(const Geom& g, int dtype, const FwdLaunch& f, const Workspace& w, hipStream_t st) {
  if (dtype == 0) {
    switch (g.d) {
      case 16: return forward_impl<float, 16>(g, f, w, st);
      case 32: return forward_impl<float, 32>(g, f, w, st);
      case 64: return forward_impl<float, 64>(g, f, w, st);
    }
  } else {
    switch (g.d) {
      case 32: return forward_impl<bf16_t, 32>(g, f, w, st);
      case 64: return forward_impl<bf16_t, 64>(g, f, w, st);
      case 128: return forward_impl<bf16_t, 128>(g, f, w, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace sinkattn
