// Sustained issue rates of the two units every band pass is bound by, for
// the roofline fractions of a run: the bf16 score MFMA
// (v_mfma_f32_16x16x32_bf16, the instruction each bf16 score tile and P.V
// product uses; 2 * 16 * 16 * 32 flops) and the exp2 of the plan entries
// (v_exp_f32, one per band entry per pass).  Published peaks assume the
// top clock; these probes give what the chip sustains under a full load at
// the clock it actually runs, which the probe also reports.
//
// Each probe keeps independent dependency chains in every wave and launches
// far more waves than the CUs hold, so that the unit, not the latency of one
// chain, sets the rate.  The MFMA probe keeps two accumulators per wave:
// with four or more the compiler moves accumulators between register files
// inside the loop and the probe measures those moves instead.  The chains'
// values are irrelevant to the rate; a run-time sentinel that the results
// never equal keeps them live without a store ever being taken.  The clock
// is s_memtime (shader clock) over s_memrealtime (fixed-rate wall clock) on
// workgroup 0.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "geom.hpp"

namespace sinkattn {

// External linkage: the compiler cannot prove the sink unread, so the
// conditional stores into it (never taken) keep the probe chains live.
__device__ float g_probe_sink[256];
__device__ unsigned long long g_probe_clock[4];  // s_memtime, s_memrealtime at the start and end of workgroup 0

namespace {

constexpr int kProbeThreads = 256;        // 4 waves
constexpr int kProbeBlocks = 256 * 8;     // 32 waves per CU, in several rounds
constexpr int kExpChains = 16;
constexpr int kMfmaChains = 2;
constexpr int kExpIters = 16384;
constexpr int kMfmaIters = 65536;
constexpr int kLdsProbeGroups = 256;  // one workgroup per CU (the ring fills most of the LDS)
constexpr int kLdsProbeIters = 200;

__device__ __forceinline__ void clock_mark(int which) {
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    g_probe_clock[2 * which] = __builtin_amdgcn_s_memtime();
    g_probe_clock[2 * which + 1] = __builtin_amdgcn_s_memrealtime();
  }
}

__global__ __launch_bounds__(kProbeThreads) void exp_probe_kernel(int iters, float sentinel) {
  clock_mark(0);
  float x[kExpChains];
#pragma unroll
  for (int c = 0; c < kExpChains; ++c) x[c] = 0.03125f * c + 1e-6f * threadIdx.x;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kExpChains; ++c) x[c] = exp2_fast(-x[c]);  // stays in (0, 1]
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kExpChains; ++c) s += x[c];
  if (s == sentinel) g_probe_sink[threadIdx.x] = s;
  __syncthreads();
  clock_mark(1);
}

__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(int iters, float sentinel) {
  clock_mark(0);
  const uint32_t lane = threadIdx.x & 63;
  // bf16 pairs near 2^-7: the accumulators stay finite over any run length
  const u4 a = {0x3c003c00u + lane, 0x3c013c00u, 0x3c003c02u, 0x3c033c00u};
  const u4 b = {0x3c003c01u, 0x3c023c00u + lane, 0x3c003c00u, 0x3c003c04u};
  f4 acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) acc[c] = (f4){0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c) acc[c] = Elt<bf16_t>::mma_chunk(acc[c], a, b);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  if (s == sentinel) g_probe_sink[threadIdx.x] = s;
  __syncthreads();
  clock_mark(1);
}

// LDS read pattern of the fused step kernel's K-tile operand reads: eight
// waves of one workgroup per CU each read, tile after tile, 17 consecutive
// tiles of a 32-tile ring of 16-row tiles (row stride RS bytes), lane (r, g)
// of a read taking the 16 bytes at 16 g + 64 c of row r (c = 0..3, one
// 128-bit read per c).  SWZ: 256-byte rows whose 16-byte chunk p sits at
// position p ^ ((r ^ 2 r) & 15) (each lane then forms four chunk offsets).
// Every workgroup records the shader cycles of its read loop.
__device__ unsigned long long g_lds_cycles[kLdsProbeGroups];

template <int RS, bool SWZ>
__global__ __launch_bounds__(512) void lds_probe_kernel(int iters, unsigned sentinel) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int TILEB = 16 * RS;
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int wave = tid >> 6;
  for (int i = tid; i < 32 * TILEB / 4; i += 512) reinterpret_cast<uint32_t*>(smem)[i] = i * 2654435761u;
  __syncthreads();
  int offc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    int pos = lg + 4 * c;
    if (SWZ) pos ^= (lr ^ (2 * lr)) & 15;
    offc[c] = lr * RS + pos * 16;  // < 16 RS: inside the tile
  }
  u4 acc = {0u, 0u, 0u, 0u};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int t = 0; t < 17; ++t) {
      const char* base = smem + ((wave + t + it) & 31) * TILEB;
#pragma unroll
      for (int c = 0; c < 4; ++c) acc ^= ld16(base + offc[c]);
    }
  }
  const unsigned h = acc.x ^ acc.y ^ acc.z ^ acc.w;
  __syncthreads();
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  if (h == sentinel) g_probe_sink[tid & 255] = 1.f;
  if (tid == 0) g_lds_cycles[blockIdx.x] = t1 - t0;
}

template <int RS, bool SWZ>
hipError_t time_lds_probe(hipStream_t st, double* cycles_per_read) {
  const size_t lds = (size_t)32 * 16 * RS;
  hipError_t e = ensure_lds(reinterpret_cast<const void*>(lds_probe_kernel<RS, SWZ>), lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((lds_probe_kernel<RS, SWZ>), dim3(kLdsProbeGroups), dim3(512), lds, st, kLdsProbeIters / 8, 0u);
  e = hipGetLastError();
  if (e == hipSuccess) {
    hipLaunchKernelGGL((lds_probe_kernel<RS, SWZ>), dim3(kLdsProbeGroups), dim3(512), lds, st, kLdsProbeIters, 0u);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  unsigned long long cyc[kLdsProbeGroups];
  if (e == hipSuccess)
    e = hipMemcpyFromSymbol(cyc, HIP_SYMBOL(g_lds_cycles), sizeof(cyc), 0, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return e;
  double sum = 0.0;
  for (int i = 0; i < kLdsProbeGroups; ++i) sum += (double)cyc[i];
  // wave-wide 128-bit reads per workgroup (the CU's LDS serves all of them)
  const double reads = (double)kLdsProbeIters * 17 * 4 * 8;
  *cycles_per_read = sum / kLdsProbeGroups / reads;
  return hipSuccess;
}

// One timed launch (after an untimed short one that brings the clocks up):
// elapsed seconds and the shader clock over workgroup 0's span.
template <typename Kernel>
hipError_t time_probe(Kernel kernel, int iters, hipStream_t st, double* seconds, double* clock_hz) {
  int dev = 0, wall_khz = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, dev);
  if (e != hipSuccess) return e;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(kernel, dim3(kProbeBlocks), dim3(kProbeThreads), 0, st, iters / 8, -1.f);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipEventRecord(e0, st);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(kernel, dim3(kProbeBlocks), dim3(kProbeThreads), 0, st, iters, -1.f);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipEventRecord(e1, st);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  float ms = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  unsigned long long clk[4] = {0, 0, 0, 0};
  if (e == hipSuccess) e = hipMemcpyFromSymbol(clk, HIP_SYMBOL(g_probe_clock), sizeof(clk), 0, hipMemcpyDeviceToHost);
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (e != hipSuccess) return e;
  *seconds = ms * 1e-3;
  const double wall_s = wall_khz > 0 && clk[3] > clk[1] ? (double)(clk[3] - clk[1]) / (wall_khz * 1e3) : 0.0;
  *clock_hz = wall_s > 0.0 && clk[2] > clk[0] ? (double)(clk[2] - clk[0]) / wall_s : 0.0;
  return hipSuccess;
}

}  // namespace

hipError_t launch_lds_probe(int row_stride, int swizzle, double* cycles_per_read, hipStream_t st) {
  if (swizzle) return row_stride == 256 ? time_lds_probe<256, true>(st, cycles_per_read) : hipErrorInvalidValue;
  switch (row_stride) {
    case 256: return time_lds_probe<256, false>(st, cycles_per_read);
    case 272: return time_lds_probe<272, false>(st, cycles_per_read);
    case 288: return time_lds_probe<288, false>(st, cycles_per_read);
    case 304: return time_lds_probe<304, false>(st, cycles_per_read);
    case 320: return time_lds_probe<320, false>(st, cycles_per_read);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_peak_probes(double* mfma_flops, double* exps, double* clock_hz, hipStream_t st) {
  double t_exp = 0.0, t_mfma = 0.0, clk_exp = 0.0, clk_mfma = 0.0;
  hipError_t e = time_probe(exp_probe_kernel, kExpIters, st, &t_exp, &clk_exp);
  if (e == hipSuccess) e = time_probe(mfma_probe_kernel, kMfmaIters, st, &t_mfma, &clk_mfma);
  if (e != hipSuccess) return e;
  const double threads = (double)kProbeBlocks * kProbeThreads;
  const double waves = threads / 64.0;
  *exps = t_exp > 0.0 ? threads * kExpIters * kExpChains / t_exp : 0.0;
  *mfma_flops = t_mfma > 0.0 ? waves * kMfmaIters * kMfmaChains * (2.0 * 16 * 16 * 32) / t_mfma : 0.0;
  if (clock_hz) *clock_hz = clk_mfma > 0.0 ? clk_mfma : clk_exp;
  return hipSuccess;
}

}  // namespace sinkattn
