// A-posteriori certificate of the stop-gradient bias and tail-depth
// selection ("Blockwise Differentiable Sinkhorn Attention", section 2.4, third
// certificate; section 4.1 reports it selecting R = 2 at tolerance 1e-5).
//
// The forward ran N = T + R_max steps and kept the tail stack u^(0..R_max),
// v^(0..R_max).  For R <= R_max, the surrogate gradient grad_R is the exact
// gradient of that same N-step forward with only its last R steps
// differentiable; it is the ordinary backward pass of depth R run on the top
// R + 1 slots of the stack (the potentials do not depend on where the
// stop-gradient sits).  Its adjoint vectors are the top R of the depth-R_max
// pass's (each is formed from the later steps only), so after one full pass
// every shallower gradient needs only the dQ and dK sweeps over those
// vectors, with the tail terms of the steps below the stop-gradient left out.
// The certificate is
//   eta_R = ||grad_Rmax - grad_R||_F / ||grad_Rmax||_F   over (dQ, dK),
// the gradient residual left by stopping the gradient after R steps, measured
// against the deepest tail available (dV does not depend on R).  With T = 0 the
// deepest tail is the full gradient through every step, so eta_R is then the
// full residual; otherwise the bias bound of section 2.4 (first certificate:
// the residual decays geometrically with R) makes it converge to the full
// residual as R_max grows.  Norms are fp64 sums in a fixed order.
#include <hip/hip_runtime.h>

#include <cmath>
#include <vector>

#include "geom.hpp"

namespace sinkattn {

hipError_t launch_backward(const Geom& g, int dtype, const BwdLaunch& f, const Workspace& w, hipStream_t st);

// part[2 blk] = sum (x - y)^2, part[2 blk + 1] = sum y^2 over a grid-stride
// slice of n4 float4 groups (fp64 accumulation).
__global__ __launch_bounds__(256) void diff_norm_parts(const float4* x, const float4* y, size_t n4, double* part) {
  const int tid = threadIdx.x;
  double dd = 0.0, yy = 0.0;
  for (size_t i = (size_t)blockIdx.x * 256 + tid; i < n4; i += (size_t)gridDim.x * 256) {
    const float4 a = x[i], b = y[i];
    const double e0 = (double)a.x - (double)b.x, e1 = (double)a.y - (double)b.y;
    const double e2 = (double)a.z - (double)b.z, e3 = (double)a.w - (double)b.w;
    dd += e0 * e0 + e1 * e1 + e2 * e2 + e3 * e3;
    yy += (double)b.x * b.x + (double)b.y * b.y + (double)b.z * b.z + (double)b.w * b.w;
  }
  __shared__ double s0[256], s1[256];
  s0[tid] = dd;
  s1[tid] = yy;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) {
      s0[tid] += s0[tid + s];
      s1[tid] += s1[tid + s];
    }
    __syncthreads();
  }
  if (tid == 0) {
    part[2 * blockIdx.x] = s0[0];
    part[2 * blockIdx.x + 1] = s1[0];
  }
}

// out[0..1] = the partials summed in a fixed order (one workgroup).
__global__ __launch_bounds__(256) void diff_norm_final(const double* part, int nparts, double* out) {
  const int tid = threadIdx.x;
  double dd = 0.0, yy = 0.0;
  for (int i = tid; i < nparts; i += 256) {
    dd += part[2 * i];
    yy += part[2 * i + 1];
  }
  __shared__ double s0[256], s1[256];
  s0[tid] = dd;
  s1[tid] = yy;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) {
      s0[tid] += s0[tid + s];
      s1[tid] += s1[tid + s];
    }
    __syncthreads();
  }
  if (tid == 0) {
    out[0] = s0[0];
    out[1] = s1[0];
  }
}

// `base` carries the inputs and the outputs of the reference pass (dQ, dK,
// dV at depth R_max); dQs, dKs receive each shallower pass.  eta: host
// [R_max + 1].  Waits for the stream before returning.
hipError_t launch_certificate(const Geom& g, int dtype, const BwdLaunch& base, int R_max, const Workspace& w,
                              float* dQs, float* dKs, double* eta, hipStream_t st) {
  const size_t n4 = (size_t)g.B * g.H * g.L * g.d / 4;  // d is a multiple of 16
  double* part = w.red;
  double* outs = w.red + 2 * kRedParts;  // [R][4]: dQ (dd, yy), dK (dd, yy)
  BwdLaunch f = base;
  f.R = R_max;
  f.slot0 = 0;
  f.vbar0 = nullptr;
  hipError_t err = launch_backward(g, dtype, f, w, st);
  if (err != hipSuccess) return err;
  for (int R = 0; R < R_max; ++R) {
    BwdLaunch fr = f;
    fr.R = R;
    fr.slot0 = R_max - R;
    fr.dQ = dQs;
    fr.dK = dKs;  // dV is the same at every depth: not recomputed
    fr.grad_only = 1;
    fr.R_vec = R_max;
    err = launch_backward(g, dtype, fr, w, st);
    if (err != hipSuccess) return err;
    const float* pairs[2][2] = {{dQs, base.dQ}, {dKs, base.dK}};
    for (int k = 0; k < 2; ++k) {
      hipLaunchKernelGGL(diff_norm_parts, dim3(kRedParts), dim3(256), 0, st,
                         reinterpret_cast<const float4*>(pairs[k][0]), reinterpret_cast<const float4*>(pairs[k][1]),
                         n4, part);
      hipLaunchKernelGGL(diff_norm_final, dim3(1), dim3(256), 0, st, part, kRedParts, outs + 4 * R + 2 * k);
    }
  }
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  std::vector<double> h((size_t)4 * (R_max > 0 ? R_max : 1), 0.0);
  if (R_max > 0) {
    err = hipMemcpyAsync(h.data(), outs, (size_t)4 * R_max * sizeof(double), hipMemcpyDeviceToHost, st);
    if (err != hipSuccess) return err;
  }
  err = hipStreamSynchronize(st);
  if (err != hipSuccess) return err;
  for (int R = 0; R < R_max; ++R) {
    const double num = h[4 * R] + h[4 * R + 2];
    const double den = h[4 * R + 1] + h[4 * R + 3];
    eta[R] = den > 0.0 ? std::sqrt(num / den) : (num > 0.0 ? INFINITY : 0.0);
  }
  eta[R_max] = 0.0;
  return hipSuccess;
}

}  // namespace sinkattn
