// Projective contraction diagnostic ("Blockwise Differentiable Sinkhorn
// Attention", section 2.4, second certificate: Hilbert's projective metric
// shows that the strictly positive active blocks of the Sinkhorn map are
// contractions).
//
// A diagonal block [s, s + B) x [s, s + B) of the support with
// B <= min(h1, h2) + 1 lies wholly inside the band, so its kernel
// K_ik = exp(S_ik) is strictly positive.  By the Birkhoff-Hopf theorem K
// contracts Hilbert's projective metric by tanh(Delta / 4), where Delta is its
// projective diameter
//   Delta = max_{i,j,k,l} log(K_ik K_jl / (K_jk K_il))
//         = max_{i,j} [ max_k (S_ik - S_jk) - min_k (S_ik - S_jk) ],
// and one Sinkhorn step (a K and a K^T scaling) restricted to the block
// contracts by at most tanh(Delta / 4)^2.  This kernel returns Delta per block
// (natural-log units) and, optionally, kappa = tanh(Delta / 4); blocks are
// laid over the real tokens of each sequence, the last one clipped to n_b.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "geom.hpp"

namespace sinkattn {

constexpr int kDiagMaxBlock = 128;

// One workgroup (256 threads) per (block, b, h).  Q and K rows of the block
// are staged in LDS as fp32 (row stride d + 1), the block's scores are formed
// in 8 x 8 register tiles and written back over the staged rows (row stride
// B + 1), then every unordered row pair takes the range of its score
// difference.
template <typename T>
__global__ __launch_bounds__(256) void block_diameter_kernel(Geom g, const T* Q, const T* K, int Bd, int nblocks,
                                                             float* delta, float* kappa) {
  extern __shared__ float sm[];
  const int blk = blockIdx.x;
  const int bh = blockIdx.y;
  const int bb = bh / g.H;
  const int n = real_len(g, bb);
  const int d = g.d;
  const int tid = threadIdx.x;
  const int s = blk * Bd;
  const size_t o = (size_t)bh * nblocks + blk;
  if (s >= n) {
    if (tid == 0) {
      delta[o] = 0.f;
      if (kappa) kappa[o] = 0.f;
    }
    return;
  }
  const int nb = min(Bd, n - s);
  const int ld = d + 1;
  float* qs = sm;                          // [nb][d + 1], later the scores [nb][nb + 1]
  float* ks = sm + kDiagMaxBlock * ld;     // [nb][d + 1] (the scores may extend over it)
  const size_t base = ((size_t)bh * g.L + s) * d;
  for (int e = tid; e < nb * d; e += 256) {
    const int r = e / d, c = e - r * d;
    qs[r * ld + c] = Elt<T>::load(Q + base, e);
    ks[r * ld + c] = Elt<T>::load(K + base, e);
  }
  __syncthreads();
  // scores: thread t forms the 8 x 8 tile at rows r0 = 8 (t / 16), columns
  // c0 = 8 (t % 16) (16 LDS reads per 64 products)
  const int r0 = 8 * (tid >> 4), c0 = 8 * (tid & 15);
  float sc[8][8];
#pragma unroll
  for (int x = 0; x < 8; ++x)
#pragma unroll
    for (int y = 0; y < 8; ++y) sc[x][y] = 0.f;
  if (r0 < nb && c0 < nb) {
    // rows and columns past nb read staged rows that exist (index clamped)
    // and are never stored
    for (int c = 0; c < d; ++c) {
      float qv[8], kv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        qv[e] = qs[min(r0 + e, nb - 1) * ld + c];
        kv[e] = ks[min(c0 + e, nb - 1) * ld + c];
      }
#pragma unroll
      for (int x = 0; x < 8; ++x)
#pragma unroll
        for (int y = 0; y < 8; ++y) sc[x][y] = __builtin_fmaf(qv[x], kv[y], sc[x][y]);
    }
  }
  __syncthreads();  // every read of the staged rows is done
  const int ls = nb + 1;
  if (r0 < nb && c0 < nb) {
#pragma unroll
    for (int x = 0; x < 8; ++x)
#pragma unroll
      for (int y = 0; y < 8; ++y)
        if (r0 + x < nb && c0 + y < nb) qs[(r0 + x) * ls + c0 + y] = sc[x][y] * g.inv_sqrt_d;
  }
  __syncthreads();
  // row pairs: item (a, q) compares row a with rows 4 q .. 4 q + 3 above it
  float best = 0.f;
  const int ng = (nb + 3) >> 2;
  for (int it = tid; it < nb * ng; it += 256) {
    const int ra = it / ng, q4 = 4 * (it - ra * ng);
    if (q4 + 3 <= ra) continue;  // no row of the group lies above ra
    float hi[4], lo[4];
    int rc[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      hi[e] = -__builtin_inff();
      lo[e] = __builtin_inff();
      rc[e] = min(q4 + e, nb - 1);
    }
    for (int k = 0; k < nb; ++k) {
      const float sa = qs[ra * ls + k];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = sa - qs[rc[e] * ls + k];
        hi[e] = fmaxf(hi[e], x);
        lo[e] = fminf(lo[e], x);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (q4 + e > ra && q4 + e < nb) best = fmaxf(best, hi[e] - lo[e]);
  }
  __shared__ float red[256];
  red[tid] = best;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
    __syncthreads();
  }
  if (tid == 0) {
    delta[o] = red[0];
    if (kappa) kappa[o] = tanhf(0.25f * red[0]);
  }
}

hipError_t launch_block_diameters(const Geom& g, int dtype, const void* Q, const void* K, int Bd, float* delta,
                                  float* kappa, hipStream_t st) {
  const int nblocks = (g.L + Bd - 1) / Bd;
  // staged Q and K rows, or the scores written over them afterwards
  const size_t stage = (size_t)2 * kDiagMaxBlock * (g.d + 1);
  const size_t scores = (size_t)kDiagMaxBlock * (kDiagMaxBlock + 1);
  const size_t lds = (stage > scores ? stage : scores) * sizeof(float);
  if (lds > 160 * 1024) return hipErrorInvalidConfiguration;
  const dim3 grid(nblocks, g.B * g.H);
  hipError_t err;
  if (dtype == 0) {
    err = ensure_lds(reinterpret_cast<const void*>(block_diameter_kernel<float>), lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(block_diameter_kernel<float>, grid, dim3(256), lds, st, g, reinterpret_cast<const float*>(Q),
                       reinterpret_cast<const float*>(K), Bd, nblocks, delta, kappa);
  } else {
    err = ensure_lds(reinterpret_cast<const void*>(block_diameter_kernel<bf16_t>), lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(block_diameter_kernel<bf16_t>, grid, dim3(256), lds, st, g,
                       reinterpret_cast<const bf16_t*>(Q), reinterpret_cast<const bf16_t*>(K), Bd, nblocks, delta, kappa);
  }
  return hipGetLastError();
}

}  // namespace sinkattn
