// Backward pass: exact adjoint of the R differentiable tail steps of banded
// Sinkhorn attention, with the stopped base held constant.
//
// "Blockwise Differentiable Sinkhorn Attention", section 2.2: the adjoint of
// the tail touches the staircase plans P^(r,r) (column updates) and
// P^(r,r-1) (row updates).  They all lie in one row/column scaling orbit of
// the reference plan P = P^(R,R):
//     P^(r,s) = P (.) alpha^(r) beta^(s)^T,
//     alpha^(r) = exp(u^(r) - u^(R)),  beta^(s) = exp(v^(s) - v^(R)),
// so every sweep below rebuilds only the reference tile
// P_ij = exp(S_ij + u^(R)_i + v^(R)_j) (S recomputed on MFMA) and applies
// O(L) vector modifiers.  With x^(r) = ubar^(r) / a and y^(r) = vbar^(r) / b:
//   vbar^(R) = E,                E_j = V_j . dV_j,  dV = P^T dO
//   ubar^(r) = [r = R] D - alpha^(r) (.) P (beta^(r) (.) y^(r)),  D_i = dO_i . O_i
//   vbar^(r-1) = -beta^(r-1) (.) P^T (alpha^(r) (.) x^(r))
//   dS = P (.) (dO V^T - sum_r [alpha^(r) (beta^(r) y^(r))^T + (alpha^(r) x^(r)) beta^(r-1)^T])
//   dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d)
// Sweeps: one column sweep (dV), R row sweeps and R column sweeps for the
// adjoint vectors (the last column sweep only when vbar^(0) is requested),
// a row sweep for dQ and a column sweep for dK.  All accumulations run in a
// fixed order inside one workgroup: results are bitwise reproducible.
//
// Units: the tail stack holds potentials in log2 units (x * log2(e)) and
// scores are taken as S * log2(e) / sqrt(d), so every plan entry and
// modifier is one exp2 of a sum; gradients come out in natural units.
//
// Row sweeps put one query row per lane (score tile = K_tile Q_strip^T);
// column sweeps put one key column per lane (score tile = Q_tile K_strip^T).
// The second operand of the output products (K for dQ, Q for dK, dO for dV)
// is staged transposed in LDS.  bf16: P and dS are split into hi + lo bf16
// operands (~16 mantissa bits).
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "geom.hpp"

namespace sinkattn {

constexpr int kMaxR = 8;

struct BwArgs {
  const void* Q;
  const void* K;
  const void* V;
  const void* dO;
  const float* O;
  const float* a;
  const float* b;
  const double* tail_u;  // [R+1][BHL] (fp64, log2 units)
  const double* tail_v;  // [R+1][BHL]
  const float* sdr;
  const float* sdc;
  float* D;             // [BHL]
  float* vbar;          // [R+1][BHL]
  float* x;             // [R+1][BHL]
  float* out;           // dQ / dK / dV
  float* e_out;         // dV sweep, no dustbin: E_j = V_j . dV_j written here (vbar^(R)), and
                        // filler rows of dV zeroed, in the sweep itself (nullptr: a later pass)
  int R;
  int r;                // pass index (vector sweeps)
  int padded_grid;
};

__device__ __forceinline__ size_t slot(int r, size_t BHL) { return (size_t)r * BHL; }

// Tile-pair product: acc[dc] += A^T-operand tile pair (C layout, lane = m
// index) times rows of a transposed LDS window (element stride `stride`).
// k slot 8*lg + e maps to window column c0 + e (e < 4) / c0 + 12 + e (e >= 4).
template <typename T, int ND>
__device__ __forceinline__ void acc_pair(f4 (&acc)[ND], const float (&p0)[4], const float (&p1)[4],
                                         bool has1, const char* tw, int stride, int c0, int lr) {
  if constexpr (sizeof(T) == 2) {
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
#pragma unroll
    for (int dc = 0; dc < ND; ++dc) {
      const uint16_t* row = reinterpret_cast<const uint16_t*>(tw) + (size_t)(dc * 16 + lr) * stride;
      const u2 x0 = *reinterpret_cast<const u2*>(row + c0);
      u2 x1 = {0u, 0u};
      if (has1) x1 = *reinterpret_cast<const u2*>(row + c0 + 16);
      const u4 vb = {x0.x, x0.y, x1.x, x1.y};
      acc[dc] = Elt<bf16_t>::mma_chunk(acc[dc], hi, vb);
      acc[dc] = Elt<bf16_t>::mma_chunk(acc[dc], lo, vb);
    }
  } else {
#pragma unroll
    for (int dc = 0; dc < ND; ++dc) {
      const float* row = reinterpret_cast<const float*>(tw) + (size_t)(dc * 16 + lr) * stride;
      const f4 v0 = *reinterpret_cast<const f4*>(row + c0);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[dc] = __builtin_amdgcn_mfma_f32_16x16x4f32(p0[r], v0[r], acc[dc], 0, 0, 0);
      if (has1) {
        const f4 v1 = *reinterpret_cast<const f4*>(row + c0 + 16);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[dc] = __builtin_amdgcn_mfma_f32_16x16x4f32(p1[r], v1[r], acc[dc], 0, 0, 0);
      }
    }
  }
}

// Stage rows [row0, row0 + nrows) of a [L, D] tensor (zero outside [0, n))
// into LDS transposed: dst[c * stride + k] = X[row0 + k][c].
template <typename T, int D>
__device__ __forceinline__ void stage_transposed(char* dst, int stride, const void* Xbh, int row0, int nrows, int n,
                                                 int tid, int nthreads) {
  constexpr int RB = D * Elt<T>::kBytes;
  constexpr int per_row = RB / 16;
  const char* X = reinterpret_cast<const char*>(Xbh);
  for (int idx = tid; idx < nrows * per_row; idx += nthreads) {
    const int k = idx / per_row, c16 = idx - k * per_row;
    const int row = row0 + k;
    u4 val = {0u, 0u, 0u, 0u};
    if (row >= 0 && row < n) val = ld16(X + (size_t)row * RB + c16 * 16);
    if constexpr (sizeof(T) == 2) {
      const uint16_t* hv = reinterpret_cast<const uint16_t*>(&val);
#pragma unroll
      for (int e = 0; e < 8; ++e) reinterpret_cast<uint16_t*>(dst)[(size_t)(c16 * 8 + e) * stride + k] = hv[e];
    } else {
      const uint32_t* fv = reinterpret_cast<const uint32_t*>(&val);
#pragma unroll
      for (int e = 0; e < 4; ++e) reinterpret_cast<uint32_t*>(dst)[(size_t)(c16 * 4 + e) * stride + k] = fv[e];
    }
  }
}

// ---------------------------------------------------------------------------
// Row sweeps.  MODE 0: adjoint vector pass r (writes x^(r)); MODE 1: dQ.
// Block = 4 strips of 16 rows; window columns [r0 - 16 TL, r0 + 64 + 16 TR).
// ---------------------------------------------------------------------------
template <typename T, int D, int MODE>
__global__ __launch_bounds__(256) void bw_row_kernel(Geom g, BwArgs p) {
  constexpr int RB = D * Elt<T>::kBytes;
  constexpr int NCH = RB / 64;
  constexpr int ND = D / 16;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int nbh = g.B * g.H;
  const int nblk = ceil_div_pos(g.L, kBwdBlock);
  const int logical = xcd_remap(blockIdx.x, p.padded_grid);
  if (logical >= nbh * nblk) return;
  const int bh = logical / nblk;
  const int blk = logical - bh * nblk;
  const int bb = bh / g.H;
  const int n = real_len(g, bb);
  const int r0 = blk * kBwdBlock;
  if (r0 >= n) return;
  const size_t L = g.L;
  const size_t BHL = (size_t)nbh * L;
  const int R = p.R;
  const int NWC = 16 * (g.TL + g.TR + kBwdWaves);
  const int tw0 = (r0 >> 4) - g.TL;
  const int tid = threadIdx.x;
  const int KTS = NWC + 8;  // transposed-K row stride (elements)

  // LDS: w [NWC] | colvec [2R or 1][NWC] | K^T [D][KTS]
  float* w2s = reinterpret_cast<float*>(smem);
  float* cv = w2s + NWC;
  const int ncv = MODE == 0 ? 1 : 2 * R;
  char* kt = reinterpret_cast<char*>(cv + (size_t)(ncv > 0 ? ncv : 1) * NWC);
  const double* vR = p.tail_v + slot(R, BHL) + bh * L;
  const double* uR = p.tail_u + slot(R, BHL) + bh * L;
  const double vref = vR[r0];  // exponents split as (u_i + vref) + (v_j - vref)
  for (int c = tid; c < NWC; c += blockDim.x) {
    const int j = tw0 * 16 + c;
    const bool ok = j >= 0 && j < n;
    w2s[c] = ok ? (float)(vR[j] - vref) : kNegInf;
    if (MODE == 0) {
      // z_j = beta^(r)_j y^(r)_j
      float z = 0.f;
      if (ok) {
        const double vr = p.tail_v[slot(p.r, BHL) + bh * L + j];
        z = exp2f(vr - vR[j]) * p.vbar[slot(p.r, BHL) + bh * L + j] / p.b[(size_t)bb * L + j];
      }
      cv[c] = z;
    } else {
      for (int k = 1; k <= R; ++k) {
        float by = 0.f, bm = 0.f;
        if (ok) {
          const double vk = p.tail_v[slot(k, BHL) + bh * L + j];
          const double vk1 = p.tail_v[slot(k - 1, BHL) + bh * L + j];
          by = exp2f(vk - vR[j]) * p.vbar[slot(k, BHL) + bh * L + j] / p.b[(size_t)bb * L + j];
          bm = exp2f(vk1 - vR[j]);
        }
        cv[(size_t)(2 * (k - 1)) * NWC + c] = by;
        cv[(size_t)(2 * (k - 1) + 1) * NWC + c] = bm;
      }
    }
  }
  if (MODE == 1) {
    stage_transposed<T, D>(kt, KTS, reinterpret_cast<const char*>(p.K) + (size_t)bh * L * RB, tw0 * 16, NWC, n,
                           tid, blockDim.x);
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

  const char* Qb = reinterpret_cast<const char*>(p.Q) + (size_t)bh * L * RB;
  const char* Kb = reinterpret_cast<const char*>(p.K) + (size_t)bh * L * RB;
  const char* Vb = reinterpret_cast<const char*>(p.V) + (size_t)bh * L * RB;
  const char* dOb = reinterpret_cast<const char*>(p.dO) + (size_t)bh * L * RB;
  const int qi = i0 + lr;
  const bool myrow = qi < n;
  u4 qb[NCH], ob[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    qb[c] = (u4){0u, 0u, 0u, 0u};
    ob[c] = (u4){0u, 0u, 0u, 0u};
    if (myrow) {
      qb[c] = ld16(Qb + (size_t)qi * RB + c * 64 + lg * 16);
      if (MODE == 1) ob[c] = ld16(dOb + (size_t)qi * RB + c * 64 + lg * 16);
    }
  }
  const float ui2 = myrow ? (float)(uR[qi] + vref) : 0.f;
  // row modifiers (MODE 1): alpha^(k)_i, alpha^(k)_i x^(k)_i
  float al[kMaxR], ax[kMaxR];
#pragma unroll
  for (int k = 0; k < kMaxR; ++k) {
    al[k] = 0.f;
    ax[k] = 0.f;
    if (MODE == 1 && k < R && myrow) {
      al[k] = exp2f(p.tail_u[slot(k + 1, BHL) + bh * L + qi] - uR[qi]);
      ax[k] = al[k] * p.x[slot(k + 1, BHL) + bh * L + qi];
    }
  }

  auto tile = [&](int t, float (&pt)[4], float (&dst)[4]) {
    if (t >= NT || t < t_lo || t > t_hi) {
#pragma unroll
      for (int r = 0; r < 4; ++r) { pt[r] = 0.f; dst[r] = 0.f; }
      return;
    }
    const int jrow = (tg0 + t) * 16 + lr;
    const bool kin = jrow >= 0 && jrow < n;
    f4 s = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      u4 ka = {0u, 0u, 0u, 0u}, va = {0u, 0u, 0u, 0u};
      if (kin) {
        ka = ld16(Kb + (size_t)jrow * RB + c * 64 + lg * 16);
        if (MODE == 1) va = ld16(Vb + (size_t)jrow * RB + c * 64 + lg * 16);
      }
      s = Elt<T>::mma_chunk(s, ka, qb[c]);
      if (MODE == 1) dp = Elt<T>::mma_chunk(dp, va, ob[c]);
    }
    const int obase = (t - g.TL) * 16 + 4 * lg - lr;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int o = obase + r;
      const int c = (wave + t) * 16 + 4 * lg + r;
      float x = __builtin_fmaf(s[r], g.scale2, w2s[c] + ui2);
      x = (o >= -g.h1 && o <= g.h2 && myrow) ? x : kNegInf;
      pt[r] = exp2_fast(x);
      if (MODE == 1) {
        float br = dp[r];
#pragma unroll
        for (int k = 0; k < kMaxR; ++k) {
          if (k < R) {
            br -= al[k] * cv[(size_t)(2 * k) * NWC + c];
            br -= ax[k] * cv[(size_t)(2 * k + 1) * NWC + c];
          }
        }
        dst[r] = pt[r] * br;
      } else {
        dst[r] = pt[r] * cv[c];
      }
    }
  };

  if (MODE == 0) {
    float acc = 0.f;
    for (int t = 0; t < NT; ++t) {
      float pt[4], pz[4];
      tile(t, pt, pz);
      acc += (pz[0] + pz[1]) + (pz[2] + pz[3]);
    }
    acc = cross_row_sum(acc);
    if (lg == 0 && myrow) {
      const int i = qi;
      if (g.dustbin) {
        // entry (i, delta): P_i,delta z_delta
        const double vRd = p.tail_v[slot(R, BHL) + bh * L + n];
        const float zd = exp2f(p.tail_v[slot(p.r, BHL) + bh * L + n] - vRd) *
                         p.vbar[slot(p.r, BHL) + bh * L + n] / p.b[(size_t)bb * L + n];
        acc += exp2f(p.sdc[bh * L + i] + uR[i] + vRd) * zd;
      }
      const float alpha = exp2f(p.tail_u[slot(p.r, BHL) + bh * L + i] - uR[i]);
      const float ub = (p.r == R ? p.D[bh * L + i] : 0.f) - alpha * acc;
      p.x[slot(p.r, BHL) + bh * L + i] = ub / p.a[(size_t)bb * L + i];
    }
  } else {
    f4 acc[ND];
#pragma unroll
    for (int dc = 0; dc < ND; ++dc) acc[dc] = (f4){0.f, 0.f, 0.f, 0.f};
    for (int t = 0; t < NT; t += 2) {
      float p0[4], s0[4], p1[4], s1[4];
      tile(t, p0, s0);
      tile(t + 1, p1, s1);
      const int c0 = (wave + t) * 16 + 4 * lg;
      acc_pair<T, ND>(acc, s0, s1, t + 1 < NT, kt, KTS, c0, lr);
    }
#pragma unroll
    for (int dc = 0; dc < ND; ++dc) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + 4 * lg + r;
        if (i < n) p.out[((size_t)bh * L + i) * D + dc * 16 + lr] = acc[dc][r] * g.inv_sqrt_d;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Column sweeps.  MODE 0: adjoint vector pass (writes vbar^(r-1));
// MODE 1: dK; MODE 2: dV (band part).
// Block = 4 strips of 16 columns; window rows [c0 - 16 TLc, c0 + 64 + 16 TRc).
// ---------------------------------------------------------------------------
template <typename T, int D, int MODE>
__global__ __launch_bounds__(256) void bw_col_kernel(Geom g, BwArgs p) {
  constexpr int RB = D * Elt<T>::kBytes;
  constexpr int NCH = RB / 64;
  constexpr int ND = D / 16;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int nbh = g.B * g.H;
  const int nblk = ceil_div_pos(g.L, kBwdBlock);
  const int logical = xcd_remap(blockIdx.x, p.padded_grid);
  if (logical >= nbh * nblk) return;
  const int bh = logical / nblk;
  const int blk = logical - bh * nblk;
  const int bb = bh / g.H;
  const int n = real_len(g, bb);
  const int c0b = blk * kBwdBlock;
  if (c0b >= n) return;
  const size_t L = g.L;
  const size_t BHL = (size_t)nbh * L;
  const int R = p.R;
  const int NWR = 16 * (g.TLc + g.TRc + kBwdWaves);
  const int tw0 = (c0b >> 4) - g.TLc;
  const int tid = threadIdx.x;
  const int XTS = NWR + 8;

  float* w2s = reinterpret_cast<float*>(smem);   // u^(R) (log2) of window rows
  float* rv = w2s + NWR;                         // row vectors
  const int nrv = MODE == 0 ? 1 : (MODE == 1 ? 2 * R : 0);
  char* xt = reinterpret_cast<char*>(rv + (size_t)(nrv > 0 ? nrv : 1) * NWR);
  const double* vR = p.tail_v + slot(R, BHL) + bh * L;
  const double* uR = p.tail_u + slot(R, BHL) + bh * L;
  const double uref = uR[c0b];  // exponents split as (u_i - uref) + (v_j + uref)
  for (int c = tid; c < NWR; c += blockDim.x) {
    const int i = tw0 * 16 + c;
    const bool ok = i >= 0 && i < n;
    w2s[c] = ok ? (float)(uR[i] - uref) : kNegInf;
    if (MODE == 0) {
      // zz_i = alpha^(r)_i x^(r)_i
      float z = 0.f;
      if (ok) z = exp2f(p.tail_u[slot(p.r, BHL) + bh * L + i] - uR[i]) * p.x[slot(p.r, BHL) + bh * L + i];
      rv[c] = z;
    } else if (MODE == 1) {
      for (int k = 1; k <= R; ++k) {
        float al = 0.f, ax = 0.f;
        if (ok) {
          al = exp2f(p.tail_u[slot(k, BHL) + bh * L + i] - uR[i]);
          ax = al * p.x[slot(k, BHL) + bh * L + i];
        }
        rv[(size_t)(2 * (k - 1)) * NWR + c] = al;
        rv[(size_t)(2 * (k - 1) + 1) * NWR + c] = ax;
      }
    }
  }
  if (MODE == 1)
    stage_transposed<T, D>(xt, XTS, reinterpret_cast<const char*>(p.Q) + (size_t)bh * L * RB, tw0 * 16, NWR, n, tid,
                           blockDim.x);
  if (MODE == 2)
    stage_transposed<T, D>(xt, XTS, reinterpret_cast<const char*>(p.dO) + (size_t)bh * L * RB, tw0 * 16, NWR, n, tid,
                           blockDim.x);
  __syncthreads();

  const int wave = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int j0 = c0b + wave * 16;
  if (j0 >= n) return;
  const int NT = g.NTc;
  const int tg0 = tw0 + wave;
  int t_lo = -tg0;
  t_lo = t_lo < 0 ? 0 : t_lo;
  int t_hi = (n - 1) / 16 - tg0;
  t_hi = t_hi > NT - 1 ? NT - 1 : t_hi;

  const char* Qb = reinterpret_cast<const char*>(p.Q) + (size_t)bh * L * RB;
  const char* Kb = reinterpret_cast<const char*>(p.K) + (size_t)bh * L * RB;
  const char* Vb = reinterpret_cast<const char*>(p.V) + (size_t)bh * L * RB;
  const char* dOb = reinterpret_cast<const char*>(p.dO) + (size_t)bh * L * RB;
  const int kj = j0 + lr;
  const bool mycol = kj < n;
  u4 kb[NCH], vb[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    kb[c] = (u4){0u, 0u, 0u, 0u};
    vb[c] = (u4){0u, 0u, 0u, 0u};
    if (mycol) {
      kb[c] = ld16(Kb + (size_t)kj * RB + c * 64 + lg * 16);
      if (MODE == 1) vb[c] = ld16(Vb + (size_t)kj * RB + c * 64 + lg * 16);
    }
  }
  const float vj2 = mycol ? (float)(vR[kj] + uref) : 0.f;
  // column modifiers (MODE 1): beta^(k)_j y^(k)_j and beta^(k-1)_j
  float by[kMaxR], bm[kMaxR];
#pragma unroll
  for (int k = 0; k < kMaxR; ++k) {
    by[k] = 0.f;
    bm[k] = 0.f;
    if (MODE == 1 && k < R && mycol) {
      by[k] = exp2f(p.tail_v[slot(k + 1, BHL) + bh * L + kj] - vR[kj]) * p.vbar[slot(k + 1, BHL) + bh * L + kj] /
              p.b[(size_t)bb * L + kj];
      bm[k] = exp2f(p.tail_v[slot(k, BHL) + bh * L + kj] - vR[kj]);
    }
  }

  auto tile = [&](int t, float (&pt)[4], float (&dst)[4]) {
    if (t >= NT || t < t_lo || t > t_hi) {
#pragma unroll
      for (int r = 0; r < 4; ++r) { pt[r] = 0.f; dst[r] = 0.f; }
      return;
    }
    const int irow = (tg0 + t) * 16 + lr;
    const bool qin = irow >= 0 && irow < n;
    f4 s = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      u4 qa = {0u, 0u, 0u, 0u}, oa = {0u, 0u, 0u, 0u};
      if (qin) {
        qa = ld16(Qb + (size_t)irow * RB + c * 64 + lg * 16);
        if (MODE == 1) oa = ld16(dOb + (size_t)irow * RB + c * 64 + lg * 16);
      }
      s = Elt<T>::mma_chunk(s, qa, kb[c]);
      if (MODE == 1) dp = Elt<T>::mma_chunk(dp, oa, vb[c]);
    }
    // lane: i = (tg0 + t) * 16 + 4 lg + r, j = j0 + lr
    const int obase = (g.TLc - t) * 16 + lr - 4 * lg;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int o = obase - r;
      const int c = (wave + t) * 16 + 4 * lg + r;
      float x = __builtin_fmaf(s[r], g.scale2, w2s[c] + vj2);
      x = (o >= -g.h1 && o <= g.h2 && mycol) ? x : kNegInf;
      pt[r] = exp2_fast(x);
      if (MODE == 1) {
        float br = dp[r];
#pragma unroll
        for (int k = 0; k < kMaxR; ++k) {
          if (k < R) {
            br -= rv[(size_t)(2 * k) * NWR + c] * by[k];
            br -= rv[(size_t)(2 * k + 1) * NWR + c] * bm[k];
          }
        }
        dst[r] = pt[r] * br;
      } else if (MODE == 0) {
        dst[r] = pt[r] * rv[c];
      } else {
        dst[r] = pt[r];
      }
    }
  };

  if (MODE == 0) {
    float acc = 0.f;
    for (int t = 0; t < NT; ++t) {
      float pt[4], pz[4];
      tile(t, pt, pz);
      acc += (pz[0] + pz[1]) + (pz[2] + pz[3]);
    }
    acc = cross_row_sum(acc);
    if (lg == 0 && mycol) {
      const int j = kj;
      if (g.dustbin) {
        // entry (delta, j): P_delta,j zz_delta
        const double uRd = p.tail_u[slot(R, BHL) + bh * L + n];
        const float zd = exp2f(p.tail_u[slot(p.r, BHL) + bh * L + n] - uRd) * p.x[slot(p.r, BHL) + bh * L + n];
        acc += exp2f(p.sdr[bh * L + j] + uRd + vR[j]) * zd;
      }
      const float beta = exp2f(p.tail_v[slot(p.r - 1, BHL) + bh * L + j] - vR[j]);
      p.vbar[slot(p.r - 1, BHL) + bh * L + j] = -beta * acc;
    }
  } else {
    f4 acc[ND];
#pragma unroll
    for (int dc = 0; dc < ND; ++dc) acc[dc] = (f4){0.f, 0.f, 0.f, 0.f};
    for (int t = 0; t < NT; t += 2) {
      float p0[4], s0[4], p1[4], s1[4];
      tile(t, p0, s0);
      tile(t + 1, p1, s1);
      const int c0 = (wave + t) * 16 + 4 * lg;
      acc_pair<T, ND>(acc, s0, s1, t + 1 < NT, xt, XTS, c0, lr);
    }
    const float sc = MODE == 1 ? g.inv_sqrt_d : 1.f;
#pragma unroll
    for (int dc = 0; dc < ND; ++dc) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = j0 + 4 * lg + r;
        if (j < n) p.out[((size_t)bh * L + j) * D + dc * 16 + lr] = acc[dc][r] * sc;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Per-token kernels (one thread per token, d-long loops).
// ---------------------------------------------------------------------------
// Per-token kernels below use 16 lanes per token (one DPP row): lane c
// handles head-dimension columns c, c + 16, ... so row reads coalesce.
constexpr int kTokPerBlock = 16;  // 256 threads

// D_i = dO_i . O_i on active rows.
template <typename T, int D>
__global__ __launch_bounds__(256) void bw_rowdot(Geom g, const T* dO, const float* O, float* Dv) {
  constexpr int V = D / 16;  // contiguous elements per lane (16 lanes per token; one vector load each)
  const int bh = blockIdx.y;
  const int i = blockIdx.x * kTokPerBlock + (threadIdx.x >> 4);
  const int c0 = (threadIdx.x & 15) * V;
  const int n = real_len(g, bh / g.H);
  const int nact = n + (g.dustbin ? 1 : 0);
  const size_t o = (size_t)bh * g.L + (i < g.L ? i : 0);
  float s = 0.f;
  if (i < nact) {
    // rows are 16-byte aligned (checked at the boundary) and c0 is a multiple of V
    T a[V];
    float b[V];
    __builtin_memcpy(a, __builtin_assume_aligned(dO + o * D + c0, V * sizeof(T)), sizeof(a));
    __builtin_memcpy(b, __builtin_assume_aligned(O + o * D + c0, V * sizeof(float)), sizeof(b));
#pragma unroll
    for (int c = 0; c < V; ++c) s = __builtin_fmaf(Elt<T>::load(a, c), b[c], s);
  }
  s = row16_sum(s);
  if (i < g.L && (threadIdx.x & 15) == 0) Dv[o] = s;
}

// After the dV sweep: add the dustbin-row entry (delta, j) for real j, zero
// filler rows, E_j = V_j . dV_j, vbar^(R)_j = E_j.
template <typename T>
__global__ __launch_bounds__(256) void bw_finish_dv(Geom g, const T* V, const T* dO, const double* tail_u,
                                                    const double* tail_v, const float* sdr, int R, float* dV,
                                                    float* vbarR) {
  const int bh = blockIdx.y;
  const int j = blockIdx.x * kTokPerBlock + (threadIdx.x >> 4);
  const int c0 = threadIdx.x & 15;
  if (j >= g.L) return;  // whole 16-lane rows exit together
  const int n = real_len(g, bh / g.H);
  const size_t L = g.L;
  const size_t BHL = (size_t)g.B * g.H * L;
  const size_t o = (size_t)bh * L + j;
  const int d = g.d;
  if (j >= n) {
    if (!(g.dustbin && j == n)) {
      for (int c = c0; c < d; c += 16) dV[o * d + c] = 0.f;
      if (c0 == 0) vbarR[o] = 0.f;
    }
    return;
  }
  float pdj = 0.f;
  if (g.dustbin) {
    const double uRd = tail_u[slot(R, BHL) + bh * L + n];
    pdj = exp2f((float)((double)sdr[o] + uRd + tail_v[slot(R, BHL) + o]));
  }
  const size_t od = (size_t)bh * L + n;
  float e = 0.f;
  for (int c = c0; c < d; c += 16) {
    float dv = dV[o * d + c];
    if (g.dustbin) dv = __builtin_fmaf(pdj, Elt<T>::load(dO, od * d + c), dv);
    dV[o * d + c] = dv;
    e = __builtin_fmaf(Elt<T>::load(V, o * d + c), dv, e);
  }
  e = row16_sum(e);
  if (c0 == 0) vbarR[o] = e;
}

// After the dQ (IS_K = 0) or dK (IS_K = 1) sweep: add the dustbin entry of
// every real token and zero filler rows.
//   dQ_i += dS_i,delta K_delta / sqrt(d);  dK_j += dS_delta,j Q_delta / sqrt(d)
template <typename T, int IS_K>
__global__ void bw_finish_grad(Geom g, BwArgs p) {
  const int bh = blockIdx.y;
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= g.L) return;
  const int bb = bh / g.H;
  const int n = real_len(g, bb);
  const size_t L = g.L;
  const size_t BHL = (size_t)g.B * g.H * L;
  const int d = g.d;
  const int R = p.R;
  const size_t o = (size_t)bh * L + t;
  if (t >= n) {
    if (!(g.dustbin && t == n))
      for (int c = 0; c < d; ++c) p.out[o * d + c] = 0.f;
    return;
  }
  if (!g.dustbin) return;
  const T* Q = reinterpret_cast<const T*>(p.Q);
  const T* K = reinterpret_cast<const T*>(p.K);
  const T* V = reinterpret_cast<const T*>(p.V);
  const T* dO = reinterpret_cast<const T*>(p.dO);
  const size_t od = (size_t)bh * L + n;
  const double* uR = p.tail_u + slot(R, BHL);
  const double* vR = p.tail_v + slot(R, BHL);
  // the entry: row i, column j
  const size_t oi = IS_K ? od : o;
  const size_t oj = IS_K ? o : od;
  const float s = IS_K ? p.sdr[o] : p.sdc[o];
  const float P = exp2f(s + uR[oi] + vR[oj]);
  float dP = 0.f;
  for (int c = 0; c < d; ++c) dP = __builtin_fmaf(Elt<T>::load(dO, oi * d + c), Elt<T>::load(V, oj * d + c), dP);
  const int bi = IS_K ? n : t, bj = IS_K ? t : n;
  float br = dP;
  for (int k = 1; k <= R; ++k) {
    const float al = exp2f(p.tail_u[slot(k, BHL) + oi] - uR[oi]);
    const float x = p.x[slot(k, BHL) + oi];
    const float by = exp2f(p.tail_v[slot(k, BHL) + oj] - vR[oj]) * p.vbar[slot(k, BHL) + oj] / p.b[(size_t)bb * L + bj];
    const float bm = exp2f(p.tail_v[slot(k - 1, BHL) + oj] - vR[oj]);
    br -= al * by + al * x * bm;
  }
  (void)bi;
  const float dS = P * br * g.inv_sqrt_d;
  const T* X = IS_K ? Q : K;  // the other side's dustbin vector
  const size_t ox = IS_K ? oi : oj;
  for (int c = 0; c < d; ++c) p.out[o * d + c] = __builtin_fmaf(dS, Elt<T>::load(X, ox * d + c), p.out[o * d + c]);
}

// Dustbin row and column (full length).
//   mode 0: dV_delta = sum_i P_i,delta dO_i, vbar^(R)_delta = V_delta . dV_delta
//   mode 1: x^(r)_delta (row pass r)
//   mode 2: vbar^(r-1)_delta (column pass r)
//   mode 3: dQ_delta (row),  mode 4: dK_delta (column)
// The tokens go in chunks of 256, one workgroup per (chunk, (b, h)): each
// thread forms the coefficient w_t of one token (modes 1, 2: its term of the
// sum; modes 0, 3, 4: the plan entry times dO (mode 0), or times the adjoint
// of its score), and the chunk's partial sum goes to `dpart` (modes 1, 2: one
// value; modes 0, 3, 4: out[c] = sum_t w_t X_t[c], 256 / d threads per column
// c each taking every (256 / d)-th token).  bw_dustbin_fin then adds the
// chunks in a fixed order and finishes the output.
template <typename T>
__global__ __launch_bounds__(256) void bw_dustbin_part(Geom g, BwArgs p, int mode, float* dpart) {
  const int bh = blockIdx.y;
  const int chunk = blockIdx.x;
  const int bb = bh / g.H;
  const int n = real_len(g, bb);
  const size_t L = g.L;
  const size_t BHL = (size_t)g.B * g.H * L;
  const int d = g.d;
  const int R = p.R;
  const int tid = threadIdx.x;
  const int t0 = chunk * 256;
  float* out = dpart + ((size_t)bh * gridDim.x + chunk) * d;
  if (t0 > n) return;  // a chunk past the dustbin (the finish reads only the chunks up to it)
  const size_t od = (size_t)bh * L + n;
  const double* uR = p.tail_u + slot(R, BHL);
  const double* vR = p.tail_v + slot(R, BHL);
  const T* Q = reinterpret_cast<const T*>(p.Q);
  const T* K = reinterpret_cast<const T*>(p.K);
  const T* V = reinterpret_cast<const T*>(p.V);
  const T* dO = reinterpret_cast<const T*>(p.dO);
  __shared__ float red[256];
  // plan entry with the dustbin: row side (delta, t) when row = true
  auto plan = [&](int t, bool row) {
    const size_t ot = (size_t)bh * L + t;
    const float sc = row ? p.sdr[ot] : p.sdc[ot];
    return row ? exp2f(sc + uR[od] + vR[ot]) : exp2f(sc + uR[ot] + vR[od]);
  };
  const int t = t0 + tid;
  const size_t ot = (size_t)bh * L + t;
  float w = 0.f;
  if (t <= n) {
    if (mode == 1) {  // z_t = beta^(r)_t y^(r)_t over the dustbin row
      const int r = p.r;
      const float z = exp2f(p.tail_v[slot(r, BHL) + ot] - vR[ot]) * p.vbar[slot(r, BHL) + ot] / p.b[(size_t)bb * L + t];
      w = plan(t, true) * z;
    } else if (mode == 2) {  // zz_t = alpha^(r)_t x^(r)_t over the dustbin column
      const int r = p.r;
      const float z = exp2f(p.tail_u[slot(r, BHL) + ot] - uR[ot]) * p.x[slot(r, BHL) + ot];
      w = plan(t, false) * z;
    } else if (mode == 0) {
      w = plan(t, false);
    } else {
      const bool row = mode == 3;
      const size_t oi = row ? od : ot, oj = row ? ot : od;
      const int bj = row ? t : n;
      float dP = 0.f;
      for (int cc = 0; cc < d; ++cc) dP = __builtin_fmaf(Elt<T>::load(dO, oi * d + cc), Elt<T>::load(V, oj * d + cc), dP);
      float br = dP;
      for (int k = 1; k <= R; ++k) {
        const float al = exp2f(p.tail_u[slot(k, BHL) + oi] - uR[oi]);
        const float x = p.x[slot(k, BHL) + oi];
        const float by = exp2f(p.tail_v[slot(k, BHL) + oj] - vR[oj]) * p.vbar[slot(k, BHL) + oj] / p.b[(size_t)bb * L + bj];
        const float bm = exp2f(p.tail_v[slot(k - 1, BHL) + oj] - vR[oj]);
        br -= al * by + al * x * bm;
      }
      w = plan(t, row) * br;
    }
  }
  if (mode == 1 || mode == 2) {
    red[tid] = w;
    __syncthreads();
    for (int sft = 128; sft > 0; sft >>= 1) {
      if (tid < sft) red[tid] += red[tid + sft];
      __syncthreads();
    }
    if (tid == 0) out[0] = red[0];
    return;
  }
  __shared__ float wch[256];
  const int tpc = 256 / d;  // threads per output column (d divides 256)
  const int col = tid % d, part = tid / d;
  const T* X = mode == 0 ? dO : (mode == 3 ? K : Q);
  wch[tid] = w;
  __syncthreads();
  const int cnt = n + 1 - t0 < 256 ? n + 1 - t0 : 256;
  float acc = 0.f;
  for (int k = part; k < cnt; k += tpc) acc = __builtin_fmaf(wch[k], Elt<T>::load(X, ((size_t)bh * L + t0 + k) * d + col), acc);
  red[tid] = acc;
  __syncthreads();
  if (part == 0) {
    float sum = 0.f;
    for (int k = 0; k < tpc; ++k) sum += red[col + k * d];
    out[col] = sum;
  }
}

// The chunks of bw_dustbin_part added in chunk order, and the outputs of
// each mode.  One workgroup per (b, h).
template <typename T>
__global__ __launch_bounds__(256) void bw_dustbin_fin(Geom g, BwArgs p, int mode, const float* dpart, int nch) {
  const int bh = blockIdx.x;
  const int bb = bh / g.H;
  const int n = real_len(g, bb);
  const size_t L = g.L;
  const size_t BHL = (size_t)g.B * g.H * L;
  const int d = g.d;
  const int R = p.R;
  const int tid = threadIdx.x;
  const size_t od = (size_t)bh * L + n;
  const int used = (n + 1 + 255) / 256;  // chunks holding the dustbin's tokens 0 .. n
  const float* in = dpart + (size_t)bh * nch * d;
  if (mode == 1 || mode == 2) {
    if (tid == 0) {
      float acc = 0.f;
      for (int c = 0; c < used; ++c) acc += in[(size_t)c * d];
      const int r = p.r;
      const double* uR = p.tail_u + slot(R, BHL);
      const double* vR = p.tail_v + slot(R, BHL);
      if (mode == 1) {
        const float alpha = exp2f(p.tail_u[slot(r, BHL) + od] - uR[od]);
        const float ub = (r == R ? p.D[od] : 0.f) - alpha * acc;
        p.x[slot(r, BHL) + od] = ub / p.a[(size_t)bb * L + n];
      } else {
        const float beta = exp2f(p.tail_v[slot(r - 1, BHL) + od] - vR[od]);
        p.vbar[slot(r - 1, BHL) + od] = -beta * acc;
      }
    }
    return;
  }
  __shared__ float outv[256];
  __shared__ float red[256];
  for (int c = tid; c < d; c += 256) {
    float sum = 0.f;
    for (int k = 0; k < used; ++k) sum += in[(size_t)k * d + c];
    outv[c] = mode == 0 ? sum : sum * g.inv_sqrt_d;
    p.out[od * d + c] = outv[c];
  }
  if (mode == 0) {  // vbar^(R)_delta = E_delta = V_delta . dV_delta
    __syncthreads();
    const T* V = reinterpret_cast<const T*>(p.V);
    red[tid] = tid < d ? Elt<T>::load(V, od * d + tid) * outv[tid] : 0.f;
    __syncthreads();
    for (int sft = 128; sft > 0; sft >>= 1) {
      if (tid < sft) red[tid] += red[tid + sft];
      __syncthreads();
    }
    if (tid == 0) p.vbar[slot(R, BHL) + od] = red[0];
  }
}

// vbar^(0) -> caller buffer (filler = 0).
__global__ void bw_copy_vbar0(Geom g, const float* vbar0, float* out) {
  const int bh = blockIdx.y;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= g.L) return;
  const int n = real_len(g, bh / g.H);
  const int nact = n + (g.dustbin ? 1 : 0);
  const size_t o = (size_t)bh * g.L + i;
  out[o] = i < nact ? vbar0[o] : 0.f;
}

// ---------------------------------------------------------------------------
template <typename T>
__global__ void dustbin_scores_bw(Geom g, const T* Q, const T* K, float* sdr, float* sdc) {
  const int bh = blockIdx.y;
  const int n = real_len(g, bh / g.H);
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j > n) return;
  const size_t L = g.L;
  const int d = g.d;
  float sr = 0.f, sc = 0.f;
  for (int c = 0; c < d; ++c) {
    sr = __builtin_fmaf(Elt<T>::load(Q, ((size_t)bh * L + n) * d + c), Elt<T>::load(K, ((size_t)bh * L + j) * d + c), sr);
    sc = __builtin_fmaf(Elt<T>::load(Q, ((size_t)bh * L + j) * d + c), Elt<T>::load(K, ((size_t)bh * L + n) * d + c), sc);
  }
  sdr[bh * L + j] = sr * g.scale2;
  sdc[bh * L + j] = sc * g.scale2;
}

// ---------------------------------------------------------------------------
// bf16 sweeps for d = 64, 128.  Row sweeps (COL = false): MODE 0 adjoint
// vector x^(r), MODE 1 dQ.  Column sweeps (COL = true): MODE 0 vbar^(r-1),
// MODE 1 dK, MODE 2 dV.  Same results as bw_row_kernel / bw_col_kernel.
//
// One workgroup of 8 waves per block of 128 strip indices (rows i for row
// sweeps, columns j for column sweeps); wave w owns strip w (16 indices) and
// keeps its operands and accumulators in registers.  The block's window of
// NT + 7 tiles (16 indices of the other side each) streams through LDS two
// tiles at a time, double-buffered; a wave works on the tiles of its own
// band span.
//   score / dP tiles: MFMA 16x16x32, A = streamed tile (row-major LDS),
//     B = strip registers; a lane of the result holds one strip index and
//     4 consecutive indices of the other side;
//   products (dS K, dS^T Q, P^T dO): MFMA 16x16x32 with the tile pair as A
//     (4 + 4 k-slots per lane, hi + lo bf16) and the streamed rows as B, read
//     transposed straight from the row-major LDS rows (ds_read_b64_tr_b16:
//     within 16 lanes, lane 4r + q points at 4 elements of row r, and lane c
//     receives element c of the 4 rows).
// Stored rows swizzle their 16-byte chunks (sw_chunk) so that both the
// 128-bit reads of 16 consecutive rows and the transposed reads of 4
// consecutive rows are free of bank conflicts (256-byte rows).
// ---------------------------------------------------------------------------
constexpr int kSwWaves = 8;
constexpr int kSwThreads = 64 * kSwWaves;

// RX: the tail depth is exactly RM (a compile-time constant), else any R <= RM.
template <int D, bool COL, int MODE, int RM, bool RX = false>
__global__ __launch_bounds__(kSwThreads, RM <= 2 ? 4 : 2) void bw_sweep_kernel(Geom g, BwArgs p) {
  constexpr int RB = D * 2;           // bytes per row (bf16)
  constexpr int CPR = RB / 16;        // 16-byte chunks per row
  constexpr int NCH = RB / 64;        // 32-element MFMA chunks per row
  constexpr int ND = D / 16;          // 16-wide output slices
  constexpr int NTEN = MODE == 0 ? 1 : 2;   // streamed tensors
  constexpr int PT = MODE == 2 ? 1 : 0;     // streamed tensor of the product
  constexpr int TBYTES = 32 * RB;     // one tile pair of one tensor
  constexpr int NBUF = 4;             // pair buffers: three pairs in flight ahead of the one in use
  static_assert(CPR >= 8, "the chunk swizzle needs 8 chunks per row");
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int nbh = g.B * g.H;
  const int nblk = ceil_div_pos(g.L, 128);
  const int logical = xcd_remap(blockIdx.x, p.padded_grid);
  if (logical >= nbh * nblk) return;
  const int bh = logical / nblk;
  const int blk = logical - bh * nblk;
  const int bb = bh / g.H;
  const int n = real_len(g, bb);
  const int s0b = blk * 128;
  // dV with E fused: rows [s0b, s0b + 128) of dV and of E are written by this
  // workgroup even where they are filler (zeros)
  auto zero_rows = [&](int s_lo) {
    for (int e = threadIdx.x; e < 128 * D; e += kSwThreads) {
      const int s = s0b + e / D;
      if (s >= s_lo && s < g.L) p.out[((size_t)bh * g.L + s) * D + e % D] = 0.f;
    }
    for (int e = threadIdx.x; e < 128; e += kSwThreads) {
      const int s = s0b + e;
      if (s >= s_lo && s < g.L) p.e_out[(size_t)bh * g.L + s] = 0.f;
    }
  };
  if (s0b >= n) {
    if (MODE == 2 && p.e_out) zero_rows(s0b);
    return;
  }
  const size_t L = g.L;
  const size_t BHL = (size_t)nbh * L;
  const int R = RX ? RM : p.R;
  const int TLx = COL ? g.TLc : g.TL;
  const int NT = COL ? g.NTc : g.NT;
  const int NW = NT + kSwWaves - 1;   // window tiles of the block
  const int NP = (NW + 1) >> 1;       // tile pairs
  const int NWC = 2 * NP * 16;        // window indices held in LDS
  const int tw0 = blk * 8 - TLx;      // first window tile (global)
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;

  // LDS: tiles [NBUF buffers][NTEN][32 rows][RB] | wv [NWC] | window vectors [NV][NWC]
  constexpr int NVMAX = 2 * kMaxR;
  char* tbuf = smem;
  float* wv = reinterpret_cast<float*>(smem + NBUF * NTEN * TBYTES);
  float* vec = wv + NWC;
  const int NV = MODE == 0 ? 1 : (MODE == 1 ? 2 * R : 0);

  const double* uR = p.tail_u + slot(R, BHL) + bh * L;
  const double* vR = p.tail_v + slot(R, BHL) + bh * L;
  // exponent split: strip side (x_s + ref) + window side (x_w - ref)
  const double ref = COL ? uR[s0b] : vR[s0b];
  // Every load of the set-up reads a clamped, always valid index and the
  // result is selected afterwards, so that the loads carry no branch: they
  // are all in flight together instead of one round trip per condition.
  for (int c = tid; c < NWC; c += kSwThreads) {
    const int k = tw0 * 16 + c;  // window index (a column j for row sweeps, a row i for column sweeps)
    const bool ok = k >= 0 && k < n;
    const int kc = k < 0 ? 0 : (k < n ? k : n - 1);
    const double xw = COL ? uR[kc] : vR[kc];
    wv[c] = ok ? (float)(xw - ref) : kNegInf;
    if (MODE == 0) {
      float z;
      if (COL)  // zz_i = alpha^(r)_i x^(r)_i
        z = exp2f(p.tail_u[slot(p.r, BHL) + bh * L + kc] - xw) * p.x[slot(p.r, BHL) + bh * L + kc];
      else  // z_j = beta^(r)_j y^(r)_j
        z = exp2f(p.tail_v[slot(p.r, BHL) + bh * L + kc] - xw) * p.vbar[slot(p.r, BHL) + bh * L + kc] /
            p.b[(size_t)bb * L + kc];
      vec[c] = ok ? z : 0.f;
    } else if (MODE == 1) {
#pragma unroll
      for (int kk = 1; kk <= RM; ++kk) {
        if (kk <= R) {
          float m0, m1;
          if (COL) {  // row modifiers alpha^(k)_i, alpha^(k)_i x^(k)_i
            m0 = exp2f(p.tail_u[slot(kk, BHL) + bh * L + kc] - xw);
            m1 = m0 * p.x[slot(kk, BHL) + bh * L + kc];
          } else {  // column modifiers beta^(k)_j y^(k)_j, beta^(k-1)_j
            m0 = exp2f(p.tail_v[slot(kk, BHL) + bh * L + kc] - xw) * p.vbar[slot(kk, BHL) + bh * L + kc] /
                 p.b[(size_t)bb * L + kc];
            m1 = exp2f(p.tail_v[slot(kk - 1, BHL) + bh * L + kc] - xw);
          }
          vec[(size_t)(2 * (kk - 1)) * NWC + c] = ok ? m0 : 0.f;
          vec[(size_t)(2 * (kk - 1) + 1) * NWC + c] = ok ? m1 : 0.f;
        }
      }
    }
  }
  (void)NVMAX;
  (void)NV;

  // streamed tensors: [0] score side (K rows / Q rows), [1] dP side (V / dO)
  // or, for dV, the product side (dO)
  const char* X0 = reinterpret_cast<const char*>(COL ? p.Q : p.K) + (size_t)bh * L * RB;
  const char* X1 = reinterpret_cast<const char*>(COL ? p.dO : p.V) + (size_t)bh * L * RB;
  // Pairs stream into LDS by DMA (global_load_lds, 16 bytes per lane): wave
  // w fills bytes [w KB, (w + 1) KB) of each tensor's pair buffer, i.e. rows
  // RPW w .. RPW (w + 1) - 1, and the lane at chunk position pc of its row
  // loads logical chunk pc ^ f(row), which leaves the buffer in the swizzled
  // layout the reads expect (sw_chunk is an involution).  Rows outside the
  // sequence are loaded from the nearest real row: every entry they feed is
  // masked to exactly zero (their scores are -inf).
  constexpr int RPW = 1024 / RB;                  // rows per wave instruction
  const uint32_t lds_base = lds_addr(tbuf);
  constexpr int DMA_WAVES = 32 / RPW;             // waves that move a pair
  const bool dma_wave = wave < DMA_WAVES;
  auto issue_pair = [&](int pp) {
    if (dma_wave) {
      const int pos = lane * 16;
      const int r32 = wave * RPW + pos / RB;
      const int c = sw_chunk<CPR>((pos % RB) / 16, r32);
      int row = (tw0 + 2 * pp) * 16 + r32;
      row = row < 0 ? 0 : (row >= n ? n - 1 : row);
      const uint32_t dst = lds_base + (uint32_t)((pp % NBUF) * NTEN) * TBYTES + wave * 1024;
      const uint32_t off = (uint32_t)(row * RB + c * 16);
      lds_dma16(X0, off, dst);
      if (NTEN > 1) lds_dma16(X1, off, dst + TBYTES);
    }
  };
  // Barrier of the pair pipeline: this wave's LDS reads are done and its
  // DMAs of the next pair have landed (at most `later` pairs issued after it
  // still in flight: vmcnt counts this wave's DMA instructions, and the loop
  // issues no other vector memory operation), then the waves meet.  A plain
  // __syncthreads would also wait for every DMA in flight, draining the
  // prefetch at each pair.
  auto pipe_barrier = [&](int later) {
    asm volatile("" ::: "memory");
    constexpr int kLgkm0 = 0x0070;  // lgkmcnt(0), expcnt left free; vmcnt in bits 3:0
    if (later >= 2) __builtin_amdgcn_s_waitcnt(kLgkm0 | (2 * NTEN));
    else if (later == 1) __builtin_amdgcn_s_waitcnt(kLgkm0 | NTEN);
    else __builtin_amdgcn_s_waitcnt(kLgkm0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // strip operands (registers): score side (Q rows / K rows), dP side (dO / V)
  const int si = s0b + wave * 16 + lr;  // strip index of this lane (B operand row)
  const bool sok = si < n;
  const int sic = si < (int)L ? si : (int)L - 1;
  const char* S0 = reinterpret_cast<const char*>(COL ? p.K : p.Q) + (size_t)bh * L * RB;
  const char* S1 = reinterpret_cast<const char*>(COL ? p.V : p.dO) + (size_t)bh * L * RB;
  u4 sb0[NCH], sb1[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const u4 a0 = ld16(S0 + (size_t)sic * RB + c * 64 + lg * 16);
    sb0[c] = sok ? a0 : (u4){0u, 0u, 0u, 0u};
    if (MODE == 1) {
      const u4 a1 = ld16(S1 + (size_t)sic * RB + c * 64 + lg * 16);
      sb1[c] = sok ? a1 : (u4){0u, 0u, 0u, 0u};
    }
  }
  // strip-side exponent part and strip modifiers (MODE 1); clamped loads
  // (n >= 1 here: the block holds a real row)
  const int sil = sok ? si : n - 1;
  const double xs = COL ? vR[sil] : uR[sil];
  const float sbias = sok ? (float)(xs + ref) : 0.f;
  float sm0[RM], sm1[RM];  // RM >= R: tail depth bound of this instance
#pragma unroll
  for (int k = 0; k < RM; ++k) {
    sm0[k] = 0.f;
    sm1[k] = 0.f;
    if (MODE == 1 && k < R) {
      float m0, m1;
      if (COL) {  // beta^(k)_j y^(k)_j, beta^(k-1)_j
        m0 = exp2f(p.tail_v[slot(k + 1, BHL) + bh * L + sil] - xs) * p.vbar[slot(k + 1, BHL) + bh * L + sil] /
             p.b[(size_t)bb * L + sil];
        m1 = exp2f(p.tail_v[slot(k, BHL) + bh * L + sil] - xs);
      } else {  // alpha^(k)_i, alpha^(k)_i x^(k)_i
        m0 = exp2f(p.tail_u[slot(k + 1, BHL) + bh * L + sil] - xs);
        m1 = m0 * p.x[slot(k + 1, BHL) + bh * L + sil];
      }
      sm0[k] = sok ? m0 : 0.f;
      sm1[k] = sok ? m1 : 0.f;
    }
  }

  // per-lane LDS offsets: A-operand chunks of row lr; transposed B reads
  // (lane 4 r + q of its 16-lane group: row 4 lg + r, 8 bytes of chunk pair ds)
  // The swizzle is an XOR, so sw_chunk(4 c + lg, r) = 4 c ^ sw_chunk(lg, r) and
  // sw_chunk(2 ds + e, r) = 2 ds ^ sw_chunk(e, r).  The run-time-R dQ / dK
  // instance has no registers to spare for offset tables and forms each
  // offset at its read.
  constexpr bool kTab = !(MODE == 1 && !RX);
  const int rowA = lr * RB;
  int hA = sw_chunk<CPR>(lg, lr) * 16;
  const int rowB = (4 * lg + (lr >> 2)) * RB + 8 * (lr & 1);
  int hB = sw_chunk<CPR>((lr & 3) >> 1, 4 * lg + (lr >> 2)) * 16;
  int offA[kTab ? NCH : 1], offB[kTab ? ND : 1];
#pragma unroll
  for (int c = 0; c < (kTab ? NCH : 1); ++c) offA[c] = rowA + ((64 * c) ^ hA);
#pragma unroll
  for (int ds = 0; ds < (kTab ? ND : 1); ++ds) offB[ds] = rowB + ((32 * ds) ^ hB);
  auto offAat = [&](int c) { return kTab ? offA[c] : rowA + ((64 * c) ^ hA); };
  auto offBat = [&](int ds) { return kTab ? offB[ds] : rowB + ((32 * ds) ^ hB); };

  float vacc = 0.f;  // MODE 0
  f4 acc[ND];
#pragma unroll
  for (int ds = 0; ds < ND; ++ds) acc[ds] = (f4){0.f, 0.f, 0.f, 0.f};

  for (int q = 0; q < 3 && q < NP; ++q) issue_pair(q);
  pipe_barrier((NP - 1 < 2) ? NP - 1 : 2);  // pair 0 (pairs 1, 2 may still be in flight)

  const int wstart = wave;           // first window tile of this strip
  const int sidx0 = s0b + wave * 16;  // first strip index of the wave
  const bool wactive = sidx0 < n;
  for (int pp = 0; pp < NP; ++pp) {
    const int buf = pp % NBUF;
    // (no table: keep the offset parts opaque so that the compiler does not
    // hoist every offset out of the loop into registers)
    if constexpr (!kTab) asm volatile("" : "+v"(hA), "+v"(hB));
    // pair pp + 3 into the buffer pair pp - 1 used (every wave is past it)
    if (pp + 3 < NP) issue_pair(pp + 3);
    // tiles 2pp, 2pp + 1 of the window; strip-relative t = window tile - wave
    float val[2][4];
    bool any = false;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int wt = 2 * pp + tt;
      const int t = wt - wstart;
      const int tg = tw0 + wt;  // global tile
      const bool act = wactive && t >= 0 && t < NT && tg >= 0 && tg * 16 < n;
#pragma unroll
      for (int r = 0; r < 4; ++r) val[tt][r] = 0.f;
      if (act) {
        any = true;
        const char* tb0 = tbuf + (size_t)(buf * NTEN + 0) * TBYTES + tt * 16 * RB;
        f4 sacc = {0.f, 0.f, 0.f, 0.f}, dacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          const u4 a = ld16(tb0 + offAat(c));
          sacc = Elt<bf16_t>::mma_chunk(sacc, a, sb0[c]);
        }
        if (MODE == 1) {
          const char* tb1 = tbuf + (size_t)(buf * NTEN + 1) * TBYTES + tt * 16 * RB;
#pragma unroll
          for (int c = 0; c < NCH; ++c) {
            const u4 a = ld16(tb1 + offAat(c));
            dacc = Elt<bf16_t>::mma_chunk(dacc, a, sb1[c]);
          }
        }
        // lane: strip index si, window indices wi = tg * 16 + 4 lg + r
        const int cw = wt * 16 + 4 * lg;  // window position of r = 0
        // wave-uniform: every entry of the tile lies inside the band and
        // between real rows and columns, so no entry needs the mask
        const int olo = COL ? sidx0 - tg * 16 - 15 : tg * 16 - sidx0 - 15;  // lowest j - i
        const bool inner = olo >= -g.h1 && olo + 30 <= g.h2 && sidx0 + 16 <= n && tg * 16 + 16 <= n;
        const f4 w4 = *reinterpret_cast<const f4*>(wv + cw);
        f4 z4 = {0.f, 0.f, 0.f, 0.f};
        if (MODE == 0) z4 = *reinterpret_cast<const f4*>(vec + cw);
        // dP minus the tail terms, tail step by tail step: the step's two
        // window modifiers of the lane's four entries come in one 16-byte read
        // each (cw is a multiple of 4 and NWC of 16) and are used at once
        f4 br4 = dacc;
        if (MODE == 1) {
#pragma unroll
          for (int k = 0; k < RM; ++k) {
            if (k < R) {
              const f4 m0 = *reinterpret_cast<const f4*>(vec + (size_t)(2 * k) * NWC + cw);
              const f4 m1 = *reinterpret_cast<const f4*>(vec + (size_t)(2 * k + 1) * NWC + cw);
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                br4[r] -= COL ? m0[r] * sm0[k] : sm0[k] * m0[r];
                br4[r] -= COL ? m1[r] * sm1[k] : sm1[k] * m1[r];
              }
            }
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int wi = tg * 16 + 4 * lg + r;
          const int o = COL ? si - wi : wi - si;  // j - i
          float x = __builtin_fmaf(sacc[r], g.scale2, w4[r] + sbias);
          if (!inner) x = (o >= -g.h1 && o <= g.h2 && sok && wi >= 0 && wi < n) ? x : kNegInf;
          const float pe = exp2_fast(x);
          if (MODE == 0) {
            val[tt][r] = pe * z4[r];
          } else if (MODE == 2) {
            val[tt][r] = pe;
          } else {
            val[tt][r] = pe * br4[r];
          }
        }
      }
    }
    if (MODE == 0) {
      vacc += (val[0][0] + val[0][1]) + (val[0][2] + val[0][3]);
      vacc += (val[1][0] + val[1][1]) + (val[1][2] + val[1][3]);
    } else if (any) {
      u4 hi, lo;
      split_hilo(val[0], val[1], hi, lo);
      const char* pb = tbuf + (size_t)(buf * NTEN + PT) * TBYTES;
#pragma unroll
      for (int ds = 0; ds < ND; ++ds) {
        const u2 b0 = ld_tr16(pb + offBat(ds));
        const u2 b1 = ld_tr16(pb + 16 * RB + offBat(ds));
        const u4 bv = {b0.x, b0.y, b1.x, b1.y};
        acc[ds] = Elt<bf16_t>::mma_chunk(acc[ds], hi, bv);
        acc[ds] = Elt<bf16_t>::mma_chunk(acc[ds], lo, bv);
      }
    }
    // pair pp + 1 complete in every wave before the next iteration reads it
    const int later = NP - 2 - pp;  // pairs issued after pair pp + 1
    pipe_barrier(later < 0 ? 0 : (later > 2 ? 2 : later));
  }

  if (!wactive) {
    if (MODE == 2 && p.e_out) {  // filler strip: zero dV rows and E
#pragma unroll
      for (int ds = 0; ds < ND; ++ds)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int s = sidx0 + 4 * lg + r;
          if (s < (int)L) p.out[((size_t)bh * L + s) * D + ds * 16 + lr] = 0.f;
        }
      if (lr == 0)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int s = sidx0 + 4 * lg + r;
          if (s < (int)L) p.e_out[(size_t)bh * L + s] = 0.f;
        }
    }
    return;
  }
  if (MODE == 0) {
    const float tot = cross_row_sum(vacc);
    if (lg == 0 && sok) {
      if (!COL) {
        const int i = si;
        float a2 = tot;
        if (g.dustbin) {
          // entry (i, delta): P_i,delta z_delta
          const double vRd = p.tail_v[slot(R, BHL) + bh * L + n];
          const float zd = exp2f(p.tail_v[slot(p.r, BHL) + bh * L + n] - vRd) *
                           p.vbar[slot(p.r, BHL) + bh * L + n] / p.b[(size_t)bb * L + n];
          a2 += exp2f(p.sdc[bh * L + i] + uR[i] + vRd) * zd;
        }
        const float alpha = exp2f(p.tail_u[slot(p.r, BHL) + bh * L + i] - uR[i]);
        const float ub = (p.r == R ? p.D[bh * L + i] : 0.f) - alpha * a2;
        p.x[slot(p.r, BHL) + bh * L + i] = ub / p.a[(size_t)bb * L + i];
      } else {
        const int j = si;
        float a2 = tot;
        if (g.dustbin) {
          // entry (delta, j): P_delta,j zz_delta
          const double uRd = p.tail_u[slot(R, BHL) + bh * L + n];
          const float zd = exp2f(p.tail_u[slot(p.r, BHL) + bh * L + n] - uRd) * p.x[slot(p.r, BHL) + bh * L + n];
          a2 += exp2f(p.sdr[bh * L + j] + uRd + vR[j]) * zd;
        }
        const float beta = exp2f(p.tail_v[slot(p.r - 1, BHL) + bh * L + j] - vR[j]);
        p.vbar[slot(p.r - 1, BHL) + bh * L + j] = -beta * a2;
      }
    }
  } else {
    const float sc = MODE == 1 ? g.inv_sqrt_d : 1.f;
    const bool fuse_e = MODE == 2 && p.e_out != nullptr;
    float e4[4] = {0.f, 0.f, 0.f, 0.f};  // E partials of the lane's four columns
    // V at the lane's dV entries, loaded before any store (the compiler
    // cannot move a load above a store that may alias it) from clamped rows,
    // so that all of them are in flight at once
    constexpr int NVL = MODE == 2 ? ND * 4 : 1;
    unsigned short vl[NVL];
#pragma unroll
    for (int e = 0; e < NVL; ++e) vl[e] = 0;
    if (fuse_e) {
      const unsigned short* Vb = reinterpret_cast<const unsigned short*>(p.V);
#pragma unroll
      for (int ds = 0; ds < ND; ++ds)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int s = sidx0 + 4 * lg + r;
          const int sl = s < n ? s : n - 1;
          vl[(MODE == 2 ? ds * 4 + r : 0)] = Vb[((size_t)bh * L + sl) * D + ds * 16 + lr];
        }
    }
#pragma unroll
    for (int ds = 0; ds < ND; ++ds) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int s = sidx0 + 4 * lg + r;
        if (s < n) {
          p.out[((size_t)bh * L + s) * D + ds * 16 + lr] = acc[ds][r] * sc;
          if (fuse_e) e4[r] = __builtin_fmaf(bf16_to_float(vl[(MODE == 2 ? ds * 4 + r : 0)]), acc[ds][r], e4[r]);
        } else if (fuse_e && s < (int)L) {
          p.out[((size_t)bh * L + s) * D + ds * 16 + lr] = 0.f;
        }
      }
    }
    if (fuse_e) {
      // E_j = sum over d of V_jd dV_jd: the lane's 8 slices, then its 16-lane row
#pragma unroll
      for (int r = 0; r < 4; ++r) e4[r] = row16_sum(e4[r]);
      if (lr == 0)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int s = sidx0 + 4 * lg + r;
          if (s < (int)L) p.e_out[(size_t)bh * L + s] = s < n ? e4[r] : 0.f;
        }
    }
  }
}

template <typename T, int D>
static hipError_t backward_impl(const Geom& g, const BwdLaunch& f, const Workspace& w, hipStream_t st) {
  constexpr int EB = Elt<T>::kBytes;
  const int nbh = g.B * g.H;
  const size_t BHL = (size_t)nbh * g.L;
  const int R = f.R;
  const int nblk = ceil_div_pos(g.L, kBwdBlock);
  const int grid = (nbh * nblk + 7) & ~7;
  const int NWC = 16 * (g.TL + g.TR + kBwdWaves);
  const int NWR = 16 * (g.TLc + g.TRc + kBwdWaves);
  const size_t row_vec_lds = (size_t)NWC * 4 * 2 + 64;
  const size_t row_grad_lds = (size_t)NWC * 4 * (1 + 2 * (R > 0 ? R : 1)) + (size_t)D * (NWC + 8) * EB + 64;
  const size_t col_vec_lds = (size_t)NWR * 4 * 2 + 64;
  const size_t col_grad_lds = (size_t)NWR * 4 * (1 + 2 * (R > 0 ? R : 1)) + (size_t)D * (NWR + 8) * EB + 64;
  const size_t col_dv_lds = (size_t)NWR * 4 * 2 + (size_t)D * (NWR + 8) * EB + 64;
  if (row_grad_lds > 160 * 1024 || col_grad_lds > 160 * 1024 || col_dv_lds > 160 * 1024)
    return hipErrorInvalidConfiguration;
  hipError_t err;
#define SET_LDS(kern, bytes)                                                                              \
  err = ensure_lds(reinterpret_cast<const void*>(kern), (size_t)(bytes));                                 \
  if (err != hipSuccess) return err;
  SET_LDS((bw_row_kernel<T, D, 1>), row_grad_lds);
  SET_LDS((bw_col_kernel<T, D, 1>), col_grad_lds);
  SET_LDS((bw_col_kernel<T, D, 2>), col_dv_lds);
#undef SET_LDS

  // Adjoint vectors: vbar^(0..R), x^(0..R) (slot r = tail step r).  A
  // grad-only pass of depth R reads those of a full pass of depth R_vec: the
  // vectors of the last R tail steps do not depend on where the stop-gradient
  // sits (each comes from the later steps only, and every modifier is taken
  // relative to the same last step), so its slots are that pass's slots
  // R_vec - R .. R_vec.
  const bool grad_only = f.grad_only != 0;
  const int Rv = grad_only ? f.R_vec : R;
  if (grad_only && (Rv < R || f.slot0 < Rv - R)) return hipErrorInvalidValue;
  float* Dv = w.bw;
  float* vbar = Dv + align64(BHL) + (size_t)(Rv - R) * BHL;
  float* xv = Dv + align64(BHL) + align64((size_t)(Rv + 1) * BHL) + (size_t)(Rv - R) * BHL;
  BwArgs p{};
  p.Q = f.Q;
  p.K = f.K;
  p.V = f.V;
  p.dO = f.dO;
  p.O = f.O;
  p.a = f.a;
  p.b = f.b;
  // this pass's stack: slots slot0 .. slot0 + R of the forward's tail stack
  const double* tail_u = w.tail_u + (size_t)f.slot0 * BHL;
  const double* tail_v = w.tail_v + (size_t)f.slot0 * BHL;
  p.tail_u = tail_u;
  p.tail_v = tail_v;
  p.sdr = w.sdr;
  p.sdc = w.sdc;
  p.D = Dv;
  p.vbar = vbar;
  p.x = xv;
  p.R = R;
  p.padded_grid = grid;
  const dim3 tg((g.L + 255) / 256, nbh);
  const T* Qt = reinterpret_cast<const T*>(f.Q);
  const T* Kt = reinterpret_cast<const T*>(f.K);
  const T* Vt = reinterpret_cast<const T*>(f.V);
  const T* dOt = reinterpret_cast<const T*>(f.dO);
  if (g.dustbin && !grad_only) hipLaunchKernelGGL(dustbin_scores_bw<T>, tg, dim3(256), 0, st, g, Qt, Kt, w.sdr, w.sdc);
  // dustbin row / column sums: chunk partials, then the fixed-order finish
  const int dch = (g.L + 255) / 256;
  float* dpart = w.dpart;
  auto dustbin_bw = [&](int mode) {
    hipLaunchKernelGGL(bw_dustbin_part<T>, dim3(dch, nbh), dim3(256), 0, st, g, p, mode, dpart);
    hipLaunchKernelGGL(bw_dustbin_fin<T>, dim3(nbh), dim3(256), 0, st, g, p, mode, static_cast<const float*>(dpart), dch);
  };
  const dim3 tok((g.L + kTokPerBlock - 1) / kTokPerBlock, nbh);
  if (!grad_only) hipLaunchKernelGGL((bw_rowdot<T, D>), tok, dim3(256), 0, st, g, dOt, f.O, Dv);
  // bf16 with d >= 64: streamed sweeps (one workgroup per 128-index block)
  constexpr bool kSweep = sizeof(T) == 2 && D >= 64;
  const int sgrid = (nbh * ceil_div_pos(g.L, 128) + 7) & ~7;
  BwArgs ps = p;
  ps.padded_grid = sgrid;
  auto sweep_lds = [&](bool col, int mode) {
    const int NT = col ? g.NTc : g.NT;
    const int NP = (NT + kSwWaves) / 2;
    const int NWC = 2 * NP * 16;
    const int ntens = mode == 0 ? 1 : 2;
    const int nv = mode == 0 ? 1 : (mode == 1 ? 2 * R : 0);
    return (size_t)4 * ntens * 32 * D * 2 + (size_t)NWC * 4 * (1 + nv) + 64;  // 4 pair buffers
  };
  if constexpr (kSweep) {
#define SET_SW(COLV, MODEV, RMV, RXV)                                                                   \
  err = ensure_lds(reinterpret_cast<const void*>(bw_sweep_kernel<D, COLV, MODEV, RMV, RXV>),            \
                   sweep_lds(COLV, MODEV));                                                             \
  if (err != hipSuccess) return err;
    SET_SW(false, 0, 2, false) SET_SW(false, 1, 2, false) SET_SW(true, 0, 2, false) SET_SW(true, 1, 2, false)
    SET_SW(true, 2, 2, false) SET_SW(false, 1, kMaxR, false) SET_SW(true, 1, kMaxR, false)
    SET_SW(false, 1, 2, true) SET_SW(true, 1, 2, true)
#undef SET_SW
  }
  if (!grad_only) {
    // dV (band) -> add dustbin row, E, vbar^(R).  The bf16 sweep computes E and
    // zeroes filler rows itself when there is no dustbin term to add first.
    p.out = f.dV;
    ps.out = f.dV;
    const bool fuse_e = kSweep && !g.dustbin;
    ps.e_out = fuse_e ? vbar + (size_t)R * BHL : nullptr;
    if constexpr (kSweep)
      hipLaunchKernelGGL((bw_sweep_kernel<D, true, 2, 2>), dim3(sgrid), dim3(kSwThreads), sweep_lds(true, 2), st, g, ps);
    else
      hipLaunchKernelGGL((bw_col_kernel<T, D, 2>), dim3(grid), dim3(256), col_dv_lds, st, g, p);
    if (!fuse_e)
      hipLaunchKernelGGL(bw_finish_dv<T>, tok, dim3(256), 0, st, g, Vt, dOt, tail_u, tail_v, w.sdr, R, f.dV,
                         vbar + (size_t)R * BHL);
    ps.e_out = nullptr;  // the later sweeps write no E
    if (g.dustbin) dustbin_bw(0);
    // adjoint vectors through the tail
    for (int r = R; r >= 1; --r) {
      p.r = r;
      ps.r = r;
      if constexpr (kSweep)
        hipLaunchKernelGGL((bw_sweep_kernel<D, false, 0, 2>), dim3(sgrid), dim3(kSwThreads), sweep_lds(false, 0), st, g, ps);
      else
        hipLaunchKernelGGL((bw_row_kernel<T, D, 0>), dim3(grid), dim3(256), row_vec_lds, st, g, p);
      if (g.dustbin) dustbin_bw(1);
      if (r > 1 || f.vbar0) {
        if constexpr (kSweep)
          hipLaunchKernelGGL((bw_sweep_kernel<D, true, 0, 2>), dim3(sgrid), dim3(kSwThreads), sweep_lds(true, 0), st, g, ps);
        else
          hipLaunchKernelGGL((bw_col_kernel<T, D, 0>), dim3(grid), dim3(256), col_vec_lds, st, g, p);
        if (g.dustbin) dustbin_bw(2);
      }
    }
  }
  // dQ, dK
  p.out = f.dQ;
  ps.out = f.dQ;
  if constexpr (kSweep) {
    if (R == 2)  // the tail depth as a compile-time constant
      hipLaunchKernelGGL((bw_sweep_kernel<D, false, 1, 2, true>), dim3(sgrid), dim3(kSwThreads), sweep_lds(false, 1), st,
                         g, ps);
    else if (R < 2)
      hipLaunchKernelGGL((bw_sweep_kernel<D, false, 1, 2>), dim3(sgrid), dim3(kSwThreads), sweep_lds(false, 1), st, g, ps);
    else
      hipLaunchKernelGGL((bw_sweep_kernel<D, false, 1, kMaxR>), dim3(sgrid), dim3(kSwThreads), sweep_lds(false, 1), st, g,
                         ps);
  }
  else
    hipLaunchKernelGGL((bw_row_kernel<T, D, 1>), dim3(grid), dim3(256), row_grad_lds, st, g, p);
  hipLaunchKernelGGL((bw_finish_grad<T, 0>), tg, dim3(256), 0, st, g, p);
  if (g.dustbin) dustbin_bw(3);
  p.out = f.dK;
  ps.out = f.dK;
  if constexpr (kSweep) {
    if (R == 2)
      hipLaunchKernelGGL((bw_sweep_kernel<D, true, 1, 2, true>), dim3(sgrid), dim3(kSwThreads), sweep_lds(true, 1), st,
                         g, ps);
    else if (R < 2)
      hipLaunchKernelGGL((bw_sweep_kernel<D, true, 1, 2>), dim3(sgrid), dim3(kSwThreads), sweep_lds(true, 1), st, g, ps);
    else
      hipLaunchKernelGGL((bw_sweep_kernel<D, true, 1, kMaxR>), dim3(sgrid), dim3(kSwThreads), sweep_lds(true, 1), st, g,
                         ps);
  }
  else
    hipLaunchKernelGGL((bw_col_kernel<T, D, 1>), dim3(grid), dim3(256), col_grad_lds, st, g, p);
  hipLaunchKernelGGL((bw_finish_grad<T, 1>), tg, dim3(256), 0, st, g, p);
  if (g.dustbin) dustbin_bw(4);
  if (f.vbar0 && !grad_only) hipLaunchKernelGGL(bw_copy_vbar0, tg, dim3(256), 0, st, g, vbar, f.vbar0);
  return hipGetLastError();
}

hipError_t launch_backward(const Geom& g, int dtype, const BwdLaunch& f, const Workspace& w, hipStream_t st) {
  if (dtype == 0) {
    switch (g.d) {
      case 16: return backward_impl<float, 16>(g, f, w, st);
      case 32: return backward_impl<float, 32>(g, f, w, st);
      case 64: return backward_impl<float, 64>(g, f, w, st);
    }
  } else {
    switch (g.d) {
      case 32: return backward_impl<bf16_t, 32>(g, f, w, st);
      case 64: return backward_impl<bf16_t, 64>(g, f, w, st);
      case 128: return backward_impl<bf16_t, 128>(g, f, w, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace sinkattn
