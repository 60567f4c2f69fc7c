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
  double* u_tail;         // optional copy of u^(t)
  float* part_out;        // [BH][nblk][NWC] column partials of step t
  float* partd_out;       // [BH][nblk] dustbin-column partials of step t
  const double* dstate;   // dustbin state after step t-1 (nullptr => zeros)
  const float* sdr;       // dustbin row scores [BHL], log2 units
  const float* sdc;       // dustbin column scores [BHL], log2 units
  int first;              // 1 => step 1: v^(0) = 0 and exact row maxima
  int padded_grid;
};

// floor(a / b) for b > 0 and any sign of a.
__device__ __forceinline__ int floor_div(int a, int b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }

// Finish v^(t-1)_j (log2 units, fp64) for band column j (a real token) from
// the partial sums of step t-1, summed in increasing block order.
__device__ __forceinline__ double finish_v(const Geom& g, int bh, int n, int j, const double* v_prev2,
                                           const float* part_in, const float* b, int bb,
                                           const double* dstate, const float* sdr) {
  const size_t L = g.L;
  const double vprev = v_prev2 ? v_prev2[bh * L + j] : 0.0;
  const int x = j + 16 * g.TL - g.NWC;
  int rlo = floor_div(x, kBlockRows) + 1;
  rlo = rlo < 0 ? 0 : rlo;
  int rhi = (j + 16 * g.TL) / kBlockRows;
  rhi = rhi > g.nblk - 1 ? g.nblk - 1 : rhi;
  float gam = 0.f;
  for (int r = rlo; r <= rhi; ++r) {
    if (r * kBlockRows >= n) break;  // blocks without real rows wrote nothing
    gam += part_in[((size_t)bh * g.nblk + r) * g.NWC + (j - (r * kBlockRows - 16 * g.TL))];
  }
  if (g.dustbin && dstate) {
    // dustbin row entry of the row-normalised plan P^(t-1,t-2)_{delta j}
    const double* ds = dstate + 4 * bh;
    gam += exp2_fast((float)((double)sdr[bh * L + j] + vprev - ds[2])) * (float)ds[3];
  }
  return vprev + log2((double)b[(size_t)bb * L + j]) - log2((double)gam);
}

template <typename T, int D>
__global__ __launch_bounds__(512) void iter_kernel(Geom g, IterArgs p) {
  constexpr int RB = D * Elt<T>::kBytes;  // bytes per Q/K row
  constexpr int NCH = RB / 64;             // 16-byte lane chunks per row
  constexpr int RS = RB + 16;              // padded LDS row stride
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
  if (r0 >= n) return;

  const size_t L = g.L;
  const int NWC = g.NWC;
  const int tw0 = (r0 >> 4) - g.TL;  // first window tile
  char* kw = smem;                                     // [NWC][RS]
  float* w2s = reinterpret_cast<float*>(smem + (size_t)NWC * RS);  // [NWC]
  float* colbuf = w2s + NWC;                           // [8][NWC]
  float* misc = colbuf + kWaves * NWC;                 // [8]

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;

  // (0) reference potential: v^(t-1) at column r0 (a real token)
  if (tid == 0)
    sh_vref = p.part_in ? finish_v(g, bh, n, r0, p.v_prev2, p.part_in, p.b, bb, p.dstate, p.sdr) : 0.0;
  __syncthreads();
  const double vref = sh_vref;

  // (1) finish v^(t-1) on the window; owners publish it.
  for (int c = tid; c < NWC; c += blockDim.x) {
    const int j = tw0 * 16 + c;
    float w = kNegInf;
    if (j >= 0 && j < n) {
      double vj = 0.0;
      if (p.part_in) vj = finish_v(g, bh, n, j, p.v_prev2, p.part_in, p.b, bb, p.dstate, p.sdr);
      if (p.v_out && j >= r0 && j < r0 + kBlockRows) {
        p.v_out[bh * L + j] = vj;
        if (p.v_tail) p.v_tail[bh * L + j] = vj;
      }
      w = (float)(vj - vref);
    }
    w2s[c] = w;
  }
  // (2) K window -> LDS (zero outside the real tokens)
  {
    const char* Kb = reinterpret_cast<const char*>(p.K) + (size_t)bh * L * RB;
    const int per_row = RB / 16;
    for (int idx = tid; idx < NWC * per_row; idx += blockDim.x) {
      const int row = idx / per_row, c16 = idx - row * per_row;
      const int j = tw0 * 16 + row;
      u4 val = {0u, 0u, 0u, 0u};
      if (j >= 0 && j < n) val = ld16(Kb + (size_t)j * RB + c16 * 16);
      st16(kw + (size_t)row * RS + c16 * 16, val);
    }
  }
  float* cb = colbuf + wave * NWC;
  for (int c = lane; c < NWC; c += 64) cb[c] = 0.f;
  if (lane == 0) misc[wave] = 0.f;
  __syncthreads();

  const int i0 = r0 + wave * 16;
  if (i0 < n) {
    // Q strip operands (A side: row i0 + lr)
    u4 qa[NCH];
    {
      const char* Qb = reinterpret_cast<const char*>(p.Q) + (size_t)bh * L * RB;
      const int qi = i0 + lr;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        qa[c] = (u4){0u, 0u, 0u, 0u};
        if (qi < n) qa[c] = ld16(Qb + (size_t)qi * RB + c * 64 + lg * 16);
      }
    }
    const int NT = g.NT;
    // tile t covers global columns [(tw0 + wave + t) * 16, +16)
    const int tg0 = tw0 + wave;
    int t_lo = -tg0;                 // first tile with a column >= 0
    t_lo = t_lo < 0 ? 0 : t_lo;
    int t_hi = (n - 1) / 16 - tg0;   // last tile with a column < n
    t_hi = t_hi > NT - 1 ? NT - 1 : t_hi;

    float e[kMaxTiles][4];
    float shift[4];
    float rs[4];
    float ed[4] = {0.f, 0.f, 0.f, 0.f};
    bool rowok[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) rowok[r] = i0 + 4 * lg + r < n;
    // dustbin column exponent for the lane's rows, relative to vref
    float xd[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
    if (g.dustbin) {
      const double vd = p.dstate ? p.dstate[4 * bh + 1] : 0.0;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (rowok[r]) xd[r] = (float)((double)p.sdc[bh * L + i0 + 4 * lg + r] + vd - vref);
    }

    const bool partial = i0 + 16 > n;  // wave-uniform: strip holds non-real rows
    // score tile t -> x = S * log2e/sqrt(d) + w_j (band-masked)
    auto score_tile = [&](int t, float (&x)[4]) {
      f4 acc = {0.f, 0.f, 0.f, 0.f};
      const char* kb = kw + (size_t)((wave + t) * 16 + lr) * RS + lg * 16;
#pragma unroll
      for (int c = 0; c < NCH; ++c) acc = Elt<T>::mma_chunk(acc, qa[c], ld16(kb + c * 64));
      const float wj = w2s[(wave + t) * 16 + lr];
      const int obase = (t - g.TL) * 16 + lr - 4 * lg;
      const bool interior = (16 * (t - g.TL) - 15 >= -g.h1) && (16 * (t - g.TL) + 15 <= g.h2);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = __builtin_fmaf(acc[r], g.scale2, wj);
        if (!interior) {
          const int o = obase - r;
          v = (o >= -g.h1 && o <= g.h2) ? v : kNegInf;
        }
        if (partial) v = rowok[r] ? v : kNegInf;  // rows past the real tokens
        x[r] = v;
      }
    };

    bool need_safe = p.first != 0;
    if (!need_safe) {
#pragma unroll
      for (int r = 0; r < 4; ++r) { shift[r] = 0.f; rs[r] = 0.f; }
#pragma unroll
      for (int t = 0; t < kMaxTiles; ++t) {
        if (t < NT && t >= t_lo && t <= t_hi) {
          float x[4];
          score_tile(t, x);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            e[t][r] = exp2_fast(x[r]);
            rs[r] += e[t][r];
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) e[t][r] = 0.f;
        }
      }
      bool bad = false;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        rs[r] = row16_sum(rs[r]);
        if (g.dustbin) {
          ed[r] = exp2_fast(xd[r]);
          rs[r] += ed[r];
        }
        if (rowok[r]) bad |= !(rs[r] >= 0x1p-120f && rs[r] <= 0x1p120f);
      }
      need_safe = __any(bad);
    }
    if (need_safe) {
      // exact per-row maxima
      float m[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
      for (int t = 0; t < kMaxTiles; ++t) {
        if (t < NT && t >= t_lo && t <= t_hi) {
          score_tile(t, e[t]);
#pragma unroll
          for (int r = 0; r < 4; ++r) m[r] = fmaxf(m[r], e[t][r]);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) e[t][r] = kNegInf;
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        m[r] = row16_max(m[r]);
        if (g.dustbin) m[r] = fmaxf(m[r], xd[r]);
        if (!(m[r] > kNegInf)) m[r] = 0.f;  // inactive row
        shift[r] = m[r];
        rs[r] = 0.f;
      }
#pragma unroll
      for (int t = 0; t < kMaxTiles; ++t) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          e[t][r] = exp2_fast(e[t][r] - shift[r]);
          rs[r] += e[t][r];
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        rs[r] = row16_sum(rs[r]);
        ed[r] = g.dustbin ? exp2_fast(xd[r] - shift[r]) : 0.f;
        rs[r] += ed[r];
      }
    }

    // (3) u^(t) (fp64) and the row weights h_i = a_i / rho_i
    float h[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = i0 + 4 * lg + r;
      h[r] = 0.f;
      if (rowok[r]) {
        const float ai = p.a[(size_t)bb * L + i];
        h[r] = ai / rs[r];
        if (lr == 0) {
          const double u = log2((double)ai) - log2((double)rs[r]) - (double)shift[r] - vref;
          p.u_out[bh * L + i] = u;
          if (p.u_tail) p.u_tail[bh * L + i] = u;
        }
      }
    }
    // (4) column partials of this strip: sum_i e_ij h_i
#pragma unroll
    for (int t = 0; t < kMaxTiles; ++t) {
      if (t < NT && t >= t_lo && t <= t_hi) {
        float cp = e[t][0] * h[0];
        cp = __builtin_fmaf(e[t][1], h[1], cp);
        cp = __builtin_fmaf(e[t][2], h[2], cp);
        cp = __builtin_fmaf(e[t][3], h[3], cp);
        cp = cross_row_sum(cp);
        if (lg == 0) cb[(wave + t) * 16 + lr] = cp;
      }
    }
    if (g.dustbin) {
      float dp = 0.f;
      if (lr == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) dp = __builtin_fmaf(ed[r], h[r], dp);
      }
      dp = wave_sum(dp);
      if (lane == 0) misc[wave] = dp;
    }
  }
  __syncthreads();
  // (5) block sums of the column partials, fixed wave order
  float* po = p.part_out + ((size_t)bh * g.nblk + blk) * NWC;
  for (int c = tid; c < NWC; c += blockDim.x) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s += colbuf[w * NWC + c];
    po[c] = s;
  }
  if (g.dustbin && tid == 0) {
    float s = 0.f;
    for (int w = 0; w < kWaves; ++w) s += misc[w];
    p.partd_out[(size_t)bh * g.nblk + blk] = s;
  }
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
  const float* partd;   // [BH][nblk] dustbin-column partials of step t
  double* dstate;       // in: state after t-1 (ignored when first); out: after t
  const float* sdr;
  double* u_tail;       // optional: u^(t) slot
  double* v_tail;       // optional: v^(t) slot
  double* u_out;        // latest-u buffer (dustbin entry)
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
  const float* srow = p.sdr + bh * L;
  // x_j = S_delta,j + v_j (log2) over active j; the corner uses v_delta
  double m = -__builtin_inf();
  for (int j = tid; j <= n; j += blockDim.x) {
    const double vj = (j == n) ? vd_prev : (p.v_cur ? p.v_cur[bh * L + j] : 0.0);
    m = fmax(m, (double)srow[j] + vj);
  }
  redd[tid] = m;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) redd[tid] = fmax(redd[tid], redd[tid + s]);
    __syncthreads();
  }
  const double M = redd[0];
  float acc = 0.f;
  for (int j = tid; j <= n; j += blockDim.x) {
    const double vj = (j == n) ? vd_prev : (p.v_cur ? p.v_cur[bh * L + j] : 0.0);
    acc += exp2_fast((float)((double)srow[j] + vj - M));
  }
  red[tid] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  if (tid == 0) {
    const float rho = red[0];
    const float ad = p.a[(size_t)bb * L + n];
    const float bd = p.b[(size_t)bb * L + n];
    const double ud = log2((double)ad) - log2((double)rho) - M;
    const float hd = ad / rho;
    float gam = 0.f;
    for (int r = 0; r < g.nblk && r * kBlockRows < n; ++r) gam += p.partd[(size_t)bh * g.nblk + r];
    gam += exp2_fast((float)((double)srow[n] + vd_prev - M)) * hd;  // corner of P^(t,t-1)
    const double vd = vd_prev + log2((double)bd) - log2((double)gam);
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
    sh_vref = p.part_in ? finish_v(g, bh, n, r0, p.v_prev2, p.part_in, p.b, bb, p.dstate, p.sdr) : 0.0;
  __syncthreads();
  const double vref = sh_vref;

  float* w2s = reinterpret_cast<float*>(smem);                       // [NWC]
  char* vt = smem + (size_t)NWC * 4;                                 // [D][VTS] elements
  for (int c = tid; c < NWC; c += blockDim.x) {
    const int j = tw0 * 16 + c;
    float w = kNegInf;
    if (j >= 0 && j < n) {
      double vj = 0.0;
      if (p.part_in) vj = finish_v(g, bh, n, j, p.v_prev2, p.part_in, p.b, bb, p.dstate, p.sdr);
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

// Dustbin row of the output: O_delta = sum_j P_delta,j V_j over active j,
// plus u, v of the dustbin (state fp64 log2 units, outputs natural).
// One workgroup per (b, h); thread c owns column c of the head dimension.
template <typename T>
__global__ __launch_bounds__(256) void dustbin_output(Geom g, const T* V, const double* v2_real,
                                                      const double* dstate, const float* sdr,
                                                      float* O, float* u_out, float* v_out) {
  const int bh = blockIdx.x;
  const int n = real_len(g, bh / g.H);
  const size_t L = g.L;
  const int d = g.d;
  const double ud = dstate ? dstate[4 * bh + 0] : 0.0;
  const double vd = dstate ? dstate[4 * bh + 1] : 0.0;
  for (int c = threadIdx.x; c < d; c += blockDim.x) {
    float acc = 0.f;
    for (int j = 0; j <= n; ++j) {
      const double vj = (j == n) ? vd : v2_real[bh * L + j];
      const float pj = exp2_fast((float)((double)sdr[bh * L + j] + ud + vj));
      acc = __builtin_fmaf(pj, Elt<T>::load(V + ((size_t)bh * L + j) * d, c), acc);
    }
    O[((size_t)bh * L + n) * d + c] = acc;
  }
  if (threadIdx.x == 0) {
    const double ln2 = 0.6931471805599453;
    u_out[bh * L + n] = (float)(ud * ln2);
    v_out[bh * L + n] = (float)(vd * ln2);
  }
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
  const size_t iter_lds = (size_t)g.NWC * (RB + 16) + (size_t)g.NWC * 4 * (1 + kWaves) + 64;
  const size_t out_lds = (size_t)g.NWC * 4 + (size_t)D * (g.NWC + 8) * Elt<T>::kBytes + 64;
  hipError_t err;
  if (iter_lds > 150 * 1024 || out_lds > 150 * 1024) return hipErrorInvalidConfiguration;
  err = hipFuncSetAttribute(reinterpret_cast<const void*>(iter_kernel<T, D>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)iter_lds);
  if (err != hipSuccess) return err;
  err = hipFuncSetAttribute(reinterpret_cast<const void*>(output_kernel<T, D>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)out_lds);
  if (err != hipSuccess) return err;

  if (g.dustbin) {
    dim3 sg((g.L + 255) / 256, nbh);
    hipLaunchKernelGGL(dustbin_scores<T>, sg, dim3(256), 0, st, g, reinterpret_cast<const T*>(f.Q),
                       reinterpret_cast<const T*>(f.K), w.sdr, w.sdc);
  }
  const int N = f.T + f.R;
  if (f.T == 0) {
    dim3 zg((g.L + 255) / 256, nbh);
    hipLaunchKernelGGL(zero_start, zg, dim3(256), 0, st, g, w.tail_u, w.tail_v);
  }
  const size_t part_slot = (size_t)nbh * g.nblk * g.NWC;
  for (int t = 1; t <= N; ++t) {
    IterArgs a{};
    a.Q = f.Q;
    a.K = f.K;
    a.a = f.a;
    a.b = f.b;
    a.first = (t == 1);
    a.part_in = (t == 1) ? nullptr : w.part + (size_t)((t - 1) & 1) * part_slot;
    a.v_prev2 = (t <= 2) ? nullptr : w.vbuf + (size_t)((t - 2) & 1) * BHL;
    a.v_out = (t == 1) ? nullptr : w.vbuf + (size_t)((t - 1) & 1) * BHL;
    a.v_tail = (t >= 2 && t - 1 >= f.T) ? w.tail_v + (size_t)(t - 1 - f.T) * BHL : nullptr;
    a.u_out = w.ubuf;
    a.u_tail = (t >= f.T) ? w.tail_u + (size_t)(t - f.T) * BHL : nullptr;
    a.part_out = w.part + (size_t)(t & 1) * part_slot;
    a.partd_out = w.partd + (size_t)(t & 1) * nbh * g.nblk;
    a.dstate = (g.dustbin && t > 1) ? w.dstate : nullptr;
    a.sdr = w.sdr;
    a.sdc = w.sdc;
    a.padded_grid = grid;
    if (timing_enabled()) timing_mark(st, false);
    hipLaunchKernelGGL((iter_kernel<T, D>), dim3(grid), dim3(512), iter_lds, st, g, a);
    if (timing_enabled()) timing_mark(st, true);
    if (g.dustbin) {
      DustArgs da{};
      da.a = f.a;
      da.b = f.b;
      da.v_cur = (t == 1) ? nullptr : a.v_out;
      da.partd = a.partd_out;
      da.dstate = w.dstate;
      da.sdr = w.sdr;
      da.u_tail = a.u_tail;
      da.v_tail = (t >= f.T) ? w.tail_v + (size_t)(t - f.T) * BHL : nullptr;
      da.u_out = w.ubuf;
      da.first = (t == 1);
      hipLaunchKernelGGL(dustbin_step, dim3(nbh), dim3(256), 0, st, g, da);
    }
  }
  OutArgs o{};
  o.Q = f.Q;
  o.K = f.K;
  o.V = f.V;
  o.a = f.a;
  o.b = f.b;
  o.part_in = (N == 0) ? nullptr : w.part + (size_t)(N & 1) * part_slot;
  o.v_prev2 = (N <= 1) ? nullptr : w.vbuf + (size_t)((N - 1) & 1) * BHL;
  o.u_in = (N == 0) ? nullptr : w.ubuf;
  o.dstate = (g.dustbin && N >= 1) ? w.dstate : nullptr;
  o.sdr = w.sdr;
  o.sdc = w.sdc;
  o.O = f.O;
  o.u_out = f.u;
  o.v_out = f.v;
  o.v_tail = w.tail_v + (size_t)f.R * BHL;
  o.padded_grid = grid;
  hipLaunchKernelGGL((output_kernel<T, D>), dim3(grid), dim3(512), out_lds, st, g, o);
  if (g.dustbin) {
    hipLaunchKernelGGL(dustbin_output<T>, dim3(nbh), dim3(128), 0, st, g, reinterpret_cast<const T*>(f.V),
                       w.tail_v + (size_t)f.R * BHL, o.dstate, w.sdr, f.O, f.u, f.v);
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
