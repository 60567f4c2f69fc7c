/*
 * sinkattn.h -- banded, balanced, log-domain Sinkhorn attention on AMD
 * Instinct MI355X (gfx950): forward (stopped base + differentiable tail +
 * output) and the exact tail adjoint.
 *
 * The operation follows the summaries of "Blockwise Differentiable Sinkhorn
 * Attention" (arXiv 2605.08123):
 *   - section 2.1 (forward pass): attention weights are the entropic
 *     transport plan on a fixed banded support Omega of width W, with the
 *     temperature absorbed into S = Q K^T / sqrt(d); T balanced Sinkhorn
 *     steps run under a stop-gradient (the "stopped base"), then R more steps
 *     form the differentiable tail; the output is O = P V with
 *     P = exp(S + u^(R) (+) v^(R)) on Omega.
 *   - section 2.2 (R = 2 staircase, single reference tile): the backward pass
 *     is the exact adjoint of the R tail steps; every staircase plan
 *     P^(a,b) is rebuilt from the reference plan P^(R,R) through the vector
 *     modifiers exp(u^(a) - u^(R)) and exp(v^(b) - v^(R)), so only O(L)
 *     extra device memory is used and no L x L or L x W matrix is ever stored.
 *   - section 2.3 (gap-aware dustbin bridge): a learned dustbin token and
 *     inactive filler tokens are appended to Q/K/V; the dustbin row and column
 *     are fully active and the same solver runs on the enlarged state space.
 *
 * Conventions (readings where the summaries leave a step open):
 *   - Band: offsets j - i in [-floor(W/2), ceil(W/2) - 1], clipped at the
 *     ends of the real tokens (W = 17 is |i - j| <= 8).
 *   - One step = one row update u_i = log a_i - LSE_{j in Omega_i}(S_ij + v_j)
 *     followed by one column update v_j = log b_j - LSE_{i}(S_ij + u_i);
 *     the iteration starts from u = v = 0 and runs exactly T + R steps.
 *   - Potentials are natural-log, returned raw (no gauge centring).
 *   - O = P^(R,R) V (raw plan entries, no row renormalisation).
 *   - Token layout per sequence b: real tokens [0, n_b), then the dustbin at
 *     index n_b when enabled, then inactive filler up to L.  Filler has zero
 *     mass and is outside Omega: its u and v are -inf and its rows of O, dQ,
 *     dK and dV are zero.
 *
 * Memory: every pointer is a DEVICE pointer owned by the caller.  The library
 * allocates nothing and keeps no state between calls; calls on different
 * streams with different workspaces may run concurrently.  All calls are
 * stream-ordered and asynchronous; argument validation happens on the host
 * before anything is enqueued.
 */
#ifndef SINKATTN_H
#define SINKATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  Every entry point returns one of these; no exceptions
 * cross the ABI. */
typedef enum {
  SINKATTN_OK = 0,
  SINKATTN_EINVAL = -1,        /* a bad argument (NULL pointer, size, W<1, ...) */
  SINKATTN_EUNSUPPORTED = -2,  /* valid but outside the built kernels' envelope */
  SINKATTN_EHIP = -3,          /* a HIP launch or runtime call failed */
  SINKATTN_EWORKSPACE = -4,    /* workspace smaller than sinkattn_workspace_bytes */
  SINKATTN_ENONFINITE = -5,    /* debug check: a non-finite potential on an active token */
  SINKATTN_ESTALL = -6,        /* a neighbour wait of the persistent step launch gave up */
  SINKATTN_ESCRATCH = -7       /* sinkattn_forward_noalloc: the call needs more than its static scratch */
} sinkattn_status;

/* Debug checks.  With the environment variable SINKATTN_DEBUG set (to
 * anything but "" or "0"; read at every call), sinkattn_forward and
 * sinkattn_forward_converge wait for their stream after enqueueing and check
 * the results: SINKATTN_ESTALL when a neighbour wait of the persistent step
 * launch gave up (the bounded spin of one workgroup waiting for another ran
 * out: not expected, since the launch is cooperative; the outputs are then
 * invalid), else SINKATTN_ENONFINITE when the stopped base u^(0), v^(0) or the
 * returned u, v hold a non-finite value on an active token.  The outputs are
 * written either way.  Without the debug checks a wait that gave up is
 * visible only in the outputs: O[0] and u[0] are set to NaN. */

/* Element type of Q, K, V and dO.  All outputs and potentials are fp32. */
typedef enum { SINKATTN_F32 = 0, SINKATTN_BF16 = 1 } sinkattn_dtype;

/* Problem shape.
 *   B, H, L, d : batch, heads, padded sequence length, head dimension.
 *                Q, K, V, dO, O, dQ, dK, dV are [B, H, L, d], d fastest,
 *                contiguous, 16-byte aligned.
 *   dtype      : sinkattn_dtype of Q, K, V and dO.
 *   lengths    : DEVICE int32[B] real-token counts n_b, or NULL (n_b = L).
 *                Values are clamped to [0, L] (to [0, L-1] with a dustbin).
 *   dustbin    : nonzero => token n_b of sequence b is the dustbin; its row
 *                and column are active against every active token (corner
 *                included).  Requires n_b < L.
 * Supported envelope of this build: d in {16, 32, 64} for fp32 and
 * {32, 64, 128} for bf16; band tile count ceil(h1 / 16) + ceil(h2 / 16) + 1
 * <= 17 with h1 = min(floor(W/2), L-1) and h2 = min(ceil(W/2) - 1, L-1):
 * every W <= 257, and any W (the dense case W >= 2L - 1 included) when
 * L <= 129; sizes B H <= 65535, B H L <= 2^31 - 1, B H L d <= 4 (2^31 - 1)
 * and one (b, h) slice of Q under 2 GiB (L d bytes-per-element <= 2^31 - 1).
 * Anything else returns SINKATTN_EUNSUPPORTED. */
typedef struct {
  int32_t B, H, L, d;
  int32_t dtype;
  const int32_t *lengths;
  int32_t dustbin;
} sinkattn_shape;

/* Bytes of device workspace a forward/backward pair needs for (s, W, R).
 * Layout: [tail stack: u^(0..R) then v^(0..R), each fp64 [B, H, L]]
 *         [scratch: O(B*H*L) vectors and band-column partial sums].
 * The size is O(B * H * L * (R + W/128)): no L x W or L x L buffer.
 * Returns 0 for an invalid shape. */
size_t sinkattn_workspace_bytes(const sinkattn_shape *s, int W, int R);

/* Byte offset, inside the workspace, of the fp64 [B, H, L] tail-stack slot
 * u^(r) (is_v = 0) or v^(r) (is_v = 1), r in [0, R].  u^(0), v^(0) is the
 * stopped base.  Slots hold the potentials in log2 units (natural value
 * times log2(e)) on active tokens; filler entries are unspecified.
 * Returns (size_t)-1 for bad arguments. */
size_t sinkattn_tail_offset(const sinkattn_shape *s, int R, int r, int is_v);

/* Forward pass (sections 2.1 and 2.3).
 *   Q, K, V     : [B, H, L, d] of s->dtype.
 *   W           : band width (>= 1).   T : stopped-base steps (>= 0).
 *   R           : differentiable tail steps (>= 0).
 *   a, b        : fp32 [B, L] row/column marginals, shared by all heads;
 *                 positive on active tokens, zero on filler, each summing to 1
 *                 (contents are the caller's responsibility).
 *   O           : out, fp32 [B, H, L, d].
 *   u, v        : out, fp32 [B, H, L] natural-log potentials u^(R), v^(R);
 *                 -inf on filler.
 *   workspace   : device buffer of workspace_bytes >=
 *                 sinkattn_workspace_bytes(s, W, R).  On return (stream order)
 *                 it holds the tail stack the backward pass needs; keep it
 *                 unchanged until sinkattn_backward has run.
 *   stream      : HIP stream (NULL = default stream).
 * Returns SINKATTN_OK or an error before enqueueing anything. */
int sinkattn_forward(const void *Q, const void *K, const void *V, int W, int T, int R,
                     const float *a, const float *b, const sinkattn_shape *s,
                     float *O, float *u, float *v, void *workspace,
                     size_t workspace_bytes, hipStream_t stream);

/* Forward pass that allocates nothing, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Arguments and outputs as sinkattn_forward, minus
 * the workspace: the library's own static device scratch of
 * SINKATTN_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU serves instead, so the
 * tail stack is not handed back (this is an inference entry point: pair
 * sinkattn_forward with sinkattn_backward for training).  The scratch is
 * resolved once per device with hipGetSymbolAddress and kept until the
 * process ends; every call on one GPU shares it, so calls that overlap in
 * time on the same GPU race (serialise them, e.g. on one stream).  Every
 * buffer the kernels rely on is cleared by the kernels themselves.
 * Returns SINKATTN_ESCRATCH (before enqueueing anything) when the shape, W
 * and R need more than the scratch, i.e. sinkattn_workspace_bytes(s, W, R) >
 * SINKATTN_NOALLOC_SCRATCH_BYTES (the long-context shape B=1, H=8, L=32768,
 * d=128, W=256 fits at R <= 4); otherwise as sinkattn_forward. */
#define SINKATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int sinkattn_forward_noalloc(const void *Q, const void *K, const void *V, int W, int T, int R,
                             const float *a, const float *b, const sinkattn_shape *s,
                             float *O, float *u, float *v, hipStream_t stream);

/* Forward pass whose stopped base ends early once converged (section 2.1:
 * the base runs until convergence or for a fixed number of steps).
 * Arguments as sinkattn_forward, with T_max (>= 0) the largest base length
 * and R >= 1.  The convergence measure after base step c is the L1 row-
 * marginal error of its plan,
 *   e_c = sum over active rows i of | sum_j P^(c,c)_ij - a_i |,
 * P^(c,c) = exp(S + u^(c) (+) v^(c)) on the support (its column sums are b
 * exactly), per (b, h) problem, evaluated in fp64 from the potentials.  It is
 * checked for c = check_every, 2 check_every, ... while c + 2 <= T_max; the
 * base ends at the first checked c where every (b, h) has e_c < tol (so all
 * problems of a call share one base length), otherwise after T_max steps.
 * The check of c rides on the row update of step c + 1, which is then the
 * first tail step, so a passing check costs no extra step.
 *   tol         : >= 0 (0 never stops early).  Values below about 1e-6 sit
 *                 under the resolution of fp32 entry sums.
 *   check_every : >= 1.
 *   T_used      : out (host int): the base length used (the T to pass to
 *                 sinkattn_backward; any T is accepted there).
 *   err_last    : out (host double, may be NULL): the largest per-(b, h)
 *                 e_c at the last check (NaN if a check was not finite;
 *                 untouched if no check ran).
 * Blocks the calling thread at each check (a device-to-host copy of B*H
 * doubles and a stream synchronisation).  Argument errors return before
 * anything is enqueued; a HIP error found at a check returns SINKATTN_EHIP
 * after the launches before it. */
int sinkattn_forward_converge(const void *Q, const void *K, const void *V, int W, int T_max,
                              int R, const float *a, const float *b, const sinkattn_shape *s,
                              double tol, int check_every, float *O, float *u, float *v,
                              void *workspace, size_t workspace_bytes, int *T_used,
                              double *err_last, hipStream_t stream);

/* Backward pass: exact adjoint of the R tail steps with the stopped base held
 * constant (section 2.2), evaluated with the single-reference-tile schedule.
 *   Q, K, V, W, T, R, a, b, s : exactly as passed to sinkattn_forward.
 *   O           : the forward output.   dO : [B, H, L, d] upstream gradient
 *                 of s->dtype.
 *   workspace   : the forward's workspace (its tail stack is read; its
 *                 scratch region is overwritten).
 *   dQ, dK, dV  : out, fp32 [B, H, L, d] (zero rows on filler).
 *   vbar0       : optional out (may be NULL), fp32 [B, H, L]: the adjoint
 *                 that reaches v^(0) and is dropped by the stop-gradient.
 * Returns SINKATTN_OK or an error before enqueueing anything. */
int sinkattn_backward(const void *Q, const void *K, const void *V, int W, int T, int R,
                      const float *a, const float *b, const sinkattn_shape *s,
                      const float *O, const void *dO, void *workspace,
                      size_t workspace_bytes, float *dQ, float *dK, float *dV,
                      float *vbar0, hipStream_t stream);

/* A-posteriori certificate of the stop-gradient bias, for choosing the tail
 * depth (section 2.4, third certificate; section 4.1).  The forward must have
 * run with tail depth R_max (the same W, T, shape; workspace carved for
 * R_max), i.e. N = T + R_max steps.  For R in [0, R_max], grad_R is the exact
 * gradient of that N-step forward with only its last R steps differentiable
 * (what sinkattn_backward returns for a forward with T' = N - R, R).
 *   eta[R] = ||grad_Rmax - grad_R||_F / ||grad_Rmax||_F over (dQ, dK) of the
 *            whole call (dV does not depend on R), fp64; eta[R_max] = 0.
 * With T = 0, grad_Rmax is the full gradient through every step and eta[R]
 * is the exact residual of stopping the gradient after R steps; otherwise it
 * is the residual against the deepest tail computed.  The smallest R with
 * eta[R] < tau is the depth the certificate selects for tolerance tau.
 *   dQ, dK, dV  : out, fp32 [B, H, L, d]: grad_Rmax (as sinkattn_backward).
 *   dQ_scratch, dK_scratch : device fp32 [B, H, L, d] scratch.
 *   eta         : out, host double[R_max + 1].
 *   tau         : tolerance (>= 0) of the depth selection.
 *   R_selected  : optional out (host int, may be NULL): the selected depth,
 *                 the smallest R with eta[R] < tau, or R_max when none is.
 *   R_max       : 1 .. 8.
 * Runs one backward pass of depth R_max and, for every shallower depth, the
 * dQ and dK sweeps over that pass's adjoint vectors (the last R tail steps'
 * vectors do not depend on where the stop-gradient sits), then blocks the
 * calling thread until the stream has finished them.  Argument errors return
 * before anything is enqueued. */
int sinkattn_tail_certificate(const void *Q, const void *K, const void *V, int W, int T,
                              int R_max, const float *a, const float *b,
                              const sinkattn_shape *s, const float *O, const void *dO,
                              void *workspace, size_t workspace_bytes, float *dQ, float *dK,
                              float *dV, float *dQ_scratch, float *dK_scratch, double *eta,
                              double tau, int *R_selected, hipStream_t stream);

/* Projective contraction diagnostic (section 2.4, second certificate): the
 * Hilbert projective diameter of every diagonal band block.  Blocks are
 * [s, s + block) x [s, s + block) over the real tokens of each sequence
 * (s = 0, block, 2 block, ...; the last one clipped to n_b; the dustbin is
 * not part of any block).  With block <= min(floor(W/2), ceil(W/2) - 1) + 1
 * every block lies inside the band, so its kernel exp(S) is strictly
 * positive and contracts Hilbert's projective metric by
 * kappa = tanh(Delta / 4) < 1 (Birkhoff-Hopf), where
 *   Delta = max over i, j, k, l in the block of S_ik + S_jl - S_jk - S_il
 * (S = q.k / sqrt(d), natural log units); one Sinkhorn step restricted to
 * the block contracts by at most kappa^2.
 *   block  : 1 .. 128 and inside the band as above, else SINKATTN_EINVAL.
 *   delta  : out, device fp32 [B, H, ceil(L / block)]: Delta per block
 *            (0 for blocks past n_b and for one-token blocks).
 *   kappa  : optional out (may be NULL), same shape: tanh(Delta / 4).
 * Stream-ordered; returns before anything is enqueued on bad arguments. */
int sinkattn_block_contraction(const void *Q, const void *K, int W, const sinkattn_shape *s,
                               int block, float *delta, float *kappa, hipStream_t stream);

/* Diagnostics for benchmarking: timing of the fused Sinkhorn step kernel,
 * which dominates the run time.  While enabled (on != 0), sinkattn_forward
 * records HIP events on the caller's stream around its step-kernel work: one
 * pair around the single persistent launch that runs all T + R steps, or
 * around the back-to-back run of T + R per-step launches, or (with a dustbin,
 * whose own kernel runs between steps) one pair per launch; sinkattn_forward_
 * converge records none.  sinkattn_timing_collect waits for the recorded
 * events, writes the summed bracketed time in milliseconds and the number of
 * Sinkhorn steps it covers since the previous collect (or enable), and resets
 * the counters.  Process-wide state, not thread-safe; events are created
 * lazily, reused while timing stays on, and destroyed by
 * sinkattn_timing_enable(0) (call it before the HIP runtime shuts down, so
 * that no library-owned HIP object outlives it).  Returns SINKATTN_OK,
 * SINKATTN_EINVAL (NULL outputs) or SINKATTN_EHIP. */
int sinkattn_timing_enable(int on);
int sinkattn_timing_collect(double *total_ms, long long *steps);

/* Measured peaks for roofline fractions.  Runs two probes on `stream`,
 * each one untimed short launch and one timed launch of about 10 ms that
 * fill every CU, and waits for them (blocking):
 *   mfma_bf16_flops : out, sustained flop/s of v_mfma_f32_16x16x32_bf16, the
 *                     bf16 score / P.V instruction (2 * 16 * 16 * 32 flops each);
 *   exp_per_s       : out, sustained v_exp_f32 results per second (the one
 *                     exp2 per band entry of every pass);
 *   clock_hz        : optional out (may be NULL), the shader clock during the
 *                     MFMA probe (s_memtime over s_memrealtime; 0 if unknown).
 * Allocates no device memory.  Returns SINKATTN_EINVAL on NULL required
 * outputs, SINKATTN_EHIP on a launch or event failure. */
int sinkattn_measure_peaks(double *mfma_bf16_flops, double *exp_per_s, double *clock_hz,
                           hipStream_t stream);

/* LDS service rate for the operand read pattern of the fused step kernel's
 * K tiles (a measurement behind its layout; no part of the method).  One
 * workgroup of eight waves per CU reads a ring of 32 tiles of 16 rows, each
 * wave 17 consecutive tiles per pass, lane (r, g) of a 128-bit read taking
 * the 16 bytes at 16 g + 64 c of row r (c = 0..3); rows are `row_stride`
 * bytes apart (256, 272, 288, 304 or 320), and with `swizzle` = 1 (only for
 * 256-byte rows) chunk p of row r is stored at chunk position
 * p ^ ((r ^ 2 r) & 15).  Runs an untimed short launch and a timed one on
 * `stream` and waits for them (blocking):
 *   cycles_per_read : out, shader cycles per wave-wide 128-bit read per CU
 *                     (1024 bytes; 4 when the LDS serves 256 bytes per clock
 *                     without bank conflicts).
 * Allocates no device memory.  Returns SINKATTN_EINVAL on a NULL output or
 * an unsupported stride / swizzle pair, SINKATTN_EHIP on a launch or copy
 * failure. */
int sinkattn_measure_lds(int row_stride, int swizzle, double *cycles_per_read, hipStream_t stream);

/* Human-readable text for a status code (static storage). */
const char *sinkattn_status_string(int status);

/* Name of the HIP error (hipGetErrorName) behind the calling thread's most
 * recent SINKATTN_EHIP status, "hipSuccess" if there was none (static
 * storage; not reset by later successful calls). */
const char *sinkattn_last_hip_error(void);

/* Library ABI version (major * 10000 + minor * 100 + patch). */
int sinkattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SINKATTN_H */
