"""Float64 CPU oracle for banded, balanced, log-domain Sinkhorn attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this module:
only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU baseline
leg call it.  It shares no code, tables or helpers with the HIP library.

What it computes (the "Blockwise Differentiable Sinkhorn Attention" summaries,
section 2.1 "forward pass", 2.2 "R=2 staircase and single reference tile",
2.3 "gap-aware dustbin bridge"; readings of open points are listed in the
design notes):

* Support Omega (section 2.1): a fixed band of width W over the real tokens,
  offsets j - i in [-floor(W/2), ceil(W/2) - 1], clipped at the sequence
  ends.  With a dustbin (section 2.3) one extra token at index n (right after
  the n real tokens) is active against every active token, its own corner
  included.  Filler tokens are outside Omega.
* Scores with the entropic temperature absorbed (section 2.1):
  S_ij = q_i . k_j / sqrt(d) on Omega.
* Balanced log-domain Sinkhorn half-steps (section 2.1):
  U(v)_i = log a_i - LSE_{j in Omega_i}(S_ij + v_j),
  V(u)_j = log b_j - LSE_{i in Omega^j}(S_ij + u_i),
  starting from u = v = 0, row update first in every step.
* Stopped base (section 2.1): T steps treated as constants -> (u0, v0).
* Differentiable tail (section 2.1): R further steps u^(r) = U(v^(r-1)),
  v^(r) = V(u^(r)), r = 1..R.
* Convergence-controlled base (section 2.1 allows running the base until
  convergence): the L1 row-marginal error of the plan after base step c,
  sum_i |sum_j P^(c,c)_ij - a_i|, checked every k steps; a batch stops at the
  first check where every problem is below the tolerance.
* Output: P = exp(S + u^(R) (+) v^(R)) on Omega, O = P V.
* Contraction diagnostic (section 2.4, second certificate): the Hilbert
  projective diameter Delta of each diagonal band block (strictly positive
  kernel), whose Birkhoff contraction coefficient is tanh(Delta / 4).
* Bias certificate (section 2.4, third certificate): for one forward of
  N = T + R_max steps, eta_R = ||g_Rmax - g_R|| / ||g_Rmax|| over (dQ, dK),
  g_R the gradient with only the last R steps differentiable; the selected
  depth is the smallest R with eta_R below the tolerance.
* Exact tail adjoint (section 2.2): reverse-mode through the R tail steps
  with the base held constant.  Every staircase plan P^(r,s) =
  exp(S + u^(r) (+) v^(s)) is built explicitly here (for R = 2 these are
  P^(2,2), P^(2,1), P^(1,1), P^(1,0)); the GPU path instead rebuilds them
  from the reference plan P^(R,R) with the orbit identity of section 2.2.

Data layout: per (batch, head) problem the support is held as COO pairs
sorted by row, plus a column-sorted permutation, so row and column
log-sum-exps are segment reductions.  The band of S is cached (the oracle has
no memory constraint).  Products with P or dS use scipy.sparse matrices.
"""

from __future__ import annotations

import math
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np
import scipy.sparse as sp

__all__ = [
    "band_offsets", "Support", "scores", "row_update", "col_update",
    "solve", "Solution", "output", "adjoint", "Grads",
    "forward_batch", "backward_batch", "bptt_batch", "forward_backward_batch",
    "row_marginal_error", "base_errors", "select_base_length", "converged_base_length",
    "tail_depth_gradients", "certificate_eta", "select_tail_depth", "certificate_batch",
    "block_diameters", "block_contraction_batch",
]


# ---------------------------------------------------------------------------
# Support Omega
# ---------------------------------------------------------------------------

def band_offsets(W: int):
    """Allowed offsets j - i of a centred band of full width W.

    Reading: W counts every offset in the band, split as evenly as possible,
    the extra one on the left when W is even: [-floor(W/2), ceil(W/2) - 1].
    W = 17 gives |i - j| <= 8; W = 256 gives [-128, 127].
    """
    if W < 1:
        raise ValueError("W must be >= 1")
    return W // 2, (W + 1) // 2 - 1


@dataclass
class Support:
    """Omega for one sequence: sorted COO plus row/column segment tables.

    L: padded length; n: real tokens; dustbin: whether index n is the dustbin.
    rows/cols: int64 arrays sorted by (row, col).
    col_order: permutation sorting the pairs by (col, row).
    active: bool [L].
    """

    L: int
    n: int
    W: int
    dustbin: bool
    rows: np.ndarray
    cols: np.ndarray
    col_order: np.ndarray
    active: np.ndarray

    @staticmethod
    def build(L: int, n: int, W: int, dustbin: bool = False) -> "Support":
        if not (0 <= n <= L):
            raise ValueError("need 0 <= n <= L")
        if dustbin and n >= L:
            raise ValueError("dustbin needs a free slot at index n < L")
        h1, h2 = band_offsets(W)
        # band among real tokens
        i = np.repeat(np.arange(n, dtype=np.int64), h1 + h2 + 1)
        off = np.tile(np.arange(-h1, h2 + 1, dtype=np.int64), n)
        j = i + off
        keep = (j >= 0) & (j < n)
        rows, cols = [i[keep]], [j[keep]]
        if dustbin:
            dlt = n
            real = np.arange(n, dtype=np.int64)
            # column of the dustbin for every real row
            rows.append(real)
            cols.append(np.full(n, dlt, dtype=np.int64))
            # full row of the dustbin, corner included
            rows.append(np.full(n + 1, dlt, dtype=np.int64))
            cols.append(np.arange(n + 1, dtype=np.int64))
        rows = np.concatenate(rows)
        cols = np.concatenate(cols)
        order = np.lexsort((cols, rows))
        rows, cols = rows[order], cols[order]
        col_order = np.lexsort((rows, cols))
        active = np.zeros(L, dtype=bool)
        active[:n] = True
        if dustbin:
            active[n] = True
        return Support(L, n, W, dustbin, rows, cols, col_order, active)

    @property
    def nnz(self) -> int:
        return int(self.rows.size)

    def _starts(self, keys: np.ndarray):
        """Start offsets of the runs of equal keys (keys already grouped)."""
        if keys.size == 0:
            return np.zeros(0, dtype=np.int64), np.zeros(0, dtype=np.int64)
        brk = np.flatnonzero(np.diff(keys)) + 1
        starts = np.concatenate(([0], brk)).astype(np.int64)
        return starts, keys[starts]

    def row_segments(self):
        return self._starts(self.rows)

    def col_segments(self):
        return self._starts(self.cols[self.col_order])


# ---------------------------------------------------------------------------
# Scores and half-steps
# ---------------------------------------------------------------------------

def scores(q: np.ndarray, k: np.ndarray, sup: Support, chunk: int = 1 << 18) -> np.ndarray:
    """S_ij = q_i . k_j / sqrt(d) for every (i, j) in Omega (float64)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    d = q.shape[1]
    out = np.empty(sup.nnz, dtype=np.float64)
    for s in range(0, sup.nnz, chunk):
        e = slice(s, min(s + chunk, sup.nnz))
        out[e] = np.einsum("ed,ed->e", q[sup.rows[e]], k[sup.cols[e]])
    return out / math.sqrt(d)


def _segment_lse(x: np.ndarray, starts: np.ndarray) -> np.ndarray:
    """log(sum(exp(x))) over consecutive segments, shifted by each max."""
    m = np.maximum.reduceat(x, starts)
    counts = np.diff(np.append(starts, x.size))
    s = np.add.reduceat(np.exp(x - np.repeat(m, counts)), starts)
    return m + np.log(s)


def _segment_sum(x: np.ndarray, starts: np.ndarray) -> np.ndarray:
    return np.add.reduceat(x, starts)


class _Problem:
    """Cached per-(b,h) state: support tables, scores, log-marginals."""

    def __init__(self, q, k, a, b, sup: Support):
        self.sup = sup
        self.S = scores(q, k, sup)
        self.a = np.asarray(a, dtype=np.float64)
        self.b = np.asarray(b, dtype=np.float64)
        self.rstart, self.rkey = sup.row_segments()
        self.cstart, self.ckey = sup.col_segments()
        self.S_col = self.S[sup.col_order]
        self.rows_col = sup.rows[sup.col_order]
        with np.errstate(divide="ignore"):
            self.log_a = np.log(self.a)
            self.log_b = np.log(self.b)

    def U(self, v: np.ndarray) -> np.ndarray:
        """Row half-step: u_i = log a_i - LSE_j(S_ij + v_j) on active rows."""
        u = np.full(self.sup.L, -np.inf)
        lse = _segment_lse(self.S + v[self.sup.cols], self.rstart)
        u[self.rkey] = self.log_a[self.rkey] - lse
        return u

    def V(self, u: np.ndarray) -> np.ndarray:
        """Column half-step: v_j = log b_j - LSE_i(S_ij + u_i) on active cols."""
        v = np.full(self.sup.L, -np.inf)
        lse = _segment_lse(self.S_col + u[self.rows_col], self.cstart)
        v[self.ckey] = self.log_b[self.ckey] - lse
        return v

    def plan(self, u: np.ndarray, v: np.ndarray) -> np.ndarray:
        """Entries exp(S_ij + u_i + v_j) on Omega, in row-sorted order."""
        return np.exp(self.S + u[self.sup.rows] + v[self.sup.cols])

    def csr(self, vals: np.ndarray) -> sp.csr_matrix:
        L = self.sup.L
        return sp.csr_matrix((vals, (self.sup.rows, self.sup.cols)), shape=(L, L))

    def row_sums(self, vals: np.ndarray) -> np.ndarray:
        out = np.zeros(self.sup.L)
        out[self.rkey] = _segment_sum(vals, self.rstart)
        return out

    def col_sums(self, vals: np.ndarray) -> np.ndarray:
        out = np.zeros(self.sup.L)
        out[self.ckey] = _segment_sum(vals[self.sup.col_order], self.cstart)
        return out


def row_update(q, k, a, b, sup, v):
    """One row half-step U(v) for a single problem (convenience wrapper)."""
    return _Problem(q, k, a, b, sup).U(np.asarray(v, dtype=np.float64))


def col_update(q, k, a, b, sup, u):
    """One column half-step V(u) for a single problem (convenience wrapper)."""
    return _Problem(q, k, a, b, sup).V(np.asarray(u, dtype=np.float64))


# ---------------------------------------------------------------------------
# Forward: stopped base + tail + output
# ---------------------------------------------------------------------------

@dataclass
class Solution:
    """Forward results of one problem.

    us[r], vs[r] for r = 0..R: u^(r), v^(r) (us[0], vs[0] = stopped base).
    O: [L, d] output; u, v: the returned potentials u^(R), v^(R).
    """

    us: List[np.ndarray]
    vs: List[np.ndarray]
    O: np.ndarray

    @property
    def u(self):
        return self.us[-1]

    @property
    def v(self):
        return self.vs[-1]


def _inactive_to_neg_inf(x: np.ndarray, active: np.ndarray) -> np.ndarray:
    x = x.copy()
    x[~active] = -np.inf
    return x


def solve(pb: _Problem, T: int, R: int, v_init: Optional[np.ndarray] = None):
    """Stopped base of T steps then R tail steps (section 2.1).

    Starting state: u = v = 0 (or v = v_init).  A step is one row half-step
    followed by one column half-step.  Returns the tail stack (u^(0..R),
    v^(0..R)); with T = 0 the base state is the starting state itself.
    """
    L = pb.sup.L
    u = np.zeros(L)
    v = np.zeros(L) if v_init is None else np.asarray(v_init, dtype=np.float64).copy()
    for _ in range(T):
        u = pb.U(v)
        v = pb.V(u)
    us, vs = [u], [v]
    for _ in range(R):
        u = pb.U(vs[-1])
        v = pb.V(u)
        us.append(u)
        vs.append(v)
    return us, vs


def output(pb: _Problem, u: np.ndarray, v: np.ndarray, V: np.ndarray) -> np.ndarray:
    """O = P V with P = exp(S + u (+) v) on Omega (zero rows off the support)."""
    P = pb.plan(u, v)
    return pb.csr(P) @ np.asarray(V, dtype=np.float64)


def forward_one(q, k, vv, a, b, sup: Support, T: int, R: int,
                v_init: Optional[np.ndarray] = None) -> Solution:
    pb = _Problem(q, k, a, b, sup)
    us, vs = solve(pb, T, R, v_init)
    O = output(pb, us[-1], vs[-1], vv)
    act = sup.active
    us = [_inactive_to_neg_inf(x, act) for x in us]
    vs = [_inactive_to_neg_inf(x, act) for x in vs]
    return Solution(us, vs, O)


# ---------------------------------------------------------------------------
# Convergence-controlled stopped base (section 2.1: the base is run until
# convergence or for a fixed number of steps)
# ---------------------------------------------------------------------------

def row_marginal_error(pb: _Problem, u: np.ndarray, v: np.ndarray) -> float:
    """L1 row-marginal error of the plan P = exp(S + u (+) v), built
    explicitly: sum over active rows i of |sum_j P_ij - a_i|."""
    act = pb.sup.active
    rs = pb.row_sums(pb.plan(u, v))
    return float(np.sum(np.abs(rs[act] - pb.a[act])))


def base_errors(pb: _Problem, T_max: int, every: int) -> dict:
    """Run the base from u = v = 0 for T_max steps and record, for every
    checked step c (c a multiple of `every` with c + 2 <= T_max), the error
    of the plan after step c: {c: row_marginal_error(u^(c), v^(c))}."""
    L = pb.sup.L
    u = np.zeros(L)
    v = np.zeros(L)
    errs = {}
    for c in range(1, T_max + 1):
        u = pb.U(v)
        v = pb.V(u)
        if c % every == 0 and c + 2 <= T_max:
            errs[c] = row_marginal_error(pb, u, v)
    return errs


def select_base_length(errs: Sequence[dict], T_max: int, tol: float) -> int:
    """Base length for a batch of problems: the first checked step at which
    every problem's error is below tol, else T_max."""
    checks = sorted(set().union(*[set(e) for e in errs])) if errs else []
    for c in checks:
        if all(c in e and e[c] < tol for e in errs):
            return c
    return T_max


def _job_base_errors(args):
    q, k, a, b, L, n, W, dustbin, T_max, every = args
    pb = _Problem(q, k, a, b, Support.build(L, n, W, dustbin))
    return base_errors(pb, T_max, every)


def converged_base_length(Q, K, a, b, W, T_max, tol, every, lengths=None, dustbin=False,
                          processes: Optional[int] = None):
    """(T_used, per-problem error dicts) of the convergence-controlled base
    over a [B, H, L, d] batch; the forward then runs with T = T_used."""
    B, H, L, d = Q.shape
    ns = _lengths_of(L, lengths, B)
    jobs = [(Q[bi, h], K[bi, h], a[bi], b[bi], L, ns[bi], W, dustbin, T_max, every)
            for bi in range(B) for h in range(H)]
    errs = _map(_job_base_errors, jobs, processes)
    return select_base_length(errs, T_max, tol), errs


# ---------------------------------------------------------------------------
# Backward: exact adjoint of the R-step tail (section 2.2)
# ---------------------------------------------------------------------------

@dataclass
class Grads:
    dQ: np.ndarray
    dK: np.ndarray
    dV: np.ndarray
    vbar0: np.ndarray  # adjoint reaching v^(0), discarded by the stop-gradient


def adjoint(pb: _Problem, us, vs, q, k, vv, dO) -> Grads:
    """Reverse-mode derivative of O = P^(R,R) V through the R tail steps.

    The base state (us[0], vs[0]) is a constant.  Tail step r computed
    u^(r) = U(v^(r-1)) with the row-normalised plan P^(r,r-1) and then
    v^(r) = V(u^(r)) with the column-normalised plan P^(r,r).  Differentiating
    log-sum-exp gives, with y = vbar/b and x = ubar/a:
      d v^(r)_j / d S_ij = -P^(r,r)_ij / b_j,   d v^(r)_j / d u^(r)_i = same,
      d u^(r)_i / d S_ij = -P^(r,r-1)_ij / a_i, d u^(r)_i / d v^(r-1)_j = same.
    The plans are built explicitly (exp of S plus the stored potentials).
    """
    R = len(us) - 1
    sup = pb.sup
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    vv = np.asarray(vv, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    d = q.shape[1]
    act = sup.active
    a_safe = np.where(act, pb.a, 1.0)
    b_safe = np.where(act, pb.b, 1.0)

    P = pb.plan(us[R], vs[R])
    Pm = pb.csr(P)
    # dL/dP_ij = dO_i . V_j on Omega
    dP = np.empty(sup.nnz)
    ch = 1 << 18
    for s in range(0, sup.nnz, ch):
        e = slice(s, min(s + ch, sup.nnz))
        dP[e] = np.einsum("ed,ed->e", dO[sup.rows[e]], vv[sup.cols[e]])
    dV = Pm.T @ dO
    dS = P * dP
    ubar = pb.row_sums(P * dP)   # direct dependence of O on u^(R): D_i = dO_i . O_i
    vbar = pb.col_sums(P * dP)   # direct dependence on v^(R): E_j = V_j . dV_j
    for r in range(R, 0, -1):
        # column half-step v^(r) = V(u^(r)) with plan P^(r,r)
        y = np.where(act, vbar / b_safe, 0.0)
        Prr = pb.plan(us[r], vs[r])
        cy = Prr * y[sup.cols]
        dS -= cy
        ubar = ubar - pb.row_sums(cy)
        # row half-step u^(r) = U(v^(r-1)) with plan P^(r,r-1)
        x = np.where(act, ubar / a_safe, 0.0)
        Prs = pb.plan(us[r], vs[r - 1])
        cx = Prs * x[sup.rows]
        dS -= cx
        vbar = -pb.col_sums(cx)
        ubar = np.zeros(sup.L)
    dSm = pb.csr(dS)
    dQ = (dSm @ k) / math.sqrt(d)
    dK = (dSm.T @ q) / math.sqrt(d)
    return Grads(np.asarray(dQ), np.asarray(dK), np.asarray(dV), vbar)


def backward_one(q, k, vv, a, b, sup: Support, T: int, R: int, dO,
                 sol: Optional[Solution] = None) -> Grads:
    pb = _Problem(q, k, a, b, sup)
    if sol is None:
        us, vs = solve(pb, T, R)
    else:
        us = [np.where(sup.active, x, 0.0) for x in sol.us]
        vs = [np.where(sup.active, x, 0.0) for x in sol.vs]
    return adjoint(pb, us, vs, q, k, vv, dO)


def bptt_one(q, k, vv, a, b, sup: Support, T: int, R: int, dO) -> Grads:
    """Gradient through every one of the T + R steps (no stop-gradient).

    Same forward value; all steps are treated as tail from the zero start.
    """
    return backward_one(q, k, vv, a, b, sup, 0, T + R, dO)


# ---------------------------------------------------------------------------
# Batched wrappers over [B, H, L, d]
# ---------------------------------------------------------------------------

def _supports(L, lengths, W, dustbin, B):
    out = []
    for bi in range(B):
        n = L if lengths is None else int(lengths[bi])
        out.append(Support.build(L, n, W, dustbin))
    return out


def _job_forward(args):
    q, k, vv, a, b, L, n, W, dustbin, T, R = args
    sup = Support.build(L, n, W, dustbin)
    return forward_one(q, k, vv, a, b, sup, T, R)


def _job_backward(args):
    q, k, vv, a, b, L, n, W, dustbin, T, R, dO, mode = args
    sup = Support.build(L, n, W, dustbin)
    if mode == "bptt":
        return bptt_one(q, k, vv, a, b, sup, T, R, dO)
    return backward_one(q, k, vv, a, b, sup, T, R, dO)


def _map(fn, jobs, processes):
    if processes is None or processes <= 1 or len(jobs) <= 1:
        return [fn(j) for j in jobs]
    import multiprocessing as mp
    ctx = mp.get_context("fork")
    with ctx.Pool(min(processes, len(jobs))) as pool:
        return pool.map(fn, jobs)


def _lengths_of(L, lengths, B):
    return [L if lengths is None else int(lengths[bi]) for bi in range(B)]


def forward_batch(Q, K, V, a, b, W, T, R, lengths=None, dustbin=False,
                  processes: Optional[int] = None):
    """Batched forward.  Returns dict with O [B,H,L,d], u, v [B,H,L] and the
    tail stacks us, vs [R+1, B, H, L] (float64; -inf on inactive tokens)."""
    B, H, L, d = Q.shape
    ns = _lengths_of(L, lengths, B)
    jobs = [(Q[bi, h], K[bi, h], V[bi, h], a[bi], b[bi], L, ns[bi], W, dustbin, T, R)
            for bi in range(B) for h in range(H)]
    sols = _map(_job_forward, jobs, processes)
    O = np.stack([s.O for s in sols]).reshape(B, H, L, d)
    us = np.stack([np.stack(s.us) for s in sols], axis=1).reshape(R + 1, B, H, L)
    vs = np.stack([np.stack(s.vs) for s in sols], axis=1).reshape(R + 1, B, H, L)
    return {"O": O, "u": us[-1], "v": vs[-1], "us": us, "vs": vs}


def backward_batch(Q, K, V, a, b, W, T, R, dO, lengths=None, dustbin=False,
                   processes: Optional[int] = None, mode: str = "tail"):
    """Batched exact tail adjoint (mode="tail") or full BPTT (mode="bptt").
    Returns dict with dQ, dK, dV [B,H,L,d] and vbar0 [B,H,L]."""
    B, H, L, d = Q.shape
    ns = _lengths_of(L, lengths, B)
    jobs = [(Q[bi, h], K[bi, h], V[bi, h], a[bi], b[bi], L, ns[bi], W, dustbin, T, R,
             dO[bi, h], mode) for bi in range(B) for h in range(H)]
    gs = _map(_job_backward, jobs, processes)
    shp = (B, H, L, d)
    return {"dQ": np.stack([g.dQ for g in gs]).reshape(shp),
            "dK": np.stack([g.dK for g in gs]).reshape(shp),
            "dV": np.stack([g.dV for g in gs]).reshape(shp),
            "vbar0": np.stack([g.vbar0 for g in gs]).reshape(B, H, L)}


def _job_both(args):
    q, k, vv, a, b, L, n, W, dustbin, T, R, dO = args
    sup = Support.build(L, n, W, dustbin)
    sol = forward_one(q, k, vv, a, b, sup, T, R)
    return sol, backward_one(q, k, vv, a, b, sup, T, R, dO, sol=sol)


def forward_backward_batch(Q, K, V, a, b, W, T, R, dO, lengths=None, dustbin=False,
                           processes: Optional[int] = None):
    """forward_batch and backward_batch in one pass (the backward reuses the
    forward's tail stack instead of re-running the iteration)."""
    B, H, L, d = Q.shape
    ns = _lengths_of(L, lengths, B)
    jobs = [(Q[bi, h], K[bi, h], V[bi, h], a[bi], b[bi], L, ns[bi], W, dustbin, T, R, dO[bi, h])
            for bi in range(B) for h in range(H)]
    res = _map(_job_both, jobs, processes)
    sols = [r[0] for r in res]
    gs = [r[1] for r in res]
    shp = (B, H, L, d)
    us = np.stack([np.stack(s.us) for s in sols], axis=1).reshape(R + 1, B, H, L)
    vs = np.stack([np.stack(s.vs) for s in sols], axis=1).reshape(R + 1, B, H, L)
    return {"O": np.stack([s.O for s in sols]).reshape(shp), "u": us[-1], "v": vs[-1],
            "us": us, "vs": vs,
            "dQ": np.stack([g.dQ for g in gs]).reshape(shp),
            "dK": np.stack([g.dK for g in gs]).reshape(shp),
            "dV": np.stack([g.dV for g in gs]).reshape(shp),
            "vbar0": np.stack([g.vbar0 for g in gs]).reshape(B, H, L)}


# ---------------------------------------------------------------------------
# A-posteriori certificate of the stop-gradient bias (section 2.4, third
# certificate; section 4.1: it picks the smallest tail depth within a tolerance)
# ---------------------------------------------------------------------------

def tail_depth_gradients(q, k, vv, a, b, sup: Support, T: int, R_max: int, dO) -> List[Grads]:
    """grads[R], R = 0..R_max: the exact gradient of one and the same forward
    of N = T + R_max steps when only its last R steps are differentiable (the
    stop-gradient moved to step N - R)."""
    N = T + R_max
    return [backward_one(q, k, vv, a, b, sup, N - R, R, dO) for R in range(R_max + 1)]


def certificate_eta(grads: Sequence[Sequence[Grads]]) -> List[float]:
    """eta[R] = ||g_Rmax - g_R|| / ||g_Rmax|| over (dQ, dK) of a whole batch;
    grads[p][R] are the depth-R gradients of problem p."""
    R_max = len(grads[0]) - 1
    den = sum(float(np.sum(g[R_max].dQ ** 2) + np.sum(g[R_max].dK ** 2)) for g in grads)
    eta = []
    for R in range(R_max + 1):
        num = sum(float(np.sum((g[R].dQ - g[R_max].dQ) ** 2) + np.sum((g[R].dK - g[R_max].dK) ** 2))
                  for g in grads)
        eta.append(math.sqrt(num / den) if den > 0 else (math.inf if num > 0 else 0.0))
    return eta


def select_tail_depth(eta: Sequence[float], tau: float) -> int:
    """The smallest depth R with eta[R] < tau (the deepest when none is)."""
    for R, e in enumerate(eta):
        if e < tau:
            return R
    return len(eta) - 1


def _job_depths(args):
    q, k, vv, a, b, L, n, W, dustbin, T, R_max, dO = args
    return tail_depth_gradients(q, k, vv, a, b, Support.build(L, n, W, dustbin), T, R_max, dO)


def certificate_batch(Q, K, V, a, b, W, T, R_max, dO, lengths=None, dustbin=False,
                      processes: Optional[int] = None):
    """(eta, gradients at depth R_max as a dict of [B, H, L, d] arrays)."""
    B, H, L, d = Q.shape
    ns = _lengths_of(L, lengths, B)
    jobs = [(Q[bi, h], K[bi, h], V[bi, h], a[bi], b[bi], L, ns[bi], W, dustbin, T, R_max, dO[bi, h])
            for bi in range(B) for h in range(H)]
    gs = _map(_job_depths, jobs, processes)
    shp = (B, H, L, d)
    ref = {"dQ": np.stack([g[R_max].dQ for g in gs]).reshape(shp),
           "dK": np.stack([g[R_max].dK for g in gs]).reshape(shp),
           "dV": np.stack([g[R_max].dV for g in gs]).reshape(shp)}
    return certificate_eta(gs), ref


# ---------------------------------------------------------------------------
# Projective contraction diagnostic (section 2.4, second certificate: Hilbert's
# projective metric shows that strictly positive active blocks contract)
# ---------------------------------------------------------------------------

def block_diameters(q, k, L: int, n: int, W: int, block: int) -> np.ndarray:
    """Hilbert projective diameter of each diagonal block [s, s + block) of the
    n real tokens (s = 0, block, ...; the last clipped to n; 0 past n):
    Delta = max over i, j, k, l of S_ik + S_jl - S_jk - S_il, the largest log
    cross-ratio of the block's kernel exp(S).  The block must lie inside the
    band (block <= min(h1, h2) + 1), where that kernel is strictly positive;
    its Birkhoff contraction coefficient is tanh(Delta / 4)."""
    h1, h2 = band_offsets(W)
    if not 1 <= block <= min(h1, h2) + 1:
        raise ValueError("block must lie inside the band")
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    d = q.shape[1]
    out = np.zeros((L + block - 1) // block)
    for blk, s in enumerate(range(0, L, block)):
        if s >= n:
            continue
        e = min(s + block, n)
        S = q[s:e] @ k[s:e].T / math.sqrt(d)
        diff = S[:, None, :] - S[None, :, :]  # [i, j, k]: S_ik - S_jk
        M = diff.max(axis=2)                   # max over k
        out[blk] = float((M + M.T).max())      # + max over l of S_jl - S_il
    return out


def block_contraction_batch(Q, K, W, block, lengths=None):
    """block_diameters for every (b, h): [B, H, ceil(L / block)]."""
    B, H, L, d = Q.shape
    ns = _lengths_of(L, lengths, B)
    return np.stack([np.stack([block_diameters(Q[bi, h], K[bi, h], L, ns[bi], W, block)
                               for h in range(H)]) for bi in range(B)])


def bptt_batch(Q, K, V, a, b, W, T, R, dO, lengths=None, dustbin=False,
               processes: Optional[int] = None):
    return backward_batch(Q, K, V, a, b, W, T, R, dO, lengths, dustbin, processes,
                          mode="bptt")


def default_processes() -> int:
    return max(1, os.cpu_count() or 1)
