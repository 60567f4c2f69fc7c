"""Independent references used to pin the oracle (CPU only, float64).

None of these import the oracle: each is a second, differently organised
implementation of what the Blockwise Differentiable Sinkhorn Attention
summaries define (support and scores: section 2.1; the staircase adjoint and
the orbit identity: section 2.2; the dustbin as an enlarged state space:
section 2.3), or a textbook special case of it.
"""

from __future__ import annotations

import math

import numpy as np
from scipy.special import logsumexp


def support_mask(L, n, W, dustbin=False):
    """Dense boolean Omega written out pair by pair (no vectorised tricks)."""
    lo = W // 2
    hi = (W + 1) // 2 - 1
    m = np.zeros((L, L), dtype=bool)
    for i in range(n):
        for j in range(n):
            if -lo <= j - i <= hi:
                m[i, j] = True
    if dustbin:
        for t in range(n + 1):
            m[n, t] = True
            m[t, n] = True
    return m


def dense_sinkhorn(q, k, vv, a, b, mask, T, R, v_init=None):
    """Textbook log-domain Sinkhorn on the full L x L matrix (scipy logsumexp).

    Returns (us, vs, O) with us/vs lists of length R + 1 (the tail stack).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    d = q.shape[1]
    S = q @ k.T / math.sqrt(d)
    X = np.where(mask, S, -np.inf)
    act_r = mask.any(axis=1)
    act_c = mask.any(axis=0)
    with np.errstate(divide="ignore"):
        la = np.log(np.asarray(a, np.float64))
        lb = np.log(np.asarray(b, np.float64))
    L = S.shape[0]
    u = np.zeros(L)
    v = np.zeros(L) if v_init is None else np.array(v_init, np.float64)

    def rowstep(v):
        out = np.full(L, -np.inf)
        out[act_r] = la[act_r] - logsumexp(X[act_r] + v[None, :], axis=1)
        return out

    def colstep(u):
        out = np.full(L, -np.inf)
        out[act_c] = lb[act_c] - logsumexp(X[:, act_c] + u[:, None], axis=0)
        return out

    for _ in range(T):
        u = rowstep(v)
        v = colstep(u)
    us, vs = [u], [v]
    for _ in range(R):
        u = rowstep(vs[-1])
        v = colstep(u)
        us.append(u)
        vs.append(v)
    P = plan_dense(X, us[-1], vs[-1])
    O = P @ np.asarray(vv, np.float64)
    return us, vs, O


def plan_dense(X, u, v):
    """exp(X + u (+) v), zero where X = -inf or a potential is -inf."""
    Z = X + np.where(np.isfinite(u), u, -np.inf)[:, None] + \
        np.where(np.isfinite(v), v, -np.inf)[None, :]
    with np.errstate(invalid="ignore"):
        P = np.exp(Z)
    P[~np.isfinite(Z)] = 0.0
    return P


def brute_force(q, k, vv, a, b, L, n, W, T, R, dustbin=False):
    """Pure-Python loops over explicit index lists (only for L <= ~16)."""
    q = [[float(x) for x in row] for row in np.asarray(q, np.float64)]
    k = [[float(x) for x in row] for row in np.asarray(k, np.float64)]
    vv = [[float(x) for x in row] for row in np.asarray(vv, np.float64)]
    a = [float(x) for x in a]
    b = [float(x) for x in b]
    d = len(q[0])
    lo = W // 2
    hi = (W + 1) // 2 - 1
    pairs = set()
    for i in range(n):
        for j in range(max(0, i - lo), min(n - 1, i + hi) + 1):
            pairs.add((i, j))
    if dustbin:
        for t in range(n + 1):
            pairs.add((n, t))
            pairs.add((t, n))
    S = {}
    for (i, j) in pairs:
        S[(i, j)] = sum(q[i][c] * k[j][c] for c in range(d)) / math.sqrt(d)
    rows = {i: sorted(j for (ii, j) in pairs if ii == i) for i in range(L)}
    cols = {j: sorted(i for (i, jj) in pairs if jj == j) for j in range(L)}
    u = [0.0] * L
    v = [0.0] * L

    def lse(xs):
        m = max(xs)
        return m + math.log(sum(math.exp(x - m) for x in xs))

    us, vs = None, None
    for step in range(T + R):
        u = [math.log(a[i]) - lse([S[(i, j)] + v[j] for j in rows[i]]) if rows[i] else -math.inf
             for i in range(L)]
        v = [math.log(b[j]) - lse([S[(i, j)] + u[i] for i in cols[j]]) if cols[j] else -math.inf
             for j in range(L)]
    O = [[0.0] * d for _ in range(L)]
    for (i, j) in pairs:
        p = math.exp(S[(i, j)] + u[i] + v[j])
        for c in range(d):
            O[i][c] += p * vv[j][c]
    return np.array(u), np.array(v), np.array(O)


def torch_surrogate_grads(q, k, vv, a, b, mask, T, R, dO, detach_base=True):
    """Autograd of O through the unrolled iteration (torch, float64, CPU).

    detach_base=True: the T base steps run under no_grad (stop-gradient);
    False: gradient flows through all T + R steps (full BPTT).
    """
    import torch

    dt = torch.float64
    Q = torch.tensor(np.asarray(q, np.float64), dtype=dt, requires_grad=True)
    K = torch.tensor(np.asarray(k, np.float64), dtype=dt, requires_grad=True)
    Vt = torch.tensor(np.asarray(vv, np.float64), dtype=dt, requires_grad=True)
    M = torch.tensor(mask)
    act_r = M.any(dim=1)
    act_c = M.any(dim=0)
    la = torch.log(torch.tensor(np.asarray(a, np.float64), dtype=dt))
    lb = torch.log(torch.tensor(np.asarray(b, np.float64), dtype=dt))
    d = Q.shape[1]
    L = Q.shape[0]
    # a very negative finite fill keeps all-masked (filler) rows NaN-free
    ninf = torch.tensor(-1e200, dtype=dt)

    def scores():
        return torch.where(M, Q @ K.T / math.sqrt(d), ninf)

    def rowstep(X, v):
        z = torch.logsumexp(X + v[None, :], dim=1)
        return torch.where(act_r, la - torch.where(act_r, z, torch.zeros_like(z)),
                           torch.zeros_like(z))

    def colstep(X, u):
        z = torch.logsumexp(X + u[:, None], dim=0)
        return torch.where(act_c, lb - torch.where(act_c, z, torch.zeros_like(z)),
                           torch.zeros_like(z))

    u = torch.zeros(L, dtype=dt)
    v = torch.zeros(L, dtype=dt)
    if detach_base:
        with torch.no_grad():
            X0 = scores()
            for _ in range(T):
                u = rowstep(X0, v)
                v = colstep(X0, u)
        u, v = u.detach(), v.detach()
        X = scores()
        for _ in range(R):
            u = rowstep(X, v)
            v = colstep(X, u)
    else:
        X = scores()
        for _ in range(T + R):
            u = rowstep(X, v)
            v = colstep(X, u)
    P = torch.where(M, torch.exp(X + u[:, None] + v[None, :]), torch.zeros((), dtype=dt))
    O = P @ Vt
    O.backward(torch.tensor(np.asarray(dO, np.float64), dtype=dt))
    return (Q.grad.numpy(), K.grad.numpy(), Vt.grad.numpy(), O.detach().numpy())


def modifier_adjoint(q, k, vv, a, b, mask, us, vs, dO):
    """Tail adjoint from the single reference plan P = P^(R,R) (section 2.2).

    Every other staircase plan is P (.) alpha^(r) beta^(s)^T with
    alpha^(r) = exp(u^(r) - u^(R)), beta^(s) = exp(v^(s) - v^(R)).  Dense
    matrices; independent of the oracle's explicit-plan recursion.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    vv = np.asarray(vv, np.float64)
    dO = np.asarray(dO, np.float64)
    d = q.shape[1]
    R = len(us) - 1
    act_r = mask.any(axis=1)
    act_c = mask.any(axis=0)
    S = q @ k.T / math.sqrt(d)
    X = np.where(mask, S, -np.inf)
    P = plan_dense(X, us[R], vs[R])
    uz = [np.where(act_r, x, 0.0) for x in us]
    vz = [np.where(act_c, x, 0.0) for x in vs]
    alpha = [np.where(act_r, np.exp(uz[r] - uz[R]), 0.0) for r in range(R + 1)]
    beta = [np.where(act_c, np.exp(vz[s] - vz[R]), 0.0) for s in range(R + 1)]
    asafe = np.where(act_r, a, 1.0)
    bsafe = np.where(act_c, b, 1.0)
    dP = dO @ vv.T
    dV = P.T @ dO
    D = np.sum(dO * (P @ vv), axis=1)
    E = np.sum(vv * dV, axis=1)
    xs = [None] * (R + 1)
    ys = [None] * (R + 1)
    vbar = E
    for r in range(R, 0, -1):
        ys[r] = np.where(act_c, vbar / bsafe, 0.0)
        base = D if r == R else 0.0
        ubar = base - alpha[r] * (P @ (beta[r] * ys[r]))
        xs[r] = np.where(act_r, ubar / asafe, 0.0)
        vbar = -beta[r - 1] * (P.T @ (alpha[r] * xs[r]))
    corr = np.zeros_like(P)
    for r in range(1, R + 1):
        corr += np.outer(alpha[r], beta[r] * ys[r]) + np.outer(alpha[r] * xs[r], beta[r - 1])
    dS = P * (dP - corr)
    dQ = dS @ k / math.sqrt(d)
    dK = dS.T @ q / math.sqrt(d)
    return dQ, dK, dV, vbar
