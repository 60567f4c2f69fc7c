"""Pins of the float64 oracle against things other than itself (CPU only).

Each test names the fact it checks; together they are chosen so that a
plausible slip in the oracle (a dropped term, a wrong sign or index, a
transposed operand, the wrong update order, a mis-sized band, a missing
dustbin corner) fails at least one of them -- test_mutations plants such slips
and checks exactly that.
"""

import math

import numpy as np
import pytest

import oracle
import workloads
from tests import refs

RTOL_EXACT = 1e-11


def _one(prob, bi=0, h=0):
    return (prob.Q[bi, h], prob.K[bi, h], prob.V[bi, h], prob.a[bi], prob.b[bi])


def _rel(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(x)), "finite pattern differs"
    den = np.linalg.norm(ref[fin])
    return np.linalg.norm(x[fin] - ref[fin]) / (den if den > 0 else 1.0)


# --- support -----------------------------------------------------------------

@pytest.mark.parametrize("L,n,W,dust", [(16, 16, 1, False), (16, 16, 2, False),
                                         (16, 13, 5, False), (20, 12, 8, True),
                                         (9, 9, 17, False), (12, 7, 64, True)])
def test_support_matches_pairwise_definition(L, n, W, dust):
    """Omega from the vectorised builder equals the pair-by-pair definition."""
    sup = oracle.Support.build(L, n, W, dust)
    m = np.zeros((L, L), dtype=bool)
    m[sup.rows, sup.cols] = True
    assert sup.nnz == m.sum(), "duplicate pairs"
    np.testing.assert_array_equal(m, refs.support_mask(L, n, W, dust))


def test_band_offsets_readings():
    """W = 17 is |i-j| <= 8 (tiny config); even W puts the extra offset left."""
    assert oracle.band_offsets(17) == (8, 8)
    assert oracle.band_offsets(256) == (128, 127)
    assert oracle.band_offsets(128) == (64, 63)
    assert oracle.band_offsets(1) == (0, 0)


# --- P1 closed form ------------------------------------------------------------

@pytest.mark.parametrize("T,R", [(1, 0), (3, 2), (0, 1), (5, 4)])
def test_closed_form_equal_queries(T, R):
    """Full support and q_i all equal => S_ij = g_j, one step gives P = a b^T,
    hence O_i = a_i sum_j b_j V_j (non-uniform marginals)."""
    rng = np.random.default_rng(3)
    L, d = 10, 4
    q = np.tile(rng.standard_normal(d), (L, 1))
    k = rng.standard_normal((L, d)) * 2
    vv = rng.standard_normal((L, d))
    a = rng.random(L) + 0.1
    a /= a.sum()
    b = rng.random(L) + 0.1
    b /= b.sum()
    sup = oracle.Support.build(L, L, 2 * L - 1)
    sol = oracle.forward_one(q, k, vv, a, b, sup, T, R)
    expect = np.outer(a, b @ vv)
    np.testing.assert_allclose(sol.O, expect, rtol=1e-12, atol=1e-14)


# --- P2 / P3 marginals -----------------------------------------------------------

@pytest.mark.parametrize("cfg", ["tiny", "dustbin_small", "ragged"])
def test_marginal_invariants(cfg):
    """Column sums of P^(R,R) equal b exactly (a column update just ran);
    row sums of P^(R,R-1) equal a (the row update that produced u^(R))."""
    if cfg == "tiny":
        p = workloads.make(1)
        L, n, dust = p.L, p.L, False
    elif cfg == "dustbin_small":
        p = workloads.custom(B=1, H=1, L=40, d=8, W=9, T=6, R=2, lengths=[33],
                             dustbin=True, seed=5)
        L, n, dust = p.L, 33, True
    else:
        p = workloads.custom(B=1, H=1, L=48, d=8, W=12, T=4, R=3, lengths=[41],
                             seed=6, filler="random")
        L, n, dust = p.L, 41, False
    q, k, vv, a, b = _one(p)
    sup = oracle.Support.build(L, n, p.W, dust)
    sol = oracle.forward_one(q, k, vv, a, b, sup, p.T, p.R)
    mask = refs.support_mask(L, n, p.W, dust)
    X = np.where(mask, q.astype(np.float64) @ k.astype(np.float64).T / math.sqrt(p.d), -np.inf)
    P = refs.plan_dense(X, sol.us[-1], sol.vs[-1])
    np.testing.assert_allclose(P.sum(axis=0), b, rtol=1e-13, atol=1e-16)
    Prow = refs.plan_dense(X, sol.us[-1], sol.vs[-2])
    np.testing.assert_allclose(Prow.sum(axis=1), a, rtol=1e-13, atol=1e-16)
    if dust:
        assert abs(P.sum(axis=0)[n] - 0.1) < 1e-7  # dustbin column carries its mass


def test_converged_marginals_tiny():
    """Tiny config run to convergence (T = 5000): ||P 1 - a||_1 < 1e-12."""
    p = workloads.make(1)
    q, k, vv, a, b = _one(p)
    sup = oracle.Support.build(p.L, p.L, p.W)
    sol = oracle.forward_one(q, k, vv, a, b, sup, 5000, 2)
    mask = refs.support_mask(p.L, p.L, p.W)
    X = np.where(mask, q.astype(np.float64) @ k.astype(np.float64).T / 4.0, -np.inf)
    P = refs.plan_dense(X, sol.u, sol.v)
    assert np.abs(P.sum(axis=1) - a).sum() < 1e-12
    assert np.abs(P.sum(axis=0) - b).sum() < 1e-12


# --- P4 dense special case -------------------------------------------------------

@pytest.mark.parametrize("Wmul", ["2L-1", "4L"])
def test_wide_band_is_dense_sinkhorn(Wmul):
    """W >= 2L - 1 covers every pair: equals textbook dense Sinkhorn."""
    L = 24
    W = 2 * L - 1 if Wmul == "2L-1" else 4 * L
    p = workloads.custom(B=1, H=1, L=L, d=8, W=W, T=7, R=2, seed=11, scale=0.8)
    q, k, vv, a, b = _one(p)
    sup = oracle.Support.build(L, L, W)
    sol = oracle.forward_one(q, k, vv, a, b, sup, p.T, p.R)
    us, vs, O = refs.dense_sinkhorn(q, k, vv, a, b, np.ones((L, L), bool), p.T, p.R)
    assert _rel(sol.O, O) < RTOL_EXACT
    for r in range(p.R + 1):
        assert _rel(sol.us[r], us[r]) < RTOL_EXACT
        assert _rel(sol.vs[r], vs[r]) < RTOL_EXACT


def test_dustbin_full_support_is_dense_on_enlarged_space():
    """Dustbin + full band: dense Sinkhorn on the (n+1) active tokens with
    the dustbin carrying mass 0.1 (the enlarged state space of section 2.3)."""
    L, n = 20, 15
    p = workloads.custom(B=1, H=1, L=L, d=6, W=2 * L, T=9, R=2, lengths=[n],
                         dustbin=True, seed=12, scale=0.7)
    q, k, vv, a, b = _one(p)
    sup = oracle.Support.build(L, n, p.W, True)
    sol = oracle.forward_one(q, k, vv, a, b, sup, p.T, p.R)
    mask = np.zeros((L, L), bool)
    mask[: n + 1, : n + 1] = True
    us, vs, O = refs.dense_sinkhorn(q, k, vv, a, b, mask, p.T, p.R)
    assert _rel(sol.O, O) < RTOL_EXACT
    assert _rel(sol.u, us[-1]) < RTOL_EXACT
    assert _rel(sol.v, vs[-1]) < RTOL_EXACT


# --- P5 brute force -----------------------------------------------------------------

@pytest.mark.parametrize("L,n,W,T,R,dust", [
    (8, 8, 3, 4, 2, False), (10, 10, 2, 3, 1, False), (12, 9, 5, 5, 2, False),
    (12, 8, 4, 3, 2, True), (6, 6, 1, 2, 2, False), (11, 7, 64, 2, 3, True),
    (9, 0, 3, 2, 2, True)])
def test_brute_force_loops(L, n, W, T, R, dust):
    """Pure-Python loops over explicit index lists agree to 1e-12."""
    if n == 0 and dust:
        p = workloads.custom(B=1, H=1, L=L, d=3, W=W, T=T, R=R, lengths=[0],
                             dustbin=True, seed=L)
    else:
        p = workloads.custom(B=1, H=1, L=L, d=3, W=W, T=T, R=R,
                             lengths=None if n == L else [n], dustbin=dust, seed=L,
                             scale=1.3)
    q, k, vv, a, b = _one(p)
    sup = oracle.Support.build(L, n, W, dust)
    sol = oracle.forward_one(q, k, vv, a, b, sup, T, R)
    u, v, O = refs.brute_force(q, k, vv, a, b, L, n, W, T, R, dust)
    assert _rel(sol.u, u) < 1e-12
    assert _rel(sol.v, v) < 1e-12
    assert _rel(sol.O, O) < 1e-12


# --- P6 padding invariance, P7 gauge ---------------------------------------------------

def test_padding_invariance():
    """Active results do not depend on filler content or on padded length."""
    n, W, d = 30, 9, 5
    base = workloads.custom(B=1, H=1, L=n, d=d, W=W, T=6, R=2, seed=21)
    q, k, vv, a, b = _one(base)
    ref = oracle.forward_one(q, k, vv, a, b, oracle.Support.build(n, n, W), 6, 2)
    rng = np.random.default_rng(0)
    for L in (37, 64):
        pad = lambda x: np.concatenate([x, rng.standard_normal((L - n, d)).astype(np.float32)])
        a2 = np.concatenate([a, np.zeros(L - n, np.float32)])
        sol = oracle.forward_one(pad(q), pad(k), pad(vv), a2, a2.copy(),
                                 oracle.Support.build(L, n, W), 6, 2)
        np.testing.assert_allclose(sol.O[:n], ref.O, rtol=1e-14, atol=1e-15)
        assert np.all(sol.O[n:] == 0)
        np.testing.assert_allclose(sol.u[:n], ref.u, rtol=1e-14)
        assert np.all(np.isneginf(sol.u[n:])) and np.all(np.isneginf(sol.v[n:]))


def test_gauge_shift():
    """Starting from v = c instead of 0 shifts u by -c and v by +c; O is unchanged."""
    p = workloads.make(1)
    q, k, vv, a, b = _one(p)
    sup = oracle.Support.build(p.L, p.L, p.W)
    pb = oracle.Problem(q, k, a, b, sup)
    us0, vs0 = oracle.solve(pb, 5, 2)
    c = 3.25
    us1, vs1 = oracle.solve(pb, 5, 2, v_init=np.full(p.L, c))
    np.testing.assert_allclose(us1[-1], us0[-1] - c, rtol=1e-13, atol=1e-12)
    np.testing.assert_allclose(vs1[-1], vs0[-1] + c, rtol=1e-13, atol=1e-12)
    O0 = oracle.output(pb, us0[-1], vs0[-1], vv)
    O1 = oracle.output(pb, us1[-1], vs1[-1], vv)
    np.testing.assert_allclose(O1, O0, rtol=1e-12, atol=1e-14)


# --- gradients ---------------------------------------------------------------------------

def _small_problem(seed=0, L=14, n=None, W=5, d=4, T=4, R=2, dust=False, scale=0.9):
    p = workloads.custom(B=1, H=1, L=L, d=d, W=W, T=T, R=R,
                         lengths=None if n is None else [n], dustbin=dust, seed=seed,
                         scale=scale)
    n = L if n is None else n
    return p, n


def _tail_objective(q, k, vv, a, b, sup, v0, R, dO, u0=None):
    """<dO, O> of the surrogate with the base state frozen at (u0, v0)."""
    pb = oracle.Problem(q, k, a, b, sup)
    if R == 0:
        return float(np.sum(dO * oracle.output(pb, u0, v0, vv)))
    us, vs = oracle.solve(pb, 0, R, v_init=v0)
    return float(np.sum(dO * oracle.output(pb, us[-1], vs[-1], vv)))


@pytest.mark.parametrize("R,dust,n", [(2, False, None), (1, False, None), (0, False, None),
                                      (2, True, 11), (3, False, 12)])
def test_adjoint_finite_differences(R, dust, n):
    """Central differences of the frozen-base surrogate match the adjoint."""
    p, n = _small_problem(seed=7 + R, R=R, dust=dust, n=n)
    q, k, vv, a, b = (x.astype(np.float64) for x in _one(p))
    dO = p.dO[0, 0].astype(np.float64)
    sup = oracle.Support.build(p.L, n, p.W, dust)
    sol = oracle.forward_one(q, k, vv, a, b, sup, p.T, R)
    g = oracle.backward_one(q, k, vv, a, b, sup, p.T, R, dO)
    v0 = np.where(sup.active, sol.vs[0], 0.0)
    u0 = np.where(sup.active, sol.us[0], 0.0)
    rng = np.random.default_rng(99)
    h = 1e-5
    for name, X, G in (("Q", q, g.dQ), ("K", k, g.dK), ("V", vv, g.dV)):
        E = rng.standard_normal(X.shape)
        E[~sup.active] = 0.0
        args = {"Q": [q, k, vv], "K": [q, k, vv], "V": [q, k, vv]}[name]
        idx = "QKV".index(name)

        def f(s):
            xs = list(args)
            xs[idx] = X + s * E
            return _tail_objective(xs[0], xs[1], xs[2], a, b, sup, v0, R, dO, u0)

        fd = (f(h) - f(-h)) / (2 * h)
        an = float(np.sum(G * E))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


@pytest.mark.parametrize("T,R,dust", [(5, 2, False), (3, 3, False), (4, 2, True), (6, 0, False)])
def test_adjoint_matches_torch_autograd(T, R, dust):
    """Exact autodiff of the stop-gradient surrogate (torch, base detached)."""
    p, n = _small_problem(seed=31 + T, T=T, R=R, dust=dust, n=10 if dust else None, L=16)
    q, k, vv, a, b = _one(p)
    dO = p.dO[0, 0]
    sup = oracle.Support.build(p.L, n, p.W, dust)
    g = oracle.backward_one(q, k, vv, a, b, sup, T, R, dO)
    mask = refs.support_mask(p.L, n, p.W, dust)
    tq, tk, tv, tO = refs.torch_surrogate_grads(q, k, vv, a, b, mask, T, R, dO)
    sol = oracle.forward_one(q, k, vv, a, b, sup, T, R)
    assert _rel(sol.O, tO) < 1e-12
    assert _rel(g.dQ, tq) < 1e-10
    assert _rel(g.dK, tk) < 1e-10
    assert _rel(g.dV, tv) < 1e-10


def test_no_base_equals_full_bptt():
    """T = 0: the surrogate is the full unrolled gradient (torch, no detach),
    and the oracle's BPTT reference equals torch full autograd for T > 0."""
    p, n = _small_problem(seed=41, T=0, R=4)
    q, k, vv, a, b = _one(p)
    dO = p.dO[0, 0]
    sup = oracle.Support.build(p.L, n, p.W)
    mask = refs.support_mask(p.L, n, p.W)
    g = oracle.backward_one(q, k, vv, a, b, sup, 0, 4, dO)
    tq, tk, tv, _ = refs.torch_surrogate_grads(q, k, vv, a, b, mask, 0, 4, dO, detach_base=False)
    assert _rel(g.dQ, tq) < 1e-10 and _rel(g.dK, tk) < 1e-10 and _rel(g.dV, tv) < 1e-10
    gb = oracle.bptt_one(q, k, vv, a, b, sup, 5, 2, dO)
    tq, tk, tv, _ = refs.torch_surrogate_grads(q, k, vv, a, b, mask, 5, 2, dO, detach_base=False)
    assert _rel(gb.dQ, tq) < 1e-10 and _rel(gb.dK, tk) < 1e-10 and _rel(gb.dV, tv) < 1e-10


@pytest.mark.parametrize("R,dust", [(2, False), (4, False), (2, True), (1, False)])
def test_single_reference_tile_adjoint(R, dust):
    """Modifier form (one P^(R,R) plus exp(u^(r)-u^(R)), exp(v^(s)-v^(R)))
    equals the explicit staircase recursion."""
    p, n = _small_problem(seed=51 + R, R=R, T=3, dust=dust, n=12 if dust else None, L=18, W=6)
    q, k, vv, a, b = _one(p)
    dO = p.dO[0, 0]
    sup = oracle.Support.build(p.L, n, p.W, dust)
    sol = oracle.forward_one(q, k, vv, a, b, sup, p.T, R)
    g = oracle.backward_one(q, k, vv, a, b, sup, p.T, R, dO)
    mask = refs.support_mask(p.L, n, p.W, dust)
    dq, dk, dv, vbar0 = refs.modifier_adjoint(q, k, vv, a, b, mask, sol.us, sol.vs, dO)
    assert _rel(g.dQ, dq) < 1e-11
    assert _rel(g.dK, dk) < 1e-11
    assert _rel(g.dV, dv) < 1e-11
    act = sup.active
    assert _rel(g.vbar0[act], vbar0[act]) < 1e-11


def test_orbit_identity_elementwise():
    """P^(a,b) built directly equals P^(2,2) (.) exp(u^a-u^2) (.) exp(v^b-v^2)."""
    p = workloads.make(1)
    q, k, vv, a, b = _one(p)
    sup = oracle.Support.build(p.L, p.L, p.W)
    pb = oracle.Problem(q, k, a, b, sup)
    us, vs = oracle.solve(pb, p.T, 2)
    P22 = pb.plan(us[2], vs[2])
    for (ia, ib) in ((2, 1), (1, 1), (1, 0)):
        direct = pb.plan(us[ia], vs[ib])
        orbit = P22 * np.exp(us[ia] - us[2])[sup.rows] * np.exp(vs[ib] - vs[2])[sup.cols]
        np.testing.assert_allclose(orbit, direct, rtol=1e-13, atol=0)


def test_dV_and_identities():
    """dV = P^T dO and, for R = 0, dS = P (.) (dO V^T) (plain fixed-plan gradient)."""
    p, n = _small_problem(seed=61, R=0, T=5)
    q, k, vv, a, b = (x.astype(np.float64) for x in _one(p))
    dO = p.dO[0, 0].astype(np.float64)
    sup = oracle.Support.build(p.L, n, p.W)
    sol = oracle.forward_one(q, k, vv, a, b, sup, p.T, 0)
    g = oracle.backward_one(q, k, vv, a, b, sup, p.T, 0, dO)
    mask = refs.support_mask(p.L, n, p.W)
    X = np.where(mask, q @ k.T / 2.0, -np.inf)
    P = refs.plan_dense(X, sol.u, sol.v)
    np.testing.assert_allclose(g.dV, P.T @ dO, rtol=1e-12, atol=1e-14)
    dS = P * (dO @ vv.T)
    np.testing.assert_allclose(g.dQ, dS @ k / 2.0, rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(g.dK, dS.T @ q / 2.0, rtol=1e-11, atol=1e-14)


@pytest.mark.parametrize("cfg", ["tiny", "midsmall"])
def test_gradient_gap_shrinks_with_tail_depth(cfg):
    """Stop-gradient vs full BPTT gap (same N = T + R steps) falls from R = 0
    to 1 to 2; R = 4 is no worse than R = 2 (section 4.1)."""
    if cfg == "tiny":
        p = workloads.make(1)
        N = 22
    else:
        p = workloads.custom(B=1, H=1, L=96, d=16, W=24, seed=71, scale=1.0 / 2)
        N = 30
    q, k, vv, a, b = _one(p)
    dO = p.dO[0, 0]
    sup = oracle.Support.build(p.L, p.L, p.W)
    ref = oracle.bptt_one(q, k, vv, a, b, sup, N, 0, dO)
    refv = np.concatenate([ref.dQ.ravel(), ref.dK.ravel()])
    gaps = {}
    for R in (0, 1, 2, 4):
        g = oracle.backward_one(q, k, vv, a, b, sup, N - R, R, dO)
        gv = np.concatenate([g.dQ.ravel(), g.dK.ravel()])
        gaps[R] = np.linalg.norm(gv - refv) / np.linalg.norm(refv)
    assert gaps[0] > gaps[1] > gaps[2], gaps
    assert gaps[4] <= gaps[2] * 1.0001, gaps


# --- convergence-controlled base (section 2.1: "until convergence") ------------

def _dense_errors(q, k, vv, a, b, mask, T_max, every):
    """Row-marginal L1 errors of the plan after each checked step, from the
    textbook dense Sinkhorn of refs (an independent implementation)."""
    out = {}
    for c in range(every, T_max - 1, every):
        us, vs, _ = refs.dense_sinkhorn(q, k, vv, a, b, mask, c, 0)
        X = np.where(mask, np.asarray(q, np.float64) @ np.asarray(k, np.float64).T /
                     math.sqrt(q.shape[1]), -np.inf)
        P = refs.plan_dense(X, us[0], vs[0])
        act = mask.any(axis=1)
        out[c] = float(np.abs(P.sum(axis=1)[act] - np.asarray(a, np.float64)[act]).sum())
    return out


@pytest.mark.parametrize("L,n,W,dust", [(24, 24, 7, False), (24, 17, 6, True)])
def test_base_errors_match_dense_plan(L, n, W, dust):
    """e_c from the oracle equals the L1 row error of the dense textbook plan."""
    p = workloads.custom(B=1, H=1, L=L, d=4, W=W, T=12, R=1, lengths=None if n == L else [n],
                         dustbin=dust, seed=3, scale=1.5)
    q, k, vv = p.Q[0, 0], p.K[0, 0], p.V[0, 0]
    rng = np.random.default_rng(7)
    act = refs.support_mask(L, n, W, dust).any(axis=1)
    a = np.where(act, rng.random(L) + 0.3, 0.0)
    b = np.where(act, rng.random(L) + 0.3, 0.0)
    a, b = a / a.sum(), b / b.sum()
    pb = oracle.sinkhorn._Problem(q, k, a, b, oracle.Support.build(L, n, W, dust))
    got = oracle.base_errors(pb, 12, 3)
    want = _dense_errors(q, k, vv, a, b, refs.support_mask(L, n, W, dust), 12, 3)
    assert sorted(got) == sorted(want) == [3, 6, 9]
    for c in want:
        assert abs(got[c] - want[c]) <= 1e-12 * max(1.0, want[c]), (c, got[c], want[c])
        assert want[c] > 1e-8  # a non-trivial check: not yet converged


def test_base_error_closed_form_from_next_row_update():
    """After a full step the column sums are b, and the row sums of P^(c,c)
    are a_i exp(u^(c)_i - u^(c+1)_i) with u^(c+1) = U(v^(c))."""
    p = workloads.make(2)
    q, k, vv, a, b = _one(p)
    rng = np.random.default_rng(1)
    a = rng.random(p.L) + 0.5
    a = a / a.sum()
    pb = oracle.sinkhorn._Problem(q, k, a, b, oracle.Support.build(p.L, p.L, p.W))
    u = np.zeros(p.L)
    v = np.zeros(p.L)
    for c in range(1, 7):
        u = pb.U(v)
        v = pb.V(u)
        e = oracle.row_marginal_error(pb, u, v)
        closed = float(np.sum(a * np.abs(np.expm1(u - pb.U(v)))))
        assert abs(e - closed) <= 1e-12 * max(e, 1e-300), (c, e, closed)
        colerr = np.abs(pb.col_sums(pb.plan(u, v)) - pb.b).sum()
        assert colerr < 1e-14


def test_zero_scores_converge_in_one_step():
    """S = 0 on a dense support with uniform marginals: one step solves the
    problem (P = a b^T), so e_c = 0 and the base stops at the first check."""
    L = 16
    q = np.zeros((L, 4))
    a = np.full(L, 1.0 / L)
    pb = oracle.sinkhorn._Problem(q, q, a, a, oracle.Support.build(L, L, 2 * L - 1))
    errs = oracle.base_errors(pb, 10, 2)
    assert all(e < 1e-15 for e in errs.values())
    assert oracle.select_base_length([errs], 10, 1e-12) == 2


def test_select_base_length_rule():
    """The batch stops at the first check where every problem is below tol."""
    e1 = {2: 1e-2, 4: 1e-4, 6: 1e-7}
    e2 = {2: 1e-3, 4: 1e-3, 6: 1e-8}
    assert oracle.select_base_length([e1, e2], 9, 1e-2) == 4
    assert oracle.select_base_length([e1, e2], 9, 5e-3) == 4
    assert oracle.select_base_length([e1, e2], 9, 5e-4) == 6
    assert oracle.select_base_length([e1, e2], 9, 1e-9) == 9
    assert oracle.select_base_length([e1, {2: float("nan"), 4: 0.0, 6: 0.0}], 9, 1.0) == 4
    assert oracle.select_base_length([{}], 3, 1.0) == 3


# --- a-posteriori bias certificate (section 2.4, third certificate) -------------

def _torch_base_vjp(q, k, a, b, mask, M, seed):
    """Gradient w.r.t. (q, k) of <seed, v^(M)>, v^(M) the column potential
    after M Sinkhorn steps from zero, by torch float64 autograd through the
    unrolled dense iteration (independent of the oracle)."""
    import torch
    dt = torch.float64
    Q = torch.tensor(np.asarray(q, np.float64), dtype=dt, requires_grad=True)
    K = torch.tensor(np.asarray(k, np.float64), dtype=dt, requires_grad=True)
    Mk = torch.tensor(mask)
    X = torch.where(Mk, Q @ K.T / math.sqrt(q.shape[1]), torch.tensor(-1e200, dtype=dt))
    la = torch.log(torch.tensor(np.asarray(a, np.float64), dtype=dt))
    lb = torch.log(torch.tensor(np.asarray(b, np.float64), dtype=dt))
    L = q.shape[0]
    u = torch.zeros(L, dtype=dt)
    v = torch.zeros(L, dtype=dt)
    for _ in range(M):
        u = la - torch.logsumexp(X + v[None, :], dim=1)
        v = lb - torch.logsumexp(X + u[:, None], dim=0)
    (v * torch.tensor(np.asarray(seed, np.float64), dtype=dt)).sum().backward()
    return Q.grad.numpy(), K.grad.numpy()


@pytest.mark.parametrize("R,dust", [(1, False), (2, False), (2, True)])
def test_discarded_adjoint_reconstructs_full_residual(R, dust):
    """The full gradient minus the depth-R surrogate gradient is exactly the
    discarded adjoint vbar0 pulled back through the stopped base (what the
    certificate measures; section 4.1 reports this reconstruction)."""
    L, W, N = 14, 5, 7
    n = L - 1 if dust else L
    p = workloads.custom(B=1, H=1, L=L, d=4, W=W, T=N - R, R=R, lengths=[n] if dust else None,
                         dustbin=dust, seed=21, scale=1.2)
    q, k, vv, a, b, dO = p.Q[0, 0], p.K[0, 0], p.V[0, 0], p.a[0], p.b[0], p.dO[0, 0]
    sup = oracle.Support.build(L, n, W, dust)
    tail = oracle.backward_one(q, k, vv, a, b, sup, N - R, R, dO)
    full = oracle.bptt_one(q, k, vv, a, b, sup, N - R, R, dO)
    mask = refs.support_mask(L, n, W, dust)
    gq, gk = _torch_base_vjp(q, k, a, b, mask, N - R, np.where(np.isfinite(tail.vbar0), tail.vbar0, 0))
    assert _rel(full.dQ - tail.dQ, gq) < 1e-10
    assert _rel(full.dK - tail.dK, gk) < 1e-10
    assert np.linalg.norm(gq) > 1e-6 * np.linalg.norm(full.dQ)  # a non-trivial residual


def test_certificate_without_base_is_the_full_residual():
    """T = 0: the deepest tail is full BPTT, so eta_R is exactly
    ||g_BPTT - g_R|| / ||g_BPTT|| over (dQ, dK)."""
    p = workloads.custom(B=1, H=2, L=20, d=4, W=7, T=0, R=5, seed=8, scale=1.1)
    grads, fulls = [], []
    for h in range(2):
        q, k, vv, a, b, dO = p.Q[0, h], p.K[0, h], p.V[0, h], p.a[0], p.b[0], p.dO[0, h]
        sup = oracle.Support.build(p.L, p.L, p.W)
        grads.append(oracle.tail_depth_gradients(q, k, vv, a, b, sup, 0, 5, dO))
        fulls.append(oracle.bptt_one(q, k, vv, a, b, sup, 0, 5, dO))
    eta = oracle.certificate_eta(grads)
    den = sum(np.sum(f.dQ ** 2) + np.sum(f.dK ** 2) for f in fulls)
    for R in range(6):
        num = sum(np.sum((g[R].dQ - f.dQ) ** 2) + np.sum((g[R].dK - f.dK) ** 2)
                  for g, f in zip(grads, fulls))
        assert abs(eta[R] - math.sqrt(num / den)) <= 1e-12 + 1e-9 * eta[R], (R, eta[R])
    assert eta[5] == 0.0


def test_certificate_decays_with_depth():
    """Section 2.4 (first certificate): the surrogate bias shrinks
    geometrically with the tail depth on a contractive problem."""
    p = workloads.make(1)
    q, k, vv, a, b = _one(p)
    g = oracle.tail_depth_gradients(q, k, vv, a, b, oracle.Support.build(p.L, p.L, p.W), 16, 4,
                                    p.dO[0, 0])
    eta = oracle.certificate_eta([g])
    assert all(eta[R + 1] < 0.9 * eta[R] for R in range(3)), eta
    assert oracle.select_tail_depth(eta, math.sqrt(eta[1] * eta[2])) == 2
    assert oracle.select_tail_depth(eta, 0.0) == 4


# --- projective contraction diagnostic (section 2.4, second certificate) ------

def _hilbert(x, y):
    r = np.log(x) - np.log(y)
    return r.max() - r.min()


def test_block_diameter_brute_force():
    """Delta equals the largest log cross-ratio over all index quadruples."""
    rng = np.random.default_rng(2)
    L, n, W, blk, d = 13, 11, 12, 5, 3
    q = rng.normal(size=(L, d))
    k = rng.normal(size=(L, d))
    got = oracle.block_diameters(q, k, L, n, W, blk)
    assert got.shape == (3,)
    for b_, s in enumerate(range(0, L, blk)):
        e = min(s + blk, n)
        best = 0.0
        for i in range(s, e):
            for j in range(s, e):
                for kk in range(s, e):
                    for ll in range(s, e):
                        x = (q[i] @ k[kk] + q[j] @ k[ll] - q[j] @ k[kk] - q[i] @ k[ll]) / math.sqrt(d)
                        best = max(best, x)
        assert abs(got[b_] - best) < 1e-12, (b_, got[b_], best)


def test_block_diameter_closed_forms():
    """A rank-one kernel (S_ik = f_i + g_k) has diameter 0; a 2 x 2 block has
    |S_11 + S_22 - S_12 - S_21|."""
    rng = np.random.default_rng(4)
    f, g = rng.normal(size=8), rng.normal(size=8)
    q = np.stack([f, np.ones(8)], axis=1) * math.sqrt(2)
    k = np.stack([np.ones(8), g], axis=1)
    assert np.all(np.abs(oracle.block_diameters(q, k, 8, 8, 17, 8)) < 1e-12)
    q2, k2 = rng.normal(size=(2, 4)), rng.normal(size=(2, 4))
    S = q2 @ k2.T / 2.0
    got = oracle.block_diameters(q2, k2, 2, 2, 3, 2)[0]
    assert abs(got - abs(S[0, 0] + S[1, 1] - S[0, 1] - S[1, 0])) < 1e-12


def test_block_contraction_birkhoff():
    """Birkhoff-Hopf: the block kernel contracts Hilbert's projective metric by
    tanh(Delta / 4), and not by much less (random pairs come close)."""
    rng = np.random.default_rng(6)
    d, blk = 4, 6
    q, k = rng.normal(size=(blk, d)) * 0.7, rng.normal(size=(blk, d)) * 0.7
    delta = oracle.block_diameters(q, k, blk, blk, 2 * blk + 1, blk)[0]
    kappa = math.tanh(delta / 4)
    Kmat = np.exp(q @ k.T / math.sqrt(d))
    worst = 0.0
    for _ in range(4000):
        x = np.exp(rng.normal(size=blk) * 3)
        y = np.exp(rng.normal(size=blk) * 3)
        ratio = _hilbert(Kmat @ x, Kmat @ y) / _hilbert(x, y)
        assert ratio <= kappa + 1e-12
        worst = max(worst, ratio)
    assert 0.0 < kappa < 1.0 and worst > 0.5 * kappa
