"""Plant plausible slips in a copy of the oracle and check the pins catch them.

Each mutant is the oracle's source with one textual change, loaded as a fresh
module (the real oracle is untouched).  A mutant survives only if every pin
check below still passes on it; the test asserts that none survives.
"""

import importlib.util
import math
import os
import sys
import types

import numpy as np
import pytest

import workloads
from tests import refs

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "sinkhorn.py")

MUTANTS = {
    "column update first": ("    for _ in range(T):\n        u = pb.U(v)\n        v = pb.V(u)\n",
                            "    for _ in range(T):\n        v = pb.V(u)\n        u = pb.U(v)\n"),
    "symmetric band": ("return W // 2, (W + 1) // 2 - 1", "return W // 2, W // 2"),
    "no dustbin corner": ("rows.append(np.full(n + 1, dlt, dtype=np.int64))\n"
                          "            cols.append(np.arange(n + 1, dtype=np.int64))",
                          "rows.append(np.full(n, dlt, dtype=np.int64))\n"
                          "            cols.append(np.arange(n, dtype=np.int64))"),
    "row marginal in column step": ("v[self.ckey] = self.log_b[self.ckey] - lse",
                                    "v[self.ckey] = self.log_a[self.ckey] - lse"),
    "missing 1/sqrt(d)": ("return out / math.sqrt(d)", "return out"),
    "adjoint sign (column step)": ("        dS -= cy\n", "        dS += cy\n"),
    "adjoint drops row-step term": ("        dS -= cx\n", "        pass\n"),
    "adjoint wrong plan index": ("Prs = pb.plan(us[r], vs[r - 1])", "Prs = pb.plan(us[r], vs[r])"),
    "adjoint divides by a not b": ("y = np.where(act, vbar / b_safe, 0.0)",
                                   "y = np.where(act, vbar / a_safe, 0.0)"),
    "dK not transposed": ("dK = (dSm.T @ q) / math.sqrt(d)", "dK = (dSm @ q) / math.sqrt(d)"),
    "dV not transposed": ("dV = Pm.T @ dO", "dV = Pm @ dO"),
    "D term dropped": ("ubar = pb.row_sums(P * dP)", "ubar = np.zeros(sup.L)"),
    "E term dropped": ("vbar = pb.col_sums(P * dP)", "vbar = np.zeros(sup.L)"),
    "output uses previous v": ("O = output(pb, us[-1], vs[-1], vv)",
                               "O = output(pb, us[-1], vs[-2] if len(vs) > 1 else vs[-1], vv)"),
    "base check against b": ("return float(np.sum(np.abs(rs[act] - pb.a[act])))",
                             "return float(np.sum(np.abs(rs[act] - pb.b[act])))"),
    "base check on column sums": ("rs = pb.row_sums(pb.plan(u, v))",
                                  "rs = pb.col_sums(pb.plan(u, v))"),
    "base check before the column update": ("        v = pb.V(u)\n        if c % every == 0",
                                            "        if c % every == 0"),
    "certificate moves the forward": ("return [backward_one(q, k, vv, a, b, sup, N - R, R, dO)",
                                      "return [backward_one(q, k, vv, a, b, sup, T, R, dO)"),
    "diameter without the transpose": ("out[blk] = float((M + M.T).max())", "out[blk] = float((M + M).max())"),
    "diameter over rows only": ("M = diff.max(axis=2)", "M = diff.max(axis=1)"),
    "certificate ignores dK": ("num = sum(float(np.sum((g[R].dQ - g[R_max].dQ) ** 2) + np.sum((g[R].dK - g[R_max].dK) ** 2))",
                               "num = sum(float(np.sum((g[R].dQ - g[R_max].dQ) ** 2))"),
}


def _load_mutant(old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique/found: {old!r}"
    src = src.replace(old, new)
    name = "oracle_mutant_%d" % abs(hash((old, new)))
    mod = types.ModuleType(name)
    mod.__file__ = SRC
    sys.modules[name] = mod  # dataclasses resolve annotations through sys.modules
    try:
        exec(compile(src, name, "exec"), mod.__dict__)
    finally:
        sys.modules.pop(name, None)
    return mod


def _rel(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    fin = np.isfinite(ref)
    if not np.array_equal(fin, np.isfinite(x)):
        return np.inf
    den = np.linalg.norm(ref[fin])
    return np.linalg.norm(x[fin] - ref[fin]) / (den if den > 0 else 1.0)


def _random_marginals(p, seed):
    """Distinct positive a != b on the active tokens (catches a/b swaps)."""
    rng = np.random.default_rng(seed)
    n = int(p.n_active()[0])
    a = np.zeros(p.L)
    b = np.zeros(p.L)
    a[:n] = rng.random(n) + 0.2
    b[:n] = rng.random(n) + 0.2
    return a / a.sum(), b / b.sum()


def _checks(m):
    """Yield (name, passed) for a compact set of the oracle pins."""
    # brute force, banded, ragged, dustbin, even W
    for (L, n, W, T, R, dust) in [(12, 9, 4, 3, 2, False), (12, 8, 5, 3, 2, True)]:
        p = workloads.custom(B=1, H=1, L=L, d=3, W=W, T=T, R=R, lengths=[n], dustbin=dust,
                             seed=L + W, scale=1.3)
        q, k, vv = p.Q[0, 0], p.K[0, 0], p.V[0, 0]
        a, b = _random_marginals(p, L)
        sol = m.forward_one(q, k, vv, a, b, m.Support.build(L, n, W, dust), T, R)
        u, v, O = refs.brute_force(q, k, vv, a, b, L, n, W, T, R, dust)
        yield f"brute{(L, n, W, dust)}", max(_rel(sol.u, u), _rel(sol.v, v), _rel(sol.O, O)) < 1e-12
    # gradients vs torch autograd of the stop-gradient surrogate
    for (L, n, W, T, R, dust) in [(14, 14, 5, 4, 2, False), (16, 10, 5, 3, 2, True)]:
        p = workloads.custom(B=1, H=1, L=L, d=4, W=W, T=T, R=R,
                             lengths=None if n == L else [n], dustbin=dust, seed=5, scale=0.9)
        q, k, vv = p.Q[0, 0], p.K[0, 0], p.V[0, 0]
        a, b = _random_marginals(p, L + 1)
        dO = p.dO[0, 0]
        g = m.backward_one(q, k, vv, a, b, m.Support.build(L, n, W, dust), T, R, dO)
        mask = refs.support_mask(L, n, W, dust)
        tq, tk, tv, _ = refs.torch_surrogate_grads(q, k, vv, a, b, mask, T, R, dO)
        yield f"grad{(L, n, dust)}", max(_rel(g.dQ, tq), _rel(g.dK, tk), _rel(g.dV, tv)) < 1e-10
    # convergence-controlled base: errors of the dense textbook plan
    L, n, W = 14, 11, 5
    p = workloads.custom(B=1, H=1, L=L, d=4, W=W, T=9, R=1, lengths=[n], seed=9, scale=1.4)
    q, k, vv = p.Q[0, 0], p.K[0, 0], p.V[0, 0]
    a, b = _random_marginals(p, 3)
    mask = refs.support_mask(L, n, W)
    X = np.where(mask, q.astype(np.float64) @ k.astype(np.float64).T / math.sqrt(4), -np.inf)
    pb = m._Problem(q, k, a, b, m.Support.build(L, n, W))
    got = m.base_errors(pb, 9, 2)
    ok = sorted(got) == [2, 4, 6]
    for c in (2, 4, 6):
        us, vs, _ = refs.dense_sinkhorn(q, k, vv, a, b, mask, c, 0)
        want = np.abs(refs.plan_dense(X, us[0], vs[0]).sum(axis=1)[:n] - a[:n]).sum()
        ok = ok and c in got and abs(got[c] - want) <= 1e-12 * max(1.0, want)
    yield "base check", ok
    # certificate with T = 0: eta against full BPTT
    p = workloads.custom(B=1, H=1, L=12, d=3, W=5, T=0, R=3, seed=4, scale=1.2)
    q, k, vv, dO = p.Q[0, 0], p.K[0, 0], p.V[0, 0], p.dO[0, 0]
    a, b = _random_marginals(p, 5)
    sup = m.Support.build(12, 12, 5)
    eta = m.certificate_eta([m.tail_depth_gradients(q, k, vv, a, b, sup, 0, 3, dO)])
    mask = refs.support_mask(12, 12, 5)
    fq, fk, _, _ = refs.torch_surrogate_grads(q, k, vv, a, b, mask, 0, 3, dO, detach_base=False)
    ok = True
    for R in range(3):
        tq, tk, _, _ = refs.torch_surrogate_grads(q, k, vv, a, b, mask, 3 - R, R, dO)
        want = math.sqrt((np.sum((tq - fq) ** 2) + np.sum((tk - fk) ** 2)) / (np.sum(fq ** 2) + np.sum(fk ** 2)))
        ok = ok and abs(eta[R] - want) <= 1e-9 * want
    yield "certificate", ok
    # contraction diagnostic: brute-force cross ratios
    rng = np.random.default_rng(12)
    qd, kd = rng.normal(size=(9, 3)), rng.normal(size=(9, 3))
    got = m.block_diameters(qd, kd, 9, 9, 9, 4)
    ok = True
    for b_, s0 in enumerate(range(0, 9, 4)):
        e0 = min(s0 + 4, 9)
        S = qd[s0:e0] @ kd[s0:e0].T / math.sqrt(3)
        best = max(S[i, kk] + S[j, ll] - S[j, kk] - S[i, ll] for i in range(e0 - s0) for j in range(e0 - s0)
                   for kk in range(e0 - s0) for ll in range(e0 - s0))
        ok = ok and abs(got[b_] - best) < 1e-12
    yield "diameter", ok


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _load_mutant(*MUTANTS[name])
    results = dict(_checks(mod))
    assert not all(results.values()), f"mutant '{name}' survived every pin: {results}"


def test_unmutated_oracle_passes_the_same_checks():
    mod = _load_mutant("import math\n", "import math\n")
    results = dict(_checks(mod))
    assert all(results.values()), results
