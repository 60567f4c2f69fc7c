"""GPU parity of the convergence-controlled stopped base (sinkattn_forward_converge).

Section 2.1 runs the stopped base until convergence or for a fixed number of
steps.  The measure is the L1 row-marginal error of the plan after a base
step, checked every k steps; a call stops at the first check where every
(b, h) problem is below tol.  The oracle computes the same errors from the
explicitly built plan (oracle.base_errors) and picks the base length with the
same rule (oracle.select_base_length).

The stop is an integer decision taken from floating point on both sides, so
each test sets tol between two consecutive check values of the oracle's own
error sequence, at least 30% away from both; the GPU's check value (fp64 sums
of potentials computed from fp32 entry sums: absolute error ~1e-7 against
values >= 1e-5 here) cannot cross it.  Then the base length must agree
exactly and the outputs must match the oracle run at that base length to the
usual tolerances.  Two more tests check that a tolerance that never (or
immediately) passes reproduces the fixed-T forward bit for bit.
"""

import math

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import (TOL_BF16, TOL_F32, assert_parity, compare, fmt_errs, log, run_gpu,
                            run_gpu_converge, run_oracle)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import entropic_ot_banded_amd as eoba
    eoba.load_library()


def _pick_tol(prob, T_max, every, target_index):
    """tol between the batch's largest error at check c* - every and at c*
    (c* = the target_index-th check); returns (tol, c*, E(c*))."""
    _, errs = oracle.converged_base_length(prob.Q, prob.K, prob.a, prob.b, prob.W, T_max, 0.0,
                                           every, prob.lengths, prob.dustbin, processes=8)
    checks = sorted(errs[0])
    E = {c: max(e[c] for e in errs) for c in checks}
    c_star = checks[target_index]
    c_prev = checks[target_index - 1]
    assert E[c_prev] / E[c_star] > 1.3 ** 2, (E[c_prev], E[c_star])
    tol = math.sqrt(E[c_prev] * E[c_star])
    assert oracle.select_base_length(errs, T_max, tol) == c_star
    return tol, c_star, E[c_star]


CASES = [
    ("tiny", lambda: workloads.make(1), 5, 1, TOL_F32),
    ("mid-bf16", lambda: workloads.make(2, dtype="bf16"), 2, 1, TOL_BF16),
    ("protein-ragged", lambda: workloads.make(3), 2, 1, TOL_F32),
    ("dustbin", lambda: workloads.make(4), 5, 2, TOL_F32),
]


@pytest.mark.parametrize("name,mk,every,idx,tols", CASES, ids=[c[0] for c in CASES])
def test_converged_base_matches_oracle(name, mk, every, idx, tols):
    prob = mk()
    T_max = prob.T
    tol, c_star, e_star = _pick_tol(prob, T_max, every, idx)
    log(f"[converge] {name} T_max={T_max} every={every} tol={tol:.3e} -> T={c_star}")
    gpu = run_gpu_converge(prob, T_max, tol, every)
    assert gpu["T_used"] == c_star, (gpu["T_used"], c_star)
    assert abs(gpu["err_last"] - e_star) <= 1e-2 * e_star, (gpu["err_last"], e_star)
    ref = run_oracle(prob, T=c_star)
    errs = compare(gpu, ref, prob)
    log("   errors:", fmt_errs(errs))
    assert_parity(errs, tols, name)


@pytest.mark.parametrize("tol_kind", ["never", "first"])
@pytest.mark.parametrize("dust", [False, True])
def test_converge_reproduces_fixed_base(tol_kind, dust):
    """tol = 0 runs T_max steps; a huge tol stops at the first check.  Either
    way the result equals the fixed-T forward/backward with that T exactly."""
    if dust:
        prob = workloads.custom(B=2, H=2, L=96, d=32, W=20, T=9, R=2, lengths=[70, 81],
                                dustbin=True, seed=3, name="conv-dust")
    else:
        prob = workloads.custom(B=1, H=2, L=300, d=128, W=64, T=9, R=2, dtype="bf16", seed=5,
                                name="conv-bf16")
    every = 3
    tol = 0.0 if tol_kind == "never" else 1e30
    gpu = run_gpu_converge(prob, prob.T, tol, every)
    T_expect = prob.T if tol_kind == "never" else every
    assert gpu["T_used"] == T_expect
    ref = run_gpu(prob, T=T_expect)
    for k in ("O", "u", "v", "us", "vs", "dQ", "dK", "dV"):
        a, b = gpu[k], ref[k]
        if k in ("us", "vs"):  # filler entries of the tail stack are unspecified
            from tests.gpu_util import active_mask
            act = np.broadcast_to(active_mask(prob)[None, :, None, :], a.shape)
            a, b = a[act], b[act]
        np.testing.assert_array_equal(a, b, err_msg=k)


def test_converge_rejects_bad_arguments():
    import torch

    import entropic_ot_banded_amd as eoba
    prob = workloads.make(1)
    from tests.gpu_util import to_device
    t = to_device(prob)
    for kw in ({"R": 0}, {"every": 0}, {"tol": -1.0}, {"tol": float("nan")}):
        R = kw.get("R", 2)
        with pytest.raises(eoba.SinkattnError):
            eoba.forward_converge(t["Q"], t["K"], t["V"], prob.W, prob.T, R, t["a"], t["b"],
                                  kw.get("tol", 1e-3), kw.get("every", 2))
    torch.cuda.synchronize()
