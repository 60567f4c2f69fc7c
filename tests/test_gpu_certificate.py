"""GPU parity of the stop-gradient bias certificate (sinkattn_tail_certificate).

For a forward of N = T + R_max steps, eta[R] = ||g_Rmax - g_R|| / ||g_Rmax||
over (dQ, dK), g_R the gradient with only the last R steps differentiable
(section 2.4, third certificate).  The oracle computes every g_R from its
explicit-plan adjoint (oracle.tail_depth_gradients).

Bound on eta: each GPU gradient carries a normwise error eps (measured
<= 3e-6 in these cases, bounded by the parity tolerances), so a difference of
two of them is off by at most 2 eps relative to ||g||: |eta_gpu - eta| <=
2 eps, with margin: 1e-5 (fp32) and 2e-5 (bf16), plus 1% of eta.  The
selected depth is compared at a tolerance between two consecutive eta values
that lie well above those bounds.
"""

import dataclasses
import math

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import active_mask, log, rel_err, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import entropic_ot_banded_amd as eoba
    eoba.load_library()


CASES = [
    ("tiny", lambda: dataclasses.replace(workloads.make(1), T=16), 4, 1e-5, 1e-4),
    ("mid-bf16", lambda: dataclasses.replace(workloads.make(2, dtype="bf16"), T=10), 3, 2e-5, 1e-3),
    ("protein-ragged", lambda: dataclasses.replace(workloads.make(3), T=10), 3, 1e-5, 1e-4),
    ("dustbin", lambda: dataclasses.replace(workloads.make(4), T=10), 3, 1e-5, 1e-4),
    ("bf16-d128-R4", lambda: workloads.custom(B=1, H=2, L=300, d=128, W=64, T=6, R=4, dtype="bf16",
                                              seed=5, name="cert-bf16"), 4, 2e-5, 1e-3),
]


@pytest.mark.parametrize("name,mk,R_max,eta_abs,grad_tol", CASES, ids=[c[0] for c in CASES])
def test_certificate_matches_oracle(name, mk, R_max, eta_abs, grad_tol):
    import torch

    import entropic_ot_banded_amd as eoba
    prob = mk()
    T = prob.T
    log(f"[certificate] {name} T={T} R_max={R_max} shape={prob.shape}")
    t = to_device(prob)
    O, u, v, ws = eoba.forward(t["Q"], t["K"], t["V"], prob.W, T, R_max, t["a"], t["b"], t["lengths"],
                               prob.dustbin)
    dQ, dK, dV, eta, _ = eoba.tail_certificate(t["Q"], t["K"], t["V"], prob.W, T, R_max, t["a"], t["b"], O,
                                               t["dO"], ws, t["lengths"], prob.dustbin)
    torch.cuda.synchronize()
    eta_ref, gref = oracle.certificate_batch(prob.Q, prob.K, prob.V, prob.a, prob.b, prob.W, T, R_max,
                                             prob.dO, prob.lengths, prob.dustbin, processes=8)
    log("   eta gpu:", [f"{x:.3e}" for x in eta], " oracle:", [f"{x:.3e}" for x in eta_ref])
    assert len(eta) == R_max + 1 and eta[R_max] == 0.0
    for R in range(R_max):
        assert abs(eta[R] - eta_ref[R]) <= eta_abs + 1e-2 * eta_ref[R], (R, eta[R], eta_ref[R])
    act = np.broadcast_to(active_mask(prob)[:, None, :, None], prob.Q.shape)
    for k, x in (("dQ", dQ), ("dK", dK), ("dV", dV)):
        err = rel_err(x.cpu().numpy(), gref[k], act)
        log(f"   {k} rel err {err:.2e}")
        assert err <= grad_tol, (k, err)
    # the depth selected at a tolerance between two consecutive values
    for R in range(1, R_max):
        hi, lo = eta_ref[R - 1], eta_ref[R]
        if hi / lo > 1.69 and lo > 20 * eta_abs:
            tau = math.sqrt(hi * lo)
            *_, r_sel = eoba.tail_certificate(t["Q"], t["K"], t["V"], prob.W, T, R_max, t["a"], t["b"], O,
                                              t["dO"], ws, t["lengths"], prob.dustbin, tau=tau)
            assert r_sel == oracle.select_tail_depth(eta_ref, tau) == R
            *_, r_none = eoba.tail_certificate(t["Q"], t["K"], t["V"], prob.W, T, R_max, t["a"], t["b"], O,
                                               t["dO"], ws, t["lengths"], prob.dustbin, tau=0.0)
            assert r_none == R_max  # no depth meets tau = 0
            break
    else:
        pytest.fail(f"no well-separated pair of eta values: {eta_ref}")


def test_certificate_reference_pass_equals_backward():
    """The depth-R_max gradients the certificate returns are those of
    sinkattn_backward on the same forward, bit for bit."""
    import torch

    import entropic_ot_banded_amd as eoba
    prob = workloads.custom(B=2, H=2, L=96, d=32, W=20, T=6, R=3, lengths=[70, 81], dustbin=True, seed=3)
    t = to_device(prob)
    O, u, v, ws = eoba.forward(t["Q"], t["K"], t["V"], prob.W, prob.T, prob.R, t["a"], t["b"], t["lengths"],
                               prob.dustbin)
    dQ, dK, dV, _ = eoba.backward(t["Q"], t["K"], t["V"], prob.W, prob.T, prob.R, t["a"], t["b"], O, t["dO"],
                                  ws, t["lengths"], prob.dustbin)
    cQ, cK, cV, eta, _ = eoba.tail_certificate(t["Q"], t["K"], t["V"], prob.W, prob.T, prob.R, t["a"], t["b"], O,
                                               t["dO"], ws, t["lengths"], prob.dustbin)
    torch.cuda.synchronize()
    for a_, b_ in ((dQ, cQ), (dK, cK), (dV, cV)):
        assert torch.equal(a_, b_)
    assert all(math.isfinite(x) for x in eta)
