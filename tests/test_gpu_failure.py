"""Failure reporting through the C-ABI (debug checks, SINKATTN_DEBUG).

Three forwards in turn, with the debug checks on:
  * clean inputs: SINKATTN_OK;
  * a NaN in Q: the stopped base and the returned potentials hold non-finite
    values on active tokens -> SINKATTN_ENONFINITE;
  * SINKATTN_DEBUG_STALL set: every neighbour wait of the persistent step
    launch is made unsatisfiable from the host and gives up after a few
    spins, so the launch still runs to its end -> SINKATTN_ESTALL.
No kernel faults or hangs: every wait is bounded and every index stays in
its buffer whatever the data.
"""

import numpy as np
import pytest

import workloads
from tests.gpu_util import log, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import entropic_ot_banded_amd as eoba
    eoba.load_library()


def _run(prob):
    import torch

    import entropic_ot_banded_amd as eoba
    t = to_device(prob)
    try:
        O, u, v, _ = eoba.forward(t["Q"], t["K"], t["V"], prob.W, prob.T, prob.R, t["a"], t["b"], t["lengths"],
                                  prob.dustbin)
        torch.cuda.synchronize()
        return 0, O
    except eoba.SinkattnError as e:
        log("   ", e)
        torch.cuda.synchronize()
        return e.status, None


def test_debug_checks_report_nonfinite_and_stalled_waits(monkeypatch):
    import torch

    import entropic_ot_banded_amd as eoba
    monkeypatch.setenv("SINKATTN_DEBUG", "1")
    monkeypatch.delenv("SINKATTN_DEBUG_STALL", raising=False)
    # 8 blocks per sequence in 2-block segments: the persistent launch, with waits
    prob = workloads.custom(B=1, H=64, L=1024, d=64, W=64, T=6, R=2, dtype="bf16", seed=31, name="stall")
    st, O = _run(prob)
    assert st == 0, st
    bad = workloads.custom(B=1, H=64, L=1024, d=64, W=64, T=6, R=2, dtype="bf16", seed=31, name="nan")
    bad.Q[0, 5, 100, 3] = np.nan
    st, _ = _run(bad)
    assert st == eoba.binding.SINKATTN_ENONFINITE, st
    monkeypatch.setenv("SINKATTN_DEBUG_STALL", "1")
    st, _ = _run(prob)
    assert st == eoba.binding.SINKATTN_ESTALL, st
    monkeypatch.delenv("SINKATTN_DEBUG_STALL")
    st, O2 = _run(prob)
    assert st == 0 and bool(torch.isfinite(O2).all()), st
    # the run after the forced stall reproduces the first one bit for bit
    assert torch.equal(O, O2)
    # without the debug checks the results are not inspected
    monkeypatch.delenv("SINKATTN_DEBUG")
    st, _ = _run(bad)
    assert st == 0
