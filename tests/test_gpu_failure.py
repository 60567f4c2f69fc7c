"""Failure reporting through the C-ABI (debug checks, SINKATTN_DEBUG).

One child process (the library reads SINKATTN_DEBUG once per process) runs
three forwards in turn:
  * clean inputs: SINKATTN_OK;
  * a NaN in Q: the stopped base and the returned potentials hold non-finite
    values on active tokens -> SINKATTN_ENONFINITE;
  * SINKATTN_DEBUG_STALL set: every neighbour wait of the persistent step
    launch is made unsatisfiable from the host and gives up after a few
    spins, so the launch still runs to its end -> SINKATTN_ESTALL, and O[0],
    u[0] carry the NaN marker.
No kernel faults or hangs: every wait is bounded and every index stays in
its buffer whatever the data.
"""

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r'''
import os, sys
sys.path.insert(0, ROOT)
import numpy as np
import torch
import entropic_ot_banded_amd as eoba
import workloads
from tests.gpu_util import to_device

def run(prob):
    t = to_device(prob)
    try:
        O, u, v, _ = eoba.forward(t["Q"], t["K"], t["V"], prob.W, prob.T, prob.R, t["a"], t["b"], t["lengths"],
                                  prob.dustbin)
        torch.cuda.synchronize()
        return 0, O, u
    except eoba.SinkattnError as e:
        torch.cuda.synchronize()
        return e.status, None, None

# 8 blocks per sequence in 2-block segments: the persistent launch, with waits
prob = workloads.custom(B=1, H=64, L=1024, d=64, W=64, T=6, R=2, dtype="bf16", seed=31, name="stall")
st, O, u = run(prob)
print("clean", st, flush=True)
assert st == 0, st
bad = workloads.custom(B=1, H=64, L=1024, d=64, W=64, T=6, R=2, dtype="bf16", seed=31, name="nan")
bad.Q[0, 5, 100, 3] = np.nan
st, _, _ = run(bad)
print("nan", st, flush=True)
assert st == eoba.binding.SINKATTN_ENONFINITE, st
os.environ["SINKATTN_DEBUG_STALL"] = "1"
st, _, _ = run(prob)
print("stall", st, flush=True)
assert st == eoba.binding.SINKATTN_ESTALL, st
os.environ.pop("SINKATTN_DEBUG_STALL")
st, O, u = run(prob)
print("clean again", st, flush=True)
assert st == 0 and bool(torch.isfinite(O).all()), st
print("FAILURE-PATH CHECKS PASSED", flush=True)
'''


@pytest.mark.timeout(300)
def test_debug_checks_report_nonfinite_and_stalled_waits():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    env = dict(os.environ, SINKATTN_DEBUG="1")
    env.pop("SINKATTN_DEBUG_STALL", None)
    res = subprocess.run([sys.executable, "-c", f"ROOT = {ROOT!r}\n" + CHILD], capture_output=True, text=True,
                         env=env, timeout=240)
    print(res.stdout)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    assert "FAILURE-PATH CHECKS PASSED" in res.stdout
