"""GPU parity of the projective contraction diagnostic (sinkattn_block_contraction).

Section 2.4 (second certificate): strictly positive active blocks of the
Sinkhorn map contract Hilbert's projective metric.  Each diagonal band block
(inside the band, so its kernel is strictly positive) gets its projective
diameter Delta and kappa = tanh(Delta / 4).  The oracle evaluates the same
maxima in float64 (oracle.block_diameters).

Bound: the GPU forms the block scores in fp32 from the exact input values
(error ~ d * 2^-24 * max|q||k| / sqrt(d), below 1e-5 here) and Delta is a sum
of four of them, so |Delta_gpu - Delta| <= 1e-4 (1 + Delta) holds with room;
kappa inherits it (its slope is at most 1/4).
"""

import math

import numpy as np
import pytest

import oracle
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


CASES = [
    ("tiny", lambda: workloads.make(1), 9),
    ("mid-bf16", lambda: workloads.make(2, dtype="bf16"), 64),
    ("protein-ragged", lambda: workloads.make(3), 32),
    ("dustbin", lambda: workloads.make(4), 64),
    ("ragged-small-d", lambda: workloads.custom(B=2, H=1, L=200, d=16, W=40, T=1, R=1, lengths=[200, 77],
                                                seed=9, name="small-d"), 17),
    ("long-context-head0", lambda: workloads.make(5, heads=[0]), 128),
]


@pytest.mark.parametrize("name,mk,block", CASES, ids=[c[0] for c in CASES])
def test_block_contraction_matches_oracle(name, mk, block):
    import torch

    import entropic_ot_banded_amd as eoba
    prob = mk()
    t = to_device(prob)
    log(f"[contraction] {name} shape={prob.shape} W={prob.W} block={block}")
    delta, kappa = eoba.block_contraction(t["Q"], t["K"], prob.W, block, t["lengths"], prob.dustbin)
    torch.cuda.synchronize()
    ref = oracle.block_contraction_batch(prob.Q, prob.K, prob.W, block, prob.lengths)
    dg, kg = delta.cpu().numpy().astype(np.float64), kappa.cpu().numpy().astype(np.float64)
    assert dg.shape == ref.shape
    err = np.abs(dg - ref) / (1 + ref)
    log(f"   Delta max {ref.max():.4f}, kappa max {math.tanh(ref.max() / 4):.4f}, worst err {err.max():.2e}")
    assert err.max() <= 1e-4
    assert np.abs(kg - np.tanh(ref / 4)).max() <= 1e-4
    assert np.all(kg < 1.0)


def test_block_contraction_rejects_blocks_outside_the_band():
    import entropic_ot_banded_amd as eoba
    prob = workloads.make(1)  # W = 17: offsets [-8, 8], blocks up to 9
    t = to_device(prob)
    for blk in (0, 10, 129):
        with pytest.raises(eoba.SinkattnError):
            eoba.block_contraction(t["Q"], t["K"], prob.W, blk)
