"""The forward entry point that allocates nothing (sinkattn_forward_noalloc,
static per-GPU scratch) against sinkattn_forward with a caller workspace:
two calls in a row, the second with a smaller input (the scratch keeps the
first call's contents), each bitwise equal to the workspace path (same
kernels and launch configuration, deterministic arithmetic).  A shape whose
workspace exceeds the scratch is rejected before any launch."""

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


def _compare(prob):
    import torch

    import entropic_ot_banded_amd as eoba
    t = to_device(prob)
    O, u, v, _ = eoba.forward(t["Q"], t["K"], t["V"], prob.W, prob.T, prob.R, t["a"], t["b"], t["lengths"],
                              prob.dustbin)
    O2, u2, v2 = eoba.forward_noalloc(t["Q"], t["K"], t["V"], prob.W, prob.T, prob.R, t["a"], t["b"], t["lengths"],
                                      prob.dustbin)
    torch.cuda.synchronize()
    log(f"[noalloc] {prob.name} {prob.shape} dtype={prob.dtype} W={prob.W} dustbin={prob.dustbin}")
    for name, x, y in (("O", O, O2), ("u", u, u2), ("v", v, v2)):
        assert torch.equal(x, y), name


def test_noalloc_matches_workspace_forward_on_two_calls():
    # first: 2-block segments (the persistent step launch), bf16
    _compare(workloads.custom(B=2, H=32, L=1024, d=64, W=128, T=20, R=2, dtype="bf16", seed=41, name="first"))
    # second, smaller: fp32, ragged, with a dustbin (per-step launches)
    _compare(workloads.custom(B=2, H=2, L=300, d=32, W=33, T=10, R=2, lengths=[250, 299], dustbin=True, seed=42,
                              name="second"))


def test_noalloc_rejects_shapes_beyond_the_scratch():
    import torch

    import entropic_ot_banded_amd as eoba
    from entropic_ot_banded_amd import binding
    B, H, L, d = 1, 64, 32768, 128
    shape = binding.Shape(B, H, L, d, binding.SINKATTN_BF16)
    assert eoba.workspace_bytes(shape, 256, 2) > binding.NOALLOC_SCRATCH_BYTES
    Q = torch.zeros((B, H, L, d), dtype=torch.bfloat16, device="cuda")
    a = torch.full((B, L), 1.0 / L, dtype=torch.float32, device="cuda")
    with pytest.raises(eoba.SinkattnError) as e:
        eoba.forward_noalloc(Q, Q, Q, 256, 3, 2, a, a)
    assert e.value.status == binding.SINKATTN_ESCRATCH
