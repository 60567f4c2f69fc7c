"""Trainability through the autograd wrapper (the protein-like synthetic task).

Section 4.2 trains on Pfam, which is not used here; this stands in with the
protein-like shapes (B = 8, H = 8, L = 512, d = 64, 20 token ids, ragged
lengths 128..512, W = 64, T = 30, R = 2): embedding -> Q, K, V projections ->
banded Sinkhorn attention (the HIP kernels, through
entropic_ot_banded_amd.sinkhorn_attention) -> linear head, trained to
reconstruct each real token's id (cross-entropy), with and without a dustbin
token.  The attention's rows carry mass a_i, so its output is rescaled by
1 / a_i before the head.

Checks: (1) the gradients of the three projections equal those chained by
hand from the oracle's dQ, dK, dV for the same upstream dO (normwise 1e-4,
the fp32 gradient bound); (2) 30 Adam steps lower the loss below half its
start (log 20 ~ 3.0) with every step finite.
"""

import math

import numpy as np
import pytest

import oracle
from tests.gpu_util import log

pytestmark = pytest.mark.gpu

B, H, L, d, VOCAB, W, T, R = 8, 8, 512, 64, 20, 64, 30, 2
D = H * d


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import entropic_ot_banded_amd as eoba
    eoba.load_library()


def _task(dustbin, seed=0):
    """Token ids, lengths and marginals (numpy PCG64); the dustbin, when on,
    is token n_b with its own id VOCAB."""
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, VOCAB, size=(B, L))
    lengths = rng.integers(128, 512 if dustbin else 513, size=B).astype(np.int32)
    a = np.zeros((B, L), np.float32)
    for bi, n in enumerate(lengths):
        if dustbin:
            a[bi, :n] = 0.9 / n
            a[bi, n] = 0.1
            ids[bi, n] = VOCAB
        else:
            a[bi, :n] = 1.0 / n
    return ids, lengths, a


def _params(torch, dev, seed=1):
    g = torch.Generator().manual_seed(seed)
    mk = lambda *s, std: (torch.randn(*s, generator=g, dtype=torch.float64) * std).float().to(dev)  # noqa: E731
    p = {"E": mk(VOCAB + 1, D, std=0.02), "Wq": mk(D, D, std=D ** -0.5), "Wk": mk(D, D, std=D ** -0.5),
         "Wv": mk(D, D, std=D ** -0.5), "Wo": mk(D, VOCAB, std=D ** -0.5)}
    for t in p.values():
        t.requires_grad_(True)
    return p


def _loss(torch, p, ids, lengths, a, dustbin, keep=None):
    from entropic_ot_banded_amd import sinkhorn_attention
    x = p["E"][ids]  # [B, L, D]

    def heads(Wm):
        return (x @ Wm).view(B, L, H, d).permute(0, 2, 1, 3).contiguous()

    Q, K, V = heads(p["Wq"]), heads(p["Wk"]), heads(p["Wv"])
    O, _, _ = sinkhorn_attention(Q, K, V, a, a, W, T, R, lengths, dustbin)
    if keep is not None:
        O.retain_grad()
        keep.update(Q=Q, K=K, V=V, O=O, x=x)
    inv_a = torch.where(a > 0, 1.0 / a, torch.zeros_like(a))
    o = O.permute(0, 2, 1, 3).reshape(B, L, D) * inv_a[:, :, None]
    logits = o @ p["Wo"]
    real = torch.arange(L, device=ids.device)[None, :] < lengths[:, None].long()
    return torch.nn.functional.cross_entropy(logits[real], ids[real])


def _device_task(torch, dustbin):
    dev = torch.device("cuda:0")
    ids, lengths, a = _task(dustbin)
    return (torch.from_numpy(ids).to(dev), torch.from_numpy(lengths).to(dev),
            torch.from_numpy(a).to(dev), ids, lengths, a)


@pytest.mark.parametrize("dustbin", [False, True])
def test_projection_gradients_match_oracle(dustbin):
    import torch
    ids_t, len_t, a_t, ids, lengths, a = _device_task(torch, dustbin)
    p = _params(torch, ids_t.device)
    keep = {}
    loss = _loss(torch, p, ids_t, len_t, a_t, dustbin, keep)
    loss.backward()
    torch.cuda.synchronize()
    f64 = lambda t: t.detach().double().cpu().numpy()  # noqa: E731
    ref = oracle.backward_batch(f64(keep["Q"]), f64(keep["K"]), f64(keep["V"]), a.astype(np.float64),
                                a.astype(np.float64), W, T, R, f64(keep["O"].grad), lengths, dustbin,
                                processes=8)
    x = f64(keep["x"])  # [B, L, D]
    for name, g in (("Wq", "dQ"), ("Wk", "dK"), ("Wv", "dV")):
        dflat = ref[g].transpose(0, 2, 1, 3).reshape(B, L, D)
        want = np.einsum("bld,ble->de", x, dflat)
        got = f64(p[name].grad)
        err = np.linalg.norm(got - want) / np.linalg.norm(want)
        log(f"   {name} grad rel err {err:.2e}")
        assert err < 1e-4, (name, err)


@pytest.mark.parametrize("dustbin", [False, True])
def test_training_reduces_reconstruction_loss(dustbin):
    import time

    import torch
    ids_t, len_t, a_t, _, _, _ = _device_task(torch, dustbin)
    p = _params(torch, ids_t.device)
    opt = torch.optim.Adam(list(p.values()), lr=1e-2)
    losses = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(30):
        loss = _loss(torch, p, ids_t, len_t, a_t, dustbin)
        opt.zero_grad()
        loss.backward()
        opt.step()
        losses.append(float(loss))
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / 30
    log(f"   dustbin={dustbin}: loss {losses[0]:.3f} -> {losses[-1]:.4f}, "
        f"every 5: {[round(x, 3) for x in losses[::5]]}, {ms:.1f} ms/step")
    assert all(math.isfinite(x) for x in losses)
    assert abs(losses[0] - math.log(VOCAB)) < 0.5
    assert losses[-1] < 0.5 * losses[0]
