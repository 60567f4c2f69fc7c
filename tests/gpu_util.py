"""Helpers for GPU-vs-oracle parity tests (imported only by tests)."""

from __future__ import annotations

import os
import sys

import numpy as np

import oracle
import workloads


def rel_err(x, ref, mask=None):
    """Normwise relative error ||x - ref|| / ||ref|| over finite reference
    entries (and `mask` if given); the -inf patterns must agree."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    fin = np.isfinite(ref)
    if mask is not None:
        fin &= mask
    bad = np.isfinite(x) != np.isfinite(ref)
    if mask is not None:
        bad &= mask
    if bad.any():
        return np.inf
    den = np.linalg.norm(ref[fin])
    return float(np.linalg.norm(x[fin] - ref[fin]) / (den if den > 0 else 1.0))


def gauge_removed(u, v, active):
    """(u - c, v + c) with c the mean of u over active entries, per (b, h)."""
    u = np.array(u, np.float64)
    v = np.array(v, np.float64)
    for idx in np.ndindex(u.shape[:-1]):
        act = active[idx[0]]
        c = u[idx][act].mean() if act.any() else 0.0
        u[idx] = np.where(act, u[idx] - c, u[idx])
        v[idx] = np.where(act, v[idx] + c, v[idx])
    return u, v


def active_mask(prob: workloads.Problem):
    m = np.zeros((prob.B, prob.L), dtype=bool)
    for bi, n in enumerate(prob.n_active()):
        m[bi, :n] = True
    return m


def to_device(prob: workloads.Problem, device="cuda"):
    import torch

    dt = torch.bfloat16 if prob.dtype == "bf16" else torch.float32

    def up(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(device).to(dt).contiguous()

    d = {"Q": up(prob.Q), "K": up(prob.K), "V": up(prob.V), "dO": up(prob.dO),
         "a": torch.from_numpy(prob.a).to(device), "b": torch.from_numpy(prob.b).to(device),
         "lengths": None}
    if prob.lengths is not None:
        d["lengths"] = torch.from_numpy(prob.lengths.astype(np.int32)).to(device)
    return d


def run_gpu(prob: workloads.Problem, T=None, R=None, W=None, want_vbar0=False, backward=True):
    import torch

    import entropic_ot_banded_amd as eoba

    T = prob.T if T is None else T
    R = prob.R if R is None else R
    W = prob.W if W is None else W
    t = to_device(prob)
    O, u, v, ws = eoba.forward(t["Q"], t["K"], t["V"], W, T, R, t["a"], t["b"], t["lengths"],
                               prob.dustbin)
    out = {"O": O, "u": u, "v": v}
    us, vs = eoba.tail_stack(ws, t["Q"], R, t["lengths"], prob.dustbin)
    out["us"] = [x.clone() for x in us]
    out["vs"] = [x.clone() for x in vs]
    if backward:
        dQ, dK, dV, vb0 = eoba.backward(t["Q"], t["K"], t["V"], W, T, R, t["a"], t["b"], O, t["dO"],
                                        ws, t["lengths"], prob.dustbin, want_vbar0)
        out.update(dQ=dQ, dK=dK, dV=dV)
        if want_vbar0:
            out["vbar0"] = vb0
    torch.cuda.synchronize()
    res = {}
    for k, val in out.items():
        if isinstance(val, list):
            res[k] = np.stack([x.cpu().numpy() for x in val])
        else:
            res[k] = val.float().cpu().numpy()
    return res


def run_gpu_converge(prob: workloads.Problem, T_max, tol, every, R=None, W=None, backward=True):
    """forward_converge (+ backward at the base length it used).  Returns the
    same dict as run_gpu plus T_used and err_last."""
    import torch

    import entropic_ot_banded_amd as eoba

    R = prob.R if R is None else R
    W = prob.W if W is None else W
    t = to_device(prob)
    O, u, v, ws, T_used, err_last = eoba.forward_converge(
        t["Q"], t["K"], t["V"], W, T_max, R, t["a"], t["b"], tol, every, t["lengths"], prob.dustbin)
    out = {"O": O, "u": u, "v": v}
    us, vs = eoba.tail_stack(ws, t["Q"], R, t["lengths"], prob.dustbin)
    out["us"] = [x.clone() for x in us]
    out["vs"] = [x.clone() for x in vs]
    if backward:
        dQ, dK, dV, _ = eoba.backward(t["Q"], t["K"], t["V"], W, T_used, R, t["a"], t["b"], O, t["dO"],
                                      ws, t["lengths"], prob.dustbin)
        out.update(dQ=dQ, dK=dK, dV=dV)
    torch.cuda.synchronize()
    res = {}
    for k, val in out.items():
        if isinstance(val, list):
            res[k] = np.stack([x.cpu().numpy() for x in val])
        else:
            res[k] = val.float().cpu().numpy()
    res["T_used"] = T_used
    res["err_last"] = err_last
    return res


def run_oracle(prob: workloads.Problem, T=None, R=None, W=None, backward=True, processes=None):
    T = prob.T if T is None else T
    R = prob.R if R is None else R
    W = prob.W if W is None else W
    if processes is None:
        processes = min(16, os.cpu_count() or 1)
    if backward:
        return oracle.forward_backward_batch(prob.Q, prob.K, prob.V, prob.a, prob.b, W, T, R,
                                             prob.dO, prob.lengths, prob.dustbin,
                                             processes=processes)
    return oracle.forward_batch(prob.Q, prob.K, prob.V, prob.a, prob.b, W, T, R, prob.lengths,
                                prob.dustbin, processes=processes)


# Parity bounds.  Normwise relative error ||x - x*|| / ||x*|| over active
# entries (the tolerance the benchmark spec states: 1e-5 on O, u, v and 1e-4 on dQ,
# dK, dV for fp32 inputs; the bf16 bounds follow from P and dS entering the
# bf16 MFMAs as hi + lo pairs, about 16 mantissa bits), and element-wise
# max|x - x*| / max|x*| ("<key>_max"), which an error confined to a few rows
# (band ends, ragged tails, the dustbin row) cannot hide in.
TOL_F32 = {"O": 1e-5, "u": 1e-5, "v": 1e-5, "uv_gauge": 1e-5, "dQ": 1e-4, "dK": 1e-4, "dV": 1e-4,
           "O_max": 4e-5, "u_max": 2e-5, "v_max": 4e-5, "dQ_max": 4e-4, "dK_max": 4e-4, "dV_max": 4e-4}
TOL_BF16 = {"O": 1e-4, "u": 1e-4, "v": 1e-4, "uv_gauge": 1e-4, "dQ": 1e-3, "dK": 1e-3, "dV": 1e-3,
            "O_max": 4e-4, "u_max": 2e-4, "v_max": 4e-4, "dQ_max": 4e-3, "dK_max": 4e-3, "dV_max": 4e-3}
# v is held to its own per-tensor bound unless ||v*|| < V_SMALL * ||u*||:
# then v is a small remainder of the potential pair (uniform marginals put
# the scale in u), its relative error measures only the absolute rounding of
# the pair, and it is bounded against the pair's scale instead (v_pair).
V_SMALL = 0.1


def max_rel_err(x, ref, mask=None, scale=None):
    """Element-wise max|x - ref| / max|ref| over finite reference entries
    (and `mask`); `scale` replaces max|ref| when given."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    fin = np.isfinite(ref)
    if mask is not None:
        fin &= mask
    if not fin.any():
        return 0.0
    bad = np.isfinite(x) != np.isfinite(ref)
    if mask is not None:
        bad &= mask
    if bad.any():
        return np.inf
    den = np.abs(ref[fin]).max() if scale is None else scale
    return float(np.abs(x[fin] - ref[fin]).max() / (den if den > 0 else 1.0))


def compare(gpu, ref, prob, keys=("O", "u", "v", "dQ", "dK", "dV")):
    """Relative errors per output over active tokens: normwise (key) and
    element-wise ("<key>_max"); for v also the pair-scaled errors ("v_pair",
    "v_pair_max") and the ratio ||v*|| / ||u*|| ("vu_ratio"); plus the
    gauge-removed potential pair (O and the plans are invariant under
    u + c, v - c)."""
    act = active_mask(prob)
    act_bhl = np.broadcast_to(act[:, None, :], gpu["u"].shape)
    act_rows = np.broadcast_to(act[:, None, :, None], gpu["O"].shape)
    errs = {}
    for k in keys:
        if k not in gpu:
            continue
        if k in ("u", "v"):
            errs[k] = rel_err(gpu[k], ref[k], act_bhl)
            errs[k + "_max"] = max_rel_err(gpu[k], ref[k], act_bhl)
            if k == "v":
                rv = np.asarray(ref["v"], np.float64)[act_bhl]
                ru = np.asarray(ref["u"], np.float64)[act_bhl]
                nv, nu = np.linalg.norm(rv), np.linalg.norm(ru)
                errs["vu_ratio"] = float(nv / nu) if nu > 0 else np.inf
                errs["v_pair"] = errs["v"] * nv / max(nv, nu) if nv > 0 else errs["v"]
                mv = np.abs(rv).max() if rv.size else 0.0
                mu = np.abs(ru).max() if ru.size else 0.0
                errs["v_pair_max"] = max_rel_err(gpu[k], ref[k], act_bhl, scale=max(mv, mu))
        else:
            errs[k] = rel_err(gpu[k], ref[k], act_rows)
            errs[k + "_max"] = max_rel_err(gpu[k], ref[k], act_rows)
            # filler rows must be exactly zero
            if (~act_rows).any():
                assert np.all(gpu[k][~act_rows] == 0), f"{k}: nonzero filler rows"
    if "u" in gpu:
        # gauge-removed pair (u - c, v + c), relative to the raw pair's norm
        gu, gv = gauge_removed(gpu["u"], gpu["v"], act)
        ru, rv = gauge_removed(ref["u"], ref["v"], act)
        num = np.sqrt(np.sum((gu - ru)[act_bhl] ** 2) + np.sum((gv - rv)[act_bhl] ** 2))
        den = np.sqrt(np.sum(np.asarray(ref["u"], np.float64)[act_bhl] ** 2) +
                      np.sum(np.asarray(ref["v"], np.float64)[act_bhl] ** 2))
        errs["uv_gauge"] = float(num / (den if den > 0 else 1.0))
        # inactive potentials are -inf
        assert np.all(np.isneginf(gpu["u"][~act_bhl])) and np.all(np.isneginf(gpu["v"][~act_bhl]))
    return errs


def parity_failures(errs, tol, skip=()):
    """The bounds `errs` violates, as messages.  v takes its own bound when
    ||v*|| >= V_SMALL ||u*||, the pair-scaled one (v_pair, v_pair_max) when v
    is a small remainder of the pair."""
    bad = []
    small_v = errs.get("vu_ratio", np.inf) < V_SMALL
    for k, lim in tol.items():
        if k in skip or k not in errs:
            continue
        val = errs[k]
        if small_v and k in ("v", "v_max"):
            val = errs["v_pair" if k == "v" else "v_pair_max"]
            k = f"{k} (pair-scaled: ||v*|| / ||u*|| = {errs['vu_ratio']:.3f} < {V_SMALL})"
        if not (val <= lim):
            bad.append(f"{k}: {val:.3e} > {lim:.1e}")
    return bad


def assert_parity(errs, tol, label="", skip=()):
    bad = parity_failures(errs, tol, skip)
    assert not bad, f"{label}: " + "; ".join(bad)


def fmt_errs(errs):
    return {k: f"{v:.2e}" for k, v in errs.items()}


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()
