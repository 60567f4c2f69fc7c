"""torch.autograd wrapper: forward/backward both call the C-ABI kernels.

Gradients flow to Q, K and V (the marginals a, b are treated as constants);
the backward is the exact adjoint of the R tail steps with the stopped base
held constant.
"""

from __future__ import annotations

from . import binding


def _make_function():
    import torch

    class _SinkhornAttention(torch.autograd.Function):
        @staticmethod
        def forward(ctx, Q, K, V, a, b, W, T, R, lengths, dustbin, tol, check_every):
            Q, K, V = Q.contiguous(), K.contiguous(), V.contiguous()
            if tol is None:
                O, u, v, ws = binding.forward(Q, K, V, W, T, R, a, b, lengths, dustbin)
            else:
                O, u, v, ws, T, _ = binding.forward_converge(Q, K, V, W, T, R, a, b, tol, check_every,
                                                             lengths, dustbin)
            ctx.save_for_backward(Q, K, V, a, b, O, ws, *( [lengths] if lengths is not None else []))
            ctx.cfg = (W, T, R, lengths is not None, dustbin)
            ctx.mark_non_differentiable(u, v)
            return O, u, v

        @staticmethod
        def backward(ctx, dO, du, dv):
            W, T, R, has_len, dustbin = ctx.cfg
            saved = ctx.saved_tensors
            Q, K, V, a, b, O, ws = saved[:7]
            lengths = saved[7] if has_len else None
            dO = dO.to(Q.dtype).contiguous()
            dQ, dK, dV, _ = binding.backward(Q, K, V, W, T, R, a, b, O, dO, ws, lengths, dustbin)
            return (dQ.to(Q.dtype), dK.to(K.dtype), dV.to(V.dtype), None, None, None, None, None,
                    None, None, None, None)

    return _SinkhornAttention


_FN = None


def sinkhorn_attention(Q, K, V, a, b, W: int, T: int, R: int = 2, lengths=None,
                       dustbin: bool = False, tol=None, check_every: int = 5):
    """Differentiable banded Sinkhorn attention; returns (O, u, v).

    With `tol` set, T is the largest base length and the base stops once the
    row-marginal L1 error of every problem is below tol (checked every
    `check_every` steps; see binding.forward_converge)."""
    global _FN
    if _FN is None:
        _FN = _make_function()
    return _FN.apply(Q, K, V, a, b, W, T, R, lengths, dustbin, tol, check_every)
