"""Float64 CPU oracle for banded differentiable Sinkhorn attention.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; never by the library or its Python
binding.  It is written from the method's description (Blockwise
Differentiable Sinkhorn Attention, sections 2.1-2.3) in plain numpy/scipy,
float64 throughout, and shares no code with the HIP path.

Parity pins (tests/test_oracle_pins.py) tie every function here to something
other than itself: closed forms, marginal invariants, an independent dense
Sinkhorn, pure-Python brute force, finite differences and torch autograd.
"""

from .sinkhorn import (  # noqa: F401
    Grads, Solution, Support, adjoint, backward_batch, band_offsets, bptt_batch,
    col_update, default_processes, forward_backward_batch, forward_batch, output, row_update,
    scores, solve,
)
from .sinkhorn import _Problem as Problem  # noqa: F401
from .sinkhorn import backward_one, bptt_one, forward_one  # noqa: F401
from .sinkhorn import (  # noqa: F401
    base_errors, block_contraction_batch, block_diameters, certificate_batch, certificate_eta, converged_base_length, row_marginal_error,
    select_base_length, select_tail_depth, tail_depth_gradients,
)
