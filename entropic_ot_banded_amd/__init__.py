"""entropic_ot_banded_amd: banded differentiable Sinkhorn attention on MI355X.

The compute lives in libsinkattn.so (hand-written HIP for gfx950, C-ABI in
include/sinkattn.h).  This package is its thin Python binding plus an
autograd wrapper; torch supplies device memory and streams only.
"""

from .binding import (  # noqa: F401
    EXPORTED, SINKATTN_BF16, SINKATTN_F32, Shape, SinkattnError, backward, block_contraction, forward,
    forward_converge, forward_noalloc, load_library, measure_lds, measure_peaks, status_string, tail_certificate, tail_offset,
    tail_stack, timing_collect, timing_enable, workspace_bytes,
)
from .autograd import sinkhorn_attention  # noqa: F401

__version__ = "1.1.0"
