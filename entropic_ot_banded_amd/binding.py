"""ctypes binding of libsinkattn.so (the C-ABI declared in include/sinkattn.h).

Argument marshalling only: every step of the attention runs in the HIP
kernels behind the C-ABI.  torch provides device memory and the current
stream; nothing here computes on tensor values.  If the shared library is
missing the binding raises -- there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsinkattn.so")

SINKATTN_OK = 0
SINKATTN_EINVAL = -1
SINKATTN_EUNSUPPORTED = -2
SINKATTN_EHIP = -3
SINKATTN_EWORKSPACE = -4
SINKATTN_ENONFINITE = -5
SINKATTN_ESTALL = -6
SINKATTN_ESCRATCH = -7
NOALLOC_SCRATCH_BYTES = 64 << 20  # the static device scratch of sinkattn_forward_noalloc
SINKATTN_F32 = 0
SINKATTN_BF16 = 1

EXPORTED = ("sinkattn_workspace_bytes", "sinkattn_tail_offset", "sinkattn_forward",
            "sinkattn_forward_noalloc", "sinkattn_forward_converge", "sinkattn_backward", "sinkattn_tail_certificate",
            "sinkattn_block_contraction", "sinkattn_timing_enable", "sinkattn_timing_collect",
            "sinkattn_status_string", "sinkattn_last_hip_error", "sinkattn_version",
            "sinkattn_measure_peaks", "sinkattn_measure_lds")


class SinkattnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"sinkattn status {status}: {msg}")
        self.status = status


class _Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("L", ctypes.c_int32),
                ("d", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("lengths", ctypes.c_void_p), ("dustbin", ctypes.c_int32)]


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load (once) and type the shared library; raises if it is not built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise FileNotFoundError(
            f"{p} is missing: build it with `python -m entropic_ot_banded_amd.build`")
    lib = ctypes.CDLL(p)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    shp = ctypes.POINTER(_Shape)
    lib.sinkattn_workspace_bytes.argtypes = [shp, i32, i32]
    lib.sinkattn_workspace_bytes.restype = sz
    lib.sinkattn_tail_offset.argtypes = [shp, i32, i32, i32]
    lib.sinkattn_tail_offset.restype = sz
    lib.sinkattn_forward.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp, shp, vp, vp, vp, vp, sz, vp]
    lib.sinkattn_forward.restype = i32
    lib.sinkattn_forward_noalloc.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp, shp, vp, vp, vp, vp]
    lib.sinkattn_forward_noalloc.restype = i32
    lib.sinkattn_forward_converge.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp, shp, ctypes.c_double,
                                              i32, vp, vp, vp, vp, sz, ctypes.POINTER(i32),
                                              ctypes.POINTER(ctypes.c_double), vp]
    lib.sinkattn_forward_converge.restype = i32
    lib.sinkattn_backward.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp, shp, vp, vp, vp, sz,
                                      vp, vp, vp, vp, vp]
    lib.sinkattn_backward.restype = i32
    lib.sinkattn_tail_certificate.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp, shp, vp, vp, vp, sz,
                                              vp, vp, vp, vp, vp, ctypes.POINTER(ctypes.c_double),
                                              ctypes.c_double, ctypes.POINTER(i32), vp]
    lib.sinkattn_tail_certificate.restype = i32
    lib.sinkattn_block_contraction.argtypes = [vp, vp, i32, shp, i32, vp, vp, vp]
    lib.sinkattn_block_contraction.restype = i32
    lib.sinkattn_timing_enable.argtypes = [i32]
    lib.sinkattn_timing_enable.restype = i32
    lib.sinkattn_timing_collect.argtypes = [ctypes.POINTER(ctypes.c_double),
                                            ctypes.POINTER(ctypes.c_longlong)]
    lib.sinkattn_timing_collect.restype = i32
    lib.sinkattn_status_string.argtypes = [i32]
    lib.sinkattn_status_string.restype = ctypes.c_char_p
    lib.sinkattn_last_hip_error.argtypes = []
    lib.sinkattn_last_hip_error.restype = ctypes.c_char_p
    lib.sinkattn_version.argtypes = []
    lib.sinkattn_version.restype = i32
    dp = ctypes.POINTER(ctypes.c_double)
    lib.sinkattn_measure_peaks.argtypes = [dp, dp, dp, vp]
    lib.sinkattn_measure_peaks.restype = i32
    lib.sinkattn_measure_lds.argtypes = [i32, i32, dp, vp]
    lib.sinkattn_measure_lds.restype = i32
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().sinkattn_status_string(status).decode()


def _check(status: int):
    if status != SINKATTN_OK:
        msg = status_string(status)
        if status == SINKATTN_EHIP:
            msg += f" ({load_library().sinkattn_last_hip_error().decode()})"
        raise SinkattnError(status, msg)


@dataclass
class Shape:
    """Problem shape (mirrors sinkattn_shape)."""

    B: int
    H: int
    L: int
    d: int
    dtype: int = SINKATTN_F32
    lengths_ptr: int = 0  # device int32[B] pointer or 0
    dustbin: bool = False

    def c(self) -> _Shape:
        return _Shape(self.B, self.H, self.L, self.d, self.dtype,
                      ctypes.c_void_p(self.lengths_ptr or None), 1 if self.dustbin else 0)


def workspace_bytes(shape: Shape, W: int, R: int) -> int:
    s = shape.c()
    return int(load_library().sinkattn_workspace_bytes(ctypes.byref(s), W, R))


def tail_offset(shape: Shape, R: int, r: int, is_v: bool) -> int:
    s = shape.c()
    return int(load_library().sinkattn_tail_offset(ctypes.byref(s), R, r, 1 if is_v else 0))


def timing_enable(on: bool = True):
    """Start (or stop) per-launch event timing of the fused step kernel."""
    _check(load_library().sinkattn_timing_enable(1 if on else 0))


def timing_collect():
    """(total_ms, launches) of the fused step kernel since the last collect."""
    ms = ctypes.c_double(0.0)
    n = ctypes.c_longlong(0)
    _check(load_library().sinkattn_timing_collect(ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


# ---------------------------------------------------------------------------
# torch-facing wrappers (torch is plumbing: allocation, pointers, streams)
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return SINKATTN_F32
    if t.dtype == torch.bfloat16:
        return SINKATTN_BF16
    raise TypeError(f"Q/K/V/dO must be float32 or bfloat16, got {t.dtype}")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(None)


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _shape_of(Q, lengths, dustbin) -> Shape:
    B, H, L, d = Q.shape
    lp = 0
    if lengths is not None:
        lp = lengths.data_ptr()
    return Shape(B, H, L, d, _dtype_code(Q), lp, bool(dustbin))


def _validate(Q, K, V, a, b, lengths):
    torch = _torch()
    for name, t in (("Q", Q), ("K", K), ("V", V)):
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise ValueError(f"{name} must be a contiguous 4-D device tensor [B, H, L, d]")
        if t.shape != Q.shape or t.dtype != Q.dtype:
            raise ValueError(f"{name} must match Q in shape and dtype")
    B, H, L, d = Q.shape
    for name, t in (("a", a), ("b", b)):
        if t.dtype != torch.float32 or tuple(t.shape) != (B, L) or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 device tensor [B, L]")
    if lengths is not None:
        if lengths.dtype != torch.int32 or tuple(lengths.shape) != (B,) or not lengths.is_cuda:
            raise ValueError("lengths must be an int32 device tensor [B]")


def forward(Q, K, V, W: int, T: int, R: int, a, b, lengths=None, dustbin: bool = False,
            workspace=None):
    """Run the forward pass.  Returns (O, u, v, workspace).

    Q, K, V: [B, H, L, d] float32 or bfloat16 device tensors; a, b: float32
    [B, L]; lengths: optional int32 [B] (real tokens per sequence).
    The returned workspace (a uint8 device tensor) carries the tail stack to
    `backward`.
    """
    torch = _torch()
    _validate(Q, K, V, a, b, lengths)
    shape = _shape_of(Q, lengths, dustbin)
    nbytes = workspace_bytes(shape, W, R)
    if nbytes == 0:
        raise SinkattnError(SINKATTN_EINVAL, "invalid or unsupported shape/W/R (see the envelope in sinkattn.h)")
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=Q.device)
    B, H, L, d = Q.shape
    O = torch.empty((B, H, L, d), dtype=torch.float32, device=Q.device)
    u = torch.empty((B, H, L), dtype=torch.float32, device=Q.device)
    v = torch.empty((B, H, L), dtype=torch.float32, device=Q.device)
    s = shape.c()
    st = load_library().sinkattn_forward(
        _ptr(Q), _ptr(K), _ptr(V), W, T, R, _ptr(a), _ptr(b), ctypes.byref(s), _ptr(O), _ptr(u),
        _ptr(v), _ptr(workspace), workspace.numel(), _stream(Q.device))
    _check(st)
    return O, u, v, workspace


def forward_noalloc(Q, K, V, W: int, T: int, R: int, a, b, lengths=None, dustbin: bool = False, out=None):
    """Forward pass through sinkattn_forward_noalloc: the library allocates
    nothing (its static per-GPU scratch replaces the workspace; no tail stack
    is returned, so there is no backward from it).  `out` = (O, u, v) lets
    the caller supply the outputs; otherwise torch allocates them here.
    Returns (O, u, v)."""
    torch = _torch()
    _validate(Q, K, V, a, b, lengths)
    shape = _shape_of(Q, lengths, dustbin)
    B, H, L, d = Q.shape
    if out is None:
        out = (torch.empty((B, H, L, d), dtype=torch.float32, device=Q.device),
               torch.empty((B, H, L), dtype=torch.float32, device=Q.device),
               torch.empty((B, H, L), dtype=torch.float32, device=Q.device))
    O, u, v = out
    if (O.shape != (B, H, L, d) or u.shape != (B, H, L) or v.shape != (B, H, L) or
            any(t.dtype != torch.float32 or not t.is_contiguous() for t in out)):
        raise ValueError("out must be contiguous float32 tensors [B, H, L, d], [B, H, L], [B, H, L]")
    s = shape.c()
    st = load_library().sinkattn_forward_noalloc(
        _ptr(Q), _ptr(K), _ptr(V), W, T, R, _ptr(a), _ptr(b), ctypes.byref(s), _ptr(O), _ptr(u), _ptr(v),
        _stream(Q.device))
    _check(st)
    return O, u, v


def forward_converge(Q, K, V, W: int, T_max: int, R: int, a, b, tol: float, check_every: int = 1,
                     lengths=None, dustbin: bool = False, workspace=None):
    """Forward pass whose stopped base ends once every (b, h) problem's L1
    row-marginal error is below `tol` (checked every `check_every` steps, at
    most T_max steps; R >= 1).  Blocks at each check.  Returns
    (O, u, v, workspace, T_used, err_last); pass T_used to `backward`.
    err_last is the largest per-problem error at the last check (None if no
    check ran)."""
    torch = _torch()
    _validate(Q, K, V, a, b, lengths)
    shape = _shape_of(Q, lengths, dustbin)
    nbytes = workspace_bytes(shape, W, R)
    if nbytes == 0:
        raise SinkattnError(SINKATTN_EINVAL, "invalid or unsupported shape/W/R (see the envelope in sinkattn.h)")
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=Q.device)
    B, H, L, d = Q.shape
    O = torch.empty((B, H, L, d), dtype=torch.float32, device=Q.device)
    u = torch.empty((B, H, L), dtype=torch.float32, device=Q.device)
    v = torch.empty((B, H, L), dtype=torch.float32, device=Q.device)
    s = shape.c()
    t_used = ctypes.c_int32(-1)
    err = ctypes.c_double(float("-inf"))  # untouched when no check runs
    st = load_library().sinkattn_forward_converge(
        _ptr(Q), _ptr(K), _ptr(V), W, T_max, R, _ptr(a), _ptr(b), ctypes.byref(s), float(tol),
        int(check_every), _ptr(O), _ptr(u), _ptr(v), _ptr(workspace), workspace.numel(),
        ctypes.byref(t_used), ctypes.byref(err), _stream(Q.device))
    _check(st)
    err_last = None if err.value == float("-inf") else err.value
    return O, u, v, workspace, t_used.value, err_last


def backward(Q, K, V, W: int, T: int, R: int, a, b, O, dO, workspace, lengths=None,
             dustbin: bool = False, want_vbar0: bool = False):
    """Exact tail adjoint.  Returns (dQ, dK, dV, vbar0-or-None)."""
    torch = _torch()
    _validate(Q, K, V, a, b, lengths)
    if dO.shape != Q.shape or dO.dtype != Q.dtype or not dO.is_contiguous():
        raise ValueError("dO must match Q in shape and dtype and be contiguous")
    shape = _shape_of(Q, lengths, dustbin)
    dQ = torch.empty(Q.shape, dtype=torch.float32, device=Q.device)
    dK = torch.empty(Q.shape, dtype=torch.float32, device=Q.device)
    dV = torch.empty(Q.shape, dtype=torch.float32, device=Q.device)
    vbar0 = torch.empty(Q.shape[:3], dtype=torch.float32, device=Q.device) if want_vbar0 else None
    s = shape.c()
    st = load_library().sinkattn_backward(
        _ptr(Q), _ptr(K), _ptr(V), W, T, R, _ptr(a), _ptr(b), ctypes.byref(s), _ptr(O), _ptr(dO),
        _ptr(workspace), workspace.numel(), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(vbar0),
        _stream(Q.device))
    _check(st)
    return dQ, dK, dV, vbar0


def tail_certificate(Q, K, V, W: int, T: int, R_max: int, a, b, O, dO, workspace, lengths=None,
                     dustbin: bool = False, tau: float = 1e-5):
    """Stop-gradient bias certificate of a forward run with tail depth R_max.
    Returns (dQ, dK, dV, eta, R_selected): the gradients at depth R_max,
    eta[R] = ||grad_Rmax - grad_R|| / ||grad_Rmax|| over (dQ, dK) for
    R = 0..R_max, and the depth the library selects for tolerance tau (the
    smallest R with eta[R] < tau, else R_max; see sinkattn_tail_certificate).
    Blocks until done."""
    torch = _torch()
    _validate(Q, K, V, a, b, lengths)
    if dO.shape != Q.shape or dO.dtype != Q.dtype or not dO.is_contiguous():
        raise ValueError("dO must match Q in shape and dtype and be contiguous")
    shape = _shape_of(Q, lengths, dustbin)
    mk = lambda: torch.empty(Q.shape, dtype=torch.float32, device=Q.device)  # noqa: E731
    dQ, dK, dV, sQ, sK = mk(), mk(), mk(), mk(), mk()
    eta = (ctypes.c_double * (R_max + 1))()
    sel = ctypes.c_int32(-1)
    s = shape.c()
    st = load_library().sinkattn_tail_certificate(
        _ptr(Q), _ptr(K), _ptr(V), W, T, R_max, _ptr(a), _ptr(b), ctypes.byref(s), _ptr(O), _ptr(dO),
        _ptr(workspace), workspace.numel(), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(sQ), _ptr(sK), eta, float(tau),
        ctypes.byref(sel), _stream(Q.device))
    _check(st)
    return dQ, dK, dV, [float(x) for x in eta], sel.value


def block_contraction(Q, K, W: int, block: int, lengths=None, dustbin: bool = False):
    """Hilbert projective diameter Delta of every diagonal band block of size
    `block` (see sinkattn_block_contraction).  Returns (delta, kappa), device
    fp32 tensors [B, H, ceil(L / block)]; kappa = tanh(delta / 4) is the
    block's contraction coefficient."""
    torch = _torch()
    if Q.dim() != 4 or K.shape != Q.shape or K.dtype != Q.dtype:
        raise ValueError("Q and K must be [B, H, L, d] of one dtype")
    if not (Q.is_contiguous() and K.is_contiguous()):
        raise ValueError("Q and K must be contiguous")
    if lengths is not None and (lengths.dtype != torch.int32 or lengths.device != Q.device):
        raise ValueError("lengths must be an int32 tensor on Q's device")
    shape = _shape_of(Q, lengths, dustbin)
    B, H, L, _ = Q.shape
    nblk = (L + block - 1) // block if block > 0 else 1  # the library rejects block < 1
    delta = torch.empty((B, H, nblk), dtype=torch.float32, device=Q.device)
    kappa = torch.empty_like(delta)
    s = shape.c()
    st = load_library().sinkattn_block_contraction(_ptr(Q), _ptr(K), W, ctypes.byref(s), block, _ptr(delta),
                                                   _ptr(kappa), _stream(Q.device))
    _check(st)
    return delta, kappa


def measure_peaks(device=None) -> dict:
    """Sustained bf16 score-MFMA flop/s, v_exp_f32 results/s and the shader
    clock on `device` (see sinkattn_measure_peaks); blocks for about 50 ms."""
    torch = _torch()
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    mfma, ex, clk = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    with torch.cuda.device(dev):
        st = load_library().sinkattn_measure_peaks(ctypes.byref(mfma), ctypes.byref(ex), ctypes.byref(clk),
                                                   _stream(dev))
    _check(st)
    return {"mfma_bf16_flops": mfma.value, "exp_per_s": ex.value, "clock_hz": clk.value}


def measure_lds(row_stride: int, swizzle: bool = False, device=None) -> float:
    """Shader cycles per wave-wide 128-bit LDS read per CU for the step
    kernel's K-tile read pattern with the given row stride (see
    sinkattn_measure_lds); blocks for a few ms."""
    torch = _torch()
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    cyc = ctypes.c_double()
    with torch.cuda.device(dev):
        st = load_library().sinkattn_measure_lds(int(row_stride), 1 if swizzle else 0, ctypes.byref(cyc),
                                                 _stream(dev))
    _check(st)
    return cyc.value


def tail_stack(workspace, Q, R: int, lengths=None, dustbin=False):
    """Views (u^(0..R), v^(0..R)) of the fp64 tail stack inside a forward
    workspace (log2 units: natural potential times log2(e); filler entries
    unspecified)."""
    torch = _torch()
    shape = _shape_of(Q, lengths, dustbin)
    B, H, L, _ = Q.shape
    n = B * H * L
    us, vs = [], []
    for r in range(R + 1):
        for is_v, dst in ((False, us), (True, vs)):
            off = tail_offset(shape, R, r, is_v)
            dst.append(workspace[off:off + 8 * n].view(torch.float64).view(B, H, L))
    return us, vs
