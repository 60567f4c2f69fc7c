"""C-ABI checks that need no GPU: the library loads, exports every function
include/sinkattn.h declares, and rejects bad arguments on the host before
enqueueing any work."""

import ctypes
import os
import re

import pytest

import entropic_ot_banded_amd as eoba
from entropic_ot_banded_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sinkattn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from entropic_ot_banded_amd import build
        build.build()
    return eoba.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(sinkattn_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_expected_api():
    assert _declared_functions() == sorted(binding.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_status_strings_and_version(lib):
    assert eoba.status_string(0) == "ok"
    for code in (-1, -2, -3, -4, -5, -6, -7):
        assert eoba.status_string(code) not in ("ok", "unknown status")
    assert eoba.status_string(12345) == "unknown status"
    assert lib.sinkattn_version() >= 10000


def _shape(**kw):
    base = dict(B=1, H=2, L=256, d=64, dtype=binding.SINKATTN_F32, lengths_ptr=0, dustbin=False)
    base.update(kw)
    return binding.Shape(**base)


def test_workspace_is_linear_in_length(lib):
    """Extra device memory is O(L) (no L x W or L x L buffer)."""
    w1 = eoba.workspace_bytes(_shape(L=4096), 128, 2)
    w2 = eoba.workspace_bytes(_shape(L=8192), 128, 2)
    assert 1.9 < w2 / w1 < 2.1
    BHL = 2 * 4096
    # fp64 tail stack (2R+2 vectors) + O(1) vectors per token, far below W
    # floats per token
    assert w1 < 48 * BHL * 4
    assert w1 >= (2 * 2 + 2) * BHL * 8


def test_workspace_rejects_invalid(lib):
    assert eoba.workspace_bytes(_shape(d=48), 128, 2) == 0          # unsupported d
    assert eoba.workspace_bytes(_shape(), 0, 2) == 0                # W < 1
    assert eoba.workspace_bytes(_shape(), 128, -1) == 0             # R < 0
    assert eoba.workspace_bytes(_shape(L=0), 128, 2) == 0
    assert eoba.workspace_bytes(_shape(dtype=7), 128, 2) == 0
    assert eoba.workspace_bytes(_shape(), 600, 2) == 0              # band too wide for the tiles
    assert eoba.workspace_bytes(_shape(dtype=binding.SINKATTN_BF16, d=16), 64, 2) == 0
    assert eoba.workspace_bytes(_shape(dustbin=True), 64, 2) == 0   # dustbin needs lengths


def test_band_envelope(lib):
    """The half-widths are clamped to L - 1 and at most 17 tiles of 16 fit: any W
    up to 257, and dense bands (W >= 2L - 1) only while L <= 129."""
    assert eoba.workspace_bytes(_shape(), 257, 2) > 0
    assert eoba.workspace_bytes(_shape(), 258, 2) == 0
    assert eoba.workspace_bytes(_shape(L=129), 2 * 129 - 1, 2) > 0
    assert eoba.workspace_bytes(_shape(L=129), 10000, 2) > 0
    assert eoba.workspace_bytes(_shape(L=130), 2 * 130 - 1, 2) == 0
    assert eoba.workspace_bytes(_shape(L=185), 2 * 185 - 1, 2) == 0


def test_tail_offsets(lib):
    s = _shape(L=100)
    BHL = 1 * 2 * 100
    assert eoba.tail_offset(s, 2, 0, False) == 0
    assert eoba.tail_offset(s, 2, 2, False) == 2 * BHL * 8   # fp64 slots
    assert eoba.tail_offset(s, 2, 0, True) >= 3 * BHL * 8
    assert eoba.tail_offset(s, 2, 3, False) == ctypes.c_size_t(-1).value


def _fwd(lib, shape, W=64, T=3, R=2, ws_bytes=None, null=None, misalign=0):
    fake = 0x10000  # never dereferenced: validation fails first
    ptrs = {k: ctypes.c_void_p(fake) for k in ("Q", "K", "V", "a", "b", "O", "u", "v", "ws")}
    if null:
        ptrs[null] = ctypes.c_void_p(None)
    if misalign:
        ptrs["Q"] = ctypes.c_void_p(fake + misalign)
    s = shape.c()
    nb = eoba.workspace_bytes(shape, W, R) if ws_bytes is None else ws_bytes
    return lib.sinkattn_forward(ptrs["Q"], ptrs["K"], ptrs["V"], W, T, R, ptrs["a"], ptrs["b"],
                                ctypes.byref(s), ptrs["O"], ptrs["u"], ptrs["v"], ptrs["ws"], nb,
                                ctypes.c_void_p(None))


def test_forward_validation_before_launch(lib):
    sh = _shape()
    for name in ("Q", "K", "V", "a", "b", "O", "u", "v", "ws"):
        assert _fwd(lib, sh, null=name) == binding.SINKATTN_EINVAL, name
    assert _fwd(lib, sh, W=0) == binding.SINKATTN_EINVAL
    assert _fwd(lib, sh, T=-1) == binding.SINKATTN_EINVAL
    assert _fwd(lib, sh, R=-2) == binding.SINKATTN_EINVAL
    assert _fwd(lib, sh, misalign=4) == binding.SINKATTN_EINVAL
    assert _fwd(lib, _shape(d=40)) == binding.SINKATTN_EUNSUPPORTED
    assert _fwd(lib, _shape(B=0)) == binding.SINKATTN_EINVAL
    assert _fwd(lib, sh, ws_bytes=1024) == binding.SINKATTN_EWORKSPACE
    # size envelope: B H <= 65535, B H L <= 2^31 - 1, B H L d <= 4 (2^31 - 1),
    # one (b, h) slice under 2 GiB
    assert _fwd(lib, _shape(B=1, H=1, L=2 ** 24, d=128, dtype=binding.SINKATTN_BF16)) == \
        binding.SINKATTN_EUNSUPPORTED
    assert _fwd(lib, _shape(B=256, H=256, L=8)) == binding.SINKATTN_EUNSUPPORTED
    assert _fwd(lib, _shape(B=1, H=2, L=2 ** 30)) == binding.SINKATTN_EUNSUPPORTED
    assert _fwd(lib, _shape(B=1, H=4, L=2 ** 27, d=128, dtype=binding.SINKATTN_BF16)) == \
        binding.SINKATTN_EUNSUPPORTED


def test_forward_converge_validation_before_launch(lib):
    sh = _shape()
    s = sh.c()
    fake = ctypes.c_void_p(0x10000)
    nb = eoba.workspace_bytes(sh, 64, 2)
    t_used = ctypes.c_int32(-7)

    def call(T_max=10, R=2, tol=1e-3, every=2, ws=nb, tu=True):
        return lib.sinkattn_forward_converge(
            fake, fake, fake, 64, T_max, R, fake, fake, ctypes.byref(s), tol, every, fake, fake,
            fake, fake, ws, ctypes.byref(t_used) if tu else None, None, ctypes.c_void_p(None))

    assert call(R=0) == binding.SINKATTN_EINVAL       # the check rides on a tail step
    assert call(every=0) == binding.SINKATTN_EINVAL
    assert call(tol=-1.0) == binding.SINKATTN_EINVAL
    assert call(tol=float("nan")) == binding.SINKATTN_EINVAL
    assert call(T_max=-1) == binding.SINKATTN_EINVAL
    assert call(tu=False) == binding.SINKATTN_EINVAL
    assert call(ws=1024) == binding.SINKATTN_EWORKSPACE
    assert t_used.value == -7  # nothing written on a rejected call


def test_backward_validation_before_launch(lib):
    sh = _shape()
    s = sh.c()
    fake = ctypes.c_void_p(0x10000)
    nb = eoba.workspace_bytes(sh, 64, 2)
    args = [fake, fake, fake, 64, 3, 2, fake, fake, ctypes.byref(s), fake, fake, fake, nb,
            fake, fake, fake, ctypes.c_void_p(None), ctypes.c_void_p(None)]
    bad = list(args)
    bad[10] = ctypes.c_void_p(None)  # dO
    assert lib.sinkattn_backward(*bad) == binding.SINKATTN_EINVAL
    bad = list(args)
    bad[5] = 9  # R beyond the backward's tail limit
    assert lib.sinkattn_backward(*bad) == binding.SINKATTN_EUNSUPPORTED
    bad = list(args)
    bad[12] = 16  # workspace too small
    assert lib.sinkattn_backward(*bad) == binding.SINKATTN_EWORKSPACE


def test_timing_collect_without_launches(lib):
    eoba.timing_enable(True)
    assert eoba.timing_collect() == (0.0, 0)
    eoba.timing_enable(False)
    assert lib.sinkattn_timing_collect(None, None) == binding.SINKATTN_EINVAL


def test_binding_refuses_missing_library(tmp_path):
    with pytest.raises(FileNotFoundError):
        binding.load_library(str(tmp_path / "nope.so"))


def test_certificate_validation_before_launch(lib):
    sh = _shape()
    s = sh.c()
    fake = ctypes.c_void_p(0x10000)
    nb = eoba.workspace_bytes(sh, 64, 2)
    eta = (ctypes.c_double * 9)()
    sel = ctypes.c_int32(-3)

    def call(R_max=2, tau=1e-5, e=eta):
        return lib.sinkattn_tail_certificate(fake, fake, fake, 64, 3, R_max, fake, fake, ctypes.byref(s), fake, fake,
                                             fake, nb, fake, fake, fake, fake, fake, e, tau, ctypes.byref(sel),
                                             ctypes.c_void_p(None))

    assert call(R_max=0) == binding.SINKATTN_EINVAL
    assert call(R_max=9) == binding.SINKATTN_EUNSUPPORTED
    assert call(tau=-1.0) == binding.SINKATTN_EINVAL
    assert call(tau=float("nan")) == binding.SINKATTN_EINVAL
    assert call(e=None) == binding.SINKATTN_EINVAL
    assert sel.value == -3  # nothing written on a rejected call


def test_forward_noalloc_validation_before_launch(lib):
    """The no-allocation forward rejects bad arguments and shapes whose
    workspace exceeds its static scratch before anything is enqueued."""
    fake = ctypes.c_void_p(0x10000)

    def call(shape, W=64, T=3, R=2, Q=fake):
        s = shape.c()
        return lib.sinkattn_forward_noalloc(Q, fake, fake, W, T, R, fake, fake, ctypes.byref(s), fake, fake, fake,
                                            ctypes.c_void_p(None))

    assert call(_shape(), Q=ctypes.c_void_p(None)) == binding.SINKATTN_EINVAL
    assert call(_shape(), W=0) == binding.SINKATTN_EINVAL
    assert call(_shape(), R=-1) == binding.SINKATTN_EINVAL
    assert call(_shape(d=40)) == binding.SINKATTN_EUNSUPPORTED
    big = _shape(B=1, H=64, L=32768, d=128, dtype=binding.SINKATTN_BF16)
    assert eoba.workspace_bytes(big, 256, 2) > binding.NOALLOC_SCRATCH_BYTES
    assert call(big, W=256) == binding.SINKATTN_ESCRATCH
    long_ctx = _shape(B=1, H=8, L=32768, d=128, dtype=binding.SINKATTN_BF16)
    assert eoba.workspace_bytes(long_ctx, 256, 4) <= binding.NOALLOC_SCRATCH_BYTES


def test_measure_lds_validation(lib):
    c = ctypes.c_double()
    assert lib.sinkattn_measure_lds(288, 0, None, None) == binding.SINKATTN_EINVAL
    for stride, swizzle in ((280, 0), (336, 0), (240, 0), (272, 1), (256, 2)):
        assert lib.sinkattn_measure_lds(stride, swizzle, ctypes.byref(c), None) == binding.SINKATTN_EINVAL
