"""Peak probes used for the roofline fractions: sustained rates of the bf16
score MFMA and of v_exp_f32 must be positive and below what the chip's unit
counts allow at its top clock (256 CUs, 2.4 GHz: 2.5 PFLOP/s dense bf16,
at most 64 VALU lanes per CU per clock for exp)."""
import pytest

torch = pytest.importorskip("torch")

import entropic_ot_banded_amd as eoba  # noqa: E402

pytestmark = pytest.mark.gpu


def test_measure_peaks_plausible():
    print("case: sinkattn_measure_peaks on cuda:0", flush=True)
    p = eoba.measure_peaks("cuda:0")
    assert 0.2 * 2.5e15 < p["mfma_bf16_flops"] < 1.05 * 2.5e15, p
    assert 0.2 * 256 * 2.4e9 * 16 < p["exp_per_s"] < 1.05 * 256 * 2.4e9 * 64, p
    assert p["clock_hz"] == 0.0 or 0.5e9 < p["clock_hz"] < 2.6e9, p


def test_measure_lds_read_patterns():
    """The step kernel's K-tile read pattern at several row strides: no
    stride gets more than 256 bytes per clock per CU out of the LDS (at least
    4 cycles per 1 KB wave read), unpadded 256-byte rows conflict heavily,
    and 288-byte rows read faster than the 272-byte ones the kernel uses."""
    print("case: sinkattn_measure_lds on cuda:0", flush=True)
    c = {s: eoba.measure_lds(s, device="cuda:0") for s in (256, 272, 288, 304, 320)}
    cx = eoba.measure_lds(256, swizzle=True, device="cuda:0")
    print("cycles per wave-wide 128-bit read:", c, "xor-swizzled 256:", cx, flush=True)
    for v in list(c.values()) + [cx]:
        assert 3.5 < v < 64.0, (c, cx)
    assert c[256] > 2.0 * c[272], c
    assert c[288] < 0.85 * c[272], c
    assert cx < 0.5 * c[256], (c, cx)
