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
