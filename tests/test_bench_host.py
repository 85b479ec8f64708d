"""Host-side helpers of bench.py (no GPU): the peak-clock query (against a
stand-in for the HIP runtime) and the parity summary it prints next to the
CPU baseline."""
import ctypes
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402

class _FakeHip:
    """Stands in for the HIP runtime: hipDeviceGetAttribute writes `khz`."""

    def __init__(self, khz, rc=0):
        self.khz, self.rc, self.calls = khz, rc, []

    def hipDeviceGetAttribute(self, ptr, attr, dev):
        self.calls.append((attr, dev))
        ptr._obj.value = self.khz
        return self.rc


def test_max_sclk_from_the_runtime_clock_rate(monkeypatch):
    fake = _FakeHip(2400000)
    monkeypatch.setattr(ctypes, "CDLL", lambda name: fake)
    assert bench.gpu_max_sclk_mhz(0) == 2400
    assert fake.calls == [(5, 0)]  # hipDeviceAttributeClockRate


def test_max_sclk_none_on_a_failed_query(monkeypatch):
    monkeypatch.setattr(ctypes, "CDLL", lambda name: _FakeHip(2400000, rc=1))
    assert bench.gpu_max_sclk_mhz(0) is None
    monkeypatch.setattr(ctypes, "CDLL", lambda name: _FakeHip(0))
    assert bench.gpu_max_sclk_mhz(0) is None


def test_max_sclk_none_without_the_runtime(monkeypatch):
    def missing(name):
        raise OSError(name)
    monkeypatch.setattr(ctypes, "CDLL", missing)
    assert bench.gpu_max_sclk_mhz(0) is None


def test_parity_figures_counts_bf16_spacings():
    # oracle values 0.01 (judged at 1/16: spacing 2^-11), 3 (spacing 2^-6) and
    # 5 (spacing 2^-5); the GPU is off by one spacing at 3 and by half at 5
    out_o = np.array([0.01, 3.0, 5.0])
    out_g = np.array([0.01, 3.0 + 2.0 ** -6, 5.0 - 2.0 ** -6])
    lse_o = np.array([1.0, -np.inf, 2.0])
    lse_g = np.array([1.001, -np.inf, 2.0])
    f = bench.parity_figures(out_g, lse_g, out_o, lse_o)
    assert f["max_abs_err_out"] == 2.0 ** -6
    assert f["max_err_out_bf16_spacings_min_x_1_16"] == 1.0
    assert f["count_abs_oracle_ge_4"] == 1
    assert abs(f["max_abs_err_lse"] - 1e-3) < 1e-12
    assert f["lse_inf_match"] and f["elements_compared"] == 3
    lse_g[1] = 0.0  # a row the oracle leaves uncovered but the GPU does not
    assert not bench.parity_figures(out_g, lse_g, out_o, lse_o)["lse_inf_match"]
