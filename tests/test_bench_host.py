"""Host-side helpers of bench.py (no GPU): the GPU clock parser and the
parity summary it prints next to the CPU baseline."""
import os
import subprocess
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402

ROCMINFO = """*******
Agent 1
*******
  Name:                    AMD EPYC 9575F 64-Core Processor
  Max Clock Freq. (MHz):   3300
*******
Agent 2
*******
  Name:                    gfx950
  Marketing Name:          AMD Instinct MI355X
  Max Clock Freq. (MHz):   2400
  ISA Info:
    ISA 1
      Name:                    amdgcn-amd-amdhsa--gfx950:sramecc+:xnack-
"""


class _Done:
    def __init__(self, stdout):
        self.stdout = stdout


def test_max_sclk_is_the_gpu_agents(monkeypatch):
    monkeypatch.setattr(subprocess, "run", lambda *a, **k: _Done(ROCMINFO))
    assert bench.gpu_max_sclk_mhz() == 2400


def test_max_sclk_absent_without_a_gfx950_agent(monkeypatch):
    cpu_only = ROCMINFO.split("*******\nAgent 2")[0]
    monkeypatch.setattr(subprocess, "run", lambda *a, **k: _Done(cpu_only))
    assert bench.gpu_max_sclk_mhz() is None


def test_max_sclk_when_rocminfo_is_missing(monkeypatch):
    def missing(*a, **k):
        raise FileNotFoundError("rocminfo")
    monkeypatch.setattr(subprocess, "run", missing)
    assert bench.gpu_max_sclk_mhz() is None


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
