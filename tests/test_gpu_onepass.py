"""GPU parity of the one-pass forward (dilated_attn_fwd_onepass through the C
ABI: every covering pattern's keys in one online softmax, no workspace, no
merge pass) against the fp64 oracle, element by element, on the same seeded
inputs and with the bars of the two-kernel forward: max |out error| <= 2e-2
and max |lse error| <= 4e-3 for bf16 (the derivation is in
test_gpu_parity.py: the kernel sums the bf16-rounded probabilities it feeds to
the PV product). Rows no pattern gathers must hold exactly 0 and -inf;
outputs are pre-filled with NaN so an element the kernel never writes fails.

The cases cover the grouping the kernel relies on: residues mod lcm(r) that
do not divide the window gcd(w') (ragged groups), residues no pattern
covers, dilation rates that do not divide the segment length (2731 / 2730
rows per head), one pattern, w > N, causal and not, and the paper's
five-pattern mixture at its full size.
"""
import numpy as np
import pytest

import oracle
from sparse_long_sequence_attn_amd import DilatedAttnError, dilated_attn, dilated_attn_onepass
from sparse_long_sequence_attn_amd.workloads import WORKLOADS, host_inputs, random_inputs, to_torch

pytestmark = pytest.mark.gpu

TOL_OUT, TOL_LSE = 2e-2, 4e-3


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def run_onepass(torch, q, k, v, patterns, causal=True):
    qt, kt, vt = (to_torch(x) for x in (q, k, v))
    B, N, H, _ = qt.shape
    out = torch.full_like(qt, float("nan"))
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=qt.device)
    dilated_attn_onepass(qt, kt, vt, patterns, causal=causal, out=out, lse=lse)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def compare(out_g, lse_g, out_o, lse_o, label):
    assert not np.isnan(out_g).any(), f"{label}: unwritten output elements"
    assert not np.isnan(lse_g).any(), f"{label}: unwritten lse elements"
    fin = np.isfinite(lse_o)
    assert np.array_equal(np.isfinite(lse_g), fin), f"{label}: coverage differs"
    assert np.all(np.isneginf(lse_g[~fin]))
    assert np.all(out_g.transpose(0, 2, 1, 3)[~fin] == 0.0), f"{label}: uncovered rows not zero"
    err = float(np.abs(out_g - out_o).max())
    lerr = float(np.abs(lse_g[fin] - lse_o[fin]).max()) if fin.any() else 0.0
    print(f"{label}: max|out err| = {err:.3e}, max|lse err| = {lerr:.3e}, "
          f"uncovered rows {int((~fin).sum())}", flush=True)
    assert err <= TOL_OUT, f"{label}: out error {err}"
    assert lerr <= TOL_LSE, f"{label}: lse error {lerr}"


CASES = [
    # B, N, H, patterns, causal
    (1, 256, 4, [(64, 1), (128, 2)], True),                        # lcm 2, gcd 64
    (2, 384, 3, [(96, 3), (384, 6)], True),                        # 16 rows per residue
    (1, 2048, 16, [(128, 1), (256, 2), (512, 4), (1024, 6), (2048, 12)], True),  # ragged
    (1, 512, 4, [(128, 2), (512, 4)], False),                      # non-causal
    (2, 256, 4, [(64, 2), (128, 4)], True),                        # uncovered residues
    (1, 1024, 2, [(256, 4)], True),                                # one pattern
    (1, 512, 3, [(4096, 2), (128, 1)], True),                      # w > N
    (1, 1024, 6, [(1024, 6), (512, 2)], False),                    # r not dividing w'
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_onepass_matches_oracle(torch_cuda, case):
    B, N, H, pats, causal = case
    q, k, v = random_inputs(B, N, H, 64, "bf16", seed=700 + CASES.index(case))
    out_g, lse_g = run_onepass(torch_cuda, q, k, v, pats, causal)
    out_o, lse_o = oracle.fwd(q, k, v, pats, causal=causal)
    compare(out_g, lse_g, out_o, lse_o, f"{case}")


@pytest.mark.parametrize("name", ["three_pattern_b4_n8192_h12_bf16",
                                  "paper_mixture_n32768_h16_bf16"])
def test_onepass_workload_full(torch_cuda, name):
    """The workloads at full size against the oracle, and against the
    two-kernel forward (both within the bar of the oracle)."""
    w = WORKLOADS[name]
    q, k, v = host_inputs(w)
    out_g, lse_g = run_onepass(torch_cuda, q, k, v, w.patterns, w.causal)
    out_o, lse_o = oracle.fwd(q, k, v, w.patterns, causal=w.causal)
    compare(out_g, lse_g, out_o, lse_o, name)
    qt, kt, vt = (to_torch(x) for x in (q, k, v))
    out2, lse2 = dilated_attn(qt, kt, vt, w.patterns, causal=w.causal)
    d = float(np.abs(out2.float().cpu().numpy() - out_g).max())
    print(f"{name}: max|one pass - two kernels| = {d:.3e}", flush=True)
    assert d <= 2 * TOL_OUT


def test_onepass_deterministic(torch_cuda):
    w = WORKLOADS["three_pattern_b4_n8192_h12_bf16"]
    q, k, v = host_inputs(w)
    a = run_onepass(torch_cuda, q, k, v, w.patterns)
    b = run_onepass(torch_cuda, q, k, v, w.patterns)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_onepass_rejects(torch_cuda):
    torch = torch_cuda
    q, k, v = random_inputs(1, 64, 2, 64, "f32", seed=1)
    qt, kt, vt = (to_torch(x) for x in (q, k, v))
    with pytest.raises(DilatedAttnError) as e:
        dilated_attn_onepass(qt, kt, vt, [(64, 2)])
    assert e.value.code == -4  # bf16 only
    qb, kb, vb = (t.to(torch.bfloat16) for t in (qt, kt, vt))
    with pytest.raises(DilatedAttnError) as e:
        dilated_attn_onepass(qb, kb, vb, [(8, 5), (8, 7)])
    assert e.value.code == -3  # lcm(r) = 35 above gcd(w) = 8
