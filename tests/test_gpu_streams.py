"""Every launch of a call goes on the caller's stream.

The forward and backward passes run once on torch's current (default)
stream and once on a side stream of default priority. On the side stream the
results are copied to pinned host memory by copies enqueued on that same
stream right after the calls, and only that stream is synchronised. The
kernels are deterministic (no atomics), so with every launch ordered on the
side stream the results equal the default-stream ones bit for bit; a launch
left on another stream would race the copies. The workload is large enough
(three patterns, B 4, N 8K, 12 heads) that such a race would show.
"""
import numpy as np
import pytest

from sparse_long_sequence_attn_amd import BwdProblem, Problem
from sparse_long_sequence_attn_amd.workloads import (WORKLOADS, host_inputs, to_torch,
                                                     workload_grad_output)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def test_calls_run_on_the_callers_stream(torch_cuda):
    torch = torch_cuda
    w = WORKLOADS["three_pattern_b4_n8192_h12_bf16"]
    print(f"workload {w.name}", flush=True)
    q, k, v = (to_torch(x) for x in host_inputs(w))
    dout = to_torch(workload_grad_output(w))

    ref = Problem(q, k, v, w.patterns, w.causal)
    ref.run()
    rb = BwdProblem(q, k, v, ref.out, ref.lse, dout, w.patterns, w.causal)
    rb.run()
    torch.cuda.synchronize()
    expect = [t.clone() for t in (ref.out, ref.lse, rb.dq, rb.dk, rb.dv)]

    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd = Problem(q, k, v, w.patterns, w.causal)
        bwd = BwdProblem(q, k, v, fwd.out, fwd.lse, dout, w.patterns, w.causal)
        # outputs start as NaN, so results read before the kernels finish
        # cannot match by accident
        for t in (fwd.out, fwd.lse, bwd.dq, bwd.dk, bwd.dv):
            t.fill_(float("nan"))
        fwd.run()
        bwd.run()
        got = []
        for t in (fwd.out, fwd.lse, bwd.dq, bwd.dk, bwd.dv):
            h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
            h.copy_(t, non_blocking=True)
            got.append(h)
    side.synchronize()

    for name, g, e in zip(("out", "lse", "dq", "dk", "dv"), got, expect):
        same = torch.equal(g, e.cpu())
        print(f"{name}: bit-identical on the side stream: {same}", flush=True)
        assert same, f"{name} differs when computed on a side stream"
    assert not np.isnan(got[0].float().numpy()).any()
