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


def test_concurrent_calls_on_two_streams(torch_cuda):
    """The library holds no state between calls: two different problems
    (different shapes and pattern lists; one runs the 4-wave kernels, the
    other the one-wave kernels of segments of at most 32 rows) enqueued
    alternately on two side streams give the same results as each run
    alone."""
    torch = torch_cuda
    from sparse_long_sequence_attn_amd.workloads import grad_output, random_inputs

    specs = [(2, 2048, 8, [(256, 1), (512, 2), (2048, 4)], True, 21),
             (4, 1024, 6, [(64, 2), (32, 1)], False, 22)]
    probs = []
    for B, N, H, pats, causal, seed in specs:
        q, k, v = (to_torch(x) for x in random_inputs(B, N, H, 64, "bf16", seed))
        dout = to_torch(grad_output(B, N, H, 64, "bf16", seed + 100))
        f = Problem(q, k, v, pats, causal)
        f.run()
        b = BwdProblem(q, k, v, f.out, f.lse, dout, pats, causal)
        b.run()
        torch.cuda.synchronize()
        probs.append((q, k, v, dout, pats, causal,
                      [t.clone() for t in (f.out, f.lse, b.dq, b.dk, b.dv)]))

    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    runs = []
    for s, (q, k, v, dout, pats, causal, _) in zip(streams, probs):
        with torch.cuda.stream(s):
            f = Problem(q, k, v, pats, causal)
            b = BwdProblem(q, k, v, f.out, f.lse, dout, pats, causal)
            runs.append((f, b))
    for rep in range(3):  # alternate the launches between the two streams
        for s, (f, b) in zip(streams, runs):
            with torch.cuda.stream(s):
                f.run()
                b.run()
    torch.cuda.synchronize()
    for i, ((f, b), p) in enumerate(zip(runs, probs)):
        for name, g, e in zip(("out", "lse", "dq", "dk", "dv"), (f.out, f.lse, b.dq, b.dk, b.dv),
                              p[-1]):
            assert torch.equal(g, e), f"problem {i}: {name} differs under concurrency"
        print(f"problem {i}: identical under concurrency", flush=True)
