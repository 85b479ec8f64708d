"""The forward and backward calls write only inside the workspace they are
given. Each call gets exactly the size dilated_attn_workspace_bytes /
dilated_attn_bwd_workspace_bytes report, cut from a larger buffer whose 64 KiB
before and after it are filled with a fixed byte; after the call (and a
synchronisation) both guards must be unchanged. The cases cover the partial
layouts of both dtypes (the backward partials take the gradients' dtype, so
a bf16 workspace is smaller), the 4-wave and the one-wave (segments of at most
32 rows) kernels, ragged row counts and patterns with w > N. Outputs are also
checked against the oracle, so the exact-size workspace is known to suffice.
"""
import numpy as np
import pytest

import oracle
from sparse_long_sequence_attn_amd import BwdProblem, Problem
from sparse_long_sequence_attn_amd._native import bwd_workspace_bytes, workspace_bytes
from sparse_long_sequence_attn_amd.workloads import grad_output, random_inputs, to_torch

pytestmark = pytest.mark.gpu

GUARD = 1 << 16  # bytes; keeps the workspace 256-byte aligned
FILL = 0xA5
TOL = {"f32": 1e-4, "bf16": 2e-2}

CASES = [
    # B, N, H, patterns, causal, dtype
    (1, 512, 4, [(128, 1), (256, 2), (512, 4)], True, "bf16"),
    (1, 512, 4, [(128, 1), (256, 2), (512, 4)], True, "f32"),
    (2, 480, 6, [(480, 6), (160, 1), (96, 2)], False, "bf16"),      # ragged L
    (2, 128, 8, [(32, 1), (64, 2)], True, "bf16"),                  # one-wave kernels
    (1, 96, 3, [(1000, 7), (8, 1), (96, 96)], True, "f32"),         # w > N, L = 1
]


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def guarded(torch, nbytes):
    buf = torch.full((GUARD + max(nbytes, 1) + GUARD,), FILL, dtype=torch.uint8, device="cuda")
    return buf, buf[GUARD:GUARD + max(nbytes, 1)]


def guards_intact(buf, nbytes):
    host = buf.cpu().numpy()
    return bool(np.all(host[:GUARD] == FILL) and np.all(host[GUARD + max(nbytes, 1):] == FILL))


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("case", CASES, ids=[f"w{i}" for i in range(len(CASES))])
def test_calls_stay_inside_their_workspace(torch_cuda, case):
    torch = torch_cuda
    B, N, H, pats, causal, dtype = case
    label = f"{dtype} B{B} N{N} H{H} {pats} causal={causal}"
    print(label, flush=True)
    dcode = 1 if dtype == "bf16" else 0
    q, k, v = random_inputs(B, N, H, 64, dtype, seed=900 + CASES.index(case))
    dout = grad_output(B, N, H, 64, dtype, seed=950 + CASES.index(case))
    qt, kt, vt, dt = (to_torch(x) for x in (q, k, v, dout))

    fws = workspace_bytes(B, N, H, 64, pats, dcode)
    fbuf, fview = guarded(torch, fws)
    prob = Problem(qt, kt, vt, pats, causal, workspace=fview)
    prob.run()
    torch.cuda.synchronize()
    assert guards_intact(fbuf, fws), f"{label}: forward wrote outside its workspace"

    bws = bwd_workspace_bytes(B, N, H, 64, pats, dcode)
    bbuf, bview = guarded(torch, bws)
    bp = BwdProblem(qt, kt, vt, prob.out, prob.lse, dt, pats, causal, workspace=bview)
    bp.run()
    torch.cuda.synchronize()
    assert guards_intact(bbuf, bws), f"{label}: backward wrote outside its workspace"

    out_o, _ = oracle.fwd(q, k, v, pats, causal=causal)
    err = float(np.abs(host(prob.out) - out_o).max())
    assert err <= TOL[dtype], f"{label}: out error {err}"
    for name, g, o in zip(("dq", "dk", "dv"), (bp.dq, bp.dk, bp.dv),
                          oracle.bwd(q, k, v, dout, pats, causal=causal)):
        rel = float(np.abs(host(g) - o).max()) / max(1.0, float(np.abs(o).max()))
        print(f"{label} {name}: max err / scale = {rel:.3e}", flush=True)
        assert rel <= TOL[dtype], f"{label}: {name} error {rel}"
