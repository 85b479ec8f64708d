"""The allocation-free forward entry point against dilated_attn_fwd.

dilated_attn_fwd_noalloc takes its workspace from the library's own
per-GPU array. Two calls in a row, the second on a smaller problem, must
each match dilated_attn_fwd on the same inputs bit for bit (the same
kernels run; only the workspace address differs), and the oracle to the
bf16 bars.
"""
import numpy as np
import pytest

import oracle
from sparse_long_sequence_attn_amd import DA_NOALLOC_MAX_WORKSPACE_BYTES, DilatedAttnError
from sparse_long_sequence_attn_amd import dilated_attn, dilated_attn_noalloc, workspace_bytes
from sparse_long_sequence_attn_amd.workloads import random_inputs, to_torch

pytestmark = pytest.mark.gpu


def test_noalloc_matches_the_workspace_entry_point():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    cases = [  # the second is smaller: stale contents of the array must not leak in
        (1, 4096, 8, [(1024, 1), (2048, 2), (4096, 4)], 31),
        (1, 1024, 4, [(256, 1), (512, 2)], 32),
    ]
    for B, N, H, pats, seed in cases:
        need = workspace_bytes(B, N, H, 64, pats, 1)
        assert 0 < need <= DA_NOALLOC_MAX_WORKSPACE_BYTES
        print(f"noalloc: B={B} N={N} H={H} patterns={pats} workspace={need}", flush=True)
        q, k, v = random_inputs(B, N, H, 64, "bf16", seed)
        qt, kt, vt = (to_torch(x) for x in (q, k, v))
        ref_out, ref_lse = dilated_attn(qt, kt, vt, pats)
        out = torch.full_like(qt, float("nan"))
        lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=qt.device)
        dilated_attn_noalloc(qt, kt, vt, pats, out=out, lse=lse)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
        assert torch.equal(lse, ref_lse)
        o_o, l_o = oracle.fwd(q, k, v, pats)
        err = np.abs(out.float().cpu().numpy() - o_o).max()
        fin = np.isfinite(l_o)
        lerr = np.abs(lse.cpu().numpy()[fin] - l_o[fin]).max()
        print(f"noalloc: max|out err| {err:.3e} max|lse err| {lerr:.3e}", flush=True)
        assert err <= 2e-2 and lerr <= 4e-3


def test_noalloc_refuses_problems_beyond_its_array():
    import torch

    x = torch.zeros((1, 1 << 16, 16, 64), dtype=torch.bfloat16, device="cuda")
    pats = [(64, 1), (128, 2)]
    assert workspace_bytes(1, 1 << 16, 16, 64, pats, 1) > DA_NOALLOC_MAX_WORKSPACE_BYTES
    with pytest.raises(DilatedAttnError, match="DA_ERR_WORKSPACE"):
        dilated_attn_noalloc(x, x, x, pats)
    torch.cuda.synchronize()
