"""GPU parity of the qk_norm kernels (layer norm of 64-value query and key
rows) against the oracle's written-out layer norm and its backward, element
by element, with ragged row counts (partial passes and blocks).

Tolerance: the attention bars (1e-4 fp32, 2e-2 bf16) relative to each
tensor's scale; the gain and bias gradients are sums over all rows, so each
element also gets tol * ||summands||_2 (the rounding of a long sum grows with
the root of the summed squares).
"""
import numpy as np
import pytest

from oracle import module as om
from sparse_long_sequence_attn_amd import qk_norm_bwd, qk_norm_fwd
from sparse_long_sequence_attn_amd.workloads import bf16_round_bits, to_torch

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def draw(rows, dtype, seed, scale=1.0, shift=0.0):
    x = (np.random.default_rng(seed).standard_normal((rows, 64), dtype=np.float32)
         * np.float32(scale) + np.float32(shift))
    return x if dtype == "f32" else bf16_round_bits(x)


def widen(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def check(name, got, ref, dtype, noise=None):
    scale = max(1.0, float(np.abs(ref).max()))
    allowed = TOL[dtype] * scale + (TOL[dtype] * noise if noise is not None else 0.0)
    worst = float(np.max(np.abs(got - ref) / allowed))
    print(f"{name}: max err / scale = {float(np.abs(got - ref).max()) / scale:.3e}, "
          f"worst / allowed = {worst:.3f}", flush=True)
    assert worst <= 1.0, name


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rows", [1, 7, 33, 1000, 32 * 1024 + 5, 300_001])
def test_qk_norm_matches_oracle(torch_cuda, dtype, rows):
    torch = torch_cuda
    seed = rows * 7 + (dtype == "bf16")
    xq, xk = draw(rows, dtype, seed, 2.0, 0.5), draw(rows, dtype, seed + 1, 0.5, -1.0)
    dyq, dyk = draw(rows, dtype, seed + 2), draw(rows, dtype, seed + 3)
    gq, bq = draw(1, dtype, seed + 4, 0.2, 1.0)[0], draw(1, dtype, seed + 5, 0.2)[0]
    gk, bk = draw(1, dtype, seed + 6, 0.2, 1.0)[0], draw(1, dtype, seed + 7, 0.2)[0]
    t = {n: to_torch(np.ascontiguousarray(v)) for n, v in
         dict(xq=xq, xk=xk, dyq=dyq, dyk=dyk, gq=gq, bq=bq, gk=gk, bk=bk).items()}
    yq, yk = qk_norm_fwd(t["xq"], t["xk"], t["gq"], t["bq"], t["gk"], t["bk"])
    dxq, dxk, dp = qk_norm_bwd(t["xq"], t["xk"], t["dyq"], t["dyk"], t["gq"], t["gk"])
    torch.cuda.synchronize()
    f64 = lambda x: x.double().cpu().numpy()
    for tag, x, g, b, dy, y, dx, dpi in (("q", xq, gq, bq, dyq, yq, dxq, 0),
                                         ("k", xk, gk, bk, dyk, yk, dxk, 1)):
        x64, g64, b64, dy64 = widen(x), widen(g), widen(b), widen(dy)
        ref, xh, inv = om.layer_norm(x64, g64, b64)
        check(f"{dtype} rows={rows} y{tag}", f64(y), ref, dtype)
        rdx, rdg, rdb = om.layer_norm_bwd(dy64, xh, inv, g64)
        check(f"{dtype} rows={rows} dx{tag}", f64(dx), rdx, dtype)
        check(f"{dtype} rows={rows} dgain_{tag}", f64(dp[dpi, 0]), rdg, dtype,
              np.sqrt(((dy64 * xh) ** 2).sum(axis=0)))
        check(f"{dtype} rows={rows} dbias_{tag}", f64(dp[dpi, 1]), rdb, dtype,
              np.sqrt((dy64 ** 2).sum(axis=0)))


def test_qk_norm_bwd_deterministic(torch_cuda):
    torch = torch_cuda
    rows = 123_457
    t = [to_torch(draw(rows, "bf16", 50 + i)) for i in range(4)]
    g = to_torch(draw(1, "bf16", 60, 0.2, 1.0)[0].copy())
    a = qk_norm_bwd(t[0], t[1], t[2], t[3], g, g)
    b = qk_norm_bwd(t[0], t[1], t[2], t[3], g, g)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
