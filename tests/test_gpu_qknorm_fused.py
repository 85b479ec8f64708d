"""GPU parity of the fused qk_norm attention (dilated_attn_fwd_qknorm and
dilated_attn_bwd_qknorm through the C ABI): attention over layer-normalised
q and k, the normalisation done inside the attention kernels, against the
oracle's written-out layer norm, dilated attention and their backward passes
in float64, element by element.

Tolerance: the attention bars (1e-4 fp32, 2e-2 bf16) relative to each
tensor's scale, max |g - g_oracle| <= tol * max(1, max |g_oracle|), for out,
lse, dxq, dxk and dv. In bf16 the normalised q and k rows are rounded to bf16
before they enter the products (relative 2^-9 per value, as the separate
layer-norm kernels' bf16 outputs are), which moves scores and so lse by up to
a few 1e-3: lse gets the output bar here, not the tighter bar of
bf16-exact inputs. The gain and bias gradients are sums over every row, so
each element also gets tol * ||summands||_2 (rounding of a long sum grows
with the root of the summed squares). Outputs are pre-filled with NaN so an
unwritten element fails; rows the pattern does not gather must be exactly
zero in out, dxq, dxk and dv.
"""
import numpy as np
import pytest

import oracle
from oracle import module as om
from sparse_long_sequence_attn_amd import (DilatedAttnError, dilated_attn_qknorm,
                                           dilated_attn_qknorm_bwd, qknorm_fused_supported)
from sparse_long_sequence_attn_amd.workloads import bf16_round_bits, to_torch

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
EPS = 1e-5


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def draw(shape, dtype, rng, scale=1.0, shift=0.0):
    x = rng.standard_normal(shape, dtype=np.float32) * np.float32(scale) + np.float32(shift)
    return x if dtype == "f32" else bf16_round_bits(x)


def widen(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def inputs(B, N, H, dtype, seed):
    """xq, xk with a shift and scale per tensor (so the normalisation has
    work to do), v and dout standard normal, gains 1 + N(0, 0.1^2), biases
    N(0, 0.1^2): one PCG64 stream in that order."""
    rng = np.random.default_rng(seed)
    shape = (B, N, H, 64)
    a = {"xq": draw(shape, dtype, rng, 2.0, 0.5), "xk": draw(shape, dtype, rng, 0.5, -1.0),
         "v": draw(shape, dtype, rng), "dout": draw(shape, dtype, rng)}
    for n in ("gq", "gk"):
        a[n] = draw((64,), dtype, rng, 0.1, 1.0)
    for n in ("bq", "bk"):
        a[n] = draw((64,), dtype, rng, 0.1)
    return a


def oracle_ref(a, patterns, causal):
    w = {n: widen(x) for n, x in a.items()}
    q, xhq, invq = om.layer_norm(w["xq"], w["gq"], w["bq"], EPS)
    k, xhk, invk = om.layer_norm(w["xk"], w["gk"], w["bk"], EPS)
    out, lse = oracle.fwd(q, k, w["v"], patterns, causal=causal)
    dq, dk, dv = oracle.bwd(q, k, w["v"], w["dout"], patterns, causal=causal)
    dxq, dgq, dbq = om.layer_norm_bwd(dq, xhq, invq, w["gq"])
    dxk, dgk, dbk = om.layer_norm_bwd(dk, xhk, invk, w["gk"])
    red = lambda x: np.sqrt((x * x).reshape(-1, 64).sum(axis=0))
    noise = np.stack([np.stack([red(dq * xhq), red(dq)]), np.stack([red(dk * xhk), red(dk)])])
    dpar = np.stack([np.stack([dgq, dbq]), np.stack([dgk, dbk])])
    return {"out": out, "lse": lse, "dxq": dxq, "dxk": dxk, "dv": dv, "dparams": dpar,
            "noise": noise}


def gpu_run(torch, a, patterns, causal):
    t = {n: to_torch(x) for n, x in a.items()}
    nan = float("nan")
    B, N, H, _ = t["xq"].shape
    out = torch.full_like(t["xq"], nan)
    lse = torch.full((B, H, N), nan, dtype=torch.float32, device=out.device)
    dxq, dxk, dv = (torch.full_like(t["xq"], nan) for _ in range(3))
    dpar = torch.full((2, 2, 64), nan, dtype=torch.float32, device=out.device)
    dilated_attn_qknorm(t["xq"], t["xk"], t["v"], t["gq"], t["bq"], t["gk"], t["bk"], patterns,
                        EPS, causal, out=out, lse=lse)
    dilated_attn_qknorm_bwd(t["xq"], t["xk"], t["v"], t["gq"], t["bq"], t["gk"], t["bk"], out,
                            lse, t["dout"], patterns, EPS, causal, dxq=dxq, dxk=dxk, dv=dv,
                            dparams=dpar)
    torch.cuda.synchronize()
    return {"out": host(out), "lse": host(lse), "dxq": host(dxq), "dxk": host(dxk),
            "dv": host(dv), "dparams": host(dpar)}


def check(name, got, ref, dtype, noise=None, label=""):
    assert not np.isnan(got).any(), f"{label} {name}: NaN or unwritten elements"
    scale = max(1.0, float(np.abs(ref).max()))
    allowed = TOL[dtype] * scale + (TOL[dtype] * noise if noise is not None else 0.0)
    worst = float(np.max(np.abs(got - ref) / allowed))
    print(f"{label} {name}: max err / scale = {float(np.abs(got - ref).max()) / scale:.3e}, "
          f"worst / allowed = {worst:.3f}", flush=True)
    assert worst <= 1.0, f"{label} {name}"


def compare(got, ref, dtype, label):
    fin = np.isfinite(ref["lse"])
    assert np.array_equal(np.isfinite(got["lse"]), fin), f"{label}: coverage differs"
    assert np.all(np.isneginf(got["lse"][~fin]))
    unc = ~fin.transpose(0, 2, 1)  # [B, N, H]
    for n in ("out", "dxq", "dxk", "dv"):
        assert np.all(got[n][unc] == 0.0), f"{label}: {n} of uncovered rows not zero"
        check(n, got[n], ref[n], dtype, label=label)
    check("lse", np.where(fin, got["lse"], 0.0), np.where(fin, ref["lse"], 0.0), dtype,
          label=label)
    check("dparams", got["dparams"], ref["dparams"], dtype, ref["noise"], label)


CASES = [
    # B, N, H, w, r, causal, dtype
    (2, 256, 2, 64, 2, True, "f32"),     # the usage pattern, several segments
    (2, 256, 2, 64, 2, False, "bf16"),
    (1, 240, 3, 40, 3, False, "f32"),    # ragged: 14 / 13 / 13 rows, padded keys stay out
    (1, 240, 3, 40, 3, True, "bf16"),
    (3, 96, 4, 32, 1, True, "bf16"),     # 32 rows, dilation 1
    (1, 32, 5, 64, 2, False, "f32"),     # segment longer than the sequence: w' = N
    (2, 200, 2, 8, 1, True, "f32"),      # 8-row segments
    (1, 960, 16, 96, 3, True, "bf16"),   # heads past the dilation: offsets h mod r
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_fused_qknorm_matches_oracle(torch_cuda, case):
    B, N, H, w, r, causal, dtype = case
    pats = [(w, r)]
    label = f"{dtype} B{B} N{N} H{H} {pats} causal={causal}"
    print(label, flush=True)
    a = inputs(B, N, H, dtype, seed=900 + CASES.index(case))
    compare(gpu_run(torch_cuda, a, pats, causal), oracle_ref(a, pats, causal), dtype, label)


def test_fused_qknorm_usage_shape_sampled(torch_cuda):
    """The usage shape (B 32, N 8192, 8 heads, w 64, r 2, bf16, causal):
    every gradient of the gain and bias against the oracle would need the
    whole sequence, so the check takes batch entries 0 and 31 in full
    (whole-sequence oracle on those rows) and compares dparams with the
    separate kernels' backward (qk_norm_bwd after dilated_attn_bwd) at the
    bf16 bar."""
    import torch

    from sparse_long_sequence_attn_amd import (dilated_attn, dilated_attn_bwd, qk_norm_bwd,
                                               qk_norm_fwd)

    B, N, H, pats = 32, 8192, 8, [(64, 2)]
    a = inputs(B, N, H, "bf16", seed=950)
    got = gpu_run(torch_cuda, a, pats, True)
    for b in (0, B - 1):
        sub = {n: (x[b:b + 1] if x.ndim == 4 else x) for n, x in a.items()}
        ref = oracle_ref(sub, pats, True)
        part = {n: got[n][b:b + 1] for n in ("out", "dxq", "dxk", "dv")}
        part["lse"] = got["lse"][b:b + 1]
        for n in ("out", "dxq", "dxk", "dv"):
            check(n, part[n], ref[n], "bf16", label=f"usage b={b}")
        fin = np.isfinite(ref["lse"])
        check("lse", np.where(fin, part["lse"], 0.0), np.where(fin, ref["lse"], 0.0), "bf16",
              label=f"usage b={b}")
    t = {n: to_torch(x) for n, x in a.items()}
    yq, yk = qk_norm_fwd(t["xq"], t["xk"], t["gq"], t["bq"], t["gk"], t["bk"], EPS)
    out, lse = dilated_attn(yq, yk, t["v"], pats)
    dq, dk, _ = dilated_attn_bwd(yq, yk, t["v"], out, lse, t["dout"], pats)
    _, _, dp = qk_norm_bwd(t["xq"], t["xk"], dq, dk, t["gq"], t["gk"], EPS)
    sep = host(dp)
    scale = max(1.0, float(np.abs(sep).max()))
    err = float(np.abs(got["dparams"] - sep).max()) / scale
    print(f"usage dparams vs separate kernels: max err / scale = {err:.3e}", flush=True)
    assert err <= TOL["bf16"]


def test_fused_qknorm_deterministic(torch_cuda):
    a = inputs(2, 512, 4, "bf16", seed=960)
    x = gpu_run(torch_cuda, a, [(64, 2)], True)
    y = gpu_run(torch_cuda, a, [(64, 2)], True)
    for n in x:
        assert np.array_equal(x[n], y[n], equal_nan=True), n


def test_fused_qknorm_rejects_other_patterns(torch_cuda):
    assert qknorm_fused_supported(2, 256, 2, [(64, 2)], 1)
    assert not qknorm_fused_supported(2, 256, 2, [(128, 2)], 1)  # 64 rows per segment
    assert not qknorm_fused_supported(2, 256, 2, [(64, 2), (128, 4)], 1)
    a = inputs(1, 256, 2, "bf16", seed=970)
    t = {n: to_torch(x) for n, x in a.items()}
    with pytest.raises(DilatedAttnError) as e:
        dilated_attn_qknorm(t["xq"], t["xk"], t["v"], t["gq"], t["bq"], t["gk"], t["bk"],
                            [(128, 2)])
    assert e.value.code == -3
    with pytest.raises(DilatedAttnError) as e:
        dilated_attn_qknorm(t["xq"], t["xk"], t["v"], t["gq"], t["bq"], t["gk"], t["bk"],
                            [(64, 2)], eps=0.0)
    assert e.value.code == -9


@pytest.mark.parametrize("parts", [3, 4])
@pytest.mark.parametrize("case", [(2, 256, 2, 64, 2, True, "bf16"), (1, 240, 3, 40, 3, False, "f32")],
                         ids=["usage_pattern", "ragged"])
def test_fused_qknorm_packed_layout(torch_cuda, case, parts):
    """xq, xk, v as parts of one [B, N, parts, H, 64] buffer (row stride
    parts * H * 64; parts = 3 is the module's one-GEMM layout): every output,
    and the gradients written into such a buffer, equal the dense layout's
    bit for bit (the kernels do the same arithmetic on the same values)."""
    torch = torch_cuda
    B, N, H, w, r, causal, dtype = case
    pats = [(w, r)]
    a = inputs(B, N, H, dtype, seed=980 + parts)
    t = {n: to_torch(x) for n, x in a.items()}
    dense = gpu_run(torch, a, pats, causal)
    buf = torch.full((B, N, parts, H, 64), float("nan"), dtype=t["xq"].dtype, device="cuda")
    for i, n in enumerate(("xq", "xk", "v")):
        buf[:, :, i] = t[n]
    xq, xk, v = buf[:, :, 0], buf[:, :, 1], buf[:, :, 2]
    out, lse = dilated_attn_qknorm(xq, xk, v, t["gq"], t["bq"], t["gk"], t["bk"], pats, EPS,
                                   causal)
    gbuf = torch.full_like(buf, float("nan"))
    dxq, dxk, dv, dpar = dilated_attn_qknorm_bwd(xq, xk, v, t["gq"], t["bq"], t["gk"], t["bk"],
                                                 out, lse, t["dout"], pats, EPS, causal,
                                                 dxq=gbuf[:, :, 0], dxk=gbuf[:, :, 1],
                                                 dv=gbuf[:, :, 2])
    torch.cuda.synchronize()
    got = {"out": host(out), "lse": host(lse), "dxq": host(dxq), "dxk": host(dxk),
           "dv": host(dv), "dparams": host(dpar)}
    for n in got:
        assert np.array_equal(got[n], dense[n], equal_nan=True), n
    if parts == 4:  # the fourth part is no one's: untouched
        assert torch.isnan(gbuf[:, :, 3]).all().item()
