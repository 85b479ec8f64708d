"""GPU parity of the DilatedAttention module (projections, optional
qk_norm, the library's dilated attention, output projection) against the
module oracle in float64: the output and every gradient (input, the four
projection weights, biases, layer-norm gains and biases), element by
element, on the parameter and input values the GPU module actually holds.

Tolerance: the attention bars (1e-4 fp32, 2e-2 bf16) relative to each
tensor's scale, max |g - g_oracle| <= tol * max(1, max |g_oracle|). In bf16
every projection output, layer-norm output and gradient is rounded to bf16
(relative <= 2^-8), on top of the attention kernels' own rounding.

Parameter gradients are sums over all B * N rows. Each summand carries an
error of up to tol of its own scale with independent signs, so the sum's
error grows with the root of the summed squares, not with the sum itself;
each parameter-gradient element is allowed tol * ||summands||_2 on top of
the bar above. This matters where the exact sum is zero: adding one vector
to every key leaves every softmax unchanged, so the key-side biases (the
projection's and the layer norm's) have exactly zero gradient, and the GPU
value is the rounding left over from summing 10^3 to 10^6 bf16 rows.
"""
import numpy as np
import pytest

from oracle import module as om
from sparse_long_sequence_attn_amd.workloads import module_params, module_x

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


PARAM_OF = {"wq": "to_q.weight", "wk": "to_k.weight", "wv": "to_v.weight", "wo": "to_out.weight",
            "bq": "to_q.bias", "bk": "to_k.bias", "bv": "to_v.bias", "bo": "to_out.bias",
            "q_gain": "q_norm.weight", "q_bias": "q_norm.bias", "k_gain": "k_norm.weight",
            "k_bias": "k_norm.bias"}


def run_case(torch, B, N, heads, sizes, rates, qk_norm, bias, causal, dtype, seed):
    from sparse_long_sequence_attn_amd.module import DilatedAttention

    dim = heads * 64
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    mod = DilatedAttention(dim, heads, rates, sizes, qk_norm=qk_norm, causal=causal, bias=bias,
                           device="cuda", dtype=tdt)
    params = module_params(dim, heads, qk_norm, bias, seed)
    named = dict(mod.named_parameters())
    with torch.no_grad():
        for k, v in params.items():
            if v is not None:
                named[PARAM_OF[k]].copy_(torch.from_numpy(v))
    x = torch.from_numpy(module_x(B, N, dim, seed + 1)).to("cuda", tdt).requires_grad_()
    dy = torch.from_numpy(module_x(B, N, dim, seed + 2)).to("cuda", tdt)
    y = mod(x)
    y.backward(dy)
    torch.cuda.synchronize()

    # the oracle sees the values the GPU module holds, widened exactly
    f64 = lambda t: t.detach().double().cpu().numpy()
    p64 = {k: (f64(named[PARAM_OF[k]]) if v is not None else None) for k, v in params.items()}
    y_o, cache = om.module_fwd(f64(x), p64, heads, list(mod.patterns), qk_norm, causal)
    dx_o, g_o, l2 = om.module_bwd(f64(dy), cache, terms=True)

    def check(name, got, ref, noise=None):
        assert not np.isnan(got).any(), f"{name}: NaN"
        scale = max(1.0, float(np.abs(ref).max()))
        tol = TOL[dtype]
        allowed = tol * scale + (tol * noise if noise is not None else 0.0)
        worst = float(np.max(np.abs(got - ref) / allowed))
        err = float(np.abs(got - ref).max()) / scale
        print(f"{dtype} B{B} N{N} H{heads} {mod.patterns} qk_norm={qk_norm} bias={bias} "
              f"{name}: max err / scale = {err:.3e} (scale {scale:.3g}), "
              f"worst error / allowed = {worst:.3f}", flush=True)
        assert worst <= 1.0, f"{name}: error {err}"

    check("y", f64(y), y_o)
    check("dx", f64(x.grad), dx_o)
    for k in g_o:
        check("d" + k, f64(named[PARAM_OF[k]].grad), g_o[k], l2[k])


CASES = [
    # B, N, heads, sizes, rates, qk_norm, bias, causal, dtype
    (2, 256, 2, [64, 128], [2, 1], True, False, True, "f32"),
    (2, 256, 2, [64, 128], [2, 1], True, True, True, "bf16"),
    (1, 512, 4, 128, 4, False, True, False, "bf16"),
    (1, 512, 4, [128, 256, 512], [1, 2, 4], True, False, True, "bf16"),
    (1, 384, 3, [96, 384], [3, 6], False, False, True, "f32"),
    # one pattern of at most 32 rows per segment: qk_norm inside the attention kernels
    (2, 256, 2, 64, 2, True, False, True, "f32"),
    (1, 240, 3, 40, 3, True, True, False, "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=[f"m{i}" for i in range(len(CASES))])
def test_module_small(torch_cuda, case):
    run_case(torch_cuda, *case, seed=300 + CASES.index(case))


def test_module_readme_usage_shape(torch_cuda):
    """The README's usage example at full size: dim 512, 8 heads,
    dilation_rate 2, segment_size 64, qk_norm, batch 32, sequence 8192."""
    run_case(torch_cuda, 32, 8192, 8, 64, 2, True, False, True, "bf16", seed=400)


def test_module_rejects_bad_config(torch_cuda):
    from sparse_long_sequence_attn_amd.module import DilatedAttention

    with pytest.raises(ValueError):
        DilatedAttention(500, 8, 2, 64)
    with pytest.raises(ValueError):
        DilatedAttention(512, 8, [2, 4], [64])
