"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every output element is compared with the fp64 oracle on the same seeded
inputs: max-abs error <= 1e-4 for fp32 inputs and <= 2e-2 for bf16 inputs;
rows that no pattern gathers must hold exactly 0 and -inf. Outputs are
pre-filled with NaN so an element the kernels never write fails the check.

Log-sum-exp tolerance (no figure is given for it, so it is derived): the bf16
kernel sums the bf16-rounded probabilities it feeds to the PV product, so its
row sum carries each term's relative rounding error, at most the bf16 unit
roundoff u = 2^-8 (8-bit significand, round to nearest even), and ln of the
sum is off by at most about u = 3.9e-3. Scores are accumulated in fp32
(relative error ~2^-24 of sum |q_d k_d|) and exp2/log2 add ~1e-6, so 4e-3
for bf16. The fp32 kernel keeps probabilities in fp32: 1e-4.
"""
import math

import numpy as np
import pytest

import oracle
from sparse_long_sequence_attn_amd import Problem, coverage_map, dilated_attn, gather_map
from sparse_long_sequence_attn_amd.workloads import (WORKLOADS, device_inputs, from_torch_bits,
                                                     host_inputs, random_inputs, to_torch)

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-4, 1e-4), "bf16": (2e-2, 4e-3)}


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def run_gpu(torch, q, k, v, patterns, causal=True, scale=None):
    qt, kt, vt = (to_torch(x) for x in (q, k, v))
    B, N, H, Dh = qt.shape
    out = torch.full_like(qt, float("nan"))
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=qt.device)
    dilated_attn(qt, kt, vt, patterns, causal=causal, scale=scale, out=out, lse=lse)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def compare(out_g, lse_g, out_o, lse_o, dtype, label=""):
    tol_o, tol_l = TOL[dtype]
    assert not np.isnan(out_g).any(), f"{label}: unwritten output elements"
    assert not np.isnan(lse_g).any(), f"{label}: unwritten lse elements"
    err = np.abs(out_g - out_o).max()
    fin = np.isfinite(lse_o)
    assert np.array_equal(np.isfinite(lse_g), fin), f"{label}: coverage differs"
    assert np.all(np.isneginf(lse_g[~fin]))
    assert np.all(out_g.transpose(0, 2, 1, 3)[~fin] == 0.0), f"{label}: uncovered rows not zero"
    lerr = np.abs(lse_g[fin] - lse_o[fin]).max() if fin.any() else 0.0
    print(f"{label}: max|out err| = {err:.3e}, max|lse err| = {lerr:.3e}", flush=True)
    assert err <= tol_o, f"{label}: out error {err}"
    assert lerr <= tol_l, f"{label}: lse error {lerr}"
    return err


# ---------------------------------------------------------------- small shapes, every code path

SMALL_CASES = [
    # (B, N, H, patterns, causal, scale) - comments name the path exercised
    (2, 256, 3, [(256, 1)], True, None),                  # one segment, two 128-row tiles
    (1, 384, 2, [(384, 1)], False, None),                 # non-causal, three tiles
    (2, 200, 5, [(200, 3)], True, None),                  # ragged L (67/67/66), odd H
    (1, 512, 4, [(128, 1), (256, 2), (512, 4)], True, None),
    (1, 480, 6, [(480, 6), (160, 1), (96, 2)], True, None),
    (3, 64, 4, [(16, 2), (32, 4), (64, 1)], True, None),
    (2, 128, 8, [(64, 2)], True, None),                   # 32-row path, zero rows written
    (2, 128, 8, [(32, 1), (64, 2)], False, None),         # 32-row path, merge, non-causal
    (1, 96, 4, [(1000, 7), (8, 1), (96, 96)], True, None),  # w > N, r = w (one row)
    (1, 256, 2, [(128, 2)], True, 0.05),                  # explicit scale
    (1, 256, 4, [(256, 16)], True, None),                 # r = 16: 15 zero rows per query
    (1, 4096, 2, [(4096, 1)], True, None),                # 32 query tiles
    (1, 2560, 3, [(2560, 5), (512, 1)], False, None),     # long non-causal with tails
    (2, 192, 7, [(192, 3), (192, 3)], True, None),        # a pattern listed twice
    (1, 512, 3, [(512, 1), (256, 2), (128, 4), (64, 8), (512, 8), (256, 1), (128, 2), (64, 1)],
     True, None),                                          # the maximum of 8 patterns
    # merge over the rows that need it (some pattern has r = 1): patterns
    # that do not nest, a duplicated dense pattern, rates that divide no w
    (1, 600, 3, [(600, 1), (200, 3), (300, 2)], True, None),
    (2, 256, 5, [(64, 1), (64, 1), (256, 4)], False, None),
    (1, 1020, 4, [(1020, 3), (510, 1), (204, 5)], True, None),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", SMALL_CASES, ids=[f"c{i}" for i in range(len(SMALL_CASES))])
def test_small_shapes(torch_cuda, dtype, case):
    B, N, H, pats, causal, scale = case
    q, k, v = random_inputs(B, N, H, 64, dtype, seed=7 + B * N + H)
    out_o, lse_o = oracle.fwd(q, k, v, pats, causal=causal, scale=scale)
    out_g, lse_g = run_gpu(torch_cuda, q, k, v, pats, causal, scale)
    compare(out_g, lse_g, out_o, lse_o, dtype, f"{dtype} {case}")


def test_softmax_range_with_boosted_keys(torch_cuda):
    from sparse_long_sequence_attn_amd.workloads import bf16_round_bits, generate_f32

    q, k, v = generate_f32(1, 1024, 4, 64, 99, k_boost_frac=0.1, k_boost_factor=16.0,
                           k_boost_seed=5)
    q, k, v = (bf16_round_bits(x) for x in (q, k, v))
    pats = [(1024, 1), (256, 4)]
    out_o, lse_o = oracle.fwd(q, k, v, pats)
    out_g, lse_g = run_gpu(torch_cuda, q, k, v, pats)
    compare(out_g, lse_g, out_o, lse_o, "bf16", "boosted keys")


@pytest.mark.parametrize("causal", [True, False])
def test_scores_growing_far_beyond_the_first_block(torch_cuda, causal):
    """Keys in the second half of every 1024-row segment are 64 times larger
    (exact in bf16), so a row's scores jump, block after block, far past the
    running max its first blocks set (by hundreds in the log2 domain): the
    kernels must rebase the running max instead of overflowing."""
    q, k, v = random_inputs(1, 2048, 4, 64, "f32", seed=77)
    for s0 in (0, 1024):
        k[:, s0 + 512:s0 + 1024] *= np.float32(64.0)
        k[:, s0 + 768:s0 + 1024] *= np.float32(4.0)
    from sparse_long_sequence_attn_amd.workloads import bf16_round_bits
    q, k, v = (bf16_round_bits(x) for x in (q, k, v))
    pats = [(1024, 1), (2048, 2)]
    out_o, lse_o = oracle.fwd(q, k, v, pats, causal=causal)
    out_g, lse_g = run_gpu(torch_cuda, q, k, v, pats, causal=causal)
    assert np.isfinite(out_g).all()
    compare(out_g, lse_g, out_o, lse_o, "bf16", f"growing scores causal={causal}")


# ---------------------------------------------------------------- the five workloads

@pytest.mark.parametrize("name", [
    "w64r2_n512_h8_f32",
    "w64r2_b32_n8192_h8_bf16",
    "three_pattern_b4_n8192_h12_bf16",
    "paper_mixture_n32768_h16_bf16",
])
def test_workload_full(torch_cuda, name):
    w = WORKLOADS[name]
    q, k, v = host_inputs(w)
    out_g, lse_g = run_gpu(torch_cuda, q, k, v, w.patterns, w.causal)
    out_o, lse_o = oracle.fwd(q, k, v, w.patterns, causal=w.causal)
    compare(out_g, lse_g, out_o, lse_o, w.dtype, name)


def sample_rows(w, per_head=128, seed=0):
    """Rows to check on the million-token workload: for every pattern the
    first and last gathered row of its first and last segments, plus evenly
    spaced and random positions, for every head."""
    rng = np.random.default_rng(seed)
    rows = set()
    for h in range(w.H):
        ts = set()
        for (pw, r) in w.patterns:
            wp = min(pw, w.N)
            off = h % r
            L = -(-(wp - off) // r)
            for s in (0, w.N // wp - 1):
                ts.add(s * wp + off)
                ts.add(s * wp + off + (L - 1) * r)
                ts.add(s * wp + off + 1)  # a position this pattern does not gather
        ts.update(np.linspace(0, w.N - 1, per_head // 2).astype(int).tolist())
        ts.update(rng.integers(0, w.N, per_head // 2).tolist())
        rows.update((0, int(t), h) for t in ts)
    return np.array(sorted(rows), dtype=np.int64)


def test_million_token_workload_sampled(torch_cuda):
    torch = torch_cuda
    w = WORKLOADS["paper_mixture_plus_w65536_n1m_h16_bf16"]
    qt, kt, vt = device_inputs(w)
    prob = Problem(qt, kt, vt, w.patterns, w.causal)
    prob.out.fill_(float("nan"))
    prob.lse.fill_(float("nan"))
    prob.run()
    torch.cuda.synchronize()
    assert not torch.isnan(prob.out).any().item()
    assert not torch.isnan(prob.lse).any().item()
    rr = sample_rows(w)
    q, k, v = (from_torch_bits(x) for x in (qt, kt, vt))
    out_o, lse_o = oracle.rows(q, k, v, w.patterns, rr, causal=w.causal)
    ridx = torch.from_numpy(rr).to(qt.device)
    out_g = prob.out[ridx[:, 0], ridx[:, 1], ridx[:, 2]].float().cpu().numpy().astype(np.float64)
    lse_g = prob.lse[ridx[:, 0], ridx[:, 2], ridx[:, 1]].cpu().numpy().astype(np.float64)
    err = np.abs(out_g - out_o).max()
    fin = np.isfinite(lse_o)
    assert np.array_equal(np.isfinite(lse_g), fin)
    lerr = np.abs(lse_g[fin] - lse_o[fin]).max()
    print(f"1M tokens, {len(rr)} rows: max|out err| = {err:.3e}, max|lse err| = {lerr:.3e}")
    assert err <= TOL["bf16"][0] and lerr <= TOL["bf16"][1]


# ---------------------------------------------------------------- maps, determinism, API paths

MAP_CASES = [(32768, 16, p) for p in WORKLOADS["paper_mixture_n32768_h16_bf16"].patterns] + [
    (16, 4, (8, 2)), (96, 5, (1000, 7)), (120, 9, (40, 6)), (64, 3, (64, 64)), (1 << 20, 16, (65536, 16)),
]


@pytest.mark.parametrize("N,H,pat", MAP_CASES)
def test_maps_bit_exact(torch_cuda, N, H, pat):
    for h in range(H):
        ref = oracle.gather_map(N, pat[0], pat[1], h)
        nseg, L = ref.shape
        dev = gather_map(N, H, pat, h).cpu().numpy()
        lmax = dev.shape[1]
        assert dev.shape[0] == nseg and lmax >= L
        assert np.array_equal(dev[:, :L], ref)
        assert np.all(dev[:, L:] == -1)
        inv = np.full(N, -1, dtype=np.int64)
        for s in range(nseg):
            inv[ref[s]] = s * lmax + np.arange(L)
        assert np.array_equal(coverage_map(N, H, pat, h).cpu().numpy(), inv)


def test_deterministic_and_stage_split(torch_cuda):
    torch = torch_cuda
    w = WORKLOADS["three_pattern_b4_n8192_h12_bf16"]
    q, k, v = (to_torch(x) for x in host_inputs(w))
    p1 = Problem(q, k, v, w.patterns)
    o1, l1 = (x.clone() for x in p1.run())
    p2 = Problem(q, k, v, w.patterns)
    p2.out.fill_(float("nan"))
    p2.lse.fill_(float("nan"))
    p2.attention_stage()
    p2.merge_stage()
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), p2.out.view(torch.int16))
    assert torch.equal(l1, p2.lse)
    o3, l3 = p1.run()
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16)) and torch.equal(l1, l3)


def test_empty_inputs_and_errors(torch_cuda):
    torch = torch_cuda
    from sparse_long_sequence_attn_amd import DilatedAttnError

    q = torch.empty((0, 64, 4, 64), dtype=torch.bfloat16, device="cuda")
    out, lse = dilated_attn(q, q, q, [(16, 2)])
    assert out.shape == q.shape and lse.shape == (0, 4, 64)
    x = torch.zeros((1, 60, 4, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(DilatedAttnError, match="DA_ERR_SHAPE"):
        dilated_attn(x, x, x, [(16, 2)])
    y = torch.zeros((1, 64, 4, 32), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(DilatedAttnError, match="DA_ERR_HEADDIM"):
        dilated_attn(y, y, y, [(16, 2)])
    with pytest.raises(ValueError):
        dilated_attn(x.cpu(), x.cpu(), x.cpu(), [(16, 2)])


def test_caller_buffers_checked_before_launch(torch_cuda):
    """The C ABI cannot tell host memory from device memory, so the binding
    rejects caller-given outputs and workspaces that are on the host, on
    another device or strided, with ValueError and before any launch."""
    torch = torch_cuda
    from sparse_long_sequence_attn_amd import BwdProblem, dilated_attn_bwd, qk_norm_fwd

    x = torch.zeros((1, 64, 4, 64), dtype=torch.bfloat16, device="cuda")
    pats = [(16, 2), (64, 1)]
    good_out = torch.empty_like(x)
    good_lse = torch.empty((1, 4, 64), dtype=torch.float32, device="cuda")
    bad = {
        "out": [good_out.cpu(), torch.empty((1, 64, 64, 4), dtype=torch.bfloat16,
                                            device="cuda").transpose(2, 3)],
        "lse": [good_lse.cpu(), torch.empty((1, 64, 4), dtype=torch.float32,
                                            device="cuda").transpose(1, 2)],
        "workspace": [torch.empty(1 << 20, dtype=torch.uint8),
                      torch.empty(2 << 20, dtype=torch.uint8, device="cuda")[::2]],
    }
    for name, cases in bad.items():
        for t in cases:
            with pytest.raises(ValueError, match=name):
                dilated_attn(x, x, x, pats, **{name: t})
    fp = Problem(x, x, x, pats)
    fp.run()
    for name in ("dq", "dk", "dv"):
        with pytest.raises(ValueError, match=name):
            dilated_attn_bwd(x, x, x, fp.out, fp.lse, x, pats, **{name: good_out.cpu()})
    with pytest.raises(ValueError, match="workspace"):
        BwdProblem(x, x, x, fp.out, fp.lse, x, pats, workspace=torch.empty(1 << 20,
                                                                           dtype=torch.uint8))
    g = torch.ones(64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="yq"):
        qk_norm_fwd(x, x, g, g, g, g, yq=good_out.cpu())
    torch.cuda.synchronize()


def test_single_pattern_equals_full_attention_sdpa(torch_cuda):
    """w = N, r = 1 against torch's own attention on the GPU in fp32 (an
    independent check of the kernel besides the oracle)."""
    torch = torch_cuda
    q, k, v = random_inputs(2, 1024, 4, 64, "f32", seed=3)
    out_g, lse_g = run_gpu(torch, q, k, v, [(1024, 1)])
    tq, tk, tv = (torch.from_numpy(x).cuda().transpose(1, 2).contiguous() for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    ref = ref.transpose(1, 2).cpu().numpy()
    assert np.abs(out_g - ref).max() < 1e-4
    assert math.isfinite(lse_g.max())
