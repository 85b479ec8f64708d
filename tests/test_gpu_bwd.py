"""GPU parity of the backward pass: dq, dk, dv from the HIP kernels (through
the C ABI, fed with the GPU forward pass's out and lse) against the fp64
oracle's gradients on the same seeded inputs, element by element.

Tolerance. The forward bar (max abs error 1e-4 for fp32, 2e-2 for bf16) is
stated for outputs of order one. Gradients have no fixed scale (dv of an
early key sums the weights of every later query), so the same bar is applied
relative to each tensor's scale: max |g - g_oracle| <= tol * max(1,
max |g_oracle|). What fills the bf16 budget: every gradient is stored in
bf16 (relative rounding <= u = 2^-8 of the largest element); P and dS enter
their MFMA products rounded to bf16 (relative error <= u per term, summed
with random signs); D = dout . out is taken from the forward pass's
bf16-rounded out (relative error <= u per term). Scores, products and sums
run in fp32. For fp32 inputs every step is fp32 and the forward pass's out
is fp32, so the fp32 bar holds with a wide margin. Gradient buffers are
pre-filled with NaN, so an element the kernels never write fails the check;
rows no pattern gathers must be exactly zero.
"""
import numpy as np
import pytest

import oracle
from sparse_long_sequence_attn_amd import (DA_BWD_KV, DA_BWD_MERGE, DA_BWD_PREP, DA_BWD_Q,
                                           BwdProblem, DilatedAttnError, Problem,
                                           dilated_attn_bwd)
from sparse_long_sequence_attn_amd.workloads import (WORKLOADS, grad_output, host_inputs,
                                                     random_inputs, to_torch,
                                                     workload_grad_output)

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def gpu_grads(torch, q, k, v, dout, patterns, causal=True, scale=None):
    qt, kt, vt, dt = (to_torch(x) for x in (q, k, v, dout))
    fwd = Problem(qt, kt, vt, patterns, causal, scale)
    fwd.run()
    bp = BwdProblem(qt, kt, vt, fwd.out, fwd.lse, dt, patterns, causal, scale)
    for t in (bp.dq, bp.dk, bp.dv):
        t.fill_(float("nan"))
    bp.run()
    torch.cuda.synchronize()
    return tuple(t.float().cpu().numpy().astype(np.float64) for t in (bp.dq, bp.dk, bp.dv))


def covered_mask(N, H, patterns):
    m = np.zeros((N, H), dtype=bool)
    for (w, r) in patterns:
        wp = min(w, N)
        for h in range(H):
            for s in range(N // wp):
                m[np.arange(s * wp, (s + 1) * wp)[h % r::r], h] = True
    return m


def compare_grads(got, ref, dtype, patterns, label=""):
    N, H = ref[0].shape[1], ref[0].shape[2]
    cov = covered_mask(N, H, patterns)
    errs = []
    for name, g, o in zip(("dq", "dk", "dv"), got, ref):
        assert not np.isnan(g).any(), f"{label}: unwritten {name} elements"
        assert np.all(g[:, ~cov] == 0.0), f"{label}: {name} of uncovered rows not zero"
        scale = max(1.0, float(np.abs(o).max()))
        err = float(np.abs(g - o).max()) / scale
        rel = float(np.linalg.norm(g - o) / max(np.linalg.norm(o), 1e-30))
        errs.append(err)
        print(f"{label} {name}: max err / scale = {err:.3e} (scale {scale:.2f}), "
              f"relative Frobenius = {rel:.3e}", flush=True)
        assert err <= TOL[dtype], f"{label}: {name} error {err}"
    return errs


# ---------------------------------------------------------------- small shapes, every code path

BWD_CASES = [
    # (B, N, H, patterns, causal, scale) - comments name the path exercised
    (2, 256, 3, [(256, 1)], True, None),                  # one segment, two 128-row tiles
    (1, 384, 2, [(384, 1)], False, None),                 # non-causal, three tiles
    (2, 200, 5, [(200, 3)], True, None),                  # ragged L (67/67/66), odd H
    (1, 512, 4, [(128, 1), (256, 2), (512, 4)], True, None),
    (1, 480, 6, [(480, 6), (160, 1), (96, 2)], True, None),
    (3, 64, 4, [(16, 2), (32, 4), (64, 1)], True, None),
    (2, 128, 8, [(64, 2)], True, None),                   # 32-row path, zero rows
    (2, 128, 8, [(32, 1), (64, 2)], False, None),         # 32-row path, partials, non-causal
    (1, 96, 4, [(1000, 7), (8, 1), (96, 96)], True, None),  # w > N, r = w (one row)
    (1, 256, 2, [(128, 2)], True, 0.05),                  # explicit scale
    (1, 256, 4, [(256, 16)], True, None),                 # r = 16: 15 zero rows per query
    (1, 2048, 2, [(2048, 1)], True, None),                # 16 tiles each way
    (1, 1280, 3, [(1280, 5), (256, 1)], False, None),     # long non-causal with tails
    (2, 192, 7, [(192, 3), (192, 3)], True, None),        # a pattern listed twice
    (1, 512, 3, [(512, 1), (256, 2), (128, 4), (64, 8), (512, 8), (256, 1), (128, 2), (64, 1)],
     True, None),                                          # the maximum of 8 patterns
    (2, 90, 3, [(30, 1), (90, 4)], True, None),           # one-wave fused path: ragged L, partials
    (1, 50, 2, [(50, 2)], False, None),                   # one-wave fused path: L = 25, non-causal
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", BWD_CASES, ids=[f"c{i}" for i in range(len(BWD_CASES))])
def test_bwd_small_shapes(torch_cuda, dtype, case):
    B, N, H, pats, causal, scale = case
    seed = 11 + B * N + H
    q, k, v = random_inputs(B, N, H, 64, dtype, seed=seed)
    dout = grad_output(B, N, H, 64, dtype, seed + 1)
    ref = oracle.bwd(q, k, v, dout, pats, causal=causal, scale=scale)
    got = gpu_grads(torch_cuda, q, k, v, dout, pats, causal, scale)
    compare_grads(got, ref, dtype, pats, f"{dtype} {case}")


def test_bwd_boosted_keys(torch_cuda):
    """Keys scaled x16 on 10% of positions: wide score range, near-one-hot
    softmax rows."""
    from sparse_long_sequence_attn_amd.workloads import bf16_round_bits, generate_f32

    q, k, v = generate_f32(1, 1024, 4, 64, 99, k_boost_frac=0.1, k_boost_factor=16.0,
                           k_boost_seed=5)
    q, k, v = (bf16_round_bits(x) for x in (q, k, v))
    dout = grad_output(1, 1024, 4, 64, "bf16", 98)
    pats = [(1024, 1), (256, 4)]
    ref = oracle.bwd(q, k, v, dout, pats)
    got = gpu_grads(torch_cuda, q, k, v, dout, pats)
    compare_grads(got, ref, "bf16", pats, "boosted keys")


# ---------------------------------------------------------------- workloads at full size

@pytest.mark.parametrize("name", [
    "w64r2_n512_h8_f32",
    "w64r2_b32_n8192_h8_bf16",
    "three_pattern_b4_n8192_h12_bf16",
    "paper_mixture_n32768_h16_bf16",
])
def test_bwd_workload_full(torch_cuda, name):
    w = WORKLOADS[name]
    q, k, v = host_inputs(w)
    dout = workload_grad_output(w)
    got = gpu_grads(torch_cuda, q, k, v, dout, w.patterns, w.causal)
    ref = oracle.bwd(q, k, v, dout, w.patterns, causal=w.causal)
    compare_grads(got, ref, w.dtype, w.patterns, name)


# ---------------------------------------------------------------- one GPU's million tokens

def test_bwd_million_token_workload_sampled(torch_cuda):
    """The million-token workload (six patterns, drawn on the GPU): dq on
    sampled rows and dk, dv on sampled key rows against the oracle's row
    formulation, plus identities of the full gradients (the key gradients of
    a (batch, head) sum to zero; the value gradients sum to the summed dout,
    every row being gathered; <q, dq> = <k, dk>), with the summation-noise
    allowance tol * ||summands||_2."""
    import oracle as orc_mod
    from sparse_long_sequence_attn_amd.workloads import DOUT_SEED_OFFSET, device_inputs
    from tests.test_gpu_parity import sample_rows

    torch = torch_cuda
    w = WORKLOADS["paper_mixture_plus_w65536_n1m_h16_bf16"]
    qt, kt, vt = device_inputs(w)
    g = torch.Generator(device="cuda")
    g.manual_seed(w.seed + DOUT_SEED_OFFSET)
    dt = torch.randn(qt.shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    fwd = Problem(qt, kt, vt, w.patterns, w.causal)
    fwd.run()
    bp = BwdProblem(qt, kt, vt, fwd.out, fwd.lse, dt, w.patterns, w.causal)
    for t in (bp.dq, bp.dk, bp.dv):
        t.fill_(float("nan"))
    bp.run()
    torch.cuda.synchronize()
    for t in (bp.dq, bp.dk, bp.dv):
        assert not torch.isnan(t).any().item()

    from sparse_long_sequence_attn_amd.workloads import from_torch_bits
    q, k, v, d = (from_torch_bits(x) for x in (qt, kt, vt, dt))
    rq = sample_rows(w, per_head=48, seed=1)
    rng = np.random.default_rng(2)
    rk = []
    for h in range(w.H):
        for (pw, r) in w.patterns[:2]:  # last gathered row of a segment: few queries see it
            off = h % r
            L = -(-(min(pw, w.N) - off) // r)
            rk.append((0, off + (L - 1) * r, h))
        rk.append((0, int(rng.integers(0, w.N)), h))
    rk = np.array(rk, dtype=np.int64)
    oq, _, _ = orc_mod.bwd_rows(q, k, v, d, w.patterns, rq, causal=w.causal, want_dkv=False)
    _, ok, ov = orc_mod.bwd_rows(q, k, v, d, w.patterns, rk, causal=w.causal, want_dq=False)

    def rows_of(t, rr):
        i = torch.from_numpy(rr).to(t.device)
        return t[i[:, 0], i[:, 1], i[:, 2]].float().cpu().numpy().astype(np.float64)

    for name, got, ref in (("dq", rows_of(bp.dq, rq), oq), ("dk", rows_of(bp.dk, rk), ok),
                           ("dv", rows_of(bp.dv, rk), ov)):
        scale = max(1.0, float(np.abs(ref).max()))
        err = float(np.abs(got - ref).max()) / scale
        print(f"1M tokens {name}, {len(ref)} rows: max err / scale = {err:.3e}", flush=True)
        assert err <= TOL["bf16"], name

    tol = TOL["bf16"]
    dk64, dv64 = bp.dk.double(), bp.dv.double()
    sk = dk64.sum(dim=1)
    nk = dk64.pow(2).sum(dim=1).sqrt()
    assert bool((sk.abs() <= tol * nk).all()), float((sk.abs() / nk).max())
    sv = dv64.sum(dim=1) - dt.double().sum(dim=1)
    nv = dv64.pow(2).sum(dim=1).sqrt()
    assert bool((sv.abs() <= tol * nv).all()), float((sv.abs() / nv).max())
    qdq = (qt.double() * bp.dq.double()).sum(dim=(1, 3))
    kdk = (kt.double() * dk64).sum(dim=(1, 3))
    nq = (qt.double() * bp.dq.double()).pow(2).sum(dim=(1, 3)).sqrt()
    assert bool(((qdq - kdk).abs() <= tol * (nq + (kt.double() * dk64).pow(2).sum(dim=(1, 3)).sqrt())).all())


# ---------------------------------------------------------------- independent check, API paths

def test_bwd_full_window_equals_torch_autograd(torch_cuda):
    """w = N, r = 1 against torch autograd of its own fp32 attention on the
    GPU (a check of the kernels besides the oracle)."""
    torch = torch_cuda
    q, k, v = random_inputs(2, 512, 4, 64, "f32", seed=21)
    dout = grad_output(2, 512, 4, 64, "f32", 22)
    got = gpu_grads(torch, q, k, v, dout, [(512, 1)])
    tq, tk, tv = (torch.from_numpy(x).cuda().transpose(1, 2).contiguous().requires_grad_()
                  for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    o.backward(torch.from_numpy(dout).cuda().transpose(1, 2))
    for g, t in zip(got, (tq, tk, tv)):
        ref = t.grad.transpose(1, 2).cpu().numpy()
        assert np.abs(g - ref).max() <= 1e-4 * max(1.0, float(np.abs(ref).max()))


@pytest.mark.parametrize("name", ["three_pattern_b4_n8192_h12_bf16", "w64r2_b32_n8192_h8_bf16"])
def test_bwd_deterministic_and_stage_split(torch_cuda, name):
    """Stages run one by one equal the whole pass bit for bit (for segments
    of at most 32 rows the KV stage runs the one fused kernel and the PREP
    and Q stages launch nothing), and repeated runs agree bit for bit."""
    torch = torch_cuda
    w = WORKLOADS[name]
    q, k, v = (to_torch(x) for x in host_inputs(w))
    dout = to_torch(workload_grad_output(w))
    f = Problem(q, k, v, w.patterns)
    f.run()
    g1 = [x.clone() for x in dilated_attn_bwd(q, k, v, f.out, f.lse, dout, w.patterns)]
    bp = BwdProblem(q, k, v, f.out, f.lse, dout, w.patterns)
    for t in (bp.dq, bp.dk, bp.dv):
        t.fill_(float("nan"))
    for st in (DA_BWD_PREP, DA_BWD_KV, DA_BWD_Q, DA_BWD_MERGE):
        bp.run(st)
    torch.cuda.synchronize()
    for a, b in zip(g1, (bp.dq, bp.dk, bp.dv)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    g3 = dilated_attn_bwd(q, k, v, f.out, f.lse, dout, w.patterns)
    torch.cuda.synchronize()
    for a, b in zip(g1, g3):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_bwd_empty_and_errors(torch_cuda):
    torch = torch_cuda
    q = torch.empty((0, 64, 4, 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((0, 4, 64), dtype=torch.float32, device="cuda")
    dq, dk, dv = dilated_attn_bwd(q, q, q, q, lse, q, [(16, 2)])
    assert dq.shape == dk.shape == dv.shape == q.shape
    x = torch.zeros((1, 64, 4, 64), dtype=torch.bfloat16, device="cuda")
    l = torch.zeros((1, 4, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(DilatedAttnError, match="DA_ERR_ALIAS"):
        dilated_attn_bwd(x, x, x, x, l, x, [(16, 2)], dq=x)
    with pytest.raises(ValueError):
        dilated_attn_bwd(x, x, x, x, l[:, :2], x, [(16, 2)])
    with pytest.raises(ValueError):
        dilated_attn_bwd(x, x, x, x.float(), l, x, [(16, 2)])
