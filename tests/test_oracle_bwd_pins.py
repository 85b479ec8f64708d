"""Pins for the oracle's backward pass (gradients of sum(dout * out)).

The oracle differentiates the union-softmax form of the merged output (each
row: one softmax over the multiset of keys its covering patterns give it).
The pins below tie it to things other than itself: torch's autograd through
its CPU scaled-dot-product attention (one full window; one pattern cut into
sparsified segments with NumPy step slicing), torch's autograd through a
brute-force union softmax written without the oracle's structure, central
finite differences of the oracle's segment-and-merge forward pass (which
has pins of its own), and identities the definition implies.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tests.brute_force import union_softmax_torch
from tests.mutants import build_mutant, pins_catching


def rand4(B, N, H, Dh, seed):
    r = np.random.default_rng(seed)
    return [r.standard_normal((B, N, H, Dh)) for _ in range(4)]


def torch_grads(fn, q, k, v, dout):
    """Gradients of sum(dout * fn(q, k, v)) by torch autograd in float64."""
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    out = fn(tq, tk, tv)
    (out * torch.from_numpy(dout)).sum().backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


def sdpa_bnhd(q, k, v, causal, scale=None):
    """torch scaled_dot_product_attention on [B, N, H, Dh] tensors."""
    o = torch.nn.functional.scaled_dot_product_attention(
        q.transpose(1, 2), k.transpose(1, 2), v.transpose(1, 2), is_causal=causal, scale=scale)
    return o.transpose(1, 2)


def close(a, b, tol=1e-11):
    scale = max(1.0, float(np.abs(b).max()))
    err = float(np.abs(a - b).max()) / scale
    assert err < tol, f"max relative error {err:.3e}"


# ---------------------------------------------------------------- library routine

def pin_bwd_full_window_equals_sdpa(orc, causal=True):
    """w = N, r = 1 is plain attention: gradients equal torch autograd's."""
    q, k, v, do = rand4(2, 80, 3, 64, 11)
    got = orc.bwd(q, k, v, do, [(80, 1)], causal=causal)
    ref = torch_grads(lambda a, b, c: sdpa_bnhd(a, b, c, causal), q, k, v, do)
    for g, r in zip(got, ref):
        close(g, r)


def pin_bwd_single_pattern_equals_segment_sdpa(orc, N=96, w=32, r=5, H=6, causal=True):
    """One pattern: each head's sparsified segments (NumPy step slicing) are
    independent dense attentions; positions a head does not gather get
    exactly zero gradient."""
    B, Dh = 2, 64
    q, k, v, do = rand4(B, N, H, Dh, 12)
    scale = 0.2
    got = orc.bwd(q, k, v, do, [(w, r)], causal=causal, scale=scale)
    ref = [np.zeros_like(q) for _ in range(3)]
    gathered = np.zeros((B, N, H), dtype=bool)
    for h in range(H):
        for s in range(N // w):
            pos = np.arange(s * w, (s + 1) * w)[h % r::r]
            sl = lambda x: np.ascontiguousarray(x[:, pos][:, :, h:h + 1])
            g = torch_grads(lambda a, b, c: sdpa_bnhd(a, b, c, causal, scale),
                            sl(q), sl(k), sl(v), sl(do))
            for dst, src in zip(ref, g):
                dst[:, pos, h] = src[:, :, 0]
            gathered[:, pos, h] = True
    for g, rr in zip(got, ref):
        close(g, rr)
        assert np.all(g[~gathered] == 0.0)


# ---------------------------------------------------------------- brute force

BWD_CASES = [
    (16, [(4, 1), (8, 2), (16, 4)]),      # the blog's doubling walk-through at N = 16
    (24, [(8, 1), (12, 5)]),              # w not a multiple of r, uncovered rows
    (24, [(12, 5), (4, 2), (12, 5)]),     # a pattern listed twice
    (28, [(1000, 7), (4, 1)]),            # w > N
    (16, [(2, 2), (4, 4), (8, 8)]),       # r = w: one row per segment
]


def pin_bwd_union_softmax_autograd(orc, N=24, pats=((12, 5), (4, 2), (12, 5)), causal=True):
    """Every gradient element against torch autograd through the brute-force
    union softmax."""
    q, k, v, do = rand4(1, N, 3, 8, 13)
    got = orc.bwd(q, k, v, do, list(pats), causal=causal)
    ref = torch_grads(lambda a, b, c: union_softmax_torch(a, b, c, list(pats), causal), q, k, v, do)
    for g, r in zip(got, ref):
        close(g, r)


# ---------------------------------------------------------------- finite differences

def pin_bwd_matches_finite_differences(orc):
    """Directional derivatives of L = sum(dout * out), with out from the
    oracle's segment-and-merge forward pass, by central differences."""
    N, H, Dh = 48, 5, 16
    pats = [(16, 3), (48, 2), (8, 1)]
    q, k, v, do = rand4(2, N, H, Dh, 14)
    grads = orc.bwd(q, k, v, do, pats)
    rng = np.random.default_rng(15)
    eps = 1e-5
    for i in range(3):
        u = rng.standard_normal(q.shape)
        x = [q, k, v]
        xp = list(x)
        xm = list(x)
        xp[i] = x[i] + eps * u
        xm[i] = x[i] - eps * u
        lp = float((do * orc.fwd(*xp, pats)[0]).sum())
        lm = float((do * orc.fwd(*xm, pats)[0]).sum())
        fd = (lp - lm) / (2 * eps)
        an = float((grads[i] * u).sum())
        assert abs(fd - an) < 1e-6 * max(1.0, abs(an)), (i, fd, an)


# ---------------------------------------------------------------- identities

def pin_bwd_identities(orc):
    """Identities of softmax attention that hold per (batch, head):
    * adding one vector to every key shifts each row's scores by a constant,
      so the key gradients sum to zero;
    * adding one vector to every value shifts each covered row's output by
      it, so the value gradients sum to the covered rows' dout;
    * q -> a q, k -> k / a leaves every score unchanged, so
      <q, dq> = <k, dk>;
    * rows no pattern gathers have zero dq, and positions no pattern gathers
      for a head have zero dk and dv."""
    B, N, H, Dh = 2, 60, 6, 32
    pats = [(12, 5), (20, 4)]
    q, k, v, do = rand4(B, N, H, Dh, 16)
    dq, dk, dv = orc.bwd(q, k, v, do, pats)
    covered = np.zeros((N, H), dtype=bool)
    for (w, r) in pats:
        for h in range(H):
            for s in range(N // w):
                covered[np.arange(s * w, (s + 1) * w)[h % r::r], h] = True
    assert not covered.all()  # the case has uncovered rows
    scale = max(1.0, float(np.abs(dk).max()))
    assert np.abs(dk.sum(axis=1)).max() < 1e-11 * scale * N
    assert np.abs(dv.sum(axis=1) - (do * covered[None, :, :, None]).sum(axis=1)).max() < 1e-10
    qdq = (q * dq).sum(axis=(1, 3))
    kdk = (k * dk).sum(axis=(1, 3))
    assert np.abs(qdq - kdk).max() < 1e-10 * max(1.0, float(np.abs(qdq).max()))
    assert np.all(dq[:, ~covered] == 0.0)
    assert np.all(dk[:, ~covered] == 0.0) and np.all(dv[:, ~covered] == 0.0)


def pin_bwd_zero_query_closed_form(orc):
    """With q = 0 every weight of row t is 1 / |U(t)| and, for one full
    window, dv_j = sum over t >= j of dout_t / (t + 1) (causal)."""
    B, N, H, Dh = 1, 40, 2, 16
    q = np.zeros((B, N, H, Dh))
    _, k, v, do = rand4(B, N, H, Dh, 17)
    _, _, dv = orc.bwd(q, k, v, do, [(N, 1)])
    w = 1.0 / (np.arange(N) + 1.0)
    ref = np.cumsum((do * w[None, :, None, None])[:, ::-1], axis=1)[:, ::-1]
    assert np.abs(dv - ref).max() < 1e-12


def pin_bwd_f32_tracks_f64(orc):
    q, k, v, do = rand4(1, 64, 4, 64, 18)
    pats = [(16, 1), (32, 2), (64, 4)]
    g64 = orc.bwd(q, k, v, do, pats)
    g32 = orc.bwd(q.astype(np.float32), k.astype(np.float32), v.astype(np.float32),
                  do.astype(np.float32), pats, precision="f32")
    g64w = orc.bwd(*(x.astype(np.float32) for x in (q, k, v, do)), pats)
    for a, b in zip(g32, g64w):
        assert np.abs(a - b).max() < 2e-4
    for a, b in zip(g64w, g64):
        assert np.abs(a - b).max() < 1e-4


# ---------------------------------------------------------------- tests

@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("causal", [True, False])
def test_bwd_full_window_equals_sdpa(orc, causal):
    pin_bwd_full_window_equals_sdpa(orc, causal)


@pytest.mark.parametrize("N,w,r,H,causal", [(96, 32, 5, 6, True), (96, 32, 5, 6, False),
                                            (64, 64, 1, 2, True), (90, 30, 30, 3, True)])
def test_bwd_single_pattern_equals_segment_sdpa(orc, N, w, r, H, causal):
    pin_bwd_single_pattern_equals_segment_sdpa(orc, N, w, r, H, causal)


@pytest.mark.parametrize("N,pats", BWD_CASES)
@pytest.mark.parametrize("causal", [True, False])
def test_bwd_union_softmax_autograd(orc, N, pats, causal):
    pin_bwd_union_softmax_autograd(orc, N, pats, causal)


def test_bwd_matches_finite_differences(orc):
    pin_bwd_matches_finite_differences(orc)


def test_bwd_identities(orc):
    pin_bwd_identities(orc)


def test_bwd_zero_query_closed_form(orc):
    pin_bwd_zero_query_closed_form(orc)


def test_bwd_f32_tracks_f64(orc):
    pin_bwd_f32_tracks_f64(orc)


@pytest.mark.parametrize("causal", [True, False])
def test_bwd_rows_match_full_backward(orc, causal):
    """The row formulation (used where the full backward is too large)
    against the full backward on every row, including rows no pattern
    gathers and a pattern listed twice."""
    q, k, v, do = rand4(2, 48, 5, 16, 19)
    pats = [(16, 3), (48, 2), (8, 1), (16, 3)]
    dq, dk, dv = orc.bwd(q, k, v, do, pats, causal=causal)
    rows = np.array([(b, t, h) for b in range(2) for t in range(48) for h in range(5)])
    gq, gk, gv = orc.bwd_rows(q, k, v, do, pats, rows, causal=causal)
    idx = (rows[:, 0], rows[:, 1], rows[:, 2])
    for g, r in ((gq, dq), (gk, dk), (gv, dv)):
        assert np.abs(g - r[idx]).max() < 1e-12
    only_q = orc.bwd_rows(q, k, v, do, pats, rows[:7], causal=causal, want_dkv=False)
    assert only_q[1] is None and np.array_equal(only_q[0], gq[:7])


def test_bwd_empty_batch(orc):
    q = np.zeros((0, 16, 2, 8))
    dq, dk, dv = orc.bwd(q, q, q, q, [(8, 2)])
    assert dq.shape == dk.shape == dv.shape == q.shape


# ---------------------------------------------------------------- planted mistakes

BWD_MUTANTS = [
    ("const REAL ds = s[j] * (dp[j] - D);", "const REAL ds = s[j] * (dp[j] + D);",
     "sign of the dout.out correction flipped"),
    ("D += s[j] * dp[j];", "D += dp[j];", "correction term not weighted by P"),
    ("dq[qbase + d] += sc * ds *", "dq[qbase + d] += ds *", "scale dropped from dq"),
    ("dk[kbase + d] += sc * ds * qt[d];", "dk[kbase + d] += sc * ds * dot[d];",
     "dout used where q belongs in dk"),
    ("dv[kbase + d] += s[j] * dot[d];", "dv[kbase + d] += ds * dot[d];", "dS used where P belongs"),
    ("const int64_t last = causal ? m : L - 1;", "const int64_t last = causal ? m - 1 : L - 1;",
     "backward drops the diagonal key"),
    ("keys[nk++] = seg0 + off + mm * pats[pi].r;", "keys[nk++] = seg0 + mm * pats[pi].r;",
     "head offset dropped from the backward gather"),
    ("const int64_t rel = t - seg0 - off;", "const int64_t rel = t - seg0;",
     "backward membership ignores the head offset"),
    ("const REAL LSE = M + RLOG(Z);", "const REAL LSE = RLOG(Z);", "backward lse loses its max"),
    ("dq[qbase + d] += sc * ds * (REAL)orc_load(k,", "dq[qbase + d] += sc * ds * (REAL)orc_load(v,",
     "V used where K belongs in dq"),
    ("accv += dot[d] * (REAL)orc_load(v, in_dtype, kbase + d);",
     "accv += dot[d] * (REAL)orc_load(k, in_dtype, kbase + d);", "dP built from K instead of V"),
]

BWD_PIN_SUITE = [
    pin_bwd_full_window_equals_sdpa,
    pin_bwd_single_pattern_equals_segment_sdpa,
    pin_bwd_union_softmax_autograd,
    pin_bwd_matches_finite_differences,
    pin_bwd_identities,
    pin_bwd_zero_query_closed_form,
]


@pytest.mark.parametrize("mutant", BWD_MUTANTS, ids=[m[2] for m in BWD_MUTANTS])
def test_bwd_planted_mistakes_are_caught(tmp_path, mutant):
    old, new, _ = mutant
    lib = build_mutant(tmp_path, "oracle_core.inc", old, new)
    caught = pins_catching(lib, "tests.test_oracle_bwd_pins", "BWD_PIN_SUITE")
    assert caught, "no pin rejects this planted mistake"
