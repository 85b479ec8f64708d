"""Pins for the CPU oracle: checks against things other than the oracle.

Each pin compares the oracle with a library routine (torch's CPU
scaled-dot-product attention), a brute-force union softmax written another
way, a closed form, a fixture from the pages, or an invariant the definition
implies. Every pin is a function of an oracle instance so that
test_planted_mistakes_are_caught can run the same pins against copies of the
oracle with a mistake planted in them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from tests.brute_force import union_softmax
from tests.mutants import build_mutant, pins_catching

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand(B, N, H, Dh, seed):
    r = np.random.default_rng(seed)
    return [r.standard_normal((B, N, H, Dh)) for _ in range(3)]


def sdpa(q, k, v, causal, scale=None):
    """torch CPU scaled_dot_product_attention in float64 on [B, N, H, Dh]."""
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x.transpose(0, 2, 1, 3))) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    return o.numpy().transpose(0, 2, 1, 3)


# ---------------------------------------------------------------- library routine

def pin_full_window_equals_sdpa(orc, causal=True):
    """w = N, r = 1 is plain attention over the whole sequence."""
    q, k, v = rand(2, 96, 3, 64, 1)
    out, lse = orc.fwd(q, k, v, [(96, 1)], causal=causal)
    assert np.abs(out - sdpa(q, k, v, causal)).max() < 1e-12


def pin_window_larger_than_sequence(orc):
    q, k, v = rand(1, 64, 2, 64, 2)
    out, _ = orc.fwd(q, k, v, [(1 << 20, 1)])
    assert np.abs(out - sdpa(q, k, v, True)).max() < 1e-12


def pin_single_pattern_equals_segment_sdpa(orc, N=120, w=40, r=6, H=8, causal=True):
    """One pattern = dense attention on each head's sparsified segments (cut
    out with NumPy step slicing), scattered back; positions a head does not
    gather stay exactly 0 / -inf."""
    B, Dh = 2, 64
    q, k, v = rand(B, N, H, Dh, 3)
    scale = 0.3
    out, lse = orc.fwd(q, k, v, [(w, r)], causal=causal, scale=scale)
    ref = np.zeros_like(out)
    covered = np.zeros((B, N, H), dtype=bool)
    for h in range(H):
        for s in range(N // w):
            pos = np.arange(s * w, (s + 1) * w)[h % r::r]
            o = sdpa(q[:, pos][:, :, h:h + 1], k[:, pos][:, :, h:h + 1], v[:, pos][:, :, h:h + 1],
                     causal, scale)
            ref[:, pos, h] = o[:, :, 0]
            covered[:, pos, h] = True
    assert np.abs(out - ref).max() < 1e-12
    assert np.all(out[~covered] == 0.0)
    lse_bnh = lse.transpose(0, 2, 1)
    assert np.all(np.isneginf(lse_bnh[~covered]))
    assert np.all(np.isfinite(lse_bnh[covered]))


# ---------------------------------------------------------------- brute force

CASES = [
    (16, [(4, 1), (8, 2), (16, 4)]),      # the blog's doubling walk-through at N = 16
    (48, [(8, 1), (16, 3)]),              # w not a multiple of r
    (64, [(4, 2), (64, 1)]),              # sparse short range + full window
    (48, [(16, 5), (8, 2), (16, 5)]),     # a pattern listed twice
    (56, [(1000, 7), (8, 1)]),            # w > N
    (64, [(2, 2), (4, 4), (8, 8)]),       # r = w: one row per segment
]


def pin_merge_equals_union_softmax(orc, N=48, pats=((8, 1), (16, 3)), causal=True):
    q, k, v = rand(2, N, 5, 64, 4)
    out, lse = orc.fwd(q, k, v, list(pats), causal=causal)
    bo, bl = union_softmax(q, k, v, list(pats), causal=causal)
    assert np.abs(out - bo).max() < 1e-12
    fin = np.isfinite(bl)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.abs(lse[fin] - bl[fin]).max() < 1e-12


def pin_rows_equal_union_softmax(orc, causal=True):
    """The row formulation against the brute force, on every row."""
    N, H = 48, 5
    pats = [(16, 3), (48, 2), (8, 1)]
    q, k, v = rand(1, N, H, 64, 16)
    bo, bl = union_softmax(q, k, v, pats, causal=causal)
    rr = np.array([(0, t, h) for t in range(N) for h in range(H)])
    ro, rl = orc.rows(q, k, v, pats, rr, causal=causal)
    assert np.abs(ro - bo[0].reshape(N * H, 64)).max() < 1e-12
    assert np.abs(rl - bl[0].T.reshape(-1)).max() < 1e-12


# ---------------------------------------------------------------- closed forms

def pin_zero_query_closed_form(orc):
    """Q = 0 makes every score 0: a pattern's lse is ln(#keys) and the merged
    output is the mean of V over all (pattern, key) pairs. With V = position
    and a causal row at gathered index m of segment start s0, one pattern
    contributes m+1 keys with position sum (m+1)(s0+off) + r m(m+1)/2."""
    B, N, H, Dh = 1, 96, 6, 64
    pats = [(96, 1), (24, 2), (48, 3), (12, 6)]
    q = np.zeros((B, N, H, Dh))
    k = np.random.default_rng(5).standard_normal((B, N, H, Dh))
    v = np.broadcast_to(np.arange(N, dtype=np.float64)[None, :, None, None], (B, N, H, Dh)).copy()
    out, lse = orc.fwd(q, k, v, pats)
    for h in range(H):
        for t in range(N):
            cnt, tot = 0, 0.0
            for (w, r) in pats:
                s0 = (t // w) * w
                off = h % r
                if (t - s0) % r != off:
                    continue
                m = (t - s0 - off) // r
                cnt += m + 1
                tot += (m + 1) * (s0 + off) + r * m * (m + 1) / 2
            assert cnt > 0
            assert abs(lse[0, h, t] - math.log(cnt)) < 1e-12
            assert np.abs(out[0, t, h] - tot / cnt).max() < 1e-9


def pin_golden_worked_example(orc):
    with open(os.path.join(GOLDEN, "worked_example_windows.json")) as f:
        g = json.load(f)
    N = g["N"]
    for m in g["maps"]:
        got = orc.gather_map(N, m["w"], m["r"], m["h"])
        assert got.tolist() == m["segments"], m
    # how many of the three patterns gather each position, for head 0
    q, k, v = rand(1, N, 1, 64, 6)
    _, _, _, pl = orc.fwd(q, k, v, [(4, 1), (8, 2), (16, 4)], return_patterns=True)
    counts = np.isfinite(pl[:, 0, 0, :]).sum(0)
    assert counts.tolist() == g["row_coverage_h0"]["counts"]


def pin_golden_paper_mixture(orc):
    with open(os.path.join(GOLDEN, "paper_mixture_rows_per_head.json")) as f:
        g = json.load(f)
    for p in g["patterns"]:
        for h in range(g["H"]):
            wp, nseg, off, L = orc.geometry(g["N"], p["w"], p["r"], h)
            assert (nseg, L) == (p["nseg"], p["L"][h]), (p["w"], h)


def pin_golden_usage_example(orc):
    with open(os.path.join(GOLDEN, "usage_example_shape.json")) as f:
        g = json.load(f)
    Dh = g["dim"] // g["heads"]
    for h in range(g["heads"]):
        wp, nseg, off, L = orc.geometry(g["seq_len"], g["segment_size"], g["dilation_rate"], h)
        assert (Dh, L, nseg) == (g["derived"]["Dh"], g["derived"]["rows_per_segment_per_head"],
                                 g["derived"]["segments"])


# ---------------------------------------------------------------- invariants

def pin_duplicate_pattern_adds_ln2(orc):
    q, k, v = rand(1, 64, 4, 64, 7)
    o1, l1 = orc.fwd(q, k, v, [(16, 2)])
    o2, l2 = orc.fwd(q, k, v, [(16, 2), (16, 2)])
    fin = np.isfinite(l1)
    assert np.array_equal(np.isfinite(l2), fin)
    assert np.abs(o1 - o2).max() < 1e-13
    assert np.abs(l2[fin] - l1[fin] - math.log(2)).max() < 1e-13


def pin_pattern_order_invariance(orc):
    q, k, v = rand(1, 64, 4, 64, 8)
    pats = [(8, 1), (16, 2), (64, 4)]
    o1, l1 = orc.fwd(q, k, v, pats)
    o2, l2 = orc.fwd(q, k, v, pats[::-1])
    assert np.abs(o1 - o2).max() < 1e-13
    assert np.abs(l1 - l2).max() < 1e-13


def pin_constant_v(orc):
    """Constant V gives that constant on every covered row."""
    q, k, _ = rand(2, 64, 5, 64, 9)
    v = np.full_like(q, 0.7)
    out, lse = orc.fwd(q, k, v, [(16, 2), (32, 4)])
    cov = np.isfinite(lse).transpose(0, 2, 1)
    assert cov.any() and (~cov).any()
    assert np.abs(out[cov] - 0.7).max() < 1e-13
    assert np.all(out[~cov] == 0.0)


def pin_convex_combination(orc):
    """Each covered output lies within the range of its head's V values."""
    q, k, v = rand(2, 64, 5, 64, 10)
    q *= 3.0
    out, lse = orc.fwd(q, k, v, [(16, 2), (32, 4), (64, 1)])
    vmin = v.min(axis=1, keepdims=True)
    vmax = v.max(axis=1, keepdims=True)
    cov = np.isfinite(lse).transpose(0, 2, 1)[..., None]
    assert np.all(np.where(cov, out >= vmin - 1e-12, True))
    assert np.all(np.where(cov, out <= vmax + 1e-12, True))


def pin_causality_and_segment_independence(orc):
    """Changing K, V after position t leaves rows <= t bit-identical; changing
    them outside every segment of a row leaves that row bit-identical."""
    N = 64
    q, k, v = rand(1, N, 3, 64, 11)
    pats = [(16, 1), (32, 2)]
    o, l = orc.fwd(q, k, v, pats)
    t = 40
    k2, v2 = k.copy(), v.copy()
    k2[:, t + 1:] += 1.0
    v2[:, t + 1:] -= 2.0
    o2, l2 = orc.fwd(q, k2, v2, pats)
    assert np.array_equal(o[:, :t + 1], o2[:, :t + 1])
    assert np.array_equal(l[:, :, :t + 1], l2[:, :, :t + 1])
    assert not np.array_equal(o[:, t + 1:], o2[:, t + 1:])
    k3, v3 = k.copy(), v.copy()
    k3[:, 32:] *= -1.0
    v3[:, 32:] += 5.0
    o3, l3 = orc.fwd(q, k3, v3, pats, causal=False)
    o4, l4 = orc.fwd(q, k, v, pats, causal=False)
    assert np.array_equal(o3[:, :32], o4[:, :32])
    assert np.array_equal(l3[:, :, :32], l4[:, :, :32])


def pin_uncovered_rows_exact(orc):
    q, k, v = rand(1, 128, 8, 64, 13)
    out, lse = orc.fwd(q, k, v, [(64, 2)])
    for h in range(8):
        other = np.arange(128) % 2 != h % 2
        assert np.all(out[0, other, h] == 0.0)
        assert np.all(np.isneginf(lse[0, h, other]))
        assert np.all(np.isfinite(lse[0, h, ~other]))


# ---------------------------------------------------------------- formulations and precision

def pin_row_formulation_matches_segment_formulation(orc, causal=True):
    pats = [(32, 1), (64, 3), (128, 6)]
    q, k, v = rand(2, 128, 7, 64, 14)
    out, lse = orc.fwd(q, k, v, pats, causal=causal)
    rr = np.random.default_rng(12345).integers(0, [2, 128, 7], size=(300, 3))
    ro, rl = orc.rows(q, k, v, pats, rr, causal=causal)
    assert np.abs(ro - out[rr[:, 0], rr[:, 1], rr[:, 2]]).max() < 1e-13
    assert np.abs(rl - lse[rr[:, 0], rr[:, 2], rr[:, 1]]).max() < 1e-13


def pin_inputs_widened_exactly(orc):
    from sparse_long_sequence_attn_amd.workloads import bf16_round_bits, bf16_bits_to_f32

    q, k, v = (x.astype(np.float32) for x in rand(1, 64, 2, 64, 15))
    qb, kb, vb = (bf16_round_bits(x) for x in (q, k, v))
    o1, l1 = orc.fwd(qb, kb, vb, [(16, 2)])
    o2, l2 = orc.fwd(*(bf16_bits_to_f32(x).astype(np.float64) for x in (qb, kb, vb)), [(16, 2)])
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    o3, _ = orc.fwd(q, k, v, [(16, 2)])
    o4, _ = orc.fwd(*(x.astype(np.float64) for x in (q, k, v)), [(16, 2)])
    assert np.array_equal(o3, o4)


def pin_f32_tracks_f64_on_small_workload(orc):
    from sparse_long_sequence_attn_amd.workloads import WORKLOADS, SMALL, host_inputs

    w = WORKLOADS[SMALL]
    q, k, v = host_inputs(w)
    o64, l64 = orc.fwd(q, k, v, w.patterns)
    o32, l32 = orc.fwd(q, k, v, w.patterns, precision="f32")
    assert np.abs(o64 - o32).max() < 5e-6
    fin = np.isfinite(l64)
    assert np.array_equal(fin, np.isfinite(l32))
    assert np.abs(l64[fin] - l32[fin]).max() < 5e-6


# ---------------------------------------------------------------- pytest entry points

@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("causal", [True, False])
def test_full_window_equals_sdpa(orc, causal):
    pin_full_window_equals_sdpa(orc, causal)


def test_window_larger_than_sequence(orc):
    pin_window_larger_than_sequence(orc)


@pytest.mark.parametrize("N,w,r,H", [(256, 64, 4, 6), (120, 40, 6, 8), (64, 64, 3, 5), (32, 8, 8, 9)])
@pytest.mark.parametrize("causal", [True, False])
def test_single_pattern_equals_segment_sdpa(orc, N, w, r, H, causal):
    pin_single_pattern_equals_segment_sdpa(orc, N, w, r, H, causal)


@pytest.mark.parametrize("N,pats", CASES)
@pytest.mark.parametrize("causal", [True, False])
def test_merge_equals_union_softmax(orc, N, pats, causal):
    pin_merge_equals_union_softmax(orc, N, pats, causal)


@pytest.mark.parametrize("causal", [True, False])
def test_rows_equal_union_softmax(orc, causal):
    pin_rows_equal_union_softmax(orc, causal)


def test_zero_query_closed_form(orc):
    pin_zero_query_closed_form(orc)


def test_golden_worked_example(orc):
    pin_golden_worked_example(orc)


def test_golden_paper_mixture(orc):
    pin_golden_paper_mixture(orc)


def test_golden_usage_example(orc):
    pin_golden_usage_example(orc)


def test_duplicate_pattern_adds_ln2(orc):
    pin_duplicate_pattern_adds_ln2(orc)


def test_pattern_order_invariance(orc):
    pin_pattern_order_invariance(orc)


def test_constant_v(orc):
    pin_constant_v(orc)


def test_convex_combination(orc):
    pin_convex_combination(orc)


def test_causality_and_segment_independence(orc):
    pin_causality_and_segment_independence(orc)


def test_uncovered_rows_exact(orc):
    pin_uncovered_rows_exact(orc)


@pytest.mark.parametrize("causal", [True, False])
def test_row_formulation_matches_segment_formulation(orc, causal):
    pin_row_formulation_matches_segment_formulation(orc, causal)


def test_inputs_widened_exactly(orc):
    pin_inputs_widened_exactly(orc)


def test_f32_tracks_f64_on_small_workload(orc):
    pin_f32_tracks_f64_on_small_workload(orc)


# ---------------------------------------------------------------- planted mistakes

# (file, exact text, replacement, what the mistake is). Each is a plausible
# slip in the oracle; the pins above must reject every one of them.
MUTANTS = [
    ("oracle_core.inc", "s[j] = scale * dot;", "s[j] = dot;", "softmax scale dropped"),
    ("oracle_core.inc", "const int64_t nk = causal ? m + 1 : L;",
     "const int64_t nk = causal ? (m + 2 < L ? m + 2 : L) : L;", "causal mask one key too wide"),
    ("oracle_core.inc", "o[d] += e * vrows[j][d];", "o[d] += e * krows[j][d];",
     "K used where V belongs"),
    ("oracle_core.inc", "REAL wgt = REXP(lses[i] - LSE);", "REAL wgt = REXP(lses[i] - Mx);",
     "merge weights not normalised"),
    ("oracle_core.inc", "REAL LSE = Mx + RLOG(sum);", "REAL LSE = RLOG(sum);",
     "merged lse loses its max shift"),
    ("oracle_core.inc", "return M + RLOG(Z);", "return M - RLOG(Z);", "lse sign slip"),
    ("oracle_core.inc", "REAL e = REXP(s[j] - M);", "REAL e = REXP(s[j]);",
     "softmax max shift dropped from the weights"),
    ("oracle_core.inc", "for (int32_t d = 0; d < Dh; ++d) o[d] /= Z;", "",
     "softmax normalisation dropped"),
    ("oracle_core.inc", "idx[m] = sg * wp + off + m * r;", "idx[m] = sg * wp + m * r;",
     "head offset dropped from the gather"),
    ("dilated_oracle.c", "int64_t l = o < wpv ? (wpv - o + r - 1) / r : 0;",
     "int64_t l = o < wpv ? (wpv - o) / r : 0;", "rows per segment rounded down"),
    ("dilated_oracle.c", "int64_t o = (int64_t)(h % r);", "int64_t o = (int64_t)((h + 1) % r);",
     "heads shifted by one"),
    ("dilated_oracle.c", "return ((t - s0) % r) == (int64_t)(h % r);", "return ((t - s0) % r) == 0;",
     "row formulation ignores the head offset"),
    ("oracle_core.inc", "if (causal && tk > t) continue;", "if (causal && tk >= t) continue;",
     "row formulation drops the diagonal"),
    ("oracle_core.inc", "for (int32_t d = 0; d < Dh; ++d) dot += qrow[d] * krows[j][d];",
     "for (int32_t d = 0; d + 1 < Dh; ++d) dot += qrow[d] * krows[j][d];",
     "last head dimension dropped from the dot product"),
]

PIN_SUITE = [
    pin_full_window_equals_sdpa,
    pin_single_pattern_equals_segment_sdpa,
    pin_merge_equals_union_softmax,
    pin_rows_equal_union_softmax,
    pin_zero_query_closed_form,
    pin_golden_worked_example,
    pin_golden_paper_mixture,
    pin_duplicate_pattern_adds_ln2,
    pin_constant_v,
    pin_convex_combination,
    pin_causality_and_segment_independence,
    pin_uncovered_rows_exact,
    pin_row_formulation_matches_segment_formulation,
]


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m[3] for m in MUTANTS])
def test_planted_mistakes_are_caught(tmp_path, mutant):
    fname, old, new, _ = mutant
    lib = build_mutant(tmp_path, fname, old, new)
    assert pins_catching(lib, "tests.test_oracle_pins", "PIN_SUITE"), \
        "no pin rejects this planted mistake"
