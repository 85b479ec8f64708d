"""The work/traffic model used for reporting, against hand-derived counts."""
import json
import os

from sparse_long_sequence_attn_amd.costs import bwd_cost, cost

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_paper_mixture_flops_from_rows_per_head():
    with open(os.path.join(GOLDEN, "paper_mixture_rows_per_head.json")) as f:
        g = json.load(f)
    N, H, Dh = g["N"], g["H"], 64
    # causal segment of L rows: L(L+1)/2 (query, key) pairs, 4*Dh flops each
    # (2*Dh for the score, 2*Dh for the weighted value sum)
    alg = sum(p["nseg"] * 2 * Dh * L * (L + 1) for p in g["patterns"] for L in p["L"])
    rows = sum(p["nseg"] * L for p in g["patterns"] for L in p["L"])
    c = cost(1, N, H, Dh, [(p["w"], p["r"]) for p in g["patterns"]], True, 2)
    assert c.flops_alg == alg
    assert c.gathered_rows == rows
    assert abs(c.flops_alg / 1e9 - 286.47) < 0.01
    # nominal count: 4 N (w/r) Dh H per pattern, halved for causal
    ns = sum(4 * N * (p["w"] / p["r"]) * Dh * H / 2 for p in g["patterns"])
    assert abs(c.flops_ns - ns) < 1e-3 * ns


def test_single_pattern_bytes():
    # usage-example shape: half of q, k, v gathered (r = 2), out + lse written once
    c = cost(32, 8192, 8, 64, [(64, 2)], True, 2)
    half = 32 * 8192 * 8 * 64 * 2 // 2
    assert c.attn_read_bytes == 3 * half
    assert c.attn_write_bytes == 32 * 8192 * 8 * 64 * 2 + 32 * 8 * 8192 * 4
    assert c.merge_bytes == 0


def test_non_causal_pairs():
    c = cost(1, 64, 2, 64, [(64, 1)], False, 4)
    assert c.flops_alg == 2 * 64 * 4 * 64 * 64


def test_merge_traffic_split():
    # patterns (4, 1) and (8, 2) at N = 16, one head (offset 0): even
    # positions are gathered by both patterns, odd ones by the first only
    c = cost(1, 16, 1, 64, [(4, 1), (8, 2)], True, 2)
    assert c.gathered_rows == 16 + 8
    out_row, part_row = 64 * 2 + 4, 65 * 4
    assert c.attn_write_bytes == 8 * out_row + 16 * part_row
    assert c.merge_read_bytes == 16 * part_row
    assert c.merge_write_bytes == 8 * out_row



def test_bwd_partial_traffic_split():
    # patterns (64, 1) and (128, 2) at N = 128, one head (offset 0): the 64
    # even positions are gathered by both patterns (128 partial slots per
    # gradient), the 64 odd ones by the first only (final rows). Partial rows
    # have the gradients' dtype (es bytes an element); the merge reads them
    # and writes the 64 summed rows of each of the 3 gradients.
    for es in (2, 4):
        c = bwd_cost(1, 128, 1, 64, [(64, 1), (128, 2)], True, es)
        assert not c.fused
        row = 64 * es
        assert c.merge_bytes == 3 * 128 * row + 3 * 64 * row
        reads = (128 + 64) * (4 * row + 8)  # q, k, v, dout rows + lse, D
        assert c.kv_bytes == reads + 2 * (64 * row + 128 * row)
        assert c.q_bytes == reads + (64 * row + 128 * row)
        assert c.prep_bytes == 128 * (2 * row + 4)


def test_bwd_fused_short_segments_traffic():
    # segments of at most 32 gathered rows: one kernel reads q, k, v, dout,
    # out rows + lse once and writes final rows or partials (same split as
    # above at N = 16 with patterns (4, 1) and (8, 2))
    for es in (2, 4):
        c = bwd_cost(1, 16, 1, 64, [(4, 1), (8, 2)], True, es)
        assert c.fused
        row = 64 * es
        assert c.kv_bytes == (16 + 8) * (5 * row + 4) + 3 * 8 * row + 3 * 16 * row
        assert c.merge_bytes == 3 * 16 * row + 3 * 8 * row
