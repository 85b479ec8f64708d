"""Work and traffic of one forward call, for reporting against rooflines.

Counts follow the method's structure (segments of min(w, N), head offset
h mod r, L = ceil((w' - off) / r) gathered rows per head and segment):

* algorithmic FLOPs: the useful multiply-adds of the two dense products per
  (batch, head, segment): S = Q K^T and O = P V, 2 * Dh flops per
  (query, key) pair each. Causal rows see m + 1 keys, so a segment costs
  2 * Dh * L * (L + 1); non-causal 4 * Dh * L^2.
* nominal count: 4 * N * (w / r) * Dh * H per pattern and batch row,
  halved for causal, with real-valued w / r. It counts every position as a
  query of every pattern, r times the rows a head gathers, so it exceeds the
  algorithmic count by about r for each pattern.
* bytes: each kernel's compulsory HBM traffic - gathered q, k, v rows read
  once. A row that exactly one pattern gathers is written once as output by
  the attention kernel; a row several patterns gather is written once per
  covering pattern as an fp32 partial (Dh floats + lse), read back once by
  the merge kernel, which also writes its output; a row no pattern gathers
  is written (zeros) by the merge kernel.
"""
import math
from dataclasses import dataclass
from typing import List, Sequence, Tuple

import numpy as np

Pattern = Tuple[int, int]


def rows_per_head(N: int, w: int, r: int, h: int) -> Tuple[int, int]:
    """(segments, gathered rows per segment) of pattern (w, r) for head h."""
    wp = min(w, N)
    off = h % r
    return N // wp, (-(-(wp - off) // r) if off < wp else 0)


def lmax(N: int, w: int, r: int) -> int:
    wp = min(w, N)
    return -(-wp // r)


@dataclass
class Cost:
    flops_alg: float        # useful flops of both contractions
    flops_ns: float         # nominal count
    exps: float             # softmax exponentials (one per useful score)
    gathered_rows: int      # sum over patterns, batches, heads, segments of L
    attn_read_bytes: float  # gathered q, k, v rows
    attn_write_bytes: float  # final out + lse (one pattern) or partials (several)
    merge_read_bytes: float
    merge_write_bytes: float

    @property
    def attn_bytes(self):
        return self.attn_read_bytes + self.attn_write_bytes

    @property
    def merge_bytes(self):
        return self.merge_read_bytes + self.merge_write_bytes


def cost(B: int, N: int, H: int, Dh: int, patterns: Sequence[Pattern], causal: bool = True,
         elem_bytes: int = 2) -> Cost:
    flops_alg = 0.0
    exps = 0.0
    rows = 0
    slots = 0  # partial-buffer row slots (lmax per segment)
    for (w, r) in patterns:
        for h in range(H):
            nseg, L = rows_per_head(N, w, r, h)
            pairs = L * (L + 1) / 2 if causal else L * L
            flops_alg += B * nseg * 4.0 * Dh * pairs
            exps += B * nseg * pairs
            rows += B * nseg * L
    flops_ns = 0.0
    for (w, r) in patterns:
        wp = min(w, N)
        flops_ns += B * 4.0 * N * (wp / r) * Dh * H * (0.5 if causal else 1.0)
    out_row = Dh * elem_bytes + 4  # output row + its lse
    part_row = (Dh + 1) * 4.0        # fp32 partial row + its lse
    attn_read = 3.0 * rows * Dh * elem_bytes
    if len(patterns) == 1:
        attn_write = float(B * N * H * out_row)
        merge_read = merge_write = 0.0
    else:
        single = multi_slots = multi_rows = none = 0
        t = np.arange(N, dtype=np.int64)
        for h in range(H):
            count = np.zeros(N, dtype=np.int64)
            for (w, r) in patterns:
                wp = min(w, N)
                count += ((t % wp) % r) == (h % r)
            single += int((count == 1).sum())
            none += int((count == 0).sum())
            multi_rows += int((count >= 2).sum())
            multi_slots += int(count[count >= 2].sum())
        attn_write = B * (single * out_row + multi_slots * part_row)
        merge_read = B * multi_slots * part_row
        merge_write = B * (multi_rows + none) * float(out_row)
    return Cost(flops_alg, flops_ns, exps, rows, attn_read, attn_write, merge_read, merge_write)


@dataclass
class BwdCost:
    """Per-stage work of one backward call. With fused set (every segment
    gathers at most 32 rows) the KV stage is the one-wave kernel that
    computes D and all three gradients, and the PREP and Q stages are empty."""
    pairs: float            # useful (query, key) pairs, summed over patterns
    flops_alg: float        # five products per pair (S recomputed, dP, dV, dK, dQ): 10 Dh
    flops_kv: float         # the KV-stage kernel's products: S, dP, dV, dK (8 Dh per pair),
                            # fused: all five (10 Dh)
    flops_q: float          # the dQ kernel's products (S, dP, dQ): 6 Dh per pair; fused: 0
    exps: float             # exponentials, once per pair in each kernel that forms P
    prep_bytes: float       # out and dout read, D written; fused: 0
    kv_bytes: float         # gathered q, k, v, dout rows + lse, D read; dk, dv written;
                            # fused: q, k, v, dout, out rows + lse read; dq, dk, dv written
    q_bytes: float          # gathered q, k, v, dout rows + lse, D read; dq written; fused: 0
    merge_bytes: float      # partials read, sums and zero rows written
    fused: bool = False


def bwd_cost(B: int, N: int, H: int, Dh: int, patterns: Sequence[Pattern], causal: bool = True,
             elem_bytes: int = 2) -> BwdCost:
    """Work and compulsory HBM traffic of one backward call.

    Each gathered row of each pattern is read once by each of the two main
    kernels (q, k, v, dout rows plus its lse and D); rows one pattern
    gathers are written once as final gradients, rows several patterns
    gather once per covering pattern as partials in the gradients' dtype
    (Dh elements per gradient), which the merge kernel reads back before
    writing the sums
    and the zero rows of positions no pattern gathers. When every segment
    gathers at most 32 rows one kernel reads each gathered row's q, k, v,
    dout, out and lse once and writes its three gradients (D is formed on
    the way, never stored)."""
    fwd = cost(B, N, H, Dh, patterns, causal, elem_bytes)
    pairs = fwd.flops_alg / (4.0 * Dh)
    rows = fwd.gathered_rows
    row = Dh * elem_bytes
    prow = Dh * elem_bytes  # partial rows have the gradients' dtype
    t = np.arange(N, dtype=np.int64)
    single = multi_slots = multi_rows = none = 0
    for h in range(H):
        count = np.zeros(N, dtype=np.int64)
        for (w, r) in patterns:
            wp = min(w, N)
            count += ((t % wp) % r) == (h % r)
        single += int((count == 1).sum())
        none += int((count == 0).sum())
        multi_rows += int((count >= 2).sum())
        multi_slots += int(count[count >= 2].sum())
    merge = B * (multi_slots * 3.0 * prow + (multi_rows + none) * 3.0 * row)
    if max(lmax(N, w, r) for (w, r) in patterns) <= 32:
        fused = rows * (5.0 * row + 4.0) + B * (single * 3.0 * row + multi_slots * 3.0 * prow)
        return BwdCost(pairs, 10.0 * Dh * pairs, 10.0 * Dh * pairs, 0.0, pairs, 0.0, fused, 0.0,
                       merge, fused=True)
    reads = rows * (4.0 * row + 8.0)
    kv_write = B * (single * 2.0 * row + multi_slots * 2.0 * prow)
    q_write = B * (single * row + multi_slots * prow)
    prep = B * N * H * (2.0 * row + 4.0)
    return BwdCost(pairs, 10.0 * Dh * pairs, 8.0 * Dh * pairs, 6.0 * Dh * pairs, 2.0 * pairs,
                   prep, reads + kv_write, reads + q_write, merge)


# MI355X published peaks (dense)
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def peak_tflops(dtype: str) -> float:
    return PEAK_BF16_TFLOPS if dtype == "bf16" else PEAK_FP32_MFMA_TFLOPS
