"""Work and traffic of one forward call, for reporting against rooflines.

Counts follow the method's structure (segments of min(w, N), head offset
h mod r, L = ceil((w' - off) / r) gathered rows per head and segment):

* algorithmic FLOPs: the useful multiply-adds of the two dense products per
  (batch, head, segment): S = Q K^T and O = P V, 2 * Dh flops per
  (query, key) pair each. Causal rows see m + 1 keys, so a segment costs
  2 * Dh * L * (L + 1); non-causal 4 * Dh * L^2.
* spec count: 4 * N * (w / r) * Dh * H per pattern and batch row,
  halved for causal, with real-valued w / r. It counts every position as a
  query of every pattern, r times the rows a head gathers, so it exceeds the
  algorithmic count by about r for each pattern.
* bytes: each kernel's compulsory HBM traffic - gathered q, k, v rows read
  once, outputs and partials written once, partials read once by the merge.
"""
import math
from dataclasses import dataclass
from typing import List, Sequence, Tuple

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
    flops_ns: float         # spec formula
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
    out_bytes = B * N * H * Dh * elem_bytes + B * H * N * 4
    attn_read = 3.0 * rows * Dh * elem_bytes
    if len(patterns) == 1:
        attn_write = float(out_bytes)
        merge_read = merge_write = 0.0
    else:
        attn_write = rows * (Dh + 1) * 4.0
        merge_read = attn_write
        merge_write = float(out_bytes)
    return Cost(flops_alg, flops_ns, exps, rows, attn_read, attn_write, merge_read, merge_write)


# MI355X published peaks (dense)
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def peak_tflops(dtype: str) -> float:
    return PEAK_BF16_TFLOPS if dtype == "bf16" else PEAK_FP32_MFMA_TFLOPS
