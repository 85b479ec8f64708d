"""Seeded synthetic inputs for the dilated-attention forward pass.

This module only draws random numbers and lays them out; it holds none of
the attention arithmetic. The GPU tests, the benchmark and the oracle side of
the tests all take their inputs from here, so both sides see the same bits.

Recipe (all q, k, v are [B, N, H, Dh], Dh = 64):
  * a NumPy PCG64 generator seeded per workload draws float32 standard
    normals for Q, then K, then V from one stream;
  * optional exact power-of-two scalings (Q * 1/8, chosen K rows * 8);
  * bf16 workloads round the float32 values to bf16 with round-to-nearest-
    even; both the GPU and the oracle consume the rounded values.
The million-token workload is drawn on the GPU with torch's generator
instead (12 GB of host float32 would be needed otherwise); the oracle then
reads back the exact bf16 bits it checks. The backward pass's output
gradient dout comes from a PCG64 stream of its own (workload seed + 100000),
drawn and rounded the same way.
"""
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

# The pattern mixture of the LongNet experiments (segment lengths and
# dilation rates of the language-model runs on the dakule.com news page,
# section "实验评估").
PAPER_MIXTURE: List[Tuple[int, int]] = [(2048, 1), (4096, 2), (8192, 4), (16384, 6), (32768, 12)]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    N: int
    H: int
    Dh: int
    dtype: str  # "f32" or "bf16"
    patterns: Tuple[Tuple[int, int], ...]
    seed: int
    causal: bool = True
    q_scale: float = 1.0
    k_boost_frac: float = 0.0  # fraction of token rows of K scaled by k_boost_factor
    k_boost_factor: float = 1.0
    k_boost_seed: int = 0
    device_generated: bool = False
    note: str = field(default="", compare=False)

    @property
    def tokens(self) -> int:
        return self.B * self.N


WORKLOADS = {
    w.name: w
    for w in [
        Workload("w64r2_n512_h8_f32", 1, 512, 8, 64, "f32", ((64, 2),), 1001,
                 note="single pattern, fp32, oracle runs in well under a second"),
        Workload("w64r2_b32_n8192_h8_bf16", 32, 8192, 8, 64, "bf16", ((64, 2),), 1002,
                 q_scale=1.0 / 8.0,
                 note="the DilatedAttention usage example's shape (dim 512, 8 heads)"),
        Workload("three_pattern_b4_n8192_h12_bf16", 4, 8192, 12, 64, "bf16",
                 ((2048, 1), (4096, 2), (8192, 4)), 1003),
        Workload("paper_mixture_n32768_h16_bf16", 1, 32768, 16, 64, "bf16",
                 tuple(PAPER_MIXTURE), 1004, k_boost_frac=0.05, k_boost_factor=8.0,
                 k_boost_seed=2004,
                 note="5% of K token rows scaled x8 to stretch the softmax range"),
        Workload("paper_mixture_plus_w65536_n1m_h16_bf16", 1, 1 << 20, 16, 64, "bf16",
                 tuple(PAPER_MIXTURE) + ((65536, 16),), 1005, device_generated=True,
                 note="one GPU's share of a million-token sequence"),
    ]
}

SMALL = "w64r2_n512_h8_f32"
BENCH = "paper_mixture_n32768_h16_bf16"


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even.

    Inputs here are finite normals, so no NaN handling is needed."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def boosted_rows(N: int, frac: float, seed: int) -> np.ndarray:
    """Token indices whose K rows are scaled: round(frac*N) of them, drawn
    without replacement from their own seeded stream."""
    count = int(round(frac * N))
    return np.sort(np.random.default_rng(seed).choice(N, size=count, replace=False))


def generate_f32(B, N, H, Dh, seed, q_scale=1.0, k_boost_frac=0.0, k_boost_factor=1.0,
                 k_boost_seed=0):
    """Draw float32 q, k, v of shape [B, N, H, Dh] (Q, then K, then V)."""
    rng = np.random.default_rng(seed)
    shape = (B, N, H, Dh)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if q_scale != 1.0:
        q *= np.float32(q_scale)
    if k_boost_frac > 0.0:
        rows = boosted_rows(N, k_boost_frac, k_boost_seed)
        k[:, rows] *= np.float32(k_boost_factor)
    return q, k, v


def host_inputs(w: Workload):
    """Host inputs of a workload.

    Returns (q, k, v) as float32 arrays for f32 workloads, or as uint16 bf16
    bit patterns for bf16 workloads."""
    if w.device_generated:
        raise ValueError(f"{w.name} is drawn on the GPU; use device_inputs()")
    q, k, v = generate_f32(w.B, w.N, w.H, w.Dh, w.seed, w.q_scale, w.k_boost_frac,
                           w.k_boost_factor, w.k_boost_seed)
    if w.dtype == "f32":
        return q, k, v
    return bf16_round_bits(q), bf16_round_bits(k), bf16_round_bits(v)


# Offset between a workload's seed and the seed of its output gradient.
DOUT_SEED_OFFSET = 100_000


def grad_output(B, N, H, Dh, dtype, seed):
    """The gradient dout of the loss with respect to the output, for the
    backward pass: float32 standard normals of shape [B, N, H, Dh] from a
    PCG64 generator of its own, rounded to bf16 bits for bf16."""
    d = np.random.default_rng(seed).standard_normal((B, N, H, Dh), dtype=np.float32)
    return d if dtype == "f32" else bf16_round_bits(d)


def workload_grad_output(w: Workload):
    """dout of a workload (seed = workload seed + DOUT_SEED_OFFSET)."""
    return grad_output(w.B, w.N, w.H, w.Dh, w.dtype, w.seed + DOUT_SEED_OFFSET)


def module_params(dim, heads, qk_norm, bias, seed):
    """Parameters of the DilatedAttention module, float32: the four
    projection weights [dim, dim] (out-features first) drawn N(0, 1/dim),
    optional biases N(0, 0.01), and with qk_norm the layer-norm gains
    1 + N(0, 0.01) and biases N(0, 0.01) over the 64 head values; one PCG64
    stream in that order."""
    rng = np.random.default_rng(seed)
    p = {}
    for n in ("wq", "wk", "wv", "wo"):
        p[n] = (rng.standard_normal((dim, dim), dtype=np.float32) / np.float32(np.sqrt(dim)))
    for n in ("bq", "bk", "bv", "bo"):
        p[n] = (rng.standard_normal(dim, dtype=np.float32) * np.float32(0.1)) if bias else None
    if qk_norm:
        Dh = dim // heads
        for n in ("q_gain", "k_gain"):
            p[n] = np.float32(1.0) + np.float32(0.1) * rng.standard_normal(Dh, dtype=np.float32)
        for n in ("q_bias", "k_bias"):
            p[n] = np.float32(0.1) * rng.standard_normal(Dh, dtype=np.float32)
    return p


def module_x(B, N, dim, seed):
    """Module input x [B, N, dim]: float32 standard normals."""
    return np.random.default_rng(seed).standard_normal((B, N, dim), dtype=np.float32)


def random_inputs(B, N, H, Dh, dtype, seed, q_scale=1.0):
    """Ad-hoc shapes for tests: same recipe as host_inputs()."""
    q, k, v = generate_f32(B, N, H, Dh, seed, q_scale)
    if dtype == "f32":
        return q, k, v
    return bf16_round_bits(q), bf16_round_bits(k), bf16_round_bits(v)


def to_torch(a: np.ndarray, device="cuda"):
    """NumPy input (float32, or uint16 bf16 bits) -> torch tensor on device."""
    import torch

    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def from_torch_bits(t) -> np.ndarray:
    """torch bf16 or float32 tensor -> NumPy (uint16 bits or float32), host copy."""
    import torch

    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def device_inputs(w: Workload, device="cuda"):
    """q, k, v of a device-generated workload, drawn with torch's generator
    on the GPU (float32 normals, then bf16 rounding), Q then K then V."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(w.seed)
    shape = (w.B, w.N, w.H, w.Dh)
    out = []
    for _ in range(3):
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        out.append(x.to(torch.bfloat16))
        del x
    return tuple(out)
