"""The DilatedAttention module and an autograd-aware attention call.

``dilated_attention(q, k, v, patterns)`` runs the forward kernels through the
C ABI and, under autograd, the backward kernels (which take the forward
pass's out and lse). ``DilatedAttention`` is the drop-in module of the
LongNet package README (parameters dim, heads, dilation_rate, segment_size,
qk_norm and the usage example: x [B, N, dim] -> [B, N, dim]). Its insides
follow the plainest reading of the pages: queries, keys and values are
linear maps of x (LONGNET blog, "About the Transformer model" and "Token
expansion reaches 1 billion+"), qk_norm layer-normalises each head's query
and key vectors, the dilated attention runs in this library's kernels, and
an output projection maps the heads back to dim. The projections and the
layer norms are plain library operations (torch's GEMMs and LayerNorm).
"""
from typing import Optional, Sequence, Tuple, Union

import torch

from . import BwdProblem, Problem

Pattern = Tuple[int, int]


class DilatedAttnFunction(torch.autograd.Function):
    """out = dilated attention(q, k, v); q, k, v contiguous [B, N, H, 64]."""

    @staticmethod
    def forward(ctx, q, k, v, patterns, causal, scale):
        prob = Problem(q, k, v, patterns, causal, scale)
        out, lse = prob.run()
        ctx.save_for_backward(q, k, v, out, lse)
        ctx.patterns, ctx.causal, ctx.scale = patterns, causal, scale
        ctx.mark_non_differentiable(lse)
        return out, lse

    @staticmethod
    def backward(ctx, dout, dlse):
        q, k, v, out, lse = ctx.saved_tensors
        bp = BwdProblem(q, k, v, out, lse, dout.contiguous(), ctx.patterns, ctx.causal, ctx.scale)
        dq, dk, dv = bp.run()
        return dq, dk, dv, None, None, None


def dilated_attention(q, k, v, patterns: Sequence[Pattern], causal: bool = True,
                      scale: Optional[float] = None, return_lse: bool = False):
    """Dilated attention with autograd support. q, k, v: [B, N, H, 64] GPU
    tensors (bf16 or fp32); patterns: (w, r) pairs. Returns out (and lse)."""
    pats = tuple((int(w), int(r)) for (w, r) in patterns)
    out, lse = DilatedAttnFunction.apply(q.contiguous(), k.contiguous(), v.contiguous(), pats,
                                         bool(causal), scale)
    return (out, lse) if return_lse else out


def _as_list(x):
    return list(x) if isinstance(x, (list, tuple)) else [x]


class DilatedAttention(torch.nn.Module):
    """x [B, N, dim] -> [B, N, dim].

    dilation_rate and segment_size are ints (one pattern, as in the README's
    usage) or equal-length sequences (a mixture of patterns, as in LongNet's
    experiments). heads * 64 must equal dim. qk_norm adds one LayerNorm over
    the 64 values of every head's query and one for keys (gain and bias
    shared by all heads). bias adds biases to the four projections."""

    HEAD_DIM = 64

    def __init__(self, dim: int, heads: int, dilation_rate: Union[int, Sequence[int]],
                 segment_size: Union[int, Sequence[int]], qk_norm: bool = False,
                 causal: bool = True, bias: bool = False, scale: Optional[float] = None,
                 ln_eps: float = 1e-5, device=None, dtype=None):
        super().__init__()
        if heads < 1 or dim != heads * self.HEAD_DIM:
            raise ValueError(f"dim must be heads * {self.HEAD_DIM} (got dim={dim}, heads={heads})")
        rates, sizes = _as_list(dilation_rate), _as_list(segment_size)
        if len(rates) != len(sizes) or not rates:
            raise ValueError("dilation_rate and segment_size must pair up")
        self.dim, self.heads = dim, heads
        self.patterns = tuple((int(w), int(r)) for w, r in zip(sizes, rates))
        self.causal, self.scale, self.qk_norm = bool(causal), scale, bool(qk_norm)
        f = {"device": device, "dtype": dtype}
        self.to_q = torch.nn.Linear(dim, dim, bias=bias, **f)
        self.to_k = torch.nn.Linear(dim, dim, bias=bias, **f)
        self.to_v = torch.nn.Linear(dim, dim, bias=bias, **f)
        self.to_out = torch.nn.Linear(dim, dim, bias=bias, **f)
        if self.qk_norm:
            self.q_norm = torch.nn.LayerNorm(self.HEAD_DIM, eps=ln_eps, **f)
            self.k_norm = torch.nn.LayerNorm(self.HEAD_DIM, eps=ln_eps, **f)

    def forward(self, x):
        B, N, _ = x.shape
        shape = (B, N, self.heads, self.HEAD_DIM)
        q = self.to_q(x).view(shape)
        k = self.to_k(x).view(shape)
        v = self.to_v(x).view(shape)
        if self.qk_norm:
            q = self.q_norm(q)
            k = self.k_norm(k)
        o = dilated_attention(q, k, v, self.patterns, self.causal, self.scale)
        return self.to_out(o.view(B, N, self.dim))
