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
an output projection maps the heads back to dim. The projections are plain
library GEMMs (torch), with the weight gradients split over the long row
dimension so that they fill the chip. qk_norm runs inside the attention
kernels where the library supports it (one pattern whose segments gather at
most 32 rows, as in the README's usage example): q and k are normalised as
the kernels load them and never stored, and the backward kernel turns the
attention gradients into gradients of the un-normalised rows and of the
gains and biases. There q, k and v come from one GEMM as one [B, N, 3,
heads, 64] tensor, which the kernels read in place, and their gradients go
back through one GEMM the same way. Elsewhere it runs in this library's layer-norm kernels
(both tensors in one launch each way) before the attention.
"""
from typing import Optional, Sequence, Tuple, Union

import torch

from . import (BwdProblem, Problem, _dtype_code, dilated_attn_qknorm, dilated_attn_qknorm_bwd,
               qk_norm_bwd, qk_norm_fwd, qknorm_fused_supported)

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


class QKNormFunction(torch.autograd.Function):
    """(yq, yk) = layer norm of every 64-value row of xq and xk."""

    @staticmethod
    def forward(ctx, xq, xk, gq, bq, gk, bk, eps):
        xq, xk = xq.contiguous(), xk.contiguous()
        yq, yk = qk_norm_fwd(xq, xk, gq, bq, gk, bk, eps)
        ctx.save_for_backward(xq, xk, gq, gk)
        ctx.eps = eps
        return yq, yk

    @staticmethod
    def backward(ctx, dyq, dyk):
        xq, xk, gq, gk = ctx.saved_tensors
        dxq, dxk, dp = qk_norm_bwd(xq, xk, dyq.contiguous(), dyk.contiguous(), gq, gk, ctx.eps)
        dp = dp.to(gq.dtype)
        return dxq, dxk, dp[0, 0], dp[0, 1], dp[1, 0], dp[1, 1], None


class QKNormAttnFunction(torch.autograd.Function):
    """out = dilated attention(qk_norm(xq), qk_norm(xk), v) with the layer
    norm inside the attention kernels; the normalised q and k never exist in
    memory. xq, xk, v are the parts of one [B, N, 3, H, 64] tensor (one
    projection GEMM writes them) and its gradient comes back in that layout
    (one GEMM takes it)."""

    @staticmethod
    def forward(ctx, qkv, gq, bq, gk, bk, eps, patterns, causal, scale):
        xq, xk, v = qkv.unbind(2)
        out, lse = dilated_attn_qknorm(xq, xk, v, gq, bq, gk, bk, patterns, eps, causal, scale)
        ctx.save_for_backward(qkv, gq, bq, gk, bk, out, lse)
        ctx.eps, ctx.patterns, ctx.causal, ctx.scale = eps, patterns, causal, scale
        return out

    @staticmethod
    def backward(ctx, dout):
        qkv, gq, bq, gk, bk, out, lse = ctx.saved_tensors
        dqkv = torch.empty_like(qkv)
        dxq, dxk, dv = dqkv.unbind(2)
        _, _, _, dp = dilated_attn_qknorm_bwd(*qkv.unbind(2), gq, bq, gk, bk, out, lse,
                                              dout.contiguous(), ctx.patterns, ctx.eps,
                                              ctx.causal, ctx.scale, dxq=dxq, dxk=dxk, dv=dv)
        dp = dp.to(gq.dtype)
        return dqkv, dp[0, 0], dp[0, 1], dp[1, 0], dp[1, 1], None, None, None, None


def _weight_grad(dy2, x2):
    """dW = dy2^T x2 for [R, out] and [R, in] row-major operands. A single
    GEMM over R = B * N rows leaves most of the chip idle (a 512 x 512 output
    is only a few dozen tiles), so long R is split into 32 chunks, one
    batched GEMM computes the chunk products (left operand a transposed view,
    right operand contiguous). Each chunk product leaves the GEMM rounded to
    the operands' dtype (its accumulation is float32); the 32 chunks are then
    summed in float32 and rounded once more, so a bf16 gradient carries two
    roundings instead of one."""
    R = dy2.shape[0]
    S = 32
    if R % S == 0 and R // S >= 2048:
        part = torch.bmm(dy2.view(S, R // S, -1).transpose(1, 2), x2.view(S, R // S, -1))
        acc = torch.float32 if dy2.dtype in (torch.bfloat16, torch.float16) else dy2.dtype
        return part.sum(0, dtype=acc).to(dy2.dtype)
    return torch.mm(dy2.t(), x2)


class ProjectionFunction(torch.autograd.Function):
    """(y_1 .. y_n) = (x W_1^T + b_1, ..., x W_n^T + b_n) for one input x
    [R, in]; the backward accumulates dx over the n products in place (an
    out-of-place addmm would first copy its addend into a new [R, in]
    tensor)."""

    @staticmethod
    def forward(ctx, x2, n, *wb):
        ws, bs = wb[:n], wb[n:]
        ctx.save_for_backward(x2, *ws)
        ctx.n, ctx.has_bias = n, [b is not None for b in bs]
        return tuple(torch.nn.functional.linear(x2, w, b) for w, b in zip(ws, bs))

    @staticmethod
    def backward(ctx, *dys):
        x2, *ws = ctx.saved_tensors
        dx = None
        dws, dbs = [], []
        for dy, w, hb in zip(dys, ws, ctx.has_bias):
            dy = dy.contiguous()
            dx = torch.mm(dy, w) if dx is None else dx.addmm_(dy, w)
            dws.append(_weight_grad(dy, x2))
            dbs.append(dy.sum(0) if hb else None)
        return (dx, None, *dws, *dbs)


class PackedProjectionFunction(torch.autograd.Function):
    """y = x [W_1; ...; W_n]^T (+ [b_1; ...; b_n]) as one GEMM for one input
    x [R, in]: the n outputs side by side in y [R, n out]. The backward
    takes dy in that layout: dx is one GEMM over K = n out, the weight
    gradient one (row-split) GEMM, split back into the n weights."""

    @staticmethod
    def forward(ctx, x2, n, *wb):
        ws, bs = wb[:n], wb[n:]
        w = torch.cat(ws, 0)
        b = torch.cat(bs, 0) if bs[0] is not None else None
        ctx.save_for_backward(x2, w)
        ctx.n, ctx.has_bias = n, bs[0] is not None
        return torch.nn.functional.linear(x2, w, b)

    @staticmethod
    def backward(ctx, dy):
        x2, w = ctx.saved_tensors
        dy = dy.contiguous()
        dx = torch.mm(dy, w)
        dws = _weight_grad(dy, x2).chunk(ctx.n, 0)
        dbs = dy.sum(0).chunk(ctx.n, 0) if ctx.has_bias else (None,) * ctx.n
        return (dx, None, *dws, *dbs)


def _project_packed(x, layers):
    """Apply nn.Linear layers that share the input x [..., in] (all with or
    all without bias) as one GEMM; returns [..., n * out]."""
    lead = x.shape[:-1]
    x2 = x.reshape(-1, x.shape[-1])
    if not x2.is_contiguous():
        x2 = x2.contiguous()
    y = PackedProjectionFunction.apply(x2, len(layers), *[l.weight for l in layers],
                                       *[l.bias for l in layers])
    return y.view(*lead, y.shape[-1])


def _project(x, layers):
    """Apply nn.Linear layers that share the input x [..., in]."""
    lead = x.shape[:-1]
    x2 = x.reshape(-1, x.shape[-1])
    if not x2.is_contiguous():
        x2 = x2.contiguous()
    ys = ProjectionFunction.apply(x2, len(layers), *[l.weight for l in layers],
                                  *[l.bias for l in layers])
    return [y.view(*lead, y.shape[-1]) for y in ys]


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
    experiments). heads * 64 must equal dim. qk_norm adds one layer norm over
    the 64 values of every head's query and one for keys (gain and bias
    shared by all heads, held by the q_norm / k_norm LayerNorm containers and
    applied by the library's kernels). bias adds biases to the four
    projections."""

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
        self.fuse_qk_norm = True  # set False to run qk_norm as separate kernels
        self._fusable = {}

    def _fused(self, x, B, N):
        if not (self.qk_norm and self.fuse_qk_norm and self.q_norm.eps == self.k_norm.eps):
            return False
        key = (B, N, x.dtype)
        if key not in self._fusable:
            self._fusable[key] = qknorm_fused_supported(B, N, self.heads, self.patterns,
                                                        _dtype_code(x))
        return self._fusable[key]

    def forward(self, x):
        B, N, _ = x.shape
        shape = (B, N, self.heads, self.HEAD_DIM)
        if self._fused(x, B, N):
            # q, k, v from one GEMM, read by the attention kernels in place
            qkv = _project_packed(x, [self.to_q, self.to_k, self.to_v])
            o = QKNormAttnFunction.apply(qkv.view(B, N, 3, self.heads, self.HEAD_DIM),
                                         self.q_norm.weight, self.q_norm.bias,
                                         self.k_norm.weight, self.k_norm.bias, self.q_norm.eps,
                                         self.patterns, self.causal, self.scale)
            return _project(o.view(B, N, self.dim), [self.to_out])[0]
        q, k, v = (t.view(shape) for t in _project(x, [self.to_q, self.to_k, self.to_v]))
        if self.qk_norm:
            q, k = QKNormFunction.apply(q, k, self.q_norm.weight, self.q_norm.bias,
                                        self.k_norm.weight, self.k_norm.bias, self.q_norm.eps)
        o = dilated_attention(q, k, v, self.patterns, self.causal, self.scale)
        return _project(o.view(B, N, self.dim), [self.to_out])[0]
