"""CPU oracle of the DilatedAttention module: projections around dilated
attention, forward and backward, in float64 NumPy.

TEST INFRASTRUCTURE ONLY, like the rest of this package.

The module (LongNet package README: the DilatedAttention parameters dim,
heads, dilation_rate, segment_size, qk_norm and its usage example) maps
x [B, N, dim] to y [B, N, dim]. The pages give its interface, not its
insides; this oracle takes the plainest reading the pages support:

* queries, keys and values are linear maps of x (LONGNET blog, "About the
  Transformer model": Q, K, V are sequence-length x model-size matrices;
  "Token expansion reaches 1 billion+": each device projects its fragment
  into queries, keys and values): q = x Wq^T, k = x Wk^T, v = x Wv^T, each
  [B, N, heads * 64] viewed as [B, N, heads, 64], plus optional biases;
* qk_norm: each head's q and k vectors are layer-normalised over their 64
  values (mean and biased variance, eps), then scaled and shifted by a
  per-value gain and bias shared by all heads;
* dilated attention with the module's (segment_size, dilation_rate)
  patterns: the attention oracle of this package;
* y = o Wo^T (+ bo), o the attention output viewed as [B, N, dim].

Matrix products use NumPy's matmul (a library primitive).
"""
import numpy as np

import oracle as _oracle

LN_EPS = 1e-5


def layer_norm(x, gain, bias, eps=LN_EPS):
    """Normalise the last axis: (x - mean) / sqrt(var + eps) * gain + bias,
    with the biased variance. Returns the output and the normalised values
    and inverse deviations the backward pass needs."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    inv = 1.0 / np.sqrt(var + eps)
    xh = (x - mu) * inv
    return xh * gain + bias, xh, inv


def layer_norm_bwd(dy, xh, inv, gain):
    """Gradients of layer_norm: with g = dy * gain and n values per row,
    dx = inv * (g - mean(g) - xh * mean(g * xh)); dgain and dbias sum
    dy * xh and dy over every row."""
    g = dy * gain
    dx = inv * (g - g.mean(axis=-1, keepdims=True) - xh * (g * xh).mean(axis=-1, keepdims=True))
    red = tuple(range(dy.ndim - 1))
    return dx, (dy * xh).sum(axis=red), dy.sum(axis=red)


def module_fwd(x, params, heads, patterns, qk_norm=False, causal=True, orc=None):
    """y = module(x) for float64 x [B, N, dim].

    params: dict with wq, wk, wv, wo ([dim, dim], torch Linear layout:
    out-features first), optional bq, bk, bv, bo ([dim]), and with qk_norm
    q_gain, q_bias, k_gain, k_bias ([64]). Returns (y, cache)."""
    orc = orc or _oracle.default()
    B, N, dim = x.shape
    Dh = dim // heads

    def lin(name, b):
        y = x @ params[name].T
        return y + params[b] if params.get(b) is not None else y

    q = lin("wq", "bq").reshape(B, N, heads, Dh)
    k = lin("wk", "bk").reshape(B, N, heads, Dh)
    v = lin("wv", "bv").reshape(B, N, heads, Dh)
    cache = {"x": x, "params": params, "heads": heads, "patterns": patterns,
             "qk_norm": qk_norm, "causal": causal, "orc": orc}
    if qk_norm:
        q, cache["q_xh"], cache["q_inv"] = layer_norm(q, params["q_gain"], params["q_bias"])
        k, cache["k_xh"], cache["k_inv"] = layer_norm(k, params["k_gain"], params["k_bias"])
    o, lse = orc.fwd(np.ascontiguousarray(q), np.ascontiguousarray(k), np.ascontiguousarray(v),
                     patterns, causal=causal)
    o2 = o.reshape(B, N, dim)
    y = o2 @ params["wo"].T
    if params.get("bo") is not None:
        y = y + params["bo"]
    cache.update(q=q, k=k, v=v, o=o2, lse=lse)
    return y, cache


def module_bwd(dy, cache, terms=False):
    """Gradients of sum(dy * y): returns (dx, grads), grads keyed like params.

    Every parameter gradient is a sum over the B * N rows. With terms=True
    a third result gives, per parameter, the root of the sum over rows of
    the squared per-row contributions (same shape as the gradient), the
    scale of that sum's accumulated rounding."""
    p = cache["params"]
    x, o2 = cache["x"], cache["o"]
    B, N, dim = x.shape
    heads = cache["heads"]
    Dh = dim // heads
    grads = {}
    l2 = {}

    def outer_l2(a, b):  # sqrt(sum over rows of (a_i b_j)^2)
        return np.sqrt((a * a).T @ (b * b))

    def sum_l2(a):  # sqrt(sum over rows of a^2), a [rows, n]
        return np.sqrt((a * a).sum(axis=0))

    # y = o Wo^T + bo
    dy2 = dy.reshape(-1, dim)
    grads["wo"] = dy2.T @ o2.reshape(-1, dim)
    l2["wo"] = outer_l2(dy2, o2.reshape(-1, dim))
    if p.get("bo") is not None:
        grads["bo"] = dy.sum(axis=(0, 1))
        l2["bo"] = sum_l2(dy2)
    do = (dy @ p["wo"]).reshape(B, N, heads, Dh)
    dq, dk, dv = cache["orc"].bwd(np.ascontiguousarray(cache["q"]), np.ascontiguousarray(cache["k"]),
                                  np.ascontiguousarray(cache["v"]), np.ascontiguousarray(do),
                                  cache["patterns"], causal=cache["causal"])
    if cache["qk_norm"]:
        for t in ("q", "k"):
            g_out = dq if t == "q" else dk
            l2[t + "_gain"] = sum_l2((g_out * cache[t + "_xh"]).reshape(-1, Dh))
            l2[t + "_bias"] = sum_l2(g_out.reshape(-1, Dh))
        dq, grads["q_gain"], grads["q_bias"] = layer_norm_bwd(dq, cache["q_xh"], cache["q_inv"],
                                                             p["q_gain"])
        dk, grads["k_gain"], grads["k_bias"] = layer_norm_bwd(dk, cache["k_xh"], cache["k_inv"],
                                                             p["k_gain"])
    dx = np.zeros_like(x)
    x2 = x.reshape(-1, dim)
    for name, b, d in (("wq", "bq", dq), ("wk", "bk", dk), ("wv", "bv", dv)):
        d2 = d.reshape(-1, dim)
        grads[name] = d2.T @ x2
        l2[name] = outer_l2(d2, x2)
        if p.get(b) is not None:
            grads[b] = d2.sum(axis=0)
            l2[b] = sum_l2(d2)
        dx += (d2 @ p[name]).reshape(B, N, dim)
    return (dx, grads, l2) if terms else (dx, grads)
