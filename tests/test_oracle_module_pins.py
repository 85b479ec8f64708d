"""Pins for the oracle of the DilatedAttention module (projections, optional
qk_norm, dilated attention, output projection) and its backward pass.

The oracle composes NumPy products, a written-out layer norm and the
attention oracle. It is checked against torch's autograd through torch's own
CPU float64 linear and layer_norm routines wrapped around the brute-force
union softmax (tests/brute_force.py), which shares nothing with the oracle,
on every output and gradient element.
"""
import importlib.util

import numpy as np
import pytest
import torch

from oracle import module as om
from tests.brute_force import union_softmax_torch


def make_params(dim, heads, qk_norm, bias, seed):
    r = np.random.default_rng(seed)
    Dh = dim // heads
    p = {n: r.standard_normal((dim, dim)) / np.sqrt(dim) for n in ("wq", "wk", "wv", "wo")}
    for n in ("bq", "bk", "bv", "bo"):
        p[n] = r.standard_normal(dim) * 0.1 if bias else None
    if qk_norm:
        for n in ("q_gain", "k_gain"):
            p[n] = 1.0 + 0.1 * r.standard_normal(Dh)
        for n in ("q_bias", "k_bias"):
            p[n] = 0.1 * r.standard_normal(Dh)
    return p


def torch_module(x, p, heads, patterns, qk_norm, causal):
    """Forward and gradients by torch autograd (float64, CPU)."""
    F = torch.nn.functional
    t = {n: (torch.tensor(v, requires_grad=True) if v is not None else None) for n, v in p.items()}
    tx = torch.tensor(x, requires_grad=True)
    B, N, dim = x.shape
    Dh = dim // heads
    q = F.linear(tx, t["wq"], t["bq"]).view(B, N, heads, Dh)
    k = F.linear(tx, t["wk"], t["bk"]).view(B, N, heads, Dh)
    v = F.linear(tx, t["wv"], t["bv"]).view(B, N, heads, Dh)
    if qk_norm:
        q = F.layer_norm(q, (Dh,), t["q_gain"], t["q_bias"], om.LN_EPS)
        k = F.layer_norm(k, (Dh,), t["k_gain"], t["k_bias"], om.LN_EPS)
    o = union_softmax_torch(q, k, v, patterns, causal)
    y = F.linear(o.reshape(B, N, dim), t["wo"], t["bo"])
    dy = torch.from_numpy(np.random.default_rng(99).standard_normal(y.shape))
    (y * dy).sum().backward()
    grads = {n: v.grad.numpy() for n, v in t.items() if v is not None}
    return y.detach().numpy(), tx.grad.numpy(), grads, dy.numpy()


def close(a, b, tol=1e-11):
    scale = max(1.0, float(np.abs(b).max()))
    assert float(np.abs(a - b).max()) / scale < tol


def pin_module_matches_torch_autograd(mod, qk_norm=True, bias=True, causal=True,
                                      patterns=((8, 2), (4, 1))):
    B, N, heads, dim = 2, 16, 2, 16
    p = make_params(dim, heads, qk_norm, bias, 5)
    x = np.random.default_rng(6).standard_normal((B, N, dim))
    y_t, dx_t, g_t, dy = torch_module(x, p, heads, list(patterns), qk_norm, causal)
    y, cache = mod.module_fwd(x, p, heads, list(patterns), qk_norm, causal)
    close(y, y_t)
    dx, g = mod.module_bwd(dy, cache)
    close(dx, dx_t)
    assert set(g) == set(g_t)
    for n in g:
        close(g[n], g_t[n])


def pin_layer_norm_matches_torch(mod):
    x = np.random.default_rng(7).standard_normal((3, 5, 64)) * 3 + 1
    gain = np.random.default_rng(8).standard_normal(64)
    bias = np.random.default_rng(9).standard_normal(64)
    y, xh, _ = mod.layer_norm(x, gain, bias)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (64,), torch.from_numpy(gain),
                                         torch.from_numpy(bias), mod.LN_EPS).numpy()
    close(y, ref, 1e-12)
    assert np.abs(xh.mean(-1)).max() < 1e-12


@pytest.mark.parametrize("qk_norm", [True, False])
@pytest.mark.parametrize("bias", [True, False])
@pytest.mark.parametrize("causal", [True, False])
def test_module_matches_torch_autograd(qk_norm, bias, causal):
    pin_module_matches_torch_autograd(om, qk_norm, bias, causal)


def test_module_single_pattern_usage_form():
    """The README's form: one (segment_size, dilation_rate) pattern."""
    pin_module_matches_torch_autograd(om, True, False, True, ((8, 2),))


def test_layer_norm_matches_torch():
    pin_layer_norm_matches_torch(om)


MODULE_MUTANTS = [
    ("var = ((x - mu) ** 2).mean(", "var = ((x - mu) ** 2).sum(", "variance summed, not averaged"),
    ("inv = 1.0 / np.sqrt(var + eps)", "inv = 1.0 / np.sqrt(var)", "layer-norm eps dropped"),
    ("return xh * gain + bias, xh, inv", "return xh * gain, xh, inv", "layer-norm bias dropped"),
    (" - xh * (g * xh).mean(axis=-1, keepdims=True))", ")",
     "layer-norm backward loses the variance term"),
    ('grads["wo"] = dy2.T @ o2.reshape(-1, dim)', 'grads["wo"] = o2.reshape(-1, dim).T @ dy2',
     "output weight gradient transposed"),
    ('do = (dy @ p["wo"])', 'do = (dy @ p["wo"].T)', "output projection backward transposed"),
    ("y = x @ params[name].T", "y = x @ params[name]", "input projections transposed"),
    ("dx += (d2 @ p[name])", "dx += (d2 @ p[name].T)", "input gradient through W^T"),
    ("grads[b] = d2.sum(axis=0)", "grads[b] = d2.mean(axis=0)", "bias gradient averaged"),
]


@pytest.mark.parametrize("mutant", MODULE_MUTANTS, ids=[m[2] for m in MODULE_MUTANTS])
def test_module_planted_mistakes_are_caught(tmp_path, mutant):
    old, new, _ = mutant
    src = open(om.__file__).read()
    assert src.count(old) >= 1, f"mutation site not found: {old!r}"
    path = tmp_path / "module_mutant.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("module_mutant", str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    caught = 0
    with np.errstate(all="ignore"):
        for pin in (pin_module_matches_torch_autograd, pin_layer_norm_matches_torch):
            try:
                pin(mod)
            except (AssertionError, ValueError, RuntimeError):
                caught += 1
    assert caught, "no pin rejects this planted mistake"
