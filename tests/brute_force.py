"""Brute-force dilated attention for tiny inputs (a pin for the oracle).

Written without the oracle's structure: every pattern's sparsified segment is
cut out with NumPy step slicing (segment view, then [off::r]), and each row
takes ONE softmax over the multiset union of the keys that all of its
covering patterns give it. That union softmax equals the log-sum-exp merge
of per-pattern softmaxes, so the two formulations pin each other.
"""
import math

import numpy as np


def sparsified_positions(N, w, r, h, t):
    """Positions of the dilated segment that contains t for head h, or None
    when t is not among them."""
    wp = min(w, N)
    seg = t // wp
    positions = np.arange(seg * wp, (seg + 1) * wp)[h % r::r]
    return positions if t in positions else None


def union_softmax(q, k, v, patterns, causal=True, scale=None):
    """q, k, v float64 [B, N, H, Dh] -> out [B, N, H, Dh], lse [B, H, N]."""
    B, N, H, Dh = q.shape
    sc = scale if scale else 1.0 / math.sqrt(Dh)
    out = np.zeros((B, N, H, Dh))
    lse = np.full((B, H, N), -np.inf)
    for b in range(B):
        for h in range(H):
            for t in range(N):
                keys = []
                for (w, r) in patterns:
                    pos = sparsified_positions(N, w, r, h, t)
                    if pos is None:
                        continue
                    keys.extend(int(p) for p in pos if (not causal) or p <= t)
                if not keys:
                    continue
                kk = np.array(keys)
                s = sc * (k[b, kk, h, :] @ q[b, t, h, :])
                mx = s.max()
                e = np.exp(s - mx)
                lse[b, h, t] = mx + math.log(e.sum())
                out[b, t, h, :] = (e[:, None] * v[b, kk, h, :]).sum(0) / e.sum()
    return out, lse


def union_softmax_torch(q, k, v, patterns, causal=True, scale=None):
    """The same union softmax on torch float64 tensors [B, N, H, Dh], built
    from differentiable torch ops only, so torch's autograd gives the exact
    gradients of the definition (tiny inputs: one Python loop per row)."""
    import torch

    B, N, H, Dh = q.shape
    sc = scale if scale else 1.0 / math.sqrt(Dh)
    rows = []
    for b in range(B):
        for t in range(N):
            for h in range(H):
                keys = []
                for (w, r) in patterns:
                    pos = sparsified_positions(N, w, r, h, t)
                    if pos is None:
                        continue
                    keys.extend(int(p) for p in pos if (not causal) or p <= t)
                if not keys:
                    rows.append(torch.zeros(Dh, dtype=q.dtype))
                    continue
                kk = torch.tensor(keys)
                s = sc * (k[b, kk, h, :] @ q[b, t, h, :])
                rows.append(torch.softmax(s, dim=0) @ v[b, kk, h, :])
    return torch.stack(rows).reshape(B, N, H, Dh)
