"""Brute-force attention and LayerNorm in pure Python (test infrastructure only).

The literal textbook formulas with ``math.exp`` and ``math.fsum`` and no
max-subtraction, for tiny inputs only (S <= 16, D <= 8).  This is what the
fp64 oracle is pinned against; it shares nothing with ``oracle.c``.
"""
from __future__ import annotations

import math


def softmax_attention(q, k, v, scale, mask=None):
    """q: list of query vectors, k/v: lists of key/value vectors, mask: list or None.

    o_i = sum_j exp(scale*<q_i,k_j> + mask_j) v_j / sum_j exp(scale*<q_i,k_j> + mask_j)
    """
    out = []
    for qi in q:
        w = []
        for j, kj in enumerate(k):
            z = scale * math.fsum(a * b for a, b in zip(qi, kj)) + (mask[j] if mask else 0.0)
            w.append(0.0 if z == -math.inf else math.exp(z))
        den = math.fsum(w)
        out.append([math.fsum(w[j] * v[j][d] for j in range(len(k))) / den for d in range(len(v[0]))])
    return out


def layernorm_row(x, gamma=None, beta=None, eps=1e-6):
    n = len(x)
    mu = math.fsum(x) / n
    var = math.fsum((t - mu) ** 2 for t in x) / n
    r = 1.0 / math.sqrt(var + eps)
    g = gamma if gamma is not None else [1.0] * n
    b = beta if beta is not None else [0.0] * n
    return [(t - mu) * r * g[i] + b[i] for i, t in enumerate(x)], mu, r
