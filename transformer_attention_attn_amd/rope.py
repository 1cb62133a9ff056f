"""Host-side rotary position tables for the encoder's fused RoPE prologue.

V-JEPA2 ViT-L Encoder NKI Kernels for AWS Trainium2, "Repository layout",
builds its 3D RoPE tables on the host; vit-encoder-neuron-kernels, "Kernels",
names the two lane pairings the kernel applies; gte-encoder-neuron-kernels
(introduction) uses rotate-half RoPE with NTK scaling.  The kernel reads one
(cos, sin) pair per token and rotation pair, so every positional layout is
decided here:

* ``grid_positions(*shape, prefix_tokens=0)``: the coordinates of a token grid
  (frames x rows x columns, rows x columns, or a 1D sequence) in row-major
  order, after ``prefix_tokens`` tokens that are not rotated (class and
  register tokens);
* ``rope_tables(positions, head_dim, base, ntk_factor, rotate)``: cos/sin
  [S, head_dim/2] fp32.  The head_dim/2 rotation pairs are split into one
  contiguous group per axis, of floor(head_dim/2 / axes) pairs each; pairs
  left over after the groups, and the rows of unrotated tokens, get angle 0
  (cos 1, sin 0).  Pair i of an axis group of P pairs turns by
  position * b^(-i/P) with b = base * ntk_factor^(P/(P-1)), the NTK-aware
  rescaling of the base (identity for ntk_factor = 1).

The pages give neither the split of the pairs over the axes nor the NTK
formula; the plainest readings are taken and the kernel does not depend on
them.  Plain host code (numpy, fp64 then rounded to fp32); nothing here runs
on the GPU.
"""
from __future__ import annotations

import numpy as np

__all__ = ["grid_positions", "rope_tables"]


def grid_positions(*shape: int, prefix_tokens: int = 0):
    """Coordinates of a row-major token grid after ``prefix_tokens``
    unrotated tokens.  Returns (positions float64 [S, len(shape)], rotate
    bool [S]) with S = prefix_tokens + prod(shape)."""
    if not shape or any(int(n) <= 0 for n in shape):
        raise ValueError("grid_positions: every extent must be positive")
    axes = np.meshgrid(*[np.arange(int(n), dtype=np.float64) for n in shape], indexing="ij")
    grid = np.stack([a.reshape(-1) for a in axes], axis=1)
    pre = np.zeros((prefix_tokens, len(shape)))
    rotate = np.concatenate([np.zeros(prefix_tokens, dtype=bool), np.ones(grid.shape[0], dtype=bool)])
    return np.concatenate([pre, grid], axis=0), rotate


def rope_tables(positions, head_dim: int, base: float = 10000.0, ntk_factor: float = 1.0, rotate=None):
    """cos/sin tables [S, head_dim/2] fp32 for ``positions`` [S] or [S, A]."""
    pos = np.asarray(positions, dtype=np.float64)
    if pos.ndim == 1:
        pos = pos[:, None]
    if pos.ndim != 2 or head_dim % 2:
        raise ValueError("rope_tables: positions [S] or [S, A] and an even head_dim")
    S, A = pos.shape
    pairs = head_dim // 2
    P = pairs // A
    if P < 1:
        raise ValueError("rope_tables: fewer rotation pairs than axes")
    if not (base > 1.0 and ntk_factor > 0.0):
        raise ValueError("rope_tables: base > 1 and ntk_factor > 0")
    b = base * ntk_factor ** (P / (P - 1)) if P > 1 else base * ntk_factor
    inv = b ** (-np.arange(P, dtype=np.float64) / P)
    theta = np.zeros((S, pairs))
    for a in range(A):
        theta[:, a * P:(a + 1) * P] = pos[:, a:a + 1] * inv[None, :]
    if rotate is not None:
        theta[~np.asarray(rotate, dtype=bool)] = 0.0
    return np.cos(theta).astype(np.float32), np.sin(theta).astype(np.float32)
