"""Rotary position embedding with global positions, fp64 (test infrastructure only).

"Context Parallelism v.s. Sequence Parallelism (Megatron-LM)", section
"Implementation quirk: symmetric chunk assignment": rotary embeddings use each
token's position, so a rank holding chunks r and 2cp-1-r must rotate its tokens
by their *global* positions, never by a local renumbering 0, 1, 2, ...

The page gives no formula; the plain reading is the standard rotary embedding:
dimension pairs (a_j, b_j), j = 0 .. D/2-1, rotated by the angle pos * theta_j
with theta_j = base^(-2j/D):
    a' = a cos(pos theta_j) - b sin(pos theta_j)
    b' = a sin(pos theta_j) + b cos(pos theta_j).
Two pairings are in common use and both are provided: INTERLEAVED pairs
(2j, 2j+1); HALF pairs (j, j + D/2). A token with position -1 (a pad) is left
unchanged.
"""

from __future__ import annotations

import numpy as np

INTERLEAVED = 0
HALF = 1


def rope_pairs(d: int, style: int):
    """Index arrays (a, b) of the D/2 rotated pairs."""
    j = np.arange(d // 2)
    if style == INTERLEAVED:
        return 2 * j, 2 * j + 1
    if style == HALF:
        return j, j + d // 2
    raise ValueError("unknown rotary style")


def rope_theta(d: int, base: float):
    """Angular frequency of each pair: theta_j = base^(-2j/D), j = 0 .. D/2-1."""
    return np.power(float(base), -2.0 * np.arange(d // 2) / d)


def rope(x, pos, base: float = 10000.0, style: int = INTERLEAVED):
    """x [..., L, D] rotated by positions pos [L] (-1 = leave the row unchanged)."""
    x = np.asarray(x, dtype=np.float64)
    pos = np.asarray(pos)
    d = x.shape[-1]
    if d % 2:
        raise ValueError("D must be even")
    a, b = rope_pairs(d, style)
    theta = rope_theta(d, base)
    ang = pos.astype(np.float64)[:, None] * theta[None, :]          # [L, D/2]
    c, s = np.cos(ang), np.sin(ang)
    out = x.copy()
    xa, xb = x[..., a], x[..., b]
    ra = xa * c - xb * s
    rb = xa * s + xb * c
    keep = pos < 0
    out[..., a] = np.where(keep[:, None], xa, ra)
    out[..., b] = np.where(keep[:, None], xb, rb)
    return out
