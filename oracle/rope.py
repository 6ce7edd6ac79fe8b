"""Rotary position embedding (RoPE) of queries and keys, in float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

[SWA-theory] §Rolling Buffer KV Cache (its subsection on position encoding): a rolling buffer stores
keys out of time order, which does no harm because RoPE puts each token's absolute position into its
query and key vectors, so a score q_i·k_j depends on the positions i and j and not on the slot a key
sits in.  The page names RoPE without writing it out; the definition used here is the published one
(Su et al., "RoFormer: Enhanced Transformer with Rotary Position Embedding", 2021, §3.2-§3.4):

* the head dimension d (even) is split into d/2 coordinate pairs; pair i is rotated by the angle
  p * theta_i at position p, with theta_i = base^(-2i/d), i = 0 .. d/2-1 (base 10000 in the paper);
* the rotation of a pair (x, y) by phi is (x cos phi - y sin phi, x sin phi + y cos phi), i.e. the
  pair read as the complex number x + iy is multiplied by e^(i phi).

Which coordinates form pair i is a layout choice the paper and later models make differently; both
are offered (the reading is a per-pool setting):

* ``"pairs"``: coordinates (2i, 2i+1), the paper's own layout;
* ``"halves"``: coordinates (i, i + d/2), the split-halves layout of GPT-NeoX-style models.

The two give the same rotation up to a fixed permutation of coordinates.
"""
from __future__ import annotations

import numpy as np

STYLES = ("pairs", "halves")


def frequencies(d: int, base: float = 10000.0) -> np.ndarray:
    """theta_i = base^(-2i/d) for i = 0 .. d/2-1 (float64)."""
    if d < 2 or d % 2:
        raise ValueError("head dimension must be even and >= 2")
    if not base > 0:
        raise ValueError("base must be positive")
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / d)


def pair_index(d: int, style: str) -> tuple[np.ndarray, np.ndarray]:
    """Coordinates (first, second) of each pair i = 0 .. d/2-1 under a layout."""
    i = np.arange(d // 2)
    if style == "pairs":
        return 2 * i, 2 * i + 1
    if style == "halves":
        return i, i + d // 2
    raise ValueError(f"unknown RoPE style {style!r}")


def rope(x, positions, base: float = 10000.0, style: str = "pairs") -> np.ndarray:
    """RoPE of ``x`` ([n, H, d] or [n, d]): row r is at position ``positions[r]`` (all heads of a row
    share it).  Every pair is rotated by positions[r] * theta_i, computed in float64."""
    x = np.asarray(x, dtype=np.float64)
    squeeze = x.ndim == 2
    if squeeze:
        x = x[:, None, :]
    n, _, d = x.shape
    pos = np.asarray(positions, dtype=np.float64).reshape(-1)
    if pos.shape[0] != n:
        raise ValueError("one position per row")
    a, b = pair_index(d, style)
    phi = pos[:, None] * frequencies(d, base)[None, :]          # [n, d/2]
    c = np.cos(phi)[:, None, :]
    s = np.sin(phi)[:, None, :]
    out = np.empty_like(x)
    out[..., a] = x[..., a] * c - x[..., b] * s
    out[..., b] = x[..., a] * s + x[..., b] * c
    return out[:, 0, :] if squeeze else out
