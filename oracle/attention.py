"""fp64 causal sliding-window attention, written out from its definition.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Everything is indexed by absolute token position (0-based, as in the page's mask code), never by
where a key sits in a cache.  A query at position i sees the keys W(i) (Eq.(1)); scores are
q·k/sqrt(d) on W(i) and -inf elsewhere (Eq.(2)-(3)); weights are a softmax over the row (Eq.(4));
the output is the weighted sum of the values in W(i) (Eq.(5)).  [SWA-theory, §数学的定義]

The softmax is computed in two passes (row max, then exp and sum) in float64, with no tiling, no
online rescaling and no split over keys.  Tiling, online softmax and split-K reach the same real
number, so this plain definition is the oracle for all of them.
"""
from __future__ import annotations

import math

import numpy as np


def key_range(i: int, w: int | None) -> tuple[int, int]:
    """Half-open range [lo, i+1) of the key positions a query at position ``i`` may see.

    [SWA-theory, §数学的定義, Eq.(1)]: W(i) = {j : max(0, i-w+1) <= j <= i}.  The window holds
    the query's own position, so at most w keys.  ``w=None`` is full causal attention (all j <= i).
    """
    if i < 0:
        raise ValueError("position must be >= 0")
    if w is None:
        return 0, i + 1
    if w < 1:
        raise ValueError("window must be >= 1")
    return max(0, i - w + 1), i + 1


def mask(n: int, w: int | None) -> np.ndarray:
    """Dense boolean mask M (n x n), M[i, j] = 1 iff j in W(i).  [SWA-theory, Eq.(2)]"""
    m = np.zeros((n, n), dtype=bool)
    for i in range(n):
        lo, hi = key_range(i, w)
        m[i, lo:hi] = True
    return m


def mask_nonzeros(n: int, w: int | None) -> int:
    """Number of (query, key) pairs in an n-token causal window mask: sum over i of |W(i)|."""
    return sum(hi - lo for lo, hi in (key_range(i, w) for i in range(n)))


def kv_head_of(h: int, n_q_heads: int, n_kv_heads: int) -> int:
    """KV head shared by query head ``h`` under grouped-query attention.

    [SWA-theory, §MistralにおけるSWAの採用]: several query heads share one KV head (32 q heads over
    8 KV heads in Mistral).  The page does not say which heads share; the reading taken here is
    contiguous groups of G = Hq/Hkv query heads.
    """
    if n_q_heads % n_kv_heads:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    return h // (n_q_heads // n_kv_heads)


def attend_row(q: np.ndarray, k: np.ndarray, v: np.ndarray, i: int, w: int | None) -> np.ndarray:
    """Output for the query vectors ``q`` ([R, d], all at position ``i``, all using the same KV head).

    ``k`` and ``v`` are that KV head's logical keys and values by position ([T, d], T > i).
    Eq.(3): s_j = q·k_j / sqrt(d) for j in W(i) (keys outside W(i) have -inf and weight 0, so they
    are left out).  Eq.(4): weights exp(s_j - max s) / sum exp(s - max s).  Eq.(5): o = sum a_j v_j.
    """
    q = np.asarray(q, dtype=np.float64)
    lo, hi = key_range(i, w)
    if hi > k.shape[0]:
        raise ValueError("history shorter than the query position")
    kk = np.asarray(k[lo:hi], dtype=np.float64)
    vv = np.asarray(v[lo:hi], dtype=np.float64)
    s = (q @ kk.T) / math.sqrt(q.shape[-1])          # [R, |W(i)|]
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    return (p @ vv) / p.sum(axis=-1, keepdims=True)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, pos0: int, w: int | None,
              rows=None) -> np.ndarray:
    """Causal (sliding-window when ``w`` is set) attention for a block of queries.

    q     [n, Hq, d_k]  queries at positions pos0 .. pos0+n-1 (post-RoPE; RoPE itself is out of scope)
    k, v  [T, Hkv, d_k], [T, Hkv, d_v]  logical keys/values at positions 0 .. T-1, T >= pos0 + n
    rows  optional iterable of row indices into q to compute (others are left as NaN)
    Returns fp64 [n, Hq, d_v].
    """
    q = np.asarray(q)
    n, hq, _ = q.shape
    hkv = k.shape[1]
    out = np.full((n, hq, v.shape[-1]), np.nan, dtype=np.float64)   # d_v may differ from d_k
    g_size = hq // hkv
    kv_head_of(0, hq, hkv)  # validates the head counts
    for r in (range(n) if rows is None else rows):
        i = pos0 + r
        for g in range(hkv):
            hs = slice(g * g_size, (g + 1) * g_size)
            out[r, hs] = attend_row(q[r, hs], k[:, g], v[:, g], i, w)
    return out


def decode_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, prior_len: int, w: int | None) -> np.ndarray:
    """A decode / verify step: ``q`` [q_len, Hq, d] at positions prior_len .. prior_len+q_len-1 over
    the logical history ``k``/``v`` [prior_len+q_len, Hkv, d] (prior tokens then the new ones).
    The same formula as prefill, evaluated at the new positions."""
    return attention(q, k, v, prior_len, w)


def attention_flops(n: int, pos0: int, w: int | None, n_q_heads: int, d: int) -> int:
    """Algorithmic flops of a block: 4·d per (query, key) pair in W(i), per query head
    (2·d for q·k and 2·d for the weighted sum of v).  Cost O(n·w·d) [SWA-theory, §計算量の分析]."""
    pairs = sum(hi - lo for lo, hi in (key_range(pos0 + r, w) for r in range(n)))
    return 4 * d * pairs * n_q_heads
