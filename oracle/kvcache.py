"""Models of the dual-pool KV cache, the window-safe prefix length and KV byte accounting.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).  These are position-level models: they say
which token position each slot or page row must hold, never how the device arena is laid out.

Sources: [SWA-theory] §Rolling Buffer KV Cache (Eq.(7)), §MistralにおけるSWAの採用 (KV size per
layer), §計算時間・メモリ比較実験 (KV size calculator), §窓サイズと有効受容野 (Eq.(6));
[MiMo-review] §アーキテクチャ (hybrid stack, KV ratio) and §潜在力を本番へ (dual pool,
window-safe length).
"""
from __future__ import annotations

import numpy as np

from .attention import key_range


# --------------------------------------------------------------------------------------------
# Hybrid stack layer map
# --------------------------------------------------------------------------------------------

def layer_is_full(layer: int, period: int = 7) -> bool:
    """[MiMo-review, §アーキテクチャ]: of 70 layers, 10 use full attention and 60 use a 128-token
    window (about one global layer in seven).  The page does not say where the full layers sit;
    the reading taken here is every ``period``-th layer, 0-based ``layer % 7 == 6``."""
    return layer % period == period - 1


# --------------------------------------------------------------------------------------------
# Rolling buffer (one SWA layer, one sequence, one KV head)
# --------------------------------------------------------------------------------------------

class RollingBuffer:
    """w-slot ring: the token at position t goes to slot t mod w.  [SWA-theory, Eq.(7)]

    ``tags[s]`` is the position whose key/value slot ``s`` holds (-1 if never written).
    """

    def __init__(self, w: int, d: int):
        if w < 1:
            raise ValueError("window must be >= 1")
        self.w = w
        self.k = np.zeros((w, d))
        self.v = np.zeros((w, d))
        self.tags = np.full(w, -1, dtype=np.int64)
        self.length = 0

    def append(self, k_rows, v_rows) -> None:
        for kr, vr in zip(np.atleast_2d(k_rows), np.atleast_2d(v_rows)):
            s = self.length % self.w           # Eq.(7)
            self.k[s] = kr
            self.v[s] = vr
            self.tags[s] = self.length
            self.length += 1

    def copy(self) -> "RollingBuffer":
        c = RollingBuffer(self.w, self.k.shape[1])
        c.k, c.v, c.tags, c.length = self.k.copy(), self.v.copy(), self.tags.copy(), self.length
        return c

    def resident_positions(self) -> list[int]:
        return sorted(int(t) for t in self.tags if t >= 0)

    def read(self, p: int):
        """Key/value of position ``p``; raises if the slot no longer (or never) held it."""
        s = p % self.w
        if self.tags[s] != p:
            raise KeyError(f"position {p} not resident (slot {s} holds {self.tags[s]})")
        return self.k[s], self.v[s]

    def read_unchecked(self, p: int):
        """What a reader that trusts the slot rule without checking tags would get."""
        s = p % self.w
        return self.k[s], self.v[s]

    def memory_bytes(self, n_heads: int, elem_bytes: int) -> int:
        """Fixed buffer size for ``n_heads`` heads: K and V, w slots each.  [SWA-theory,
        §Rolling Buffer KV Cacheの実装: the buffer holds w·H·d elements for K and as many for V]"""
        return 2 * self.w * n_heads * self.k.shape[1] * elem_bytes


def resident_after(length: int, w: int) -> list[int]:
    """Positions a w-slot ring holds after ``length`` appends: the last min(length, w)."""
    return list(range(max(0, length - w), length))


def slot_of(p: int, w: int) -> int:
    """[SWA-theory, Eq.(7)] idx(t) = t mod w."""
    return p % w


def decode_via_buffer(q_row, buf: RollingBuffer, k_new, v_new, i: int, w: int, checked=True):
    """Attention for one query row at position ``i`` = buf.length (one new token) where every prior
    key comes out of the ring by its position and the new key from ``k_new``/``v_new``.

    Computed with the same Eq.(3)-(5) as ``attention.attend_row`` but gathering keys through the
    buffer model, so that comparing the two checks "rolling buffer = masked full cache"."""
    lo, hi = key_range(i, w)
    ks, vs = [], []
    for p in range(lo, hi):
        if p == i:
            ks.append(k_new)
            vs.append(v_new)
        else:
            kk, vv = buf.read(p) if checked else buf.read_unchecked(p)
            ks.append(kk)
            vs.append(vv)
    kk = np.asarray(ks, dtype=np.float64)
    vv = np.asarray(vs, dtype=np.float64)
    q = np.asarray(q_row, dtype=np.float64)
    s = kk @ q / np.sqrt(q.shape[-1])
    p_ = np.exp(s - s.max())
    return (p_ @ vv) / p_.sum()


# --------------------------------------------------------------------------------------------
# Paged full-attention pool placement
# --------------------------------------------------------------------------------------------

def page_placement(p: int, page_table: list[int], page_tokens: int) -> tuple[int, int]:
    """Where position ``p`` of a sequence lives in the paged O(N) pool: (page id, row in page).
    The page size (16 tokens) is this build's choice, not the pages'."""
    return page_table[p // page_tokens], p % page_tokens


def pages_needed(length: int, page_tokens: int) -> int:
    return -(-length // page_tokens)


# --------------------------------------------------------------------------------------------
# Window-safe prefix length  [MiMo-review, §潜在力を本番へ]
# --------------------------------------------------------------------------------------------

def window_safe_len(tags_per_layer, donor_len: int, match_len: int, w: int) -> int:
    """Brute force.  A prefix of length m' of the donor may be reused only if, in every SWA layer,
    every position p in the last W tokens before m', i.e. [max(0, m'-w), m'), still has a valid
    slot (tag[p mod w] == p).  The result is the largest such m' <= min(match_len, donor_len);
    m' = 0 always qualifies.  The page's "last W tokens" is taken literally (w positions), which is
    never less safe than Eq.(1)'s w-1 earlier keys.  One m' truncates both pools."""
    hi = min(match_len, donor_len)
    for m in range(hi, -1, -1):
        ok = True
        for tags in tags_per_layer:
            for p in range(max(0, m - w), m):
                if tags[p % w] != p:
                    ok = False
                    break
            if not ok:
                break
        if ok:
            return m
    return 0


def window_safe_len_closed(donor_len: int, match_len: int, w: int) -> int:
    """Closed form for a pure rolling buffer that has taken ``donor_len`` contiguous appends:
    it holds positions [donor_len - w, donor_len), so a cut m' < donor_len is safe only when the
    whole history still fits (donor_len <= w) and m' = donor_len is always safe."""
    m = min(match_len, donor_len)
    if donor_len <= w or m == donor_len:
        return m
    return 0


def reusable_len(sources, match_len: int, w: int) -> int:
    """Prefix-cache reuse with ring snapshots ([MiMo-review] §潜在力を本番へ: the prefix cache tree is
    rebuilt around the window-safe length).  ``sources`` are (length, tags_per_layer) pairs: the
    donor itself and every retained snapshot of it (a copy of its rings taken at that length).  Each
    source offers its own window-safe length for the match; the reusable length is the largest.
    Brute force over window_safe_len."""
    best = 0
    for length, tags in sources:
        best = max(best, window_safe_len(tags, length, match_len, w))
    return best


def reusable_len_closed(donor_len: int, snapshot_lens, match_len: int, w: int) -> int:
    """Closed form for contiguous appends: the best of the closed-form window-safe lengths of the
    donor and of each snapshot (a snapshot of length s holds [s - w, s), so it serves a match of
    at least s exactly at s, and any cut when s <= w)."""
    cands = [window_safe_len_closed(donor_len, match_len, w)]
    cands += [window_safe_len_closed(s, match_len, w) for s in snapshot_lens]
    return max(cands)


# --------------------------------------------------------------------------------------------
# KV byte accounting
# --------------------------------------------------------------------------------------------

def kv_cache_size_mb(seq_len: int, num_layers: int, num_kv_heads: int, head_dim: int,
                     window_size: int | None = None, dtype_bytes: int = 2) -> float:
    """KV size in MiB for a stack whose layers keep ``window_size`` tokens (or all ``seq_len``).
    K and V, per layer, per KV head.  Restates the page's KV size calculator
    [SWA-theory, §計算時間・メモリ比較実験, KVキャッシュサイズの比較]."""
    kept = window_size if window_size else seq_len
    return 2 * num_layers * num_kv_heads * kept * head_dim * dtype_bytes / 2**20


def dual_pool_bytes(lengths, layer_full, w: int, n_kv_heads: int, head_dim: int, elem_bytes: int,
                    page_tokens: int, shared_pages: int = 0):
    """Bytes the dual pool holds for sequences of the given lengths.

    SWA layers: the ring is allocated at w slots (``allocated``) and holds min(L, w) live tokens
    (``resident``).  Full layers: ceil(L/page)·page token rows, allocated and resident alike.
    ``shared_pages`` (per full layer) are pages counted once although several sequences map them.
    Returns (allocated, resident).
    """
    tok = 2 * n_kv_heads * head_dim * elem_bytes
    alloc = res = 0
    for L in lengths:
        for full in layer_full:
            if full:
                b = pages_needed(L, page_tokens) * page_tokens * tok
                alloc += b
                res += b
            else:
                alloc += w * tok
                res += min(L, w) * tok
    n_full = sum(1 for f in layer_full if f)
    alloc -= shared_pages * n_full * page_tokens * tok
    res -= shared_pages * n_full * page_tokens * tok
    return alloc, res


def hybrid_kv_ratio(N: int, W: int, n_swa: int = 60, n_full: int = 10) -> float:
    """[MiMo-review, §アーキテクチャ]: total KV relative to an all-full stack,
    (n_swa·W + n_full·N) / ((n_swa+n_full)·N), with W replaced by min(N, W) so that short
    sequences (which never fill the window) give 1 rather than more than 1."""
    return (n_swa * min(N, W) + n_full * N) / ((n_swa + n_full) * N)


# --------------------------------------------------------------------------------------------
# Receptive field of a stack of window layers (self-check of mask composition)
# --------------------------------------------------------------------------------------------

def receptive_field_formula(L: int, w: int) -> int:
    """[SWA-theory, §窓サイズと有効受容野, Eq.(6)] R(L) = L(w-1) + 1."""
    return L * (w - 1) + 1


def receptive_field_brute(L: int, w: int, n: int, target: int) -> int:
    """Number of input positions whose information can reach ``target`` through L window layers,
    by composing the Eq.(2) mask L times (boolean matrix reachability)."""
    m = np.zeros(n, dtype=bool)
    m[target] = True
    for _ in range(L):
        nxt = np.zeros(n, dtype=bool)
        for pos in np.nonzero(m)[0]:
            lo, hi = key_range(int(pos), w)
            nxt[lo:hi] = True
        m = nxt
    return int(m.sum())
