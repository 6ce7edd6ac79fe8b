"""Synthetic workloads on the 70-layer hybrid stack, built through the C ABI.

These builders only draw seeded inputs (``synth``) and drive the library's public calls; all
attention, commit and planning work runs in libswa.  They are shared by ``bench.py`` and the
full-size GPU tests.

Hybrid stack ([MiMo-review] §アーキテクチャ): 70 layers, layer l is full attention iff
l % 7 == 6 (10 layers), the other 60 use a 128-token window; 32 query heads over 4 KV heads,
d = 128, bf16.  Full layers keep 16-token pages; SWA layers a 128-slot ring per sequence.

Logical token streams.  Every sequence is a list of segments (start, stop, stream id): position p
of the sequence carries row p of stream ``stream id`` (K and V drawn per (seed, layer, stream) in
4096-token blocks, see ``synth.TokenStream``).  A fork that reuses a donor's prefix has the donor's
stream below the match length (same tokens, same K/V) and its own stream after it.

For SWA layers only the last w positions of a sequence are ever read (the ring), so the commit of a
long history passes a buffer whose last min(n, w) rows hold the stream's rows and whose earlier
rows are zero: kvpool_append reads only those last rows of an SWA layer, and the logical stream of
an SWA layer is defined as zero below the last w positions (no query can see them).
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

import synth

from . import swa as S

N_LAYERS, WINDOW, HQ, HKV, D = 70, 128, 32, 4, 128
CHUNK = 16384
DT = torch.bfloat16


def layer_full(l: int) -> bool:
    return l % 7 == 6


@dataclasses.dataclass
class Seq:
    sid: int                      # pool sequence id
    prior: int                    # committed length
    segments: list                # [(start, stop, stream_id)]


class Streams:
    """Device-drawn logical K/V of every (layer, stream id) for one seed."""

    def __init__(self, seed: int, device="cuda"):
        self.seed, self.device = seed, device

    def _ts(self, kind, layer, stream):
        return synth.TokenStream((self.seed, kind, layer, stream), HKV, D, DT, self.device)

    def rows(self, layer, segments, a, b):
        """K, V rows of positions [a, b) of a sequence made of `segments`."""
        ks, vs = [], []
        for (s0, s1, sid) in segments:
            lo, hi = max(a, s0), min(b, s1)
            if lo < hi:
                ks.append(self._ts("k", layer, sid).rows(lo, hi))
                vs.append(self._ts("v", layer, sid).rows(lo, hi))
        if not ks:
            e = torch.empty((0, HKV, D), dtype=DT, device=self.device)
            return e, e
        return (torch.cat(ks) if len(ks) > 1 else ks[0]), (torch.cat(vs) if len(vs) > 1 else vs[0])


def make_desc(pages_per_full_layer: int, max_seqs: int, max_seq_len: int, kv=DT, max_snapshots=0,
              decode_plan="uniform"):
    """The hybrid stack's pool descriptor; ``kv`` is the storage dtype (bf16, or
    torch.float8_e4m3fn with unit scales for FP8 KV storage); ``decode_plan`` the full-layer
    decode planner ("uniform" or "bucketed")."""
    return S.make_desc(N_LAYERS, WINDOW, HKV, D, kv, pages_per_full_layer, max_seqs, max_seq_len,
                       max_snapshots=max_snapshots, decode_plan=decode_plan)


class HybridPool:
    """A 70-layer hybrid pool over a torch-allocated arena (or a planning pool if plan=True)."""

    def __init__(self, pages_per_full_layer: int, max_seqs: int, max_seq_len: int, plan=False, kv=DT,
                 max_snapshots=0, decode_plan="uniform"):
        self.desc = make_desc(pages_per_full_layer, max_seqs, max_seq_len, kv, max_snapshots, decode_plan)
        self.kv = kv
        self.plan = plan
        if plan:
            self.arena = None
            self.h = S.kvpool_create(self.desc)
        else:
            nbytes = S.kvpool_arena_bytes(self.desc)
            self.arena = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
            self.h = S.kvpool_create(self.desc, self.arena, nbytes)
        self.max_seq_len = max_seq_len
        self._zero = None

    def close(self):
        if self.h:
            if not self.plan:
                torch.cuda.synchronize()
            S.kvpool_destroy(self.h)
            self.h = None
        self.arena = None

    def commit(self, streams: Streams | None, seq: Seq, a: int, b: int, layers=None):
        """Append positions [a, b) of `seq` to every layer, or to `layers` (layers are independent;
        the sequence's committed length in each is a)."""
        if b <= a:
            return
        for l in (range(N_LAYERS) if layers is None else layers):
            if self.plan:
                S.kvpool_append(self.h, seq.sid, l, None, None, b - a)
                continue
            if layer_full(l):
                for c0 in range(a, b, CHUNK):
                    c1 = min(b, c0 + CHUNK)
                    k, v = streams.rows(l, seq.segments, c0, c1)
                    S.kvpool_append(self.h, seq.sid, l, k, v)
            else:
                n = b - a
                tail = min(n, WINDOW)
                kt, vt = streams.rows(l, seq.segments, b - tail, b)
                if tail == n:
                    S.kvpool_append(self.h, seq.sid, l, kt, vt)
                else:
                    kz, vz = self._zero_rows(n)
                    kz[n - tail:n].copy_(kt)
                    vz[n - tail:n].copy_(vt)
                    S.kvpool_append(self.h, seq.sid, l, kz[:n], vz[:n])

    def _zero_rows(self, n):
        """A reusable [>= n, HKV, D] buffer pair; only its rows [n - min(n, w), n) are ever read
        by an SWA-layer commit, so the rest may hold anything."""
        if self._zero is None or self._zero[0].shape[0] < n:
            m = max(n, 1 << 16)
            self._zero = (torch.zeros((m, HKV, D), dtype=DT, device="cuda"),
                          torch.zeros((m, HKV, D), dtype=DT, device="cuda"))
        return self._zero


# ----------------------------------------------------------------------------------------------
# Batched decode on the hybrid stack: 256 sequences, contexts U{1..65536}, half of them forks
# ----------------------------------------------------------------------------------------------

@dataclasses.dataclass
class DecodeSetup:
    pool: HybridPool
    streams: Streams
    seqs: list
    forks: dict                   # sid -> (donor sid, kind, match, window-safe length)
    q: list                       # per layer [n, 1, HQ, D]
    kn: list                      # per layer [n, 1, HKV, D]
    vn: list
    ws: torch.Tensor


def _decode_plan(n_seqs: int, seed: int, max_ctx: int):
    rng = np.random.default_rng(seed)
    ctx = rng.integers(1, max_ctx + 1, size=n_seqs)        # context length includes the new token
    prior = ctx - 1
    n_don = n_seqs // 2
    kinds = {}
    for f in range(n_don, n_seqs):
        d = int(rng.integers(0, n_don))
        if f < n_don + (n_seqs - n_don) // 2:
            prior[f] = max(prior[f], prior[d])             # continue the donor
            kinds[f] = (d, "continue", int(prior[d]))
        else:
            m = int(rng.integers(0, min(prior[d], prior[f]) + 1))
            kinds[f] = (d, "branch", m)
    return [int(x) for x in prior], kinds


def _build_decode(pool: HybridPool, streams, prior, kinds):
    n = len(prior)
    seqs, forks = [], {}
    n_don = n // 2
    for i in range(n_don):
        sid = S.kvpool_seq_open(pool.h)
        s = Seq(sid, prior[i], [(0, prior[i], i)])
        pool.commit(streams, s, 0, prior[i])
        seqs.append(s)
    for f in range(n_don, n):
        d, kind, m = kinds[f]
        don = seqs[d]
        m_safe = S.kvpool_window_safe_len(pool.h, don.sid, m)
        sid = S.kvpool_seq_fork(pool.h, don.sid, m_safe)
        # positions below m are the donor's tokens (its own segment list), after m the fork's own
        segs = _restrict(seqs[d].segments, 0, m) + [(m, prior[f], f)]
        s = Seq(sid, prior[f], [x for x in segs if x[1] > x[0]])
        pool.commit(streams, s, m_safe, prior[f])
        seqs.append(s)
        forks[sid] = (don.sid, kind, m, m_safe)
    return seqs, forks


def _restrict(segments, a, b):
    out = []
    for (s0, s1, sid) in segments:
        lo, hi = max(a, s0), min(b, s1)
        if lo < hi:
            out.append((lo, hi, sid))
    return out


def build_decode(n_seqs=256, seed=4, max_ctx=65536, steps=16, device="cuda", kv=DT,
                 decode_plan="uniform") -> DecodeSetup:
    prior, kinds = _decode_plan(n_seqs, seed, max_ctx)
    max_len = max_ctx + steps + 16
    # size the page pool with a planning pool (metadata only), then build for real
    upper = n_seqs * (max_len // 16 + 2)            # every sequence holding its own pages
    plan = HybridPool(upper, n_seqs, max_len, plan=True, kv=kv)
    _build_decode(plan, None, prior, kinds)
    used = upper - S.kvpool_free_pages(plan.h, 6)
    plan.close()
    pages = used + n_seqs * ((steps + 15) // 16 + 2) + 64
    pool = HybridPool(pages, n_seqs, max_len, kv=kv, decode_plan=decode_plan)
    streams = Streams(seed, device)
    seqs, forks = _build_decode(pool, streams, prior, kinds)
    q = [synth.normal((n_seqs, 1, HQ, D), seed, "q", l, dtype=DT, device=device) for l in range(N_LAYERS)]
    kn = [synth.normal((n_seqs, 1, HKV, D), seed, "kn", l, dtype=DT, device=device) for l in range(N_LAYERS)]
    vn = [synth.normal((n_seqs, 1, HKV, D), seed, "vn", l, dtype=DT, device=device) for l in range(N_LAYERS)]
    sids = [s.sid for s in seqs]
    ws_bytes = max(S.swa_attn_workspace_bytes(pool.h, sids, l, 1, HQ) for l in (0, 6))
    ws = torch.empty(int(ws_bytes * 1.25) + (1 << 20), dtype=torch.uint8, device=device)
    return DecodeSetup(pool, streams, seqs, forks, q, kn, vn, ws)


def decode_step(st: DecodeSetup, out: torch.Tensor, commit=True, layer_events=None):
    """One decode step: every layer's attention for one new token per sequence, then the commit."""
    sids = np.array([s.sid for s in st.seqs], dtype=np.int32)  # one int32 buffer for all 140 calls
    h = st.pool.h
    for l in range(N_LAYERS):
        if layer_events is not None:
            layer_events[l][0].record()
        if layer_full(l):
            S.full_attn(h, sids, l, st.q[l], st.kn[l], st.vn[l], 1, HQ, out, st.ws)
        else:
            S.swa_attn_decode(h, sids, l, st.q[l], st.kn[l], st.vn[l], 1, HQ, out, st.ws)
        if layer_events is not None:
            layer_events[l][1].record()
        if commit:
            S.kvpool_append_batch(h, sids, l, st.kn[l], st.vn[l], 1)
    if commit:
        for s in st.seqs:
            s.prior += 1


def decode_logical_bytes(st: DecodeSetup, q_len=1):
    """Algorithmic bytes of one decode step: K+V of every key each (sequence, KV head) reads (shared
    pages counted per sequence, at the pool's storage size: 1 byte per element for FP8), plus Q and
    O (bf16), in every layer."""
    es = 1 if st.pool.kv == torch.float8_e4m3fn else 2
    kv_tok = 2 * HKV * D * es
    qo = 2 * len(st.seqs) * q_len * HQ * D * 2
    full = sum((s.prior + q_len) * kv_tok for s in st.seqs) + qo
    swa = sum(min(s.prior + q_len, WINDOW + q_len - 1) * kv_tok for s in st.seqs) + qo
    return full, swa  # per full layer, per SWA layer


# ----------------------------------------------------------------------------------------------
# Chunked hybrid prefill (128K in 16K chunks) and the 1M-prefix long-context case
# ----------------------------------------------------------------------------------------------

@dataclasses.dataclass
class PrefillSetup:
    pool: HybridPool
    seq: Seq
    streams: Streams
    q: dict                       # (layer, chunk) -> [CHUNK, HQ, D]
    seed: int


def chunk_inputs(streams: Streams, seed, layer, chunk_idx, seq: Seq, a, b, device="cuda"):
    q = synth.normal((b - a, HQ, D), seed, "q", layer, chunk_idx, dtype=DT, device=device)
    k, v = streams.rows(layer, seq.segments, a, b)
    return q, k, v


def build_hybrid_prefill(total=131072, seed=3, device="cuda") -> PrefillSetup:
    pages = total // 16 + 64
    pool = HybridPool(pages, 2, total + 64)
    streams = Streams(seed, device)
    sid = S.kvpool_seq_open(pool.h)
    seq = Seq(sid, 0, [(0, total, 0)])
    return PrefillSetup(pool, seq, streams, {}, seed)


def prefill_chunk(st: PrefillSetup, c: int, inputs, out, commit=True, events=None):
    """One chunk through all 70 layers: attention over the pool's prefix plus the chunk, then commit.
    `inputs[(l, c)]` = (q, k, v) of the chunk in layer l."""
    h = st.pool.h
    for l in range(N_LAYERS):
        q, k, v = inputs[(l, c)]
        if events is not None:
            events[l][0].record()
        if layer_full(l):
            S.full_attn(h, [st.seq.sid], l, q, k, v, q.shape[0], HQ, out)
        else:
            S.swa_attn_prefill(h, st.seq.sid, l, q, k, v, HQ, out)
        if events is not None:
            events[l][1].record()
        if commit:
            S.kvpool_append(h, st.seq.sid, l, k, v)


def build_long(prefix=1 << 20, chunk=CHUNK, verify=4, seed=5, device="cuda", layers=None, kv=DT) -> PrefillSetup:
    total = prefix + chunk + verify + 16
    pages = total // 16 + 64
    pool = HybridPool(pages, 2, total, kv=kv)
    streams = Streams(seed, device)
    sid = S.kvpool_seq_open(pool.h)
    seq = Seq(sid, 0, [(0, total, 0)])
    pool.commit(streams, seq, 0, prefix, layers=layers)
    seq.prior = prefix
    return PrefillSetup(pool, seq, streams, {}, seed)


def flops_prefill(n, pos0, w, hq=HQ, d=D):
    """Algorithmic flops of a chunk of n queries at positions pos0..: 4·d per (query, key) pair."""
    if w is None:
        pairs = n * pos0 + n * (n + 1) // 2
    else:
        pairs = 0
        lo, hi = pos0, pos0 + n - 1
        full_from = max(lo, w - 1)
        if hi >= full_from:
            pairs += (hi - full_from + 1) * w
        a, b = lo, min(hi, w - 2)
        if b >= a:
            pairs += (b + 1) * (b + 2) // 2 - a * (a + 1) // 2
    return 4 * d * hq * pairs
