"""Seeded random sweep of shapes through the C ABI against the fp64 oracle.

Each case draws a window (including w = 1..3 and windows that are not multiples of the 64-key
tile), a committed prefix, a chunk size (1 .. 257), a GQA group, a head dimension, the layer kind
and the pool dtype (fp32, bf16 or FP8 E4M3), runs a prefill of the chunk on top of the prefix, commits
it, then a batched decode / verify step (q_len 1..4) for that sequence and a second one.  Inputs
are seeded N(0,1) draws (synth); FP8 pools are compared against the oracle on the dequantised
committed values (oracle.fp8.roundtrip) and the call's own new tokens as passed.  Bars: fp32
max|d|/max|ref| <= 1e-5, bf16 (and FP8 pools) max|d| <= 2e-2, on every output tensor."""
import numpy as np
import pytest
import torch

import synth
from oracle import attention as A
from oracle import fp8 as F8
from tests.helpers import GpuPool, assert_close, to64

pytestmark = pytest.mark.gpu
BF = torch.bfloat16
FP8 = torch.float8_e4m3fn
F32 = torch.float32

WINDOWS = [1, 2, 3, 7, 31, 32, 33, 64, 65, 127, 128, 200, 300]
CHUNKS = [1, 2, 3, 5, 17, 63, 64, 65, 130, 257]


def make_case(i):
    g = np.random.default_rng(7000 + i)
    hkv = int(g.choice([1, 2]))
    return dict(
        w=int(g.choice(WINDOWS)), d=int(g.choice([64, 128])), hkv=hkv,
        grp=int(g.choice([1, 2, 4, 8, 16, 32])), full=bool(g.integers(0, 2)),
        kv=[FP8, FP8, F32, F32, BF, BF, BF, BF, BF][int(g.integers(0, 9))], prefix=int(g.integers(0, 400)),
        n=int(g.choice(CHUNKS)), q_len=int(g.integers(1, 5)), other=int(g.integers(0, 300)))


@pytest.fixture(scope="module")
def S():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import long_context_swa_amd.swa as S
    return S


def draw(n, h, d, *key, dtype=BF):
    return synth.normal((n, h, d), *key, dtype=dtype).cuda()


def seen(k, kv):
    """What attention reads back for committed rows: FP8 pools hold E4M3 codes (unit scale)."""
    x = to64(k)
    return F8.roundtrip(x, 1.0) if kv == FP8 else x


@pytest.mark.parametrize("case", range(64))
def test_random_shapes_prefill_then_decode(S, case):
    c = make_case(case)
    print(f"[sweep] case {case}: {c}", flush=True)
    w, d, hkv, full, kv = c["w"], c["d"], c["hkv"], c["full"], c["kv"]
    hq = c["grp"] * hkv
    layer = 1 if full else 0
    win = None if full else w
    act = F32 if kv == F32 else BF      # activation dtype of the pool
    dr = lambda *a: draw(*a, dtype=act)  # noqa: E731
    pages = (c["prefix"] + c["n"] + c["other"] + 16) // 16 * 2 + 8
    with GpuPool(S, n_layers=2, window=w, hkv=hkv, d=d, dtype=kv, pages=pages, max_seqs=2,
                 max_seq_len=1024, layer_is_full=[0, 1]) as P:
        a, b = S.kvpool_seq_open(P.h), S.kvpool_seq_open(P.h)
        hk = {a: np.zeros((0, hkv, d)), b: np.zeros((0, hkv, d))}   # committed rows as read back
        hv = {a: np.zeros((0, hkv, d)), b: np.zeros((0, hkv, d))}
        for s, L, tag in ((a, c["prefix"], "pa"), (b, c["other"], "pb")):
            if L:
                k, v = dr(L, hkv, d, 90, case, tag, "k"), dr(L, hkv, d, 90, case, tag, "v")
                S.kvpool_append(P.h, s, layer, k, v)
                hk[s], hv[s] = seen(k, kv), seen(v, kv)

        # prefill of the chunk on top of the prefix
        n, L0 = c["n"], c["prefix"]
        q, k, v = dr(n, hq, d, 90, case, "q"), dr(n, hkv, d, 90, case, "k"), dr(n, hkv, d, 90, case, "v")
        out = torch.empty_like(q)
        if full and n <= 4:   # full_attn takes q_len <= 4 as a verify of one sequence
            ws = torch.empty(max(S.swa_attn_workspace_bytes(P.h, [a], layer, n, hq), 256), dtype=torch.uint8,
                             device="cuda")
            S.full_attn(P.h, [a], layer, q, k, v, n, hq, out, ws)
        elif full:
            S.full_attn(P.h, [a], layer, q, k, v, n, hq, out)
        else:
            S.swa_attn_prefill(P.h, a, layer, q, k, v, hq, out)
        ref = A.attention(to64(q), np.concatenate([hk[a], to64(k)]), np.concatenate([hv[a], to64(v)]), L0, win)
        assert_close(out, ref, act, f"case {case} prefill")
        S.kvpool_append(P.h, a, layer, k, v)
        hk[a] = np.concatenate([hk[a], seen(k, kv)])
        hv[a] = np.concatenate([hv[a], seen(v, kv)])

        # batched decode / verify for both sequences
        ql = c["q_len"]
        seqs = [a, b]
        qd = dr(2 * ql, hq, d, 91, case, "q").reshape(2, ql, hq, d)
        kd = dr(2 * ql, hkv, d, 91, case, "k").reshape(2, ql, hkv, d)
        vd = dr(2 * ql, hkv, d, 91, case, "v").reshape(2, ql, hkv, d)
        ws = torch.empty(max(S.swa_attn_workspace_bytes(P.h, seqs, layer, ql, hq), 256), dtype=torch.uint8,
                         device="cuda")
        od = torch.empty_like(qd)
        fn = S.full_attn if full else S.swa_attn_decode
        fn(P.h, seqs, layer, qd, kd, vd, ql, hq, od, ws)
        for i, s in enumerate(seqs):
            Ls = hk[s].shape[0]
            ref = A.attention(to64(qd[i]), np.concatenate([hk[s], to64(kd[i])]),
                              np.concatenate([hv[s], to64(vd[i])]), Ls, win)
            assert_close(od[i], ref, act, f"case {case} decode seq {i} at {Ls}")


def make_long_case(i):
    g = np.random.default_rng(9100 + i)
    hkv = int(g.choice([1, 2, 4]))
    return dict(
        w=int(g.choice([64, 100, 128, 500, 1000, 4096])), d=int(g.choice([64, 128])), hkv=hkv,
        grp=int(g.choice([1, 4, 8])), full=bool(g.integers(0, 2)),
        kv=[FP8, BF, BF][int(g.integers(0, 3))], prefix=int(g.integers(0, 5000)),
        n=int(g.integers(1, 600)), q_len=int(g.integers(1, 5)), n_seqs=int(g.integers(3, 7)))


@pytest.mark.parametrize("case", range(24))
def test_random_long_shapes_prefill_then_batched_decode(S, case):
    """Larger seeded shapes: prefixes up to 5000 tokens (many pages / band tiles, decode splits),
    windows up to 4096, chunks up to 600, and a batched decode / verify over 3-6 sequences of random
    lengths; sampled query rows (first, last, random) are compared with the oracle."""
    c = make_long_case(case)
    print(f"[sweep-long] case {case}: {c}", flush=True)
    w, d, hkv, full, kv = c["w"], c["d"], c["hkv"], c["full"], c["kv"]
    hq = c["grp"] * hkv
    layer = 1 if full else 0
    win = None if full else w
    g = np.random.default_rng(9200 + case)
    lens = [c["prefix"]] + [int(x) for x in g.integers(0, 3000, size=c["n_seqs"] - 1)]
    pages = sum(L + c["n"] + 8 for L in lens) // 16 + 16
    with GpuPool(S, n_layers=2, window=w, hkv=hkv, d=d, dtype=kv, pages=pages, max_seqs=c["n_seqs"],
                 max_seq_len=8192, layer_is_full=[0, 1]) as P:
        seqs = [S.kvpool_seq_open(P.h) for _ in lens]
        hk, hv = {}, {}
        for i, (s, L) in enumerate(zip(seqs, lens)):
            hk[s], hv[s] = np.zeros((0, hkv, d)), np.zeros((0, hkv, d))
            if L:
                k, v = draw(L, hkv, d, 92, case, i, "k"), draw(L, hkv, d, 92, case, i, "v")
                S.kvpool_append(P.h, s, layer, k, v)
                hk[s], hv[s] = seen(k, kv), seen(v, kv)
        # prefill of the chunk on top of the first sequence's prefix
        a, n, L0 = seqs[0], c["n"], lens[0]
        q, k, v = draw(n, hq, d, 93, case, "q"), draw(n, hkv, d, 93, case, "k"), draw(n, hkv, d, 93, case, "v")
        out = torch.empty_like(q)
        if full and n <= 4:
            ws = torch.empty(max(S.swa_attn_workspace_bytes(P.h, [a], layer, n, hq), 256), dtype=torch.uint8,
                             device="cuda")
            S.full_attn(P.h, [a], layer, q, k, v, n, hq, out, ws)
        elif full:
            S.full_attn(P.h, [a], layer, q, k, v, n, hq, out)
        else:
            S.swa_attn_prefill(P.h, a, layer, q, k, v, hq, out)
        rows = sorted({0, n - 1, *[int(x) for x in g.integers(0, n, size=6)]})
        ref = A.attention(to64(q), np.concatenate([hk[a], to64(k)]), np.concatenate([hv[a], to64(v)]), L0, win,
                          rows=rows)[rows]
        assert_close(out[rows], ref, BF, f"long case {case} prefill")
        S.kvpool_append(P.h, a, layer, k, v)
        hk[a] = np.concatenate([hk[a], seen(k, kv)])
        hv[a] = np.concatenate([hv[a], seen(v, kv)])
        # batched decode / verify over every sequence
        ql, ns = c["q_len"], len(seqs)
        qd = draw(ns * ql, hq, d, 94, case, "q").reshape(ns, ql, hq, d)
        kd = draw(ns * ql, hkv, d, 94, case, "k").reshape(ns, ql, hkv, d)
        vd = draw(ns * ql, hkv, d, 94, case, "v").reshape(ns, ql, hkv, d)
        ws = torch.empty(max(S.swa_attn_workspace_bytes(P.h, seqs, layer, ql, hq), 256), dtype=torch.uint8,
                         device="cuda")
        od = torch.empty_like(qd)
        (S.full_attn if full else S.swa_attn_decode)(P.h, seqs, layer, qd, kd, vd, ql, hq, od, ws)
        for i, s in enumerate(seqs):
            Ls = hk[s].shape[0]
            ref = A.attention(to64(qd[i]), np.concatenate([hk[s], to64(kd[i])]),
                              np.concatenate([hv[s], to64(vd[i])]), Ls, win)
            assert_close(od[i], ref, BF, f"long case {case} decode seq {i} at {Ls}")
