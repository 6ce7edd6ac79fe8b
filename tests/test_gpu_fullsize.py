"""Parity at the workloads' full sizes, in the launch configuration bench.py times, on sampled
outputs the fp64 oracle computes one row at a time.

Samples (seeded, documented here):
  * 16K-chunk SWA prefill (n=16384, w=4096, 32/8 heads, d=128): 40 query positions -- band and
    tile edges (0, 1, 63, 64, 4094..4097, 8191, 16383) plus 28 random -- all 32 heads; and, in a
    test of its own, every one of its 16,384 x 32 output rows (host cores, about a minute).
  * 70-layer batched decode (256 sequences, contexts U{1..65536}, 64 continuing and 64 branching
    forks): 8 sequences (2 donors, 3 continuing forks, 3 branching forks), SWA layers 0-3 and full
    layers 6 and 13, all heads.
  * 128K hybrid prefill in 16K chunks: layers 0, 1, 2, 3 (SWA) and 6, 13 (full) run through all 8
    chunks (layers are independent, so their outputs equal those of the 70-layer run); in chunks 0,
    3 and 7 the first and last 256 rows and every 61st row (772 rows a chunk), all heads.
  * 1M-token prefix: layers 0, 1 (SWA) and 6 (full) hold the 1,048,576-token prefix; the 16K chunk
    prefill on 64 of its 512 blocks of 32 positions (both edge rows of each) and the q_len=4 verify
    (all 4 rows), all heads.
  * The oracle runs these samples on forked host workers (16 at most, one BLAS thread each): 17 s
    for the 128K prefill's 13,896 rows and 23 s for the 1M prefix's full layer (both tests together
    49 s on an MI355X host).
  * The 256-sequence decode and the 1M-token prefix again over FP8 (E4M3) pools (tests named
    *_fp8_sampled): committed keys read as the oracle's E4M3 round trip of the same bf16 rows.
The oracle receives the exact bf16 inputs the GPU received (drawn on the device by synth, copied
to the host); it never reads the pool.  Bar: max |gpu - oracle| <= 2e-2."""
import numpy as np
import pytest
import torch

import synth
from oracle import attention as A
from tests.helpers import BF16_ABS

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def S():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import long_context_swa_amd.swa as S
    return S


def f64(t):
    return t.detach().float().cpu().double().numpy()


def check_rows(got, q, k, v, rows, pos0, w, what):
    """got: GPU output rows [len(rows), Hq, d]; q [*, Hq, d] indexed by `rows`; k, v: logical
    history by position (index 0 = position kpos0 passed implicitly via pos0 offsets)."""
    ref = A.attention(q, k, v, pos0, w, rows=rows)[rows]
    err = float(np.max(np.abs(got - ref)))
    assert err <= BF16_ABS, f"{what}: max |gpu - oracle| = {err:.3e}"
    return err


def test_swa_prefill_16k_chunk_sampled(S):
    n, w, hq, hkv, d, seed = 16384, 4096, 32, 8, 128, 2
    q = synth.normal((n, hq, d), seed, "q", dtype=torch.bfloat16, device="cuda")
    k = synth.normal((n, hkv, d), seed, "k", dtype=torch.bfloat16, device="cuda")
    v = synth.normal((n, hkv, d), seed, "v", dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    desc = S.make_desc(1, w, hkv, d, torch.bfloat16, 0, 2, n, layer_is_full=[0])
    nb = S.kvpool_arena_bytes(desc)
    arena = torch.empty(nb, dtype=torch.uint8, device="cuda")
    pool = S.kvpool_create(desc, arena, nb)
    try:
        s = S.kvpool_seq_open(pool)
        S.swa_attn_prefill(pool, s, 0, q, k, v, hq, out)
        torch.cuda.synchronize()
        assert torch.isfinite(out.float()).all()
        rng = np.random.default_rng(7)
        rows = sorted(set([0, 1, 63, 64, 4094, 4095, 4096, 4097, 8191, 16383] +
                          list(rng.integers(0, n, 30))))[:40]
        check_rows(f64(out)[rows], f64(q), f64(k), f64(v), rows, 0, w, "16K SWA prefill")
    finally:
        torch.cuda.synchronize()
        S.kvpool_destroy(pool)


_FULL = {}


def _full_rows_worker(rows):
    """One forked worker: the oracle for these query rows of the 16K chunk, all heads; returns
    the largest |gpu - oracle|."""
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)
    q, k, v, got, w = _FULL["q"], _FULL["k"], _FULL["v"], _FULL["got"], _FULL["w"]
    ref = A.attention(q, k, v, 0, w, rows=rows)[rows]
    return float(np.max(np.abs(got[rows] - ref)))


def test_swa_prefill_16k_chunk_in_full(S):
    """Every output of the 16K-chunk SWA prefill (16,384 positions x 32 heads, w = 4096) against the
    oracle, row by row, on the host's cores (forked workers, one BLAS thread each; about a minute)."""
    import multiprocessing as mp
    import os
    import time
    n, w, hq, hkv, d, seed = 16384, 4096, 32, 8, 128, 2
    q = synth.normal((n, hq, d), seed, "q", dtype=torch.bfloat16, device="cuda")
    k = synth.normal((n, hkv, d), seed, "k", dtype=torch.bfloat16, device="cuda")
    v = synth.normal((n, hkv, d), seed, "v", dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    desc = S.make_desc(1, w, hkv, d, torch.bfloat16, 0, 2, n, layer_is_full=[0])
    nb = S.kvpool_arena_bytes(desc)
    arena = torch.empty(nb, dtype=torch.uint8, device="cuda")
    pool = S.kvpool_create(desc, arena, nb)
    try:
        s = S.kvpool_seq_open(pool)
        S.swa_attn_prefill(pool, s, 0, q, k, v, hq, out)
        torch.cuda.synchronize()
    finally:
        S.kvpool_destroy(pool)
    _FULL.update(q=f64(q), k=f64(k), v=f64(v), got=f64(out), w=w)
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    parts = [list(range(a, min(a + 256, n))) for a in range(0, n, 256)]
    t0 = time.time()
    worst, done = 0.0, 0
    try:
        with mp.get_context("fork").Pool(cores) as workers:
            for err in workers.imap_unordered(_full_rows_worker, parts):
                worst, done = max(worst, err), done + 1
                if done % 16 == 0:
                    print(f"[full C2] {done}/{len(parts)} row blocks, max |d| so far {worst:.2e}, "
                          f"{time.time() - t0:.0f} s", flush=True)
    finally:
        _FULL.clear()
    assert worst <= BF16_ABS, f"16K SWA prefill, all rows: max |gpu - oracle| = {worst:.3e}"


def test_hybrid_decode_256_sequences_sampled(S):
    import long_context_swa_amd.workloads as W
    st = W.build_decode(steps=2)
    try:
        sids = [x.sid for x in st.seqs]
        n = len(sids)
        kinds = {sid: k for sid, (_, k, _, _) in st.forks.items()}
        donors = [i for i, x in enumerate(st.seqs) if x.sid not in kinds][:2]
        cont = [i for i, x in enumerate(st.seqs) if kinds.get(x.sid) == "continue"][:3]
        branch = [i for i, x in enumerate(st.seqs) if kinds.get(x.sid) == "branch"][:3]
        sample = donors + cont + branch
        out = torch.empty((n, 1, W.HQ, W.D), dtype=W.DT, device="cuda")
        for l in (0, 1, 2, 3, 6, 13):
            full = W.layer_full(l)
            fn = S.full_attn if full else S.swa_attn_decode
            fn(st.pool.h, sids, l, st.q[l], st.kn[l], st.vn[l], 1, W.HQ, out, st.ws)
            torch.cuda.synchronize()
            got = f64(out)
            for i in sample:
                seq = st.seqs[i]
                P = seq.prior
                lo = 0 if full else max(0, P - (W.WINDOW - 1))
                k, v = st.streams.rows(l, seq.segments, lo, P)
                k = np.concatenate([f64(k), f64(st.kn[l][i])])
                v = np.concatenate([f64(v), f64(st.vn[l][i])])
                qq = f64(st.q[l][i])                      # [1, HQ, D] at position P
                ref = A.attention(qq, k, v, P - lo, None if full else W.WINDOW)
                err = float(np.max(np.abs(got[i] - ref)))
                assert err <= BF16_ABS, f"layer {l} seq {i} ({kinds.get(seq.sid, 'donor')}, L={P}): {err:.3e}"
    finally:
        st.pool.close()


_JOBS = {}


def _rows_worker(job):
    """One forked worker: oracle rows of one (layer, chunk) sample against the GPU rows; returns
    (layer, chunk, largest |gpu - oracle|).  Every query row goes through the oracle on its own, at
    its absolute position, over the layer's whole logical history held in _JOBS."""
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)
    layer, chunk, idx = job
    kh, vh = _JOBS[("kv", layer)]
    q, got, pos, w = _JOBS[(layer, chunk)]
    worst = 0.0
    for r in idx:
        ref = A.attention(q[r:r + 1], kh, vh, int(pos[r]), w)[0]
        worst = max(worst, float(np.max(np.abs(got[r] - ref))))
    return layer, chunk, worst


def _check_parallel(what, batch=24):
    """Runs every sample registered in _JOBS through the oracle on the host's cores (forked
    workers, one BLAS thread each) and asserts the bar per (layer, chunk)."""
    import multiprocessing as mp
    import os
    import time
    jobs = []
    for key, val in _JOBS.items():
        if key[0] == "kv":
            continue
        n = val[0].shape[0]
        jobs += [(key[0], key[1], list(range(a, min(a + batch, n)))) for a in range(0, n, batch)]
    jobs.sort(key=lambda j: -_JOBS[(j[0], j[1])][2][j[2][-1]])  # costliest (longest history) first
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    worst = {}
    t0 = time.time()
    with mp.get_context("fork").Pool(cores) as workers:
        for done, (layer, chunk, err) in enumerate(workers.imap_unordered(_rows_worker, jobs), 1):
            worst[(layer, chunk)] = max(worst.get((layer, chunk), 0.0), err)
            if done % 32 == 0 or done == len(jobs):
                print(f"[{what}] {done}/{len(jobs)} row batches, {time.time() - t0:.0f} s", flush=True)
    for (layer, chunk), err in sorted(worst.items()):
        assert err <= BF16_ABS, f"{what}: chunk {chunk} layer {layer}: max |gpu - oracle| = {err:.3e}"
    return worst


@pytest.mark.timeout(600)
def test_hybrid_prefill_128k_sampled(S):
    """C3 sample: layers 0-3 (SWA, w = 128) and 6, 13 (full) through all eight 16K chunks; in chunks
    0, 3 and 7 the first and last 256 rows and every 61st row, all 32 heads, against the oracle over
    each layer's whole history (17 s of host time on 16 cores)."""
    import long_context_swa_amd.workloads as W
    layers = [0, 1, 2, 3, 6, 13]
    checked = (0, 3, 7)
    rows = sorted(set(range(256)) | set(range(W.CHUNK - 256, W.CHUNK)) | set(range(0, W.CHUNK, 61)))
    st = W.build_hybrid_prefill()
    _JOBS.clear()
    try:
        out = torch.empty((W.CHUNK, W.HQ, W.D), dtype=W.DT, device="cuda")
        for c in range(8):
            a, b = c * W.CHUNK, (c + 1) * W.CHUNK
            for l in layers:
                q, k, v = W.chunk_inputs(st.streams, st.seed, l, c, st.seq, a, b)
                if W.layer_full(l):
                    S.full_attn(st.pool.h, [st.seq.sid], l, q, k, v, q.shape[0], W.HQ, out)
                else:
                    S.swa_attn_prefill(st.pool.h, st.seq.sid, l, q, k, v, W.HQ, out)
                S.kvpool_append(st.pool.h, st.seq.sid, l, k, v)
                if c in checked:
                    torch.cuda.synchronize()
                    w = None if W.layer_full(l) else W.WINDOW
                    _JOBS[(l, c)] = (f64(q[rows]), f64(out[rows]), a + np.array(rows), w)
        # KV accounting after 128K tokens in the sampled layers (the other 64 layers hold none):
        # 4 rings of w live slots and 2 x 8192 pages of 16 rows
        alloc, res = S.kvpool_bytes(st.pool.h)
        tok = 2 * W.HKV * W.D * 2
        assert res == (4 * W.WINDOW + 2 * 131072) * tok
        assert alloc == (60 * W.WINDOW + 2 * 131072) * tok
        for l in layers:
            kh, vh = st.streams.rows(l, st.seq.segments, 0, 8 * W.CHUNK)
            _JOBS[("kv", l)] = (f64(kh), f64(vh))
            del kh, vh
        _check_parallel("C3 128K hybrid prefill")
    finally:
        _JOBS.clear()
        st.pool.close()


@pytest.mark.timeout(600)
def test_long_context_1m_prefix_sampled(S):
    """C5 sample: layers 0, 1 (SWA) and 6 (full) hold the 1,048,576-token prefix.  The 16K chunk is
    checked on 64 of its 512 row blocks of 32 positions (blocks 0 and 511 and 62 spread between,
    seeded), both edge rows of each block, all 32 heads, on every layer; the q_len = 4 verify on all
    4 rows (23 s of host time on 16 cores for the full layer's 128 rows of 1M keys)."""
    import long_context_swa_amd.workloads as W
    layers = [0, 1, 6]
    st = W.build_long(layers=layers)
    rng = np.random.default_rng(11)
    blocks = sorted({0, 511} | set((np.arange(62) * 8 + 4 + rng.integers(0, 4, 62)).tolist()))
    assert len(blocks) == 64
    rows = sorted([32 * b for b in blocks] + [32 * b + 31 for b in blocks])
    _JOBS.clear()
    try:
        P0 = st.seq.prior
        out = torch.empty((W.CHUNK, W.HQ, W.D), dtype=W.DT, device="cuda")
        o4 = torch.empty((1, 4, W.HQ, W.D), dtype=W.DT, device="cuda")
        for l in layers:
            full = W.layer_full(l)
            q, k, v = W.chunk_inputs(st.streams, st.seed, l, 0, st.seq, P0, P0 + W.CHUNK)
            if full:
                S.full_attn(st.pool.h, [st.seq.sid], l, q, k, v, W.CHUNK, W.HQ, out)
            else:
                S.swa_attn_prefill(st.pool.h, st.seq.sid, l, q, k, v, W.HQ, out)
            S.kvpool_append(st.pool.h, st.seq.sid, l, k, v)
            L = P0 + W.CHUNK
            q4 = synth.normal((1, 4, W.HQ, W.D), st.seed, "vq", l, dtype=W.DT, device="cuda")
            k4 = synth.normal((1, 4, W.HKV, W.D), st.seed, "vk", l, dtype=W.DT, device="cuda")
            v4 = synth.normal((1, 4, W.HKV, W.D), st.seed, "vv", l, dtype=W.DT, device="cuda")
            ws = torch.empty(S.swa_attn_workspace_bytes(st.pool.h, [st.seq.sid], l, 4, W.HQ) + 256,
                             dtype=torch.uint8, device="cuda")
            (S.full_attn if full else S.swa_attn_decode)(st.pool.h, [st.seq.sid], l, q4, k4, v4, 4, W.HQ, o4, ws)
            torch.cuda.synchronize()
            # the SWA layers' history starts a window before the chunk (older keys never matter)
            lo = 0 if full else P0 - W.WINDOW
            kh, vh = st.streams.rows(l, st.seq.segments, lo, L)
            kh, vh = f64(kh), f64(vh)
            w = None if full else W.WINDOW
            kv4 = np.concatenate([kh, f64(k4[0])]), np.concatenate([vh, f64(v4[0])])
            ref4 = A.attention(f64(q4[0]), kv4[0], kv4[1], L - lo, w)
            err = float(np.max(np.abs(f64(o4[0]) - ref4)))
            assert err <= BF16_ABS, f"1M prefix verify q_len=4, layer {l}: {err:.3e}"
            del kv4
            _JOBS.clear()
            _JOBS[("kv", l)] = (kh, vh)
            _JOBS[(l, 0)] = (f64(q[rows]), f64(out[rows]), P0 - lo + np.array(rows), w)
            del kh, vh
            _check_parallel(f"C5 1M-prefix chunk, layer {l}")
    finally:
        _JOBS.clear()
        st.pool.close()


# ---------------------------------------------------------------------------------- FP8 KV pools

def f64_fp8_seen(t):
    """What attention sees for committed bf16 rows of an FP8 pool (unit scales): the oracle's
    E4M3 round trip, by pattern lookup."""
    from oracle import fp8 as F8
    bits = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return F8.roundtrip_bf16_bits(bits, 1.0)


def test_hybrid_decode_256_sequences_fp8_sampled(S):
    """The 256-sequence decode step over FP8 pools: same sample as the bf16 test (2 donors, 3
    continuing and 3 branching forks), SWA layers 0 and 3 and full layers 6 and 13, all heads;
    committed keys read dequantised, the new token as passed."""
    import long_context_swa_amd.workloads as W
    st = W.build_decode(steps=2, kv=torch.float8_e4m3fn)
    try:
        sids = np.array([x.sid for x in st.seqs], dtype=np.int32)
        n = len(sids)
        kinds = {sid: k for sid, (_, k, _, _) in st.forks.items()}
        donors = [i for i, x in enumerate(st.seqs) if x.sid not in kinds][:2]
        cont = [i for i, x in enumerate(st.seqs) if kinds.get(x.sid) == "continue"][:3]
        branch = [i for i, x in enumerate(st.seqs) if kinds.get(x.sid) == "branch"][:3]
        out = torch.empty((n, 1, W.HQ, W.D), dtype=W.DT, device="cuda")
        for l in (0, 3, 6, 13):
            full = W.layer_full(l)
            (S.full_attn if full else S.swa_attn_decode)(st.pool.h, sids, l, st.q[l], st.kn[l], st.vn[l], 1,
                                                         W.HQ, out, st.ws)
            torch.cuda.synchronize()
            got = f64(out)
            for i in donors + cont + branch:
                seq = st.seqs[i]
                P = seq.prior
                lo = 0 if full else max(0, P - (W.WINDOW - 1))
                k, v = st.streams.rows(l, seq.segments, lo, P)
                k = np.concatenate([f64_fp8_seen(k), f64(st.kn[l][i])])
                v = np.concatenate([f64_fp8_seen(v), f64(st.vn[l][i])])
                ref = A.attention(f64(st.q[l][i]), k, v, P - lo, None if full else W.WINDOW)
                err = float(np.max(np.abs(got[i] - ref)))
                assert err <= BF16_ABS, f"fp8 layer {l} seq {i} (L={P}): {err:.3e}"
    finally:
        st.pool.close()


def test_long_context_1m_prefix_fp8_sampled(S):
    """1,048,576-token prefix in FP8 pools (layers 0 (SWA) and 6 (full)): the 16K chunk prefill
    (rows 0 and 16383) and the q_len=4 verify (all 4 rows), all heads."""
    import long_context_swa_amd.workloads as W
    layers = [0, 6]
    st = W.build_long(layers=layers, kv=torch.float8_e4m3fn)
    try:
        P0 = st.seq.prior
        out = torch.empty((W.CHUNK, W.HQ, W.D), dtype=W.DT, device="cuda")
        o4 = torch.empty((1, 4, W.HQ, W.D), dtype=W.DT, device="cuda")
        for l in layers:
            full = W.layer_full(l)
            q, k, v = W.chunk_inputs(st.streams, st.seed, l, 0, st.seq, P0, P0 + W.CHUNK)
            if full:
                S.full_attn(st.pool.h, [st.seq.sid], l, q, k, v, W.CHUNK, W.HQ, out)
            else:
                S.swa_attn_prefill(st.pool.h, st.seq.sid, l, q, k, v, W.HQ, out)
            S.kvpool_append(st.pool.h, st.seq.sid, l, k, v)
            L = P0 + W.CHUNK
            q4 = synth.normal((1, 4, W.HQ, W.D), st.seed, "vq", l, dtype=W.DT, device="cuda")
            k4 = synth.normal((1, 4, W.HKV, W.D), st.seed, "vk", l, dtype=W.DT, device="cuda")
            v4 = synth.normal((1, 4, W.HKV, W.D), st.seed, "vv", l, dtype=W.DT, device="cuda")
            ws = torch.empty(S.swa_attn_workspace_bytes(st.pool.h, [st.seq.sid], l, 4, W.HQ) + 256,
                             dtype=torch.uint8, device="cuda")
            (S.full_attn if full else S.swa_attn_decode)(st.pool.h, [st.seq.sid], l, q4, k4, v4, 4, W.HQ, o4, ws)
            torch.cuda.synchronize()
            lo = 0 if full else P0 - W.WINDOW
            kh, vh = st.streams.rows(l, st.seq.segments, lo, L)
            w = None if full else W.WINDOW
            # the chunk prefill sees the prefix dequantised and its own keys as passed
            kp = np.concatenate([f64_fp8_seen(kh[:P0 - lo]), f64(kh[P0 - lo:])])
            vp = np.concatenate([f64_fp8_seen(vh[:P0 - lo]), f64(vh[P0 - lo:])])
            rows = [0, W.CHUNK - 1]
            ref = A.attention(f64(q), kp, vp, P0 - lo, w, rows=rows)[rows]
            err = float(np.max(np.abs(f64(out)[rows] - ref)))
            assert err <= BF16_ABS, f"fp8 1M prefix chunk, layer {l}: {err:.3e}"
            del kp, vp
            # the verify sees the whole committed history (prefix and chunk) dequantised
            kv4 = (np.concatenate([f64_fp8_seen(kh), f64(k4[0])]), np.concatenate([f64_fp8_seen(vh), f64(v4[0])]))
            ref4 = A.attention(f64(q4[0]), kv4[0], kv4[1], L - lo, w)
            err = float(np.max(np.abs(f64(o4[0]) - ref4)))
            assert err <= BF16_ABS, f"fp8 1M prefix verify q_len=4, layer {l}: {err:.3e}"
            del kh, vh, kv4
    finally:
        st.pool.close()
