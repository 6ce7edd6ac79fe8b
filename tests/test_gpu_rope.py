"""GPU parity of RoPE (kvpool_rope) against the fp64 oracle, through the C ABI.

RoPE is RoFormer's rotation (oracle.rope); positions come from the pool's committed lengths.
Bars: fp32 max|d|/max|ref| <= 1e-5; bf16 each element within 2^-8 of the exact value relative to
it (one rounding to bf16 plus a few fp32 ulps), and equal to the exact value rounded to bf16
except for a tiny fraction of near-ties; attention through a RoPE pool within 2e-2 max-abs."""
import numpy as np
import pytest
import torch

import synth
from oracle import attention as A
from oracle import fp8 as F8
from oracle import rope as R
from tests.helpers import GpuPool, assert_close, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def S():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import long_context_swa_amd.swa as S
    return S


def check_rotated(got, raw, pos, base, style, dtype, what):
    """got: device result [tokens, H, d]; raw: host copy of the input; pos: position per token."""
    ref = R.rope(to64(raw), pos, base, style)
    g = to64(got)
    if dtype == torch.float32:
        err = np.max(np.abs(g - ref)) / np.max(np.abs(ref))
        assert err <= 1e-5, f"{what}: max|d|/max|ref| = {err:.2e}"
        return
    amax = np.max(np.abs(to64(raw)))
    bound = 2.0 ** -8 * np.abs(ref) + 1e-6 * amax
    assert np.all(np.abs(g - ref) <= bound), f"{what}: max excess {np.max(np.abs(g - ref) - bound):.2e}"
    rounded = to64(torch.from_numpy(ref).to(torch.bfloat16))
    frac = np.mean(g != rounded)
    assert frac <= 1e-3, f"{what}: {frac:.2e} of elements differ from the correctly rounded value"


@pytest.mark.parametrize("dtype,style,d", [(torch.bfloat16, "pairs", 128), (torch.bfloat16, "halves", 64),
                                           (torch.float32, "pairs", 64), (torch.float32, "halves", 128)])
def test_rope_matches_oracle_up_to_1_5m_positions(S, dtype, style, d):
    """Five sequences at committed lengths 0 .. 1.5M (crossing the angle table's 2048-position
    rows), three new tokens each, in one batched call; then a single-sequence call on k alone."""
    base, hq, hkv, n, w = 10000.0, 8, 2, 3, 16
    lens = [0, 5, 2045, 1048573, 1500000]
    print(f"[rope] dtype={dtype} style={style} d={d}", flush=True)
    with GpuPool(S, n_layers=1, window=w, hkv=hkv, d=d, dtype=dtype, max_seqs=6, max_seq_len=1 << 21,
                 layer_is_full=[0], rope_base=base, rope_style=style) as P:
        zeros = torch.zeros((max(lens), hkv, d), dtype=dtype, device="cuda")
        seqs = []
        for L in lens:
            s = S.kvpool_seq_open(P.h)
            if L:
                S.kvpool_append(P.h, s, 0, zeros[:L], zeros[:L])
            seqs.append(s)
        del zeros
        q = synth.normal((len(lens), n, hq, d), 70, "q", d, style, dtype=dtype).cuda()
        k = synth.normal((len(lens), n, hkv, d), 70, "k", d, style, dtype=dtype).cuda()
        q0, k0 = q.cpu(), k.cpu()
        S.kvpool_rope(P.h, seqs, 0, q, hq, k, n)
        pos = np.concatenate([np.arange(L, L + n) for L in lens])
        check_rotated(q.reshape(-1, hq, d), q0.reshape(-1, hq, d), pos, base, style, dtype, "q")
        check_rotated(k.reshape(-1, hkv, d), k0.reshape(-1, hkv, d), pos, base, style, dtype, "k")
        # one sequence (first position as a kernel argument), keys only
        k1 = k0[3].clone().cuda()
        S.kvpool_rope(P.h, [seqs[3]], 0, None, 0, k1, n)
        check_rotated(k1, k0[3], np.arange(lens[3], lens[3] + n), base, style, dtype, "k only")


def rope_bf16(x, pos, base, style):
    """Oracle RoPE rounded once to bf16: what a bf16 RoPE pool stores and attends with."""
    return torch.from_numpy(R.rope(to64(x), pos, base, style)).to(torch.bfloat16)


@pytest.mark.parametrize("kv", [torch.bfloat16, torch.float8_e4m3fn])
def test_rope_pool_prefill_decode_verify_match_oracle(S, kv):
    """Hybrid pair of layers (SWA w=32, full) with RoPE: chunked prefill, batched decode steps and a
    q_len=3 verify, each as rope -> attention -> append, against fp64 attention over the oracle's
    rotated queries and keys.  FP8 pools store the rotated bf16 keys as E4M3 codes: committed rows
    are compared on their dequantised values, the call's own tokens as passed."""
    base, style, w, hq, hkv, d = 10000.0, "pairs", 32, 8, 2, 128
    full = [0, 1]
    dt = torch.bfloat16
    fp8 = kv == torch.float8_e4m3fn
    with GpuPool(S, n_layers=2, window=w, hkv=hkv, d=d, dtype=kv, pages=64, max_seqs=4, max_seq_len=1024,
                 layer_is_full=full, rope_base=base, rope_style=style) as P:
        a, b = S.kvpool_seq_open(P.h), S.kvpool_seq_open(P.h)
        hist = {(s, l): [torch.empty((0, hkv, d), dtype=dt), torch.empty((0, hkv, d), dtype=dt)]
                for s in (a, b) for l in (0, 1)}

        def draw(kind, *key, h, rows):
            return synth.normal((rows, h, d), 71, kind, *key, dtype=dt).cuda()

        def step(seqs, q_len, tag):
            for layer in (0, 1):
                print(f"[rope pipeline] {tag} layer={layer}", flush=True)
                q = draw("q", tag, layer, h=hq, rows=len(seqs) * q_len).reshape(len(seqs), q_len, hq, d)
                k = draw("k", tag, layer, h=hkv, rows=len(seqs) * q_len).reshape(len(seqs), q_len, hkv, d)
                v = draw("v", tag, layer, h=hkv, rows=len(seqs) * q_len).reshape(len(seqs), q_len, hkv, d)
                q0, k0 = q.cpu(), k.cpu()
                lens = [S.kvpool_seq_len(P.h, s, layer) for s in seqs]
                S.kvpool_rope(P.h, seqs, layer, q, hq, k, q_len)
                out = torch.empty_like(q)
                if len(seqs) == 1 and q_len > 4:
                    if full[layer]:
                        S.full_attn(P.h, seqs, layer, q[0], k[0], v[0], q_len, hq, out[0])
                    else:
                        S.swa_attn_prefill(P.h, seqs[0], layer, q[0], k[0], v[0], hq, out[0])
                else:
                    ws = torch.empty(max(S.swa_attn_workspace_bytes(P.h, seqs, layer, q_len, hq), 256),
                                     dtype=torch.uint8, device="cuda")
                    fn = S.full_attn if full[layer] else S.swa_attn_decode
                    fn(P.h, seqs, layer, q, k, v, q_len, hq, out, ws)
                for i, s in enumerate(seqs):
                    S.kvpool_append(P.h, s, layer, k[i], v[i], q_len)
                for i, s in enumerate(seqs):
                    pos = np.arange(lens[i], lens[i] + q_len)
                    hk = hist[(s, layer)]
                    hk[0] = torch.cat([hk[0], rope_bf16(k0[i], pos, base, style)])
                    hk[1] = torch.cat([hk[1], v[i].cpu()])
                    qr = rope_bf16(q0[i], pos, base, style)
                    kk, vv = to64(hk[0]), to64(hk[1])
                    if fp8:   # rows below lens[i] were committed before this call
                        kk[:lens[i]] = F8.roundtrip(kk[:lens[i]], 1.0)
                        vv[:lens[i]] = F8.roundtrip(vv[:lens[i]], 1.0)
                    ref = A.attention(to64(qr), kk, vv, lens[i], None if full[layer] else w)
                    assert_close(out[i], ref, dt, f"{tag} layer {layer} seq {s}")

        step([a], 60, "a0")
        step([a], 40, "a1")
        step([b], 37, "b0")
        for t in range(3):
            step([a, b], 1, f"dec{t}")
        step([b, a], 3, "verify")


def test_rope_makes_ring_slot_order_harmless(S):
    """[SWA-theory] §Rolling Buffer KV Cache: the same 80-token stream attended at positions 0..79
    and at 1003..1082 (so every key sits in a different ring slot) gives the same SWA outputs for
    queries whose window lies inside the stream, because RoPE scores depend on relative positions."""
    base, w, hq, hkv, d, n, off = 10000.0, 32, 4, 1, 64, 80, 1003
    dt = torch.bfloat16
    with GpuPool(S, n_layers=1, window=w, hkv=hkv, d=d, dtype=dt, max_seqs=2, max_seq_len=4096,
                 layer_is_full=[0], rope_base=base) as P:
        x, y = S.kvpool_seq_open(P.h), S.kvpool_seq_open(P.h)
        pad = synth.normal((off, hkv, d), 72, "pad", dtype=dt).cuda()
        S.kvpool_append(P.h, y, 0, pad, pad)
        q = synth.normal((n, hq, d), 72, "q", dtype=dt)
        k = synth.normal((n, hkv, d), 72, "k", dtype=dt)
        v = synth.normal((n, hkv, d), 72, "v", dtype=dt).cuda()
        outs = []
        for s in (x, y):
            qq, kk = q.clone().cuda(), k.clone().cuda()
            S.kvpool_rope(P.h, [s], 0, qq, hq, kk, n)
            o = torch.empty_like(qq)
            S.swa_attn_prefill(P.h, s, 0, qq, kk, v, hq, o)
            S.kvpool_append(P.h, s, 0, kk, v)
            outs.append(o)
        tx, ty = S.kvpool_slot_tags(P.h, x, 0, w), S.kvpool_slot_tags(P.h, y, 0, w)
        assert all(ty[sl] - off != tx[sl] for sl in range(w))  # each slot holds another stream token
        ref = A.attention(to64(rope_bf16(q, np.arange(n), base, "pairs")),
                          to64(rope_bf16(k, np.arange(n), base, "pairs")), to64(v), 0, w)
        assert_close(outs[0], ref, dt, "stream at 0")
        assert_close(outs[1][w - 1:], ref[w - 1:], dt, "stream at 1003")
        assert_close(outs[1][w - 1:], outs[0][w - 1:], dt, "shifted vs unshifted")


# ------------------------------------------------------------------------------------------ fused RoPE

def _pipeline_pair(S, P_plain, P_fused, seqs, layer, full, q, k, v, hq, q_len):
    """One attention + commit on both pools: kvpool_rope first on the plain pool, raw q/k on the fused
    one.  Returns (plain out, fused out)."""
    q1, k1 = q.clone(), k.clone()
    S.kvpool_rope(P_plain.h, seqs, layer, q1, hq, k1, q_len)
    outs = []
    for P, qq, kk in ((P_plain, q1, k1), (P_fused, q, k)):
        out = torch.empty_like(qq)
        if len(seqs) == 1 and q_len > 4:
            if full:
                S.full_attn(P.h, seqs, layer, qq[0], kk[0], v[0], q_len, hq, out[0])
            else:
                S.swa_attn_prefill(P.h, seqs[0], layer, qq[0], kk[0], v[0], hq, out[0])
        else:
            ws = torch.empty(max(S.swa_attn_workspace_bytes(P.h, seqs, layer, q_len, hq), 256),
                             dtype=torch.uint8, device="cuda")
            fn = S.full_attn if full else S.swa_attn_decode
            fn(P.h, seqs, layer, qq, kk, v, q_len, hq, out, ws)
        if len(seqs) > 1 and q_len == 1:
            S.kvpool_append_batch(P.h, seqs, layer, kk.reshape(len(seqs), hkv_of(kk), -1),
                                  v.reshape(len(seqs), hkv_of(v), -1), 1)
        else:
            for i, s in enumerate(seqs):
                S.kvpool_append(P.h, s, layer, kk[i], v[i], q_len)
        outs.append(out)
    return outs


def hkv_of(t):
    return t.shape[-2]


@pytest.mark.parametrize("kv,style,d,g", [(torch.bfloat16, "pairs", 128, 4), (torch.bfloat16, "halves", 128, 8),
                                          (torch.bfloat16, "halves", 64, 4), (torch.float8_e4m3fn, "pairs", 128, 16)])
def test_fused_rope_equals_rope_then_attention(S, kv, style, d, g):
    """A pool with RoPE fused into attention and commit (raw q/k in, rotated inside) against the same
    pool driven as kvpool_rope -> attention -> commit: identical outputs and identical stored bytes,
    for chunked prefill (SWA and full layer), batched decode steps and verify with q_len 3 and 4
    (G x q_len up to 64 rows); outputs also against fp64 attention over the oracle's rotation.  The
    caller's q, k and v are left as passed."""
    base, w, hkv = 10000.0, 32, 2
    hq = g * hkv
    full = [0, 1]
    dt = torch.bfloat16
    fp8 = kv == torch.float8_e4m3fn
    kw = dict(n_layers=2, window=w, hkv=hkv, d=d, dtype=kv, pages=128, max_seqs=4, max_seq_len=2048,
              layer_is_full=full, rope_base=base, rope_style=style)
    with GpuPool(S, **kw) as P0, GpuPool(S, **kw, rope_fused=True, max_chunk=256) as P1:
        a0, b0 = S.kvpool_seq_open(P0.h), S.kvpool_seq_open(P0.h)
        a1, b1 = S.kvpool_seq_open(P1.h), S.kvpool_seq_open(P1.h)
        assert (a0, b0) == (a1, b1)
        a, b = a0, b0
        hist = {(s, l): [torch.empty((0, hkv, d), dtype=dt), torch.empty((0, hkv, d), dtype=dt)]
                for s in (a, b) for l in (0, 1)}

        def step(seqs, q_len, tag):
            for layer in (0, 1):
                print(f"[fused rope] {kv} {style} d={d} g={g} {tag} layer={layer}", flush=True)
                n = len(seqs)
                q = synth.normal((n * q_len, hq, d), 72, "q", tag, layer, dtype=dt).cuda().reshape(n, q_len, hq, d)
                k = synth.normal((n * q_len, hkv, d), 72, "k", tag, layer, dtype=dt).cuda().reshape(n, q_len, hkv, d)
                v = synth.normal((n * q_len, hkv, d), 72, "v", tag, layer, dtype=dt).cuda().reshape(n, q_len, hkv, d)
                q0, k0, v0 = q.cpu(), k.cpu(), v.cpu()
                lens = [S.kvpool_seq_len(P0.h, s, layer) for s in seqs]
                assert lens == [S.kvpool_seq_len(P1.h, s, layer) for s in seqs]
                out0, out1 = _pipeline_pair(S, P0, P1, seqs, layer, full[layer], q, k, v, hq, q_len)
                torch.cuda.synchronize()
                assert torch.equal(q.cpu(), q0) and torch.equal(k.cpu(), k0) and torch.equal(v.cpu(), v0)
                assert torch.equal(out1.view(torch.int16), out0.view(torch.int16)), f"{tag} layer {layer}"
                for i, s in enumerate(seqs):
                    pos = np.arange(lens[i], lens[i] + q_len)
                    hk = hist[(s, layer)]
                    hk[0] = torch.cat([hk[0], rope_bf16(k0[i], pos, base, style)])
                    hk[1] = torch.cat([hk[1], v0[i]])
                    qr = rope_bf16(q0[i], pos, base, style)
                    kk, vv = to64(hk[0]), to64(hk[1])
                    if fp8:
                        kk[:lens[i]] = F8.roundtrip(kk[:lens[i]], 1.0)
                        vv[:lens[i]] = F8.roundtrip(vv[:lens[i]], 1.0)
                    ref = A.attention(to64(qr), kk, vv, lens[i], None if full[layer] else w)
                    assert_close(out1[i], ref, dt, f"{tag} layer {layer} seq {s}")

        step([a], 60, "a0")
        step([a], 40, "a1")
        step([b], 200, "b0")
        for t in range(3):
            step([a, b], 1, f"dec{t}")
        step([b, a], 4, "verify4")
        step([a, b], 3, "verify3")
        # stored keys and values: byte-identical in both pools
        arena0, arena1 = P0.arena.cpu().numpy(), P1.arena.cpu().numpy()
        es = 1 if fp8 else 2
        for s in (a, b):
            for layer in (0, 1):
                L = S.kvpool_seq_len(P0.h, s, layer)
                lo = 0 if full[layer] else max(0, L - w)
                for pos in range(lo, L):
                    for head in range(hkv):
                        k0_, v0_, _ = S.kvpool_locate(P0.h, s, layer, pos, head)
                        k1_, v1_, _ = S.kvpool_locate(P1.h, s, layer, pos, head)
                        assert np.array_equal(arena0[k0_:k0_ + d * es], arena1[k1_:k1_ + d * es]), (s, layer, pos)
                        assert np.array_equal(arena0[v0_:v0_ + d * es], arena1[v1_:v1_ + d * es]), (s, layer, pos)


def test_fused_rope_many_sequences_and_refusals(S):
    """Fused RoPE over 300 sequences (an SWA decode step with one work item per wave, and a full
    layer whose 40 long rows are split across work items) against the unfused pipeline: long
    histories committed raw (rotated at store) versus rotated by kvpool_rope first, then one decode
    step each.  Stored bytes and outputs are identical.  A prefill chunk above max_chunk is refused
    without effect, and so are pools that ask for fusion without RoPE, on fp32 or without max_chunk."""
    base, w, hkv, d, g = 10000.0, 16, 2, 128, 4
    hq = g * hkv
    n, n_long = 300, 40
    dt = torch.bfloat16
    kw = dict(n_layers=2, window=w, hkv=hkv, d=d, dtype=dt, pages=n_long * 3000 // 16 + n + 64, max_seqs=n,
              max_seq_len=4096, layer_is_full=[0, 1], rope_base=base, rope_style="halves")
    with GpuPool(S, **kw) as P0, GpuPool(S, **kw, rope_fused=True, max_chunk=64) as P1:
        seqs = [S.kvpool_seq_open(P0.h) for _ in range(n)]
        assert seqs == [S.kvpool_seq_open(P1.h) for _ in range(n)]
        for layer in (0, 1):
            print(f"[fused rope many] history layer={layer}", flush=True)
            for i, s in enumerate(seqs[:n_long]):
                L = 1500 + 37 * i
                kz = synth.normal((L, hkv, d), 73, "h", layer, i, dtype=dt).cuda()
                kr = kz.clone()
                S.kvpool_rope(P0.h, [s], layer, None, 0, kr, L)
                S.kvpool_append(P0.h, s, layer, kr, kz)
                S.kvpool_append(P1.h, s, layer, kz, kz)
            kz = synth.normal((n - n_long, hkv, d), 73, "short", layer, dtype=dt).cuda()
            kr = kz.clone().reshape(n - n_long, 1, hkv, d)
            S.kvpool_rope(P0.h, seqs[n_long:], layer, None, 0, kr, 1)
            S.kvpool_append_batch(P0.h, seqs[n_long:], layer, kr, kz, 1)
            S.kvpool_append_batch(P1.h, seqs[n_long:], layer, kz, kz, 1)
        torch.cuda.synchronize()
        arena0, arena1 = P0.arena.cpu().numpy(), P1.arena.cpu().numpy()
        for layer in (0, 1):
            for s in seqs[:3] + seqs[n_long - 2:n_long + 2] + seqs[-2:]:
                L = S.kvpool_seq_len(P0.h, s, layer)
                for pos in sorted({max(0, L - w), max(0, L // 2 if layer else L - 2), L - 1}):
                    for head in range(hkv):
                        o0 = S.kvpool_locate(P0.h, s, layer, pos, head)[0]
                        o1 = S.kvpool_locate(P1.h, s, layer, pos, head)[0]
                        assert np.array_equal(arena0[o0:o0 + 2 * d], arena1[o1:o1 + 2 * d]), (s, layer, pos)
        for layer in (0, 1):
            print(f"[fused rope many] decode layer={layer}", flush=True)
            q = synth.normal((n, hq, d), 73, "q", layer, dtype=dt).cuda().reshape(n, 1, hq, d)
            k = synth.normal((n, hkv, d), 73, "k", layer, dtype=dt).cuda().reshape(n, 1, hkv, d)
            v = synth.normal((n, hkv, d), 73, "v", layer, dtype=dt).cuda().reshape(n, 1, hkv, d)
            q1, k1 = q.clone(), k.clone()
            S.kvpool_rope(P0.h, seqs, layer, q1, hq, k1, 1)
            outs = []
            for P, qq, kk in ((P0, q1, k1), (P1, q, k)):
                out = torch.empty_like(q)
                ws = torch.empty(max(S.swa_attn_workspace_bytes(P.h, seqs, layer, 1, hq), 256), dtype=torch.uint8,
                                 device="cuda")
                (S.full_attn if layer else S.swa_attn_decode)(P.h, seqs, layer, qq, kk, v, 1, hq, out, ws)
                outs.append(out)
            torch.cuda.synchronize()
            assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16)), f"layer {layer}"
        # a chunk above max_chunk: refused, nothing committed, out untouched
        qc = torch.zeros((65, hq, d), dtype=dt, device="cuda")
        kc = torch.zeros((65, hkv, d), dtype=dt, device="cuda")
        oc = torch.full_like(qc, 3.0)
        s = seqs[-1]
        L = S.kvpool_seq_len(P1.h, s, 0)
        with pytest.raises(S.SwaError) as e:
            S.swa_attn_prefill(P1.h, s, 0, qc, kc, kc, hq, oc)
        assert e.value.code == S.SWA_EINVAL and S.kvpool_seq_len(P1.h, s, 0) == L
        torch.cuda.synchronize()
        assert bool((oc == 3.0).all())
