"""GPU parity of the band form of the SWA prefill (small windows: one workgroup per CU walks a run
of consecutive query blocks as one stream of tiles), through the C ABI.

The band form runs for SWA layers with w <= 256 when a call has at least two blocks per CU.  Its
per-tile arithmetic is the tiled form's, and a row's result does not depend on how the chunk is
cut as long as blocks start at the same positions (tiles a row does not see add exact zeros), so
one call over a long chunk (band form) must equal, bit for bit, the same tokens prefilled in
pieces small enough for the tiled form, each committed before the next.  Sampled rows (first and
last 128, every 97th) are also checked against the fp64 oracle (bar 2e-2).  FP8 pools: against
the oracle with the prefix keys read as their E4M3 round trip."""
import numpy as np
import pytest
import torch

import synth
from oracle import attention as A
from oracle import fp8 as F8
from oracle import rope as R
from tests.helpers import BF16_ABS, GpuPool, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def S():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import long_context_swa_amd.swa as S
    return S


def sample_rows(n):
    return sorted(set(range(min(128, n))) | set(range(max(0, n - 128), n)) | set(range(0, n, 97)))


def draw(n, h, d, *key):
    return synth.normal((n, h, d), 74, *key, dtype=torch.bfloat16).cuda()


@pytest.mark.parametrize("w,hq,hkv,d,n,pre,piece", [
    (128, 32, 4, 128, 16384, 3000, 2048),   # the hybrid stack's SWA layers, ring wrapped
    (128, 32, 4, 128, 16384, 0, 2048),      # first chunk: no prefix
    (1, 16, 16, 64, 8192, 77, 2048),        # w = 1: every row sees only itself
    (100, 32, 16, 128, 4096, 250, 2048),    # window not a tile multiple, G = 2
    (256, 8, 8, 64, 16384, 1000, 4096),     # the largest band window, G = 1
    (128, 32, 4, 128, 10000, 130, 2048),    # ragged: 313 blocks in runs of 5, the last run of 3, a half block
    (64, 32, 4, 128, 4096, 64, 1024),       # exactly two blocks per CU (the smallest band call)
])
def test_band_prefill_equals_tiled_and_oracle(S, w, hq, hkv, d, n, pre, piece):
    print(f"[band] w={w} hq={hq} hkv={hkv} d={d} n={n} pre={pre}", flush=True)
    kw = dict(window=w, hkv=hkv, d=d, dtype=torch.bfloat16, max_seqs=2, max_seq_len=pre + n + 16)
    kp, vp = draw(max(pre, 1), hkv, d, "kp", w), draw(max(pre, 1), hkv, d, "vp", w)
    q, k, v = draw(n, hq, d, "q", w), draw(n, hkv, d, "k", w), draw(n, hkv, d, "v", w)
    with GpuPool(S, **kw) as PA, GpuPool(S, **kw) as PB:
        a, b = S.kvpool_seq_open(PA.h), S.kvpool_seq_open(PB.h)
        if pre:
            S.kvpool_append(PA.h, a, 0, kp, vp)
            S.kvpool_append(PB.h, b, 0, kp, vp)
        out_a = torch.empty_like(q)
        S.swa_attn_prefill(PA.h, a, 0, q, k, v, hq, out_a)       # one call: band form
        out_b = torch.empty_like(q)
        for c0 in range(0, n, piece):                            # pieces: tiled form
            c1 = min(n, c0 + piece)
            S.swa_attn_prefill(PB.h, b, 0, q[c0:c1], k[c0:c1], v[c0:c1], hq, out_b[c0:c1])
            S.kvpool_append(PB.h, b, 0, k[c0:c1], v[c0:c1])
        torch.cuda.synchronize()
        assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
    rows = sample_rows(n)
    kh = torch.cat([kp[:pre].cpu(), k.cpu()]) if pre else k.cpu()
    vh = torch.cat([vp[:pre].cpu(), v.cpu()]) if pre else v.cpu()
    qs = to64(q.cpu())
    ref = A.attention(qs, to64(kh), to64(vh), pre, w, rows=rows)[rows]
    err = float(np.max(np.abs(to64(out_a.cpu())[rows] - ref)))
    assert err <= BF16_ABS, f"max |gpu - oracle| = {err:.3e}"


def test_band_prefill_fp8_ring_prefix(S):
    """FP8 ring (w = 128, 32/4 heads, d = 128) holding 500 prefix tokens, 16K chunk in the band form,
    sampled rows against the oracle over the prefix's E4M3 round trip and the chunk's bf16 keys."""
    w, hq, hkv, d, n, pre = 128, 32, 4, 128, 16384, 500
    kp, vp = draw(pre, hkv, d, "f8kp"), draw(pre, hkv, d, "f8vp")
    q, k, v = draw(n, hq, d, "f8q"), draw(n, hkv, d, "f8k"), draw(n, hkv, d, "f8v")
    with GpuPool(S, window=w, hkv=hkv, d=d, dtype=torch.float8_e4m3fn, max_seqs=1,
                 max_seq_len=pre + n + 16) as P:
        s = S.kvpool_seq_open(P.h)
        S.kvpool_append(P.h, s, 0, kp, vp)
        out = torch.empty_like(q)
        S.swa_attn_prefill(P.h, s, 0, q, k, v, hq, out)
        torch.cuda.synchronize()
    rows = sample_rows(n)
    kh = np.concatenate([F8.roundtrip(to64(kp.cpu()), 1.0), to64(k.cpu())])
    vh = np.concatenate([F8.roundtrip(to64(vp.cpu()), 1.0), to64(v.cpu())])
    ref = A.attention(to64(q.cpu()), kh, vh, pre, w, rows=rows)[rows]
    err = float(np.max(np.abs(to64(out.cpu())[rows] - ref)))
    assert err <= BF16_ABS, f"max |gpu - oracle| = {err:.3e}"


@pytest.mark.parametrize("style", ["pairs", "halves"])
def test_band_prefill_fused_rope(S, style):
    """Fused RoPE in the band form (each block's queries turn as they load, at every block switch):
    raw q/k into a fused pool equal kvpool_rope then the same call on a plain pool, bit for bit."""
    w, hq, hkv, d, n, pre, base = 128, 32, 4, 128, 16384, 700, 10000.0
    kw = dict(window=w, hkv=hkv, d=d, dtype=torch.bfloat16, max_seqs=1, max_seq_len=pre + n + 16,
              rope_base=base, rope_style=style)
    kp, vp = draw(pre, hkv, d, "rkp"), draw(pre, hkv, d, "rvp")
    q, k, v = draw(n, hq, d, "rq"), draw(n, hkv, d, "rk"), draw(n, hkv, d, "rv")
    with GpuPool(S, **kw) as P0, GpuPool(S, **kw, rope_fused=True, max_chunk=n) as P1:
        s0, s1 = S.kvpool_seq_open(P0.h), S.kvpool_seq_open(P1.h)
        kpr = kp.clone()
        S.kvpool_rope(P0.h, [s0], 0, None, 0, kpr, pre)
        S.kvpool_append(P0.h, s0, 0, kpr, vp)
        S.kvpool_append(P1.h, s1, 0, kp, vp)
        q0, k0 = q.clone(), k.clone()
        S.kvpool_rope(P0.h, [s0], 0, q0, hq, k0, n)
        o0, o1 = torch.empty_like(q), torch.empty_like(q)
        S.swa_attn_prefill(P0.h, s0, 0, q0, k0, v, hq, o0)
        S.swa_attn_prefill(P1.h, s1, 0, q, k, v, hq, o1)
        torch.cuda.synchronize()
        assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))
    rows = sample_rows(n)
    pos = np.arange(pre + n)
    kh = torch.from_numpy(R.rope(to64(torch.cat([kp.cpu(), k.cpu()])), pos, base, style)).to(torch.bfloat16)
    qr = torch.from_numpy(R.rope(to64(q.cpu()), pos[pre:], base, style)).to(torch.bfloat16)
    ref = A.attention(to64(qr), to64(kh), to64(torch.cat([vp.cpu(), v.cpu()])), pre, w, rows=rows)[rows]
    err = float(np.max(np.abs(to64(o1.cpu())[rows] - ref)))
    assert err <= BF16_ABS, f"max |gpu - oracle| = {err:.3e}"
