"""full_attn_noalloc (the entry point for callers that cannot allocate device memory) against
full_attn with a caller workspace and against the fp64 oracle, through the C ABI.

Two calls in a row on one pool: a 6-sequence verify (q_len = 4) whose long rows are split over pages
and merged from partials held in the library's device scratch array, then a smaller 3-sequence
decode (q_len = 1), so the second call runs over whatever the first left in the array.  Both calls
must match full_attn with its own workspace exactly (same plan, same kernels) and the oracle within
the bf16 bar.  A call that needs more workspace than the array holds is refused with SWA_ENOMEM.
Inputs are seeded N(0,1) draws (synth)."""
import pytest
import torch

import synth
from oracle import attention as A
from tests.helpers import GpuPool, History, assert_close, to64

pytestmark = pytest.mark.gpu
BF = torch.bfloat16


@pytest.fixture(scope="module")
def S():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import long_context_swa_amd.swa as S
    return S


def draw(n, h, d, *key):
    return synth.normal((n, h, d), *key, dtype=BF).cuda()


def test_noalloc_full_attn_matches_workspace_call_twice(S):
    d, hkv, g, layer = 128, 4, 8, 6
    hq = g * hkv
    lens = [0, 17, 2500, 9000, 700, 6100]
    with GpuPool(S, n_layers=7, window=64, hkv=hkv, d=d, dtype=BF, pages=2048, max_seqs=len(lens),
                 max_seq_len=10000) as P:
        seqs, hists = [], []
        for i, L in enumerate(lens):
            s = S.kvpool_seq_open(P.h)
            h = History(hkv, d, BF)
            if L:
                k, v = draw(L, hkv, d, 71, "k", i), draw(L, hkv, d, 71, "v", i)
                S.kvpool_append(P.h, s, layer, k, v)
                h.extend(k, v)
            seqs.append(s)
            hists.append(h)
        for call, (sel, q_len) in enumerate([(list(range(6)), 4), ([1, 3, 4], 1)]):
            ids = [seqs[i] for i in sel]
            n = len(ids)
            q = draw(n * q_len, hq, d, 71, "q", call).reshape(n, q_len, hq, d)
            kn = draw(n * q_len, hkv, d, 71, "kn", call).reshape(n, q_len, hkv, d)
            vn = draw(n * q_len, hkv, d, 71, "vn", call).reshape(n, q_len, hkv, d)
            need = S.swa_attn_workspace_bytes(P.h, ids, layer, q_len, hq)
            assert need > (1 << 20 if call == 0 else 1 << 17)  # split rows: partials in the workspace
            ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
            ref_out = torch.empty_like(q)
            S.full_attn(P.h, ids, layer, q, kn, vn, q_len, hq, ref_out, ws)
            out = torch.full_like(q, float("nan"))
            S.full_attn_noalloc(P.h, ids, layer, q, kn, vn, q_len, hq, out)
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), f"call {call}"
            for j, i in enumerate(sel):
                h = hists[i].copy()
                h.extend(kn[j], vn[j])
                ref = A.attention(to64(q[j]), to64(h.k), to64(h.v), lens[i], None)
                assert_close(out[j], ref, BF, f"call {call} seq len {lens[i]}")


def test_noalloc_refuses_calls_beyond_the_scratch_array(S):
    """A 32-sequence verify over 60,000-token rows needs ~34 MB of partials (more than the 32 MiB array): refused, nothing run."""
    d, hkv, g, layer = 128, 4, 8, 0
    hq = g * hkv
    n, L = 32, 60000
    with GpuPool(S, n_layers=1, window=64, hkv=hkv, d=d, dtype=BF, pages=n * (L // 16 + 1), max_seqs=n,
                 max_seq_len=L + 8, layer_is_full=[1]) as P:
        ids = [S.kvpool_seq_open(P.h) for _ in range(n)]
        kz = torch.zeros((L, hkv, d), dtype=BF, device="cuda")
        for s in ids:
            S.kvpool_append(P.h, s, layer, kz, kz)
        need = S.swa_attn_workspace_bytes(P.h, ids, layer, 4, hq)
        assert need > 32 << 20
        q = torch.zeros((n, 4, hq, d), dtype=BF, device="cuda")
        kn = torch.zeros((n, 4, hkv, d), dtype=BF, device="cuda")
        out = torch.full_like(q, 7.0)
        with pytest.raises(S.SwaError) as e:
            S.full_attn_noalloc(P.h, ids, layer, q, kn, kn, 4, hq, out)
        assert e.value.code == S.SWA_ENOMEM
        torch.cuda.synchronize()
        assert bool((out == 7.0).all())
