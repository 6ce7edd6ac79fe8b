"""GPU parity of the two full-layer decode planners (uniform split, length-bucketed split) against
the fp64 oracle, on sequences in all three length buckets (0-64K, 64K-256K, 256K+), through the
C ABI.  Bar: bf16 max|d| <= 2e-2 against the oracle for both planners."""
import numpy as np
import pytest
import torch

import synth
from oracle import attention as A
from tests.helpers import GpuPool, assert_close, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def S():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import long_context_swa_amd.swa as S
    return S


LENS = [5, 4095, 70000, 262150, 300]   # buckets 0, 0, 1, 2, 0
HQ, HKV, D = 8, 2, 64


@pytest.fixture(scope="module")
def history():
    """Logical K/V of each sequence (drawn on the device, host copies kept for the oracle)."""
    out = []
    for i, L in enumerate(LENS):
        k = synth.normal((L, HKV, D), 80, "k", i, dtype=torch.bfloat16, device="cuda")
        v = synth.normal((L, HKV, D), 80, "v", i, dtype=torch.bfloat16, device="cuda")
        out.append((k, v, to64(k), to64(v)))
    return out


@pytest.mark.parametrize("plan", ["uniform", "bucketed"])
@pytest.mark.parametrize("q_len", [1, 3])
def test_decode_planners_match_oracle_across_buckets(S, history, plan, q_len):
    print(f"[planner] plan={plan} q_len={q_len}", flush=True)
    pages = sum((L + q_len + 15) // 16 + 1 for L in LENS)
    with GpuPool(S, n_layers=1, window=128, hkv=HKV, d=D, dtype=torch.bfloat16, pages=pages,
                 max_seqs=len(LENS), max_seq_len=max(LENS) + 8, layer_is_full=[1], decode_plan=plan) as P:
        h = P.h
        seqs = []
        for (k, v, _, _) in history:
            s = S.kvpool_seq_open(h)
            S.kvpool_append(h, s, 0, k, v)
            seqs.append(s)
        n = len(LENS)
        q = synth.normal((n, q_len, HQ, D), 81, "q", q_len, dtype=torch.bfloat16, device="cuda")
        kn = synth.normal((n, q_len, HKV, D), 81, "kn", q_len, dtype=torch.bfloat16, device="cuda")
        vn = synth.normal((n, q_len, HKV, D), 81, "vn", q_len, dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(max(S.swa_attn_workspace_bytes(h, seqs, 0, q_len, HQ), 256), dtype=torch.uint8,
                         device="cuda")
        out = torch.empty_like(q)
        S.full_attn(h, seqs, 0, q, kn, vn, q_len, HQ, out, ws)
        torch.cuda.synchronize()
        for i, L in enumerate(LENS):
            _, _, k64, v64 = history[i]
            kk = np.concatenate([k64, to64(kn[i])])
            vv = np.concatenate([v64, to64(vn[i])])
            ref = A.attention(to64(q[i]), kk, vv, L, None)
            assert_close(out[i], ref, torch.bfloat16, f"{plan} q_len={q_len} seq len {L}")
