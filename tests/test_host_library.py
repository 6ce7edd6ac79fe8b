"""Host-side checks of libswa on the CPU (no GPU needed): the library loads and exports every
entry point of include/swa.h; pool metadata, ring tags, page accounting, window-safe length and
fork rules (on planning pools, which keep host metadata only) agree with the oracle; every error
code can be forced from the host."""
import os
import re

import pytest
from hypothesis import given, settings, strategies as st

from oracle import kvcache as KC

# a missing or unbuilt library is a failure, not a skip: every test below needs it
import long_context_swa_amd.swa as S  # noqa: E402

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "swa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 18, names
    for n in names:
        assert hasattr(S._lib, n), f"libswa.so does not export {n}"
    assert sorted(S.EXPORTS) == names


def plan_pool(n_layers=14, w=8, hkv=2, d=64, pages=64, max_seqs=8, max_len=4096, full=None):
    desc = S.make_desc(n_layers, w, hkv, d, S.SWA_BF16, pages, max_seqs, max_len, layer_is_full=full)
    return S.kvpool_create(desc), desc


def test_default_layer_map_matches_hybrid_stack():
    p, _ = plan_pool(n_layers=70)
    assert [S.kvpool_layer_is_full(p, l) for l in range(70)] == [KC.layer_is_full(l) for l in range(70)]
    assert sum(S.kvpool_layer_is_full(p, l) for l in range(70)) == 10
    S.kvpool_destroy(p)


@given(st.integers(1, 12), st.lists(st.integers(1, 30), min_size=1, max_size=6))
@settings(max_examples=150, deadline=None)
def test_ring_tags_follow_slot_rule(w, chunks):
    p, _ = plan_pool(n_layers=1, w=w, full=[0])
    s = S.kvpool_seq_open(p)
    buf = KC.RollingBuffer(w, 1)
    for n in chunks:
        S.kvpool_append(p, s, 0, None, None, n)
        for _ in range(n):
            buf.append([0], [0])
    assert S.kvpool_slot_tags(p, s, 0, w) == list(buf.tags)
    assert S.kvpool_seq_len(p, s, 0) == buf.length
    S.kvpool_destroy(p)


@given(st.integers(1, 10), st.lists(st.integers(0, 40), min_size=1, max_size=3), st.integers(0, 50))
@settings(max_examples=300, deadline=None)
def test_window_safe_len_matches_oracle_brute_force(w, layer_lens, m):
    """Layers of one donor may have different committed lengths (mid-stack); the library must
    agree bit-exactly with the oracle's brute force over the same ring tags."""
    n = len(layer_lens)
    p, _ = plan_pool(n_layers=n + 1, w=w, full=[0] * n + [1], pages=256)
    s = S.kvpool_seq_open(p)
    for l, L in enumerate(layer_lens):
        if L:
            S.kvpool_append(p, s, l, None, None, L)
    tags = [S.kvpool_slot_tags(p, s, l, w) for l in range(n)]
    donor_len = min(layer_lens + [0])  # the full layer has 0 tokens
    got = S.kvpool_window_safe_len(p, s, m)
    assert got == KC.window_safe_len(tags, donor_len, m, w)
    S.kvpool_destroy(p)


def test_window_safe_len_closed_form_on_stack():
    w = 8
    p, _ = plan_pool(n_layers=14, w=w, pages=512)
    for L in (0, 3, 8, 9, 50):
        s = S.kvpool_seq_open(p)
        for l in range(14):
            if L:
                S.kvpool_append(p, s, l, None, None, L)
        for m in range(0, L + 3):
            assert S.kvpool_window_safe_len(p, s, m) == KC.window_safe_len_closed(L, m, w)
        S.kvpool_seq_close(p, s)
    S.kvpool_destroy(p)


def test_fork_rules_pages_and_bytes():
    w, hkv, d = 8, 2, 64
    full = [KC.layer_is_full(l) for l in range(14)]
    p, _ = plan_pool(n_layers=14, w=w, hkv=hkv, d=d, pages=40, full=full)
    tok = 2 * hkv * d * 2
    a = S.kvpool_seq_open(p)
    for l in range(14):
        S.kvpool_append(p, a, l, None, None, 50)
    # not window-safe: 20 < 50 with 50 > w
    with pytest.raises(S.SwaError) as e:
        S.kvpool_seq_fork(p, a, 20)
    assert e.value.code == S.SWA_EINVAL
    assert S.kvpool_window_safe_len(p, a, 20) == 0
    free_before = S.kvpool_free_pages(p, 6)
    b = S.kvpool_seq_fork(p, a, 50)            # continue the donor: share 3 whole pages, copy 1
    assert all(S.kvpool_seq_len(p, b, l) == 50 for l in range(14))
    assert S.kvpool_free_pages(p, 6) == free_before - 1
    assert S.kvpool_slot_tags(p, b, 0, w) == S.kvpool_slot_tags(p, a, 0, w)
    c = S.kvpool_seq_fork(p, a, 0)             # branch: nothing reusable
    assert all(S.kvpool_seq_len(p, c, l) == 0 for l in range(14))
    assert S.kvpool_slot_tags(p, c, 0, w) == [-1] * w
    alloc, res = S.kvpool_bytes(p)
    # 3 sequences x 12 SWA layers of w slots; pages: a holds 4, b shares 3 and owns 1 (x2 layers)
    assert alloc == 3 * 12 * w * tok + 2 * 5 * 16 * tok
    assert res == (12 * (w + w + 0)) * tok + 2 * 5 * 16 * tok
    exp_alloc, exp_res = KC.dual_pool_bytes([50, 50, 0], full, w, hkv, d, 2, 16, shared_pages=3)
    assert (alloc, res) == (exp_alloc, exp_res)
    # closing the donor keeps the shared pages alive for b
    S.kvpool_seq_close(p, a)
    assert S.kvpool_free_pages(p, 6) == 40 - 4
    S.kvpool_seq_close(p, b)
    S.kvpool_seq_close(p, c)
    assert S.kvpool_free_pages(p, 6) == 40
    assert S.kvpool_bytes(p) == (0, 0)
    S.kvpool_destroy(p)


def test_fork_short_donor_partial_reuse():
    w = 16
    p, _ = plan_pool(n_layers=7, w=w, pages=16)
    a = S.kvpool_seq_open(p)
    for l in range(7):
        S.kvpool_append(p, a, l, None, None, 12)
    for m in range(13):                        # donor never exceeded w: any cut is safe
        assert S.kvpool_window_safe_len(p, a, m) == m
        b = S.kvpool_seq_fork(p, a, m)
        tags = S.kvpool_slot_tags(p, b, 0, w)
        assert tags == [t if 0 <= t < m else -1 for t in S.kvpool_slot_tags(p, a, 0, w)]
        S.kvpool_seq_close(p, b)
    S.kvpool_destroy(p)


def test_locate_follows_slot_and_page_rules():
    w, hkv, d = 8, 2, 64
    p, _ = plan_pool(n_layers=7, w=w, hkv=hkv, d=d, pages=16)
    s = S.kvpool_seq_open(p)
    S.kvpool_append(p, s, 0, None, None, 20)
    S.kvpool_append(p, s, 6, None, None, 40)
    with pytest.raises(S.SwaError):
        S.kvpool_locate(p, s, 0, 11, 0)       # overwritten: 20 > 11 + w
    offs = {S.kvpool_locate(p, s, 0, q, h)[0] for q in range(12, 20) for h in range(hkv)}
    assert len(offs) == 8 * hkv
    k12, v12, st = S.kvpool_locate(p, s, 0, 12, 1)
    k13, _, _ = S.kvpool_locate(p, s, 0, 13, 1)
    assert st == 2 and k13 - k12 == d * 2 and v12 != k12
    k16, _, _ = S.kvpool_locate(p, s, 6, 16, 0)
    k17, _, _ = S.kvpool_locate(p, s, 6, 17, 0)
    k31, _, _ = S.kvpool_locate(p, s, 6, 31, 0)
    assert k17 - k16 == d * 2 and k31 - k16 == 15 * d * 2
    with pytest.raises(S.SwaError):
        S.kvpool_locate(p, s, 6, 40, 0)
    S.kvpool_destroy(p)


def test_error_codes_from_host():
    p, desc = plan_pool(n_layers=7, w=8, hkv=2, pages=2, max_seqs=2, max_len=64)

    def code(fn, *a):
        with pytest.raises(S.SwaError) as e:
            fn(*a)
        return e.value.code
    bad = S.make_desc(1, 0, 1, 64, S.SWA_F32, 0, 1, 16)
    assert code(S.kvpool_arena_bytes, bad) == S.SWA_EINVAL            # w < 1
    assert code(S.kvpool_arena_bytes, S.make_desc(1, 8, 1, 96, S.SWA_F32, 0, 1, 16)) == S.SWA_EINVAL
    assert code(S.kvpool_seq_len, p, 3, 0) == S.SWA_ENOSEQ
    assert code(S.kvpool_seq_close, p, 0) == S.SWA_ENOSEQ
    a = S.kvpool_seq_open(p)
    b = S.kvpool_seq_open(p)
    assert code(S.kvpool_seq_open, p) == S.SWA_ENOMEM                # slots exhausted
    S.kvpool_append(p, a, 6, None, None, 32)                           # takes both pages
    assert code(S.kvpool_append, p, b, 6, None, None, 1) == S.SWA_ENOMEM
    assert S.kvpool_seq_len(p, b, 6) == 0                              # no change on failure
    assert code(S.kvpool_append, p, a, 0, None, None, 0) == S.SWA_EINVAL
    assert code(S.kvpool_append, p, a, 0, None, None, 65) == S.SWA_EINVAL   # > max_seq_len
    assert code(S.kvpool_window_safe_len, p, a, -1) == S.SWA_EINVAL
    assert code(S.kvpool_free_pages, p, 0) == S.SWA_EINVAL              # SWA layer
    assert code(S.kvpool_slot_tags, p, a, 6, 8) == S.SWA_EINVAL         # full layer
    # attention on a planning pool, layer-kind mismatch, bad head counts, bad q_len
    assert code(S.swa_attn_workspace_bytes, p, [a], 0, 5, 2) == S.SWA_EINVAL   # q_len > 4
    assert code(S.swa_attn_workspace_bytes, p, [a], 0, 1, 3) == S.SWA_EINVAL   # Hq % Hkv
    assert code(S.swa_attn_workspace_bytes, p, [a, a], 0, 1, 2) == S.SWA_EINVAL  # duplicate
    assert code(S.swa_attn_workspace_bytes, p, [7], 0, 1, 2) == S.SWA_ENOSEQ
    assert S.swa_attn_workspace_bytes(p, [a], 6, 16, 2) == 0            # full prefill: none
    assert S.swa_attn_workspace_bytes(p, [a, b], 6, 1, 2) > 0
    rc = S._lib.swa_attn_prefill(p, a, 0, None, None, None, 4, 2, S.SWA_BF16, None, None)
    assert rc == S.SWA_EINVAL and "arena" in S.swa_last_error()
    S.kvpool_destroy(p)


def test_workspace_grows_with_splits():
    p, _ = plan_pool(n_layers=7, w=8, hkv=2, pages=1024, max_len=1 << 16)
    a = S.kvpool_seq_open(p)
    S.kvpool_append(p, a, 6, None, None, 16)
    small = S.swa_attn_workspace_bytes(p, [a], 6, 1, 16)
    S.kvpool_append(p, a, 6, None, None, 8000)
    big = S.swa_attn_workspace_bytes(p, [a], 6, 1, 16)
    assert big > small
    S.kvpool_destroy(p)


def test_fp8_pool_descriptors():
    """FP8 pools store one byte per element (half the bf16 arena for rings and pages) and accept
    only power-of-two scales (0 means 1)."""
    import long_context_swa_amd.swa as S
    import torch
    kw = dict(layer_is_full=None)
    bf = S.make_desc(14, 128, 4, 128, torch.bfloat16, 1024, 8, 1 << 16, **kw)
    f8 = S.make_desc(14, 128, 4, 128, torch.float8_e4m3fn, 1024, 8, 1 << 16, **kw)
    b_bf, b_f8 = S.kvpool_arena_bytes(bf), S.kvpool_arena_bytes(f8)
    # tables and the metadata zone do not shrink; KV bytes halve
    assert b_f8 < b_bf and (b_bf - b_f8) * 2 >= (b_bf - (4 << 20)) * 0.9
    for good in (1.0, 0.0, 0.25, 8.0, 2.0 ** -60):
        d = S.make_desc(7, 16, 1, 64, torch.float8_e4m3fn, 4, 2, 256, k_scale=good, v_scale=good)
        assert S.kvpool_arena_bytes(d) > 0
    for bad in (3.0, -1.0, 0.1, 2.0 ** 70):
        d = S.make_desc(7, 16, 1, 64, torch.float8_e4m3fn, 4, 2, 256, k_scale=bad)
        with pytest.raises(S.SwaError):
            S.kvpool_arena_bytes(d)


def test_snapshot_fork_release_bookkeeping():
    """Planning pool (host metadata only): a snapshot holds the full-layer pages covering its
    length after the donor closes, a fork from it starts at that length with its ring tags, and
    release returns the pages; slots run out with SWA_ENOMEM; layers at different lengths are
    rejected."""
    import long_context_swa_amd.swa as S
    import torch
    w = 16
    d = S.make_desc(7, w, 1, 64, torch.bfloat16, 64, 4, 4096, max_snapshots=2)
    p = S.kvpool_create(d)
    try:
        don = S.kvpool_seq_open(p)
        for layer in range(7):
            S.kvpool_append(p, don, layer, None, None, 40)
        snap = S.kvpool_snapshot(p, don)
        assert S.kvpool_snapshot_len(p, snap) == 40
        for layer in range(7):
            S.kvpool_append(p, don, layer, None, None, 60)        # donor moves to 100
        assert S.kvpool_window_safe_len(p, don, 40) == 0          # the live ring cannot serve 40
        free_before = S.kvpool_free_pages(p, 6)
        S.kvpool_seq_close(p, don)
        # pages 0..2 (positions 0..47) stay held by the snapshot; the donor's other 4 pages return
        assert S.kvpool_free_pages(p, 6) == free_before + 7 - 3
        f = S.kvpool_seq_fork_snapshot(p, snap)
        assert all(S.kvpool_seq_len(p, f, layer) == 40 for layer in range(7))
        tags = S.kvpool_slot_tags(p, f, 0, w)
        assert sorted(t for t in tags if t >= 0) == list(range(24, 40))
        assert S.kvpool_window_safe_len(p, f, 40) == 40
        s2 = S.kvpool_snapshot(p, f)
        with pytest.raises(S.SwaError):                            # both slots held
            S.kvpool_snapshot(p, f)
        S.kvpool_snapshot_release(p, s2)
        S.kvpool_snapshot_release(p, snap)
        with pytest.raises(S.SwaError):
            S.kvpool_snapshot_release(p, snap)                     # already released
        S.kvpool_seq_close(p, f)
        assert S.kvpool_free_pages(p, 6) == 64                     # every page back
        g = S.kvpool_seq_open(p)
        S.kvpool_append(p, g, 0, None, None, 5)                    # layer 0 at 5, the others at 0
        with pytest.raises(S.SwaError):
            S.kvpool_snapshot(p, g)
    finally:
        S.kvpool_destroy(p)


def test_rope_descriptors_and_errors():
    base = dict(n_layers=7, window=8, n_kv_heads=2, head_dim=64, kv_dtype=S.SWA_BF16,
                pages_per_full_layer=16, max_seqs=4, max_seq_len=5000)
    plain = S.kvpool_arena_bytes(S.make_desc(**base))
    roped = S.kvpool_arena_bytes(S.make_desc(**base, rope_base=10000.0, rope_style="halves"))
    # 2048 low-angle rows + ceil(5000 / 2048) = 3 high-angle rows of d/2 (cos, sin) fp32 pairs
    tables = (2048 + 3) * 32 * 8
    assert tables <= roped - plain <= tables + 2 * 4096
    for bad in (dict(rope_base=-1.0), dict(rope_base=float("nan")), dict(rope_base=float("inf")),
                dict(rope_style=2), dict(rope_base=10000.0, max_seq_len=(1 << 26) + 1)):
        with pytest.raises(S.SwaError) as e:
            S.kvpool_arena_bytes(S.make_desc(**{**base, **bad}))
        assert e.value.code == S.SWA_EINVAL
    # planning pools and pools without RoPE reject the call before touching any pointer
    for desc in (S.make_desc(**base, rope_base=10000.0), S.make_desc(**base)):
        p = S.kvpool_create(desc)
        s = S.kvpool_seq_open(p)
        ids = S._I32([s])  # held across the call: the library gets its address only
        rc = S._lib.kvpool_rope(p, 1, ids.ptr, 0, 16, 8, 16, 1, S.SWA_BF16, None)
        assert rc == S.SWA_EINVAL
        S.kvpool_destroy(p)


def test_decode_plan_descriptor():
    ok = S.make_desc(7, 8, 2, 64, S.SWA_BF16, 16, 4, 4096, decode_plan="bucketed")
    assert S.kvpool_arena_bytes(ok) == S.kvpool_arena_bytes(S.make_desc(7, 8, 2, 64, S.SWA_BF16, 16, 4, 4096))
    with pytest.raises(S.SwaError) as e:
        S.kvpool_arena_bytes(S.make_desc(7, 8, 2, 64, S.SWA_BF16, 16, 4, 4096, decode_plan=2))
    assert e.value.code == S.SWA_EINVAL


def test_clock_probe_argument_errors_from_host():
    """The clock measurement aid checks its arguments before touching the device."""
    for out, spin in ((None, 100), (8, 0), (8, 10_000_001), (12, 100)):
        with pytest.raises(S.SwaError) as e:
            S.swa_clock_probe(out, spin)
        assert e.value.code == S.SWA_EINVAL, (out, spin)
    assert S.clock_mhz([0, 2_400_000, 0, 100_000, 100_000]) == pytest.approx(2400.0)


def test_max_seq_len_limit():
    """Key indices in work items and kernels are 32-bit: a descriptor allowing 2^31 tokens or more
    is refused, so no full-layer prior can wrap when a decode call is planned."""
    ok = S.make_desc(7, 8, 2, 64, S.SWA_BF16, 16, 4, (1 << 31) - 1)
    assert S.kvpool_arena_bytes(ok) > 0
    for bad in (1 << 31, 1 << 40, 0):
        with pytest.raises(S.SwaError) as e:
            S.kvpool_arena_bytes(S.make_desc(7, 8, 2, 64, S.SWA_BF16, 16, 4, bad))
        assert e.value.code == S.SWA_EINVAL


def test_fused_rope_descriptor():
    """A pool fusing RoPE into attention and commit reserves max_chunk x Hkv x d bf16 for the rotated
    keys of a prefill chunk; it needs RoPE, a bf16 or FP8 pool and max_chunk >= 1."""
    base = dict(n_layers=7, window=8, n_kv_heads=2, head_dim=64, pages_per_full_layer=16, max_seqs=4,
                max_seq_len=5000, rope_base=10000.0)
    roped = S.kvpool_arena_bytes(S.make_desc(**base, kv_dtype=S.SWA_BF16))
    fused = S.kvpool_arena_bytes(S.make_desc(**base, kv_dtype=S.SWA_BF16, rope_fused=True, max_chunk=1000))
    assert 1000 * 2 * 64 * 2 <= fused - roped <= 1000 * 2 * 64 * 2 + 4096
    assert S.kvpool_arena_bytes(S.make_desc(**base, kv_dtype=S.SWA_FP8_E4M3, rope_fused=True, max_chunk=16)) > 0
    two = S.make_desc(**base, kv_dtype=S.SWA_BF16, rope_fused=True, max_chunk=16)
    two.rope_fused = 2
    with pytest.raises(S.SwaError) as e:
        S.kvpool_arena_bytes(two)
    assert e.value.code == S.SWA_EINVAL
    for bad in (dict(kv_dtype=S.SWA_BF16, rope_base=0.0, rope_fused=True, max_chunk=16),   # no RoPE
                dict(kv_dtype=S.SWA_F32, rope_fused=True, max_chunk=16),                    # fp32 pool
                dict(kv_dtype=S.SWA_BF16, rope_fused=True, max_chunk=0),                    # no chunk room
                dict(kv_dtype=S.SWA_BF16, max_chunk=-1)):
        with pytest.raises(S.SwaError) as e:
            S.kvpool_arena_bytes(S.make_desc(**{**base, **bad}))
        assert e.value.code == S.SWA_EINVAL, bad
