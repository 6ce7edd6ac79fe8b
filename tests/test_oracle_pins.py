"""Pins for the fp64 oracle: each test ties an oracle function to something other than itself --
values the pages print (tests/golden/*.json, cited there), closed forms, an independent library
routine (torch SDPA in float64 with a band mask built from tril/triu), high-precision brute force,
or invariants of softmax attention.  CPU only."""
import json
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from hypothesis import given, settings, strategies as st

from oracle import attention as A
from oracle import kvcache as KC

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def rng(seed):
    return np.random.default_rng(seed)


def band_mask_torch(n, w):
    """Band mask built from library routines only: lower triangle AND within w-1 of the diagonal."""
    ones = torch.ones(n, n, dtype=torch.bool)
    m = torch.tril(ones)
    if w is not None:
        m = m & torch.triu(ones, diagonal=-(w - 1))
    return m


# ------------------------------------------------------------------------------ key sets / mask

@pytest.mark.parametrize("n", list(range(1, 25)))
def test_mask_matches_library_band(n):
    for w in list(range(1, 27)) + [None]:
        assert np.array_equal(A.mask(n, w), band_mask_torch(n, w).numpy()), (n, w)


def test_mask_counts_printed():
    g = golden("swa_theory_values.json")["mask_counts"]
    n, w = g["n"], g["w"]
    assert A.mask_nonzeros(n, None) == g["full_causal_nonzeros"] == n * (n + 1) // 2
    swa = A.mask_nonzeros(n, w)
    assert swa <= g["swa_upper_bound_nw"]
    assert swa == n * w - w * (w - 1) // 2 == 228          # exact count, closed form for n >= w


def test_window_reduces_to_full_when_w_ge_n():
    for n in (1, 5, 13):
        for w in (n, n + 1, 100):
            assert np.array_equal(A.mask(n, w), A.mask(n, None))


def test_score_memory_ratios_printed():
    g = golden("swa_theory_values.json")["score_memory"]
    assert 512 * 512 * 4 == g["fp32_bytes_n512_approx_mb"] * 2**20
    assert 32768 * 32768 * 4 == g["fp32_bytes_n32768_approx_gb"] * 2**30
    r = A.mask_nonzeros(4096, 256) / 4096**2
    assert abs(r - g["swa_over_full_n4096_w256_approx"]) / g["swa_over_full_n4096_w256_approx"] < 0.04
    assert abs(1 / r - 16.51) < 0.01
    n, w = 32 * 4096, 4096
    saved = 1 - A.mask_nonzeros(n, w) / n**2
    assert abs(saved - g["saved_fraction_n_eq_32w_approx"]) < 0.005
    assert abs(saved - 0.96923) < 1e-4


# ------------------------------------------------------------------------------ attention values

@pytest.mark.parametrize("n,w,hq,hkv,d", [(1, 1, 1, 1, 4), (5, 3, 4, 2, 8), (17, 8, 4, 1, 16),
                                          (40, 50, 8, 2, 8), (33, 7, 2, 2, 5), (24, 1, 4, 4, 3)])
def test_attention_matches_torch_sdpa_with_band_mask(n, w, hq, hkv, d):
    r = rng(n * 100 + w)
    q = r.standard_normal((n, hq, d))
    k = r.standard_normal((n, hkv, d))
    v = r.standard_normal((n, hkv, d))
    ours = A.attention(q, k, v, 0, w)
    qt, kt, vt = (torch.from_numpy(x).permute(1, 0, 2)[None] for x in (q, k, v))
    ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=band_mask_torch(n, w), enable_gqa=True)
    ref = ref[0].permute(1, 0, 2).numpy()
    assert np.max(np.abs(ours - ref)) < 1e-12


def test_full_causal_matches_torch_is_causal():
    r = rng(7)
    n, hq, hkv, d = 29, 8, 2, 16
    q, k, v = r.standard_normal((n, hq, d)), r.standard_normal((n, hkv, d)), r.standard_normal((n, hkv, d))
    qt, kt, vt = (torch.from_numpy(x).permute(1, 0, 2)[None] for x in (q, k, v))
    ref = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, enable_gqa=True)[0].permute(1, 0, 2).numpy()
    for w in (None, n, n + 5):
        assert np.max(np.abs(A.attention(q, k, v, 0, w) - ref)) < 1e-12


def test_window_one_returns_own_value_and_first_row_is_v0():
    r = rng(3)
    n, d = 12, 6
    q, k, v = r.standard_normal((n, 2, d)), r.standard_normal((n, 1, d)), r.standard_normal((n, 1, d))
    o = A.attention(q, k, v, 0, 1)
    assert np.array_equal(o[:, 0], v[:, 0]) and np.array_equal(o[:, 1], v[:, 0])
    o = A.attention(q, k, v, 0, 5)
    assert np.allclose(o[0, :], v[0, 0], rtol=0, atol=1e-15)


@pytest.mark.parametrize("w", [1, 2, 5, 9, 40])
def test_zero_query_gives_window_mean(w):
    """q = 0 makes all scores equal, so each output is the plain mean of the values in W(i).
    The mean is taken from a cumulative sum (moving average), independent of the key-set code."""
    r = rng(w)
    n, d = 30, 4
    v = r.standard_normal((n, 1, d))
    o = A.attention(np.zeros((n, 1, d)), r.standard_normal((n, 1, d)), v, 0, w)
    c = np.concatenate([np.zeros((1, d)), np.cumsum(v[:, 0], axis=0)])
    for i in range(n):
        lo = max(0, i - w + 1)
        assert np.allclose(o[i, 0], (c[i + 1] - c[lo]) / (i + 1 - lo), atol=1e-13)


def test_scale_and_key_set_closed_form():
    """One-hot keys: the score of key j is beta/sqrt(d) if j is the chosen key, else 0, so the
    weights are known in closed form; this fixes the 1/sqrt(d) scale and which keys take part."""
    n, w = 16, 6
    d = n
    k = np.eye(n)[:, None, :]
    r = rng(11)
    v = r.standard_normal((n, 1, 3))
    beta = 3.0
    for i in range(n):
        lo = max(0, i - w + 1)
        jstar = (lo + i) // 2
        q = np.zeros((1, 1, d))
        q[0, 0, jstar] = beta
        qq = np.zeros((i + 1, 1, d))
        qq[i] = q[0]
        o = A.attention(qq, k[: i + 1], v[: i + 1], 0, w, rows=[i])[i, 0]
        e = math.exp(beta / math.sqrt(d))
        cnt = i + 1 - lo
        expect = (e * v[jstar, 0] + v[lo:i + 1, 0].sum(0) - v[jstar, 0]) / (e + cnt - 1)
        assert np.allclose(o, expect, atol=1e-13), i


def test_affine_in_values():
    r = rng(5)
    n, d = 20, 5
    q, k, v = r.standard_normal((n, 2, d)), r.standard_normal((n, 1, d)), r.standard_normal((n, 1, d))
    a, b = 2.5, -0.75
    assert np.allclose(A.attention(q, k, a * v + b, 0, 4), a * A.attention(q, k, v, 0, 4) + b, atol=1e-12)


def test_high_precision_dense_brute_force():
    """Eq.(2)-(5) as written (dense mask over all n keys, masked scores dropped as exp(-inf)=0),
    evaluated in 40-digit decimal arithmetic."""
    getcontext().prec = 40
    r = rng(2)
    n, d, w = 6, 3, 3
    q, k, v = r.standard_normal((n, 1, d)), r.standard_normal((n, 1, d)), r.standard_normal((n, 1, d))
    ours = A.attention(q, k, v, 0, w)
    M = band_mask_torch(n, w).numpy()
    sq = Decimal(d).sqrt()
    for i in range(n):
        s = [sum(Decimal(float(q[i, 0, t])) * Decimal(float(k[j, 0, t])) for t in range(d)) / sq
             if M[i, j] else None for j in range(n)]
        e = [x.exp() if x is not None else Decimal(0) for x in s]
        z = sum(e)
        for t in range(d):
            o = sum(e[j] * Decimal(float(v[j, 0, t])) for j in range(n)) / z
            assert abs(float(o) - ours[i, 0, t]) < 1e-14


def test_flop_count_closed_form():
    n, w, hq, d = 16384, 4096, 32, 128
    pairs = n * w - w * (w - 1) // 2
    assert pairs == 58_722_304
    assert A.attention_flops(n, 0, w, hq, d) == 4 * d * pairs * hq == 962_106_228_736
    assert A.attention_flops(10, 5, None, 1, 2) == 4 * 2 * sum(range(6, 16))


# ------------------------------------------------------------------------------ rolling buffer

def test_rolling_buffer_demo_printed():
    g = golden("swa_theory_values.json")["rolling_buffer_demo"]
    buf = KC.RollingBuffer(g["w"], g["head_dim"])
    for t in range(8):
        buf.append(np.full(g["head_dim"], t), np.full(g["head_dim"], t))
        if t == 5:
            assert list(buf.tags) == g["physical_slots_after_step5"]
        if t == 7:
            assert buf.resident_positions() == g["resident_after_step7"]
    assert buf.memory_bytes(g["num_heads"], g["elem_bytes_fp32"]) == 2 * 4 * 1 * 2 * 4 == 64


@given(st.integers(1, 20), st.integers(0, 70))
@settings(max_examples=200, deadline=None)
def test_resident_set_is_last_w(w, L):
    buf = KC.RollingBuffer(w, 1)
    for t in range(L):
        buf.append([t], [t])
    assert buf.resident_positions() == KC.resident_after(L, w) == list(range(max(0, L - w), L))
    for p in KC.resident_after(L, w):
        assert buf.read(p)[0][0] == p and KC.slot_of(p, w) == p % w


def test_decode_through_buffer_equals_prefill_row():
    """Rolling buffer = masked full cache: every decode row read through the ring equals the
    prefill row of the same position over the logical sequence (ring order != time order)."""
    r = rng(9)
    T, w, d = 45, 7, 4
    q, k, v = r.standard_normal((T, 1, d)), r.standard_normal((T, 1, d)), r.standard_normal((T, 1, d))
    full = A.attention(q, k, v, 0, w)
    buf = KC.RollingBuffer(w, d)
    for t in range(T):
        o = KC.decode_via_buffer(q[t, 0], buf, k[t, 0], v[t, 0], t, w)
        assert np.allclose(o, full[t, 0], atol=1e-13), t
        buf.append(k[t, 0], v[t, 0])


def test_raw_match_length_fork_is_silently_wrong():
    """Mutation: reusing a donor's ring at the raw match length (not the window-safe one) reads
    slots that now hold other positions; the output then differs from the definition."""
    r = rng(4)
    w, d, L_donor, m = 7, 4, 20, 12
    k, v = r.standard_normal((L_donor + 1, d)), r.standard_normal((L_donor + 1, d))
    donor = KC.RollingBuffer(w, d)
    for t in range(L_donor):
        donor.append(k[t], v[t])
    assert KC.window_safe_len([donor.tags], L_donor, m, w) == 0
    fork = donor.copy()
    fork.length = m
    q = r.standard_normal(d)
    expect = A.attend_row(q[None], k, v, m, w)[0]
    with pytest.raises(KeyError):
        KC.decode_via_buffer(q, fork, k[m], v[m], m, w, checked=True)
    wrong = KC.decode_via_buffer(q, fork, k[m], v[m], m, w, checked=False)
    assert np.max(np.abs(wrong - expect)) > 1e-3


# ------------------------------------------------------------------------------ window-safe length

@given(st.integers(1, 12), st.integers(0, 40), st.integers(0, 45))
@settings(max_examples=400, deadline=None)
def test_window_safe_len_brute_equals_closed_form(w, L, m):
    buf = KC.RollingBuffer(w, 1)
    for t in range(L):
        buf.append([t], [t])
    brute = KC.window_safe_len([buf.tags, buf.tags.copy()], L, m, w)
    assert brute == KC.window_safe_len_closed(L, m, w)
    assert 0 <= brute <= min(m, L)


@given(st.integers(1, 10), st.lists(st.integers(0, 30), min_size=1, max_size=4), st.integers(0, 35))
@settings(max_examples=300, deadline=None)
def test_window_safe_len_layers_must_all_agree(w, lengths, m):
    """Layers with different committed lengths: the safe cut must be safe in every layer, i.e.
    it lies in the intersection of each ring's safe set {0} U {len} U ([0, len] if len <= w)."""
    tags = []
    for L in lengths:
        buf = KC.RollingBuffer(w, 1)
        for t in range(L):
            buf.append([t], [t])
        tags.append(buf.tags)
    donor_len = min(lengths)
    brute = KC.window_safe_len(tags, donor_len, m, w)

    def safe_set(L):
        s = {0, L}
        if L <= w:
            s |= set(range(L + 1))
        return s
    common = set.intersection(*(safe_set(L) for L in lengths))
    expect = max(x for x in common if x <= min(m, donor_len))
    assert brute == expect


# ------------------------------------------------------------------------------ KV accounting

def test_kv_per_layer_bytes_printed():
    g = golden("swa_theory_values.json")["kv_per_layer_bytes"]
    f = g["full_mha"]
    assert KC.kv_cache_size_mb(f["n"], 1, f["heads"], f["head_dim"], None, f["dtype_bytes"]) * 2**20 == f["bytes"]
    s = g["gqa_swa"]
    assert KC.kv_cache_size_mb(10**6, 1, s["kv_heads"], s["head_dim"], s["w"], s["dtype_bytes"]) * 2**20 == s["bytes"]
    assert s["bytes"] * 32 == g["gqa_swa_32_layers_mb"] * 2**20
    buf = KC.RollingBuffer(s["w"], s["head_dim"])
    assert buf.memory_bytes(s["kv_heads"], s["dtype_bytes"]) == s["bytes"]


def test_kv_stack_sizes_printed():
    g = golden("swa_theory_values.json")["kv_stack_mb"]
    L, d, W, b = g["layers"], g["head_dim"], g["window"], g["dtype_bytes"]
    assert KC.kv_cache_size_mb(32768, L, g["full_mha_heads"], d, None, b) == g["full_mha_32k_mb"]
    assert KC.kv_cache_size_mb(32768, L, g["gqa_heads"], d, W, b) == g["swa_gqa_32k_mb"]
    assert KC.kv_cache_size_mb(131072, L, g["full_mha_heads"], d, None, b) == g["full_mha_131k_mb"]
    assert KC.kv_cache_size_mb(131072, L, g["gqa_heads"], d, W, b) == g["swa_gqa_131k_mb"]


def test_hybrid_layer_map_and_ratio():
    g = golden("mimo_hybrid.json")
    full = [KC.layer_is_full(l) for l in range(g["n_layers"])]
    assert sum(full) == g["n_full"] and len(full) - sum(full) == g["n_swa"]
    W = g["window"]
    for N in (16, 128, 1024, 16384, 131072, 1 << 20):
        _, res = KC.dual_pool_bytes([N], full, W, 4, 128, 2, 16)
        all_full = 70 * N * 2 * 4 * 128 * 2
        assert Fraction(res, all_full) == Fraction(60 * min(N, W) + 10 * N, 70 * N)
        assert abs(KC.hybrid_kv_ratio(N, W) - res / all_full) < 1e-15
    lim = Fraction(*g["ratio_limit"])
    assert abs(KC.hybrid_kv_ratio(1 << 40, W) - float(lim)) < 1e-9
    assert abs(KC.hybrid_kv_ratio(131072, W) - 0.1436942) < 1e-7
    assert abs(KC.hybrid_kv_ratio(1048576 + 16384, W) - 0.1429602) < 1e-7


def test_allocated_vs_resident_and_sharing():
    full = [KC.layer_is_full(l) for l in range(14)]
    alloc, res = KC.dual_pool_bytes([5, 300], full, 128, 4, 128, 2, 16)
    tok = 2 * 4 * 128 * 2
    assert alloc == (12 * 128 * 2 + 2 * (16 + 304)) * tok
    assert res == (12 * (5 + 128) + 2 * (16 + 304)) * tok
    a2, r2 = KC.dual_pool_bytes([5, 300], full, 128, 4, 128, 2, 16, shared_pages=3)
    assert alloc - a2 == res - r2 == 3 * 2 * 16 * tok


def test_page_placement():
    table = [7, 3, 9]
    assert [KC.page_placement(p, table, 16) for p in (0, 15, 16, 40)] == [(7, 0), (7, 15), (3, 0), (9, 8)]
    assert KC.pages_needed(0, 16) == 0 and KC.pages_needed(16, 16) == 1 and KC.pages_needed(17, 16) == 2


# ------------------------------------------------------------------------------ receptive field

def test_receptive_field():
    g = golden("swa_theory_values.json")["receptive_field"]
    assert KC.receptive_field_brute(g["L"], g["w"], g["n"], g["n"] - 1) == g["R"]
    assert KC.receptive_field_formula(g["L"], g["w"]) == g["R"]
    assert KC.receptive_field_formula(g["mistral_L"], g["mistral_w"]) == 131041 != g["mistral_R_printed"]
    for L in range(1, 6):
        for w in range(1, 6):
            assert KC.receptive_field_brute(L, w, 64, 63) == KC.receptive_field_formula(L, w)


# ------------------------------------------------------------------------------------------ FP8 KV

from oracle import fp8 as F8  # noqa: E402


def test_e4m3_codes_from_the_format_definition():
    """OFP8 E4M3 worked values: bias 7, 3 mantissa bits, subnormals m*2^-9, max 448, S.1111.111 NaN."""
    table = {0x38: 1.0, 0x30: 0.5, 0x40: 2.0, 0xC0: -2.0, 0x3C: 1.5, 0x7E: 448.0, 0x7D: 416.0,
             0x08: 2.0 ** -6, 0x07: 7 * 2.0 ** -9, 0x01: 2.0 ** -9, 0x00: 0.0, 0x77: 240.0, 0x48: 4.0}
    for c, v in table.items():
        assert F8.e4m3_decode(c) == v, hex(c)
        assert F8.e4m3_encode(v) == c, v
    assert np.isnan(F8.e4m3_decode(0x7F)) and np.isnan(F8.e4m3_decode(0xFF))
    assert F8.e4m3_decode(0x80) == 0.0 and np.signbit(F8.e4m3_decode(0x80))
    assert F8.e4m3_encode(-0.0) == 0x80 and F8.e4m3_encode(float("nan")) == 0x7F


def test_e4m3_ties_to_even_and_saturation():
    # halfway between 1.0 (m=0) and 1.125 (m=1) -> even m=0; between 1.125 and 1.25 -> m=2
    assert F8.e4m3_encode(1.0625) == 0x38
    assert F8.e4m3_encode(1.1875) == 0x3A
    assert F8.e4m3_encode(1.0625 + 1e-9) == 0x39
    # subnormal ties: 2^-10 sits between 0 and 2^-9 -> 0; 1.5*2^-9 between codes 1 and 2 -> 2
    assert F8.e4m3_encode(2.0 ** -10) == 0x00
    assert F8.e4m3_encode(1.5 * 2.0 ** -9) == 0x02
    assert F8.e4m3_encode(7.5 * 2.0 ** -9) == 0x08  # rounds up into the first normal binade
    # 432 is halfway between 416 (m=5) and 448 (m=6): even -> 448
    assert F8.e4m3_encode(432.0) == 0x7E and F8.e4m3_encode(431.9) == 0x7D
    for big in (448.0, 449.0, 480.0, 1e6):
        assert F8.e4m3_encode(big) == 0x7E and F8.e4m3_encode(-big) == 0xFE


def test_e4m3_roundtrip_and_nearest_by_brute_force():
    codes = [c for c in range(256) if c & 0x7F != 0x7F]
    vals = F8.e4m3_decode(codes)
    assert [int(x) for x in F8.e4m3_encode(vals)] == codes  # every finite code decodes and re-encodes
    finite = np.unique(vals[np.isfinite(vals)])
    rng = np.random.default_rng(11)
    xs = np.concatenate([rng.normal(0, 3, 400), rng.uniform(-500, 500, 200), rng.normal(0, 0.01, 200)])
    got = F8.e4m3_decode(F8.e4m3_encode(xs))
    for x, g in zip(xs, got):
        clipped = min(max(x, -448.0), 448.0)
        best = np.min(np.abs(finite - clipped))
        assert abs(g - clipped) == best  # no representable value is closer


def test_e4m3_matches_torch_for_every_bf16_value():
    """An independent implementation: torch's CPU float8_e4m3fn conversion (round to nearest even)
    over every finite bf16 bit pattern, within the saturation range."""
    import torch
    bits = np.arange(65536, dtype=np.uint32) << 16
    x = bits.view(np.float32)
    fin = np.isfinite(x) & (np.abs(x) <= 448.0)
    mine = F8.e4m3_encode(x[fin].astype(np.float64))
    ref = torch.from_numpy(x[fin].copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine, ref)


def test_fp8_pool_scale_is_a_power_of_two():
    x = np.array([0.3, -1.7, 5.0, 1000.0, 2.0 ** -12])
    for s in (1.0, 0.25, 8.0):
        assert np.array_equal(F8.quantize(x, s), F8.e4m3_encode(x / s))
        assert np.array_equal(F8.roundtrip(x, s), F8.e4m3_decode(F8.e4m3_encode(x / s)) * s)
    for bad in (0.0, -1.0, 3.0, 0.1):
        with pytest.raises(ValueError):
            F8.quantize(x, bad)


def test_fp8_roundtrip_table_equals_the_encoder():
    bits = np.arange(65536, dtype=np.uint16)
    vals = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    fin = np.isfinite(vals)
    for s in (1.0, 0.5):
        tab = F8.roundtrip_bf16_bits(bits, s)
        assert np.array_equal(tab[fin], F8.roundtrip(vals[fin], s))


# ------------------------------------------------------------------------------------------ snapshots

def test_snapshot_restores_decode_after_the_donor_moved_on():
    """A copy of the ring taken at length s still decodes position s exactly like attention over
    positions [0, s] after the donor has grown far past s + w (the live ring no longer can)."""
    rng = np.random.default_rng(21)
    w, d, s, L = 8, 4, 37, 90
    ks, vs = rng.normal(size=(L + 1, d)), rng.normal(size=(L + 1, d))
    buf = KC.RollingBuffer(w, d)
    buf.append(ks[:s], vs[:s])
    snap = buf.copy()
    buf.append(ks[s:L], vs[s:L])
    q = rng.normal(size=d)
    got = KC.decode_via_buffer(q, snap, ks[s], vs[s], s, w)
    ref = A.attention(q[None, None, :], ks[:s + 1, None, :], vs[:s + 1, None, :], s, w)[0, 0]
    assert np.allclose(got, ref, rtol=0, atol=1e-12)
    with pytest.raises(KeyError):  # the live ring lost position s - 1
        KC.decode_via_buffer(q, buf, ks[s], vs[s], s, w)


def test_reusable_len_with_snapshots_brute_force_equals_closed_form():
    rng = np.random.default_rng(22)
    for _ in range(300):
        w = int(rng.integers(1, 12))
        donor_len = int(rng.integers(0, 60))
        snaps = sorted(set(int(x) for x in rng.integers(0, donor_len + 1, size=int(rng.integers(0, 4)))))
        match = int(rng.integers(0, 70))
        sources = []
        for length in snaps + [donor_len]:
            b = KC.RollingBuffer(w, 1)
            b.append(np.zeros((length, 1)), np.zeros((length, 1)))
            sources.append((length, [b.tags]))
        assert KC.reusable_len(sources, match, w) == KC.reusable_len_closed(donor_len, snaps, match, w)
    # a snapshot at s serves a longer match at exactly s once the donor is past s + w
    assert KC.reusable_len_closed(100, [40], 70, 8) == 40
    assert KC.window_safe_len_closed(100, 70, 8) == 0


# ---------------------------------------------------------------------------------- RoPE
from oracle import rope as R  # noqa: E402


def test_rope_worked_example_d4():
    """d = 4, base 10000: theta = (1, 1/100).  At position 3 the first pair turns by 3 rad and the
    second by 0.03 rad, counter-clockwise (x + iy times e^(i phi)).  Values are the textbook
    cos/sin of those angles."""
    c3, s3 = -0.9899924966004454, 0.1411200080598672
    c03, s03 = 0.9995500337489875, 0.0299955002024957
    e = np.eye(4)
    got = R.rope(e, [3, 3, 3, 3], 10000.0, "pairs")
    want = np.array([[c3, s3, 0, 0], [-s3, c3, 0, 0], [0, 0, c03, s03], [0, 0, -s03, c03]])
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-15)
    got = R.rope(e, [3, 3, 3, 3], 10000.0, "halves")   # pairs (0, 2) and (1, 3)
    want = np.array([[c3, 0, s3, 0], [0, c03, 0, s03], [-s3, 0, c3, 0], [0, -s03, 0, c03]])
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-15)


def test_rope_is_multiplication_by_a_unit_complex_number():
    """Pair i read as x + iy is multiplied by exp(i p theta_i); theta from numpy.logspace (an
    independent route to base^(-2i/d)).  Positions up to 2^21."""
    g = rng(41)
    for d, base in ((128, 10000.0), (64, 500000.0), (2, 10000.0)):
        x = g.standard_normal((64, 3, d))
        pos = g.integers(0, 1 << 21, 64)
        theta = np.logspace(0.0, -(d - 2) / d * math.log10(base), d // 2)
        z = x[..., 0::2] + 1j * x[..., 1::2]
        zr = z * np.exp(1j * pos[:, None, None] * theta[None, None, :])
        got = R.rope(x, pos, base, "pairs")
        np.testing.assert_allclose(got[..., 0::2], zr.real, rtol=0, atol=1e-8)
        np.testing.assert_allclose(got[..., 1::2], zr.imag, rtol=0, atol=1e-8)


def test_rope_scores_depend_on_relative_position_only():
    """RoFormer §3.4: <R_i q, R_j k> = Re sum_m conj(q_m) k_m e^(i (j - i) theta_m); so shifting both
    positions by the same amount leaves every score unchanged."""
    g = rng(42)
    d = 128
    theta = 10000.0 ** (-np.arange(0, d, 2) / d)
    for _ in range(50):
        q, k = g.standard_normal((2, d))
        i, j = (int(t) for t in g.integers(0, 1 << 20, 2))
        sh = int(g.integers(0, 1 << 20))
        for style in R.STYLES:
            a = R.rope(q[None], [i], style=style)[0] @ R.rope(k[None], [j], style=style)[0]
            b = R.rope(q[None], [i + sh], style=style)[0] @ R.rope(k[None], [j + sh], style=style)[0]
            assert abs(a - b) < 1e-8 * d
        zq = q[0::2] + 1j * q[1::2]
        zk = k[0::2] + 1j * k[1::2]
        closed = np.real(np.sum(np.conj(zq) * zk * np.exp(1j * (j - i) * theta)))
        a = R.rope(q[None], [i])[0] @ R.rope(k[None], [j])[0]
        assert abs(a - closed) < 1e-8 * d


def test_rope_layouts_agree_up_to_a_permutation():
    """Split-halves RoPE is pairs RoPE after moving coordinate i + d/2 next to coordinate i."""
    g = rng(43)
    d = 64
    x = g.standard_normal((16, 2, d))
    pos = g.integers(0, 100000, 16)
    perm = np.stack([np.arange(d // 2), np.arange(d // 2) + d // 2], axis=1).reshape(-1)
    np.testing.assert_allclose(R.rope(x, pos, style="halves")[..., perm], R.rope(x[..., perm], pos, style="pairs"),
                               rtol=0, atol=1e-12)


def test_rope_identity_norm_and_composition():
    g = rng(44)
    x = g.standard_normal((8, 4, 128))
    np.testing.assert_array_equal(R.rope(x, np.zeros(8)), x)
    y = R.rope(x, g.integers(0, 1 << 20, 8))
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    a = g.integers(0, 1 << 19, 8)
    b = g.integers(0, 1 << 19, 8)
    np.testing.assert_allclose(R.rope(R.rope(x, a), b), R.rope(x, a + b), rtol=0, atol=1e-8)


def test_rope_makes_window_attention_shift_invariant():
    """[SWA-theory] §Rolling Buffer KV Cache: with RoPE the ring's slot order is harmless because
    scores see positions, not slots.  Consequence checked here: SWA outputs of a token stream are
    the same when every position is shifted by s (queries whose window is full of the stream)."""
    g = rng(45)
    n, hq, hkv, d, w, s = 40, 4, 2, 32, 8, 12345
    q = g.standard_normal((n, hq, d))
    k = g.standard_normal((n, hkv, d))
    v = g.standard_normal((n, hkv, d))
    pos = np.arange(n)
    o1 = A.attention(R.rope(q, pos), R.rope(k, pos), v, 0, w)
    # the same stream placed after s other tokens (their keys are never in a full window here)
    pad = g.standard_normal((s, hkv, d))
    kk = np.concatenate([pad, R.rope(k, pos + s)])
    vv = np.concatenate([pad, v])
    o2 = A.attention(R.rope(q, pos + s), kk, vv, s, w, rows=range(w - 1, n))
    np.testing.assert_allclose(o2[w - 1:], o1[w - 1:], rtol=0, atol=1e-10)
