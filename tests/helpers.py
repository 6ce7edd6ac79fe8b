"""Shared test plumbing: pools over torch-allocated arenas, tolerance checks, logical K/V history.

The logical history is what the oracle sees: every K/V row by absolute position, kept on the host
exactly as it was handed to the GPU.  The oracle never reads the pool."""
from __future__ import annotations

import numpy as np
import torch

# Parity bars (fp32: max|d| / max|ref| per tensor; bf16: max |d|).
FP32_REL = 1e-5
BF16_ABS = 2e-2


def to64(t) -> np.ndarray:
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().to("cpu", torch.float32).double().numpy()


def assert_close(got, ref, dtype, what=""):
    g, r = to64(got), to64(ref)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.max(np.abs(g - r)) if g.size else 0.0
    if dtype == torch.float32:
        scale = max(np.max(np.abs(r)), 1e-30) if r.size else 1.0
        assert err / scale <= FP32_REL, f"{what}: max|d|/max|ref| = {err / scale:.3e} > {FP32_REL}"
    else:
        assert err <= BF16_ABS, f"{what}: max|d| = {err:.3e} > {BF16_ABS}"
    return err


class GpuPool:
    """A pool over a torch-allocated device arena (the caller owns the arena)."""

    def __init__(self, S, *, n_layers=1, window=32, hkv=1, d=64, dtype=torch.float32, pages=0,
                 max_seqs=4, max_seq_len=4096, layer_is_full=None, k_scale=1.0, v_scale=1.0,
                 max_snapshots=0, rope_base=0.0, rope_style="pairs", decode_plan="uniform", rope_fused=False,
                 max_chunk=0):
        self.S = S
        self.desc = S.make_desc(n_layers, window, hkv, d, dtype, pages, max_seqs, max_seq_len,
                                layer_is_full=layer_is_full, k_scale=k_scale, v_scale=v_scale,
                                max_snapshots=max_snapshots, rope_base=rope_base, rope_style=rope_style,
                                decode_plan=decode_plan, rope_fused=rope_fused, max_chunk=max_chunk)
        nbytes = S.kvpool_arena_bytes(self.desc)
        self.arena = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        self.h = S.kvpool_create(self.desc, self.arena, nbytes)
        self.window, self.hkv, self.d, self.dtype = window, hkv, d, dtype

    def close(self):
        if self.h:
            self.S.kvpool_destroy(self.h)
            self.h = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        torch.cuda.synchronize()
        self.close()


class History:
    """Logical K/V rows of one (sequence, layer) by absolute position, on the host."""

    def __init__(self, hkv, d, dtype):
        self.k = torch.empty((0, hkv, d), dtype=dtype)
        self.v = torch.empty((0, hkv, d), dtype=dtype)

    def extend(self, k, v):
        self.k = torch.cat([self.k, k.detach().cpu()], 0)
        self.v = torch.cat([self.v, v.detach().cpu()], 0)

    def copy(self, upto=None):
        h = History(self.k.shape[1], self.k.shape[2], self.k.dtype)
        h.k, h.v = self.k[:upto].clone(), self.v[:upto].clone()
        return h

    def __len__(self):
        return self.k.shape[0]
