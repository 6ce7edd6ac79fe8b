"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module holds no attention arithmetic: it only draws i.i.d. N(0, 1) tensors (the value
distribution of every workload here) from torch's generators, keyed by a tuple such as
(seed, "q", layer, chunk).  Both the oracle side and the HIP side receive the tensors it
returns; neither side computes its inputs itself.

Determinism: the same key, shape, dtype and device give the same values.  torch's CPU and GPU
generators are different algorithms, so a tensor drawn on the GPU differs from one drawn on the
CPU with the same key; a test that needs host copies of device-drawn data copies them.

Long logical token streams (the 1M-token prefix, the 64K-token decode contexts) are cut into
fixed blocks of ``BLOCK`` tokens, each keyed by its block index, so that any position range can be
drawn again later without holding the whole stream (the oracle's sampled checks do this).
"""
from __future__ import annotations

import hashlib

import torch

BLOCK = 4096


def seed_of(*parts) -> int:
    """63-bit seed from a tuple of ints/strings (stable across processes and machines)."""
    h = hashlib.blake2b(repr(parts).encode(), digest_size=8).digest()
    return int.from_bytes(h, "little") & ((1 << 63) - 1)


def normal(shape, *key, dtype=torch.float32, device="cpu") -> torch.Tensor:
    """i.i.d. N(0, 1) of ``shape`` drawn in float32 and rounded (RNE) to ``dtype``."""
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(*key))
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32, device=device)
    return x.to(dtype)


class TokenStream:
    """K or V rows of one logical token stream: row p is the [n_heads, d] tensor of position p.

    ``key`` names the stream, e.g. (seed, "k", layer, stream_id).  Rows are drawn block by block
    (``BLOCK`` positions per draw), so ``rows(a, b)`` is identical however the range is split.
    """

    def __init__(self, key, n_heads: int, d: int, dtype=torch.bfloat16, device="cpu"):
        self.key = tuple(key)
        self.n_heads, self.d, self.dtype, self.device = n_heads, d, dtype, device

    def block(self, b: int) -> torch.Tensor:
        return normal((BLOCK, self.n_heads, self.d), *self.key, "block", b,
                      dtype=self.dtype, device=self.device)

    def rows(self, start: int, stop: int) -> torch.Tensor:
        if stop <= start:
            return torch.empty((0, self.n_heads, self.d), dtype=self.dtype, device=self.device)
        parts = []
        b0, b1 = start // BLOCK, (stop - 1) // BLOCK
        for b in range(b0, b1 + 1):
            blk = self.block(b)
            lo = max(start, b * BLOCK) - b * BLOCK
            hi = min(stop, (b + 1) * BLOCK) - b * BLOCK
            parts.append(blk[lo:hi])
        return torch.cat(parts, 0) if len(parts) > 1 else parts[0].contiguous()
