"""FP8 (E4M3) storage of K/V entries: encoding, decoding and the per-pool scale.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

[MiMo-review] §おわりに: quantisation reduces the bits of each KV entry and hybrid SWA reduces the
number of entries; the two are orthogonal and stack, i.e. the window-limited cache can itself be
stored in FP8.  The page fixes no format or scaling; the readings taken here:

* format: E4M3 as defined by the OCP 8-bit floating point specification (OFP8): 1 sign bit,
  4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 encodes subnormals m * 2^-9;
  S.1111.111 is NaN and there are no infinities, so the largest finite magnitude is 448;
* encoding: round to nearest, ties to even; magnitudes beyond 448 saturate to +-448;
* scale: one power-of-two scale per pool for K and one for V: a stored code c reads as
  decode(c) * scale and a value x is stored as encode(x / scale).  A power of two makes both
  directions exact apart from the FP8 rounding itself.

Everything here is exact: float64 holds every E4M3 value, every bf16 value, and every quotient by a
power of two in range.
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0
_NAN_CODE = 0x7F


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 code (OFP8): (-1)^s * 2^(e-7) * (1 + m/8) for e > 0, (-1)^s * m * 2^-9
    for e = 0; 0x7F and 0xFF are NaN."""
    c = np.asarray(codes, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    out = s * mag
    return np.where((c & 0x7F) == _NAN_CODE, np.nan, out)


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 code to each value (ties to the even mantissa), saturating at +-448; NaN gives
    0x7F.  The sign of zero is kept (-0.0 -> 0x80)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.uint8)
    flat = x.ravel()
    res = out.ravel()
    for i, v in enumerate(flat):
        if math.isnan(v):
            res[i] = _NAN_CODE
            continue
        sign = 0x80 if math.copysign(1.0, v) < 0 else 0
        a = abs(v)
        if a >= E4M3_MAX:
            res[i] = sign | 0x7E
            continue
        if a == 0.0:
            res[i] = sign
            continue
        # binade of a (log2 can be off by one near powers of two: fix by comparison); the
        # subnormal binade below 2^-6 shares the quantum 2^-9 of the first normal one
        e = math.floor(math.log2(a))
        if 2.0 ** (e + 1) <= a:
            e += 1
        elif 2.0 ** e > a:
            e -= 1
        e = max(e, -6)
        q = 2.0 ** (e - 3)
        n = a / q                      # exact: a has <= 53 bits, q is a power of two
        r = math.floor(n)
        frac = n - r
        if frac > 0.5 or (frac == 0.5 and r % 2 == 1):
            r += 1
        val = r * q                    # the rounded magnitude (can reach 2^(e+1): next binade)
        if val >= 2.0 ** -6:
            ev = math.floor(math.log2(val))
            if 2.0 ** (ev + 1) <= val:
                ev += 1
            elif 2.0 ** ev > val:
                ev -= 1
            m = int(val / 2.0 ** (ev - 3)) - 8
            code = ((ev + 7) << 3) | m
        else:
            code = int(val / 2.0 ** -9)  # subnormal codes 0..7 (8 would be 2^-6 = code 0x08)
        res[i] = sign | min(code, 0x7E)
    return out


def check_scale(scale: float) -> float:
    """A pool scale must be a positive power of two (the reading above)."""
    if not (scale > 0 and math.frexp(scale)[0] == 0.5):
        raise ValueError(f"FP8 pool scale must be a power of two, got {scale}")
    return float(scale)


def quantize(x, scale: float = 1.0) -> np.ndarray:
    """Stored codes of values ``x`` in a pool with this scale: encode(x / scale)."""
    s = check_scale(scale)
    return e4m3_encode(np.asarray(x, dtype=np.float64) / s)


def dequantize(codes, scale: float = 1.0) -> np.ndarray:
    """Values a pool with this scale reads back: decode(code) * scale."""
    return e4m3_decode(codes) * check_scale(scale)


def roundtrip(x, scale: float = 1.0) -> np.ndarray:
    """What attention sees for a committed value x: dequantize(quantize(x))."""
    return dequantize(quantize(x, scale), scale)


_RT_TABLES: dict = {}


def roundtrip_bf16_bits(bits, scale: float = 1.0) -> np.ndarray:
    """roundtrip() of bf16 values given as their 16-bit patterns, by lookup in a table of all 65,536
    patterns built with the encoder and decoder above (for million-row histories)."""
    s = check_scale(scale)
    if s not in _RT_TABLES:
        with np.errstate(invalid="ignore"):  # NaN patterns widen to NaN; they are masked below
            vals = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
        tab = np.full(65536, np.nan)
        fin = np.isfinite(vals)
        tab[fin] = roundtrip(vals[fin], s)
        _RT_TABLES[s] = tab
    return _RT_TABLES[s][np.asarray(bits, dtype=np.uint16).astype(np.int64)]
