"""Number formats used by the DSA caches: OCP E4M3 (FN variant), E8M0, bf16.

Test infrastructure only (see package docstring).

The pages ask for MXFP8 on the indexer ("Full MXFP8 Quantization with
Per-Group Dynamic Scaling for LI", page 3) and FP8 for the KV cache ("FP8
KVCache with Per-Token-Head-Tile Quantization for SFA", page 3) but do not
define the bit formats.  The definitions used here are the public OCP ones:
  * E4M3 ("OCP 8-bit Floating Point Specification (OFP8)", E4M3 column):
    1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities; S.1111.111
    is NaN; largest finite 448; smallest subnormal 2^-9.
  * E8M0 ("OCP Microscaling Formats (MX) v1.0", scale format): an unsigned
    biased exponent, value 2^(E-127), 0xFF is NaN.
Rounding into E4M3 is round-to-nearest, ties to even mantissa, saturating to
+-448 (satfinite); the sign is kept, so a negative value that rounds to zero
encodes as 0x80.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def _decode_e4m3_code(b: int) -> float:
    """Value of one E4M3 code straight from the bit-field definition."""
    s = (b >> 7) & 1
    e = (b >> 3) & 0xF
    m = b & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        mag = (m / 8.0) * 2.0 ** (-6)          # subnormal
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)  # normal
    return -mag if s else mag


E4M3_TABLE = np.array([_decode_e4m3_code(b) for b in range(256)], dtype=np.float64)
# non-negative finite values in code order 0x00..0x7E (strictly increasing)
E4M3_POS = E4M3_TABLE[:0x7F].copy()


def e4m3_decode(codes) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e8m0_decode(e) -> np.ndarray:
    e = np.asarray(e, dtype=np.int64)
    out = np.ldexp(1.0, e - 127)
    return np.where(e == 255, np.nan, out)


def bf16_decode(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exact."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def e4m3_encode_nearest(y) -> np.ndarray:
    """Reference encoder by exhaustive search: the finite E4M3 value nearest
    to |y|; on an exact tie the code with an even mantissa (even code) wins;
    |y| > 448 saturates to 448; the sign bit of y is kept.

    Slow (254-way search per element); used to pin `e4m3_encode`."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y).reshape(-1)
    d = np.abs(a[:, None] - E4M3_POS[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best                          # one or two candidates
    codes = np.arange(0x7F)
    even = cand & ((codes[None, :] & 1) == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    pick = np.where(a > E4M3_MAX, 0x7E, pick)
    out = pick.astype(np.uint8) | (np.signbit(y).reshape(-1).astype(np.uint8) << 7)
    return out.reshape(y.shape)


def e4m3_encode(y) -> np.ndarray:
    """Round-to-nearest-even, saturating E4M3 encoder (vectorised).

    |y| is rounded on the E4M3 grid of its binade: the grid step is
    2^(floor(log2|y|) - 3) for |y| >= 2^-6 and 2^-9 below (subnormals).
    Division by a power of two is exact in fp64 and np.rint rounds half to
    even, so this is the nearest-even rule of the format; results above 448
    are clamped to 448.  Pinned against `e4m3_encode_nearest`."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    _, ex = np.frexp(a)                       # a = m * 2^ex, m in [0.5, 1)
    binade = np.where(a > 0, ex - 1, -6)
    step = np.ldexp(1.0, np.maximum(binade, -6) - 3)
    r = np.minimum(np.rint(a / step) * step, E4M3_MAX)
    code = np.searchsorted(E4M3_POS, r).astype(np.uint8)
    return code | (np.signbit(y).astype(np.uint8) << 7)


def e4m3_half_ulp(mag) -> np.ndarray:
    """Half the E4M3 grid spacing at magnitude `mag` (<= 448)."""
    mag = np.asarray(mag, dtype=np.float64)
    _, ex = np.frexp(mag)
    binade = np.where(mag > 0, ex - 1, -6)
    return np.ldexp(0.5, np.maximum(binade, -6) - 3)
