"""Index Branch with 4-bit index keys ("Q8KV4"): oracle.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import or call this module.  It shares no
code, tables or helpers with the HIP library, and imports nothing from it.

Source: the dot-ai.myuuu.co.jp article on MiniMax M3.1 Flash, section
"MiniMax M3.1 Flashとは？428BのMoEモデルがウェイト公開" (the model card's
quantisation notes): the indexer runs with 8-bit queries and 8-bit keys and
is moving to 4-bit keys.  The index queries stay as in oracle/fp8_index.py
(readings Q1-Q5); for the keys this module takes the following readings:

F1  the 4-bit format is OCP FP4 E2M1, the element format of the OCP
    microscaling (MX) formats: sign bit, 2 exponent bits (bias 1), 1 mantissa
    bit; exponent field 0 holds the subnormal m * 0.5; magnitudes
    0, 0.5, 1, 1.5, 2, 3, 4, 6; no infinities or NaN.
F2  scales are powers of two stored as E8M0 bytes, one per 32 consecutive
    elements of a key row (the MX block size): with one scale per 128-token
    block, as for the 8-bit keys, the two exponent bits of E2M1 would flush
    most of a block to zero.  A group's exponent e is the smallest integer
    with amax * 2^-e <= 6, clamped to [-127, 127]; an all-zero group gets 0.
F3  codes are round-to-nearest, ties to the even code (mantissa bit 0), of
    x * 2^-e; the sign bit is copied from x.
F4  storage: two codes per byte, element 2i in the low nibble.
F5  the selection is the bf16 path's rule on the dequantised values.
"""
from __future__ import annotations

import numpy as np

E2M1_MAX = 6.0
E8M0_BIAS = 127
GROUP = 32


def e2m1_decode(code):
    """Value of one E2M1 nibble: sign, 2-bit exponent (bias 1), 1-bit mantissa (F1)."""
    code = int(code) & 0xF
    sign = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        return sign * m * 0.5
    return sign * (1.0 + m / 2.0) * 2.0 ** (e - 1)


def e2m1_table():
    """float64 value of each of the 16 codes."""
    return np.array([e2m1_decode(c) for c in range(16)], dtype=np.float64)


_TABLE = e2m1_table()
_POS = _TABLE[:8]              # codes 0 .. 7: the non-negative values, ascending


def e2m1_encode(x):
    """Nearest E2M1 code of each finite |x| <= 6, ties to the even code (F3)."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)) or np.any(np.abs(x) > E2M1_MAX):
        raise ValueError("e2m1_encode: finite values with |x| <= 6 only")
    a = np.abs(x)
    i = np.zeros(a.shape, dtype=np.uint8)       # index of the largest grid value <= a
    for v in _POS[1:]:
        i += a >= v
    j = np.minimum(i + 1, 7).astype(np.uint8)   # the next grid value up (i itself at 6)
    d_lo, d_hi = a - _POS[i], _POS[j] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (j != i) & (j % 2 == 0))
    code = np.where(pick_hi, j, i)
    return code | (np.signbit(x).astype(np.uint8) << 3)


def scale_exponents4(amax):
    """Elementwise: the smallest integer e with amax * 2^-e <= 6, clamped to
    [-127, 127] (F2).

    amax = f * 2^E with f in [0.5, 1): f * 2^3 <= 6 exactly when f <= 0.75,
    so e = E - 3 then, else E - 2 (f * 2^2 < 4).  amax = 0 gives 0.
    """
    a = np.asarray(amax, dtype=np.float64)
    f, E = np.frexp(a)
    e = np.where(f <= 0.75, E - 3, E - 2)
    e = np.where(a == 0.0, 0, e)
    return np.clip(e, -127, 127).astype(np.int64)


def scale_exponent4(amax):
    """scale_exponents4 of one value."""
    return int(scale_exponents4(np.array([float(amax)]))[0])


def quantize_k_idx4(k_idx, group=GROUP):
    """k_idx [total_k, d_idx] -> (codes uint8 [total_k, d_idx] in 0..15,
    E8M0 bytes uint8 [total_k, d_idx / group]); one scale per `group`
    consecutive elements of a key row (F2, F3)."""
    k = np.asarray(k_idx, dtype=np.float64)
    T, D = k.shape
    g = k.reshape(T, D // group, group)
    e = scale_exponents4(np.abs(g).max(axis=2))                  # [T, D / group]
    codes = e2m1_encode(np.ldexp(g, -e[:, :, None])).reshape(T, D)
    return codes, (e + E8M0_BIAS).astype(np.uint8)


def dequantize_k_idx4(codes, ex, group=GROUP):
    """float64 [total_k, d_idx] values of 4-bit index keys."""
    vals = _TABLE[np.asarray(codes, dtype=np.int64)]
    e = np.repeat(np.asarray(ex, dtype=np.int64) - E8M0_BIAS, group, axis=1)
    return np.ldexp(vals, e)


def pack(codes):
    """[rows, d] codes -> [rows, d / 2] bytes, element 2i in the low nibble (F4)."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack(packed):
    """Inverse of pack."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out
