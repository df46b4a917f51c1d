"""Quantised Index Branch oracle: FP8 (E4M3) index projections with power-of-two scales.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import or call this module.  It shares no
code, tables or helpers with the HIP library, and imports nothing from it.

Source: the dot-ai.myuuu.co.jp article on MiniMax M3.1 Flash, section
"MiniMax M3.1 Flashとは？428BのMoEモデルがウェイト公開" (its discussion of the
changes from M3 and of the model card's quantisation notes): the sparse
attention's indexer and Main Branch run with 8-bit queries and 8-bit keys
("Q8KV8"), moving to 4-bit keys.  The pages fix neither the 8-bit format nor
the scaling, so this module takes the following readings:

Q1  the 8-bit format is OCP FP8 E4M3 ("e4m3fn": exponent bias 7, 3 mantissa
    bits, no infinities, S.1111.111 is NaN, largest finite value 448), the
    format of the OCP 8-bit floating point specification (OFP8).
Q2  scales are powers of two, stored as E8M0 bytes (biased exponent, 127 means
    2^0), as in the OCP microscaling (MX) formats: dequantised value =
    decode(code) * 2^(byte - 127).  With a power-of-two scale, x * 2^-e is
    exact, so every quantised code is decided by one rounding.
Q3  scale granularity: one scale per (query row, group) of q_idx, one per
    (sequence, 128-token KV block) of k_idx.  A block's scale is a positive
    factor shared by all its keys, so the block max-pool of the scaled scores
    equals the scale times the max-pool of the raw code dot products.
Q4  the exponent e of a row or block is the smallest integer with
    amax * 2^-e <= 448 (amax = largest |x|), clamped to [-127, 127];
    an all-zero row or block gets e = 0.
Q5  codes are round-to-nearest, ties to even, of x * 2^-e.
Q6  the Index Branch then computes exactly what the bf16 path computes (token
    scores, block max-pool, top-k with the forced local block) on the
    dequantised values; the Main Branch is unchanged (bf16 q, k, v).
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0
E8M0_BIAS = 127
BLOCK = 128


# ----------------------------------------------------------------------------
# OCP FP8 E4M3 (reading Q1)
# ----------------------------------------------------------------------------
def e4m3_decode(code):
    """Value of one E4M3 byte: sign bit, 4-bit exponent (bias 7), 3-bit mantissa.

    Exponent field 0 holds the subnormals m/8 * 2^-6; exponent 15 with
    mantissa 7 is NaN (no infinities); everything else is (1 + m/8) * 2^(e-7).
    """
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 15 and m == 7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e4m3_table():
    """float64 value of each of the 256 codes (NaN for the two NaN codes)."""
    return np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)


_TABLE = e4m3_table()
_POS = _TABLE[:127]            # codes 0 .. 126: the non-negative finite values, ascending


def e4m3_encode(x):
    """Nearest E4M3 code of each finite |x| <= 448, ties to the even code (Q5).

    Works on the magnitude against the ascending table of the 127
    non-negative finite values and copies the sign bit of x (so -0.0 and
    negatives that round to zero give 0x80).
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)) or np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("e4m3_encode: finite values with |x| <= 448 only")
    a = np.abs(x)
    i = np.searchsorted(_POS, a, side="right") - 1          # _POS[i] <= a < _POS[i+1]
    i = np.clip(i, 0, 126)
    j = np.minimum(i + 1, 126)
    lo, hi = _POS[i], _POS[j]
    d_lo, d_hi = a - lo, hi - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (j != i) & (j % 2 == 0))
    code = np.where(pick_hi, j, i).astype(np.uint8)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


# ----------------------------------------------------------------------------
# power-of-two scales (readings Q2, Q4)
# ----------------------------------------------------------------------------
def scale_exponent(amax):
    """Smallest integer e with amax * 2^-e <= 448, clamped to [-127, 127] (Q4).

    With amax = f * 2^E, f in [0.5, 1): f * 2^9 <= 448 exactly when
    f <= 0.875, so e = E - 9 then, else E - 8 (f * 2^8 < 256 <= 448 and
    f * 2^9 > 448).  amax = 0 gives 0.
    """
    amax = float(amax)
    if amax == 0.0:
        return 0
    f, E = math.frexp(amax)
    e = E - 9 if f <= 0.875 else E - 8
    return max(-127, min(127, e))


def quantize(x, e):
    """Codes of x at exponent e: e4m3_encode(x * 2^-e) (Q2, Q5)."""
    return e4m3_encode(np.ldexp(np.asarray(x, dtype=np.float64), -int(e)))


def dequantize(codes, e):
    """decode(code) * 2^e in float64 (exact)."""
    return np.ldexp(_TABLE[np.asarray(codes, dtype=np.int64)], int(e))


# ----------------------------------------------------------------------------
# the index projections (reading Q3)
# ----------------------------------------------------------------------------
def quantize_q_idx(q_idx):
    """q_idx [T, G, d_idx] -> (codes uint8 [T, G, d_idx], E8M0 bytes uint8 [T, G]).

    One scale per (query row, group).
    """
    q = np.asarray(q_idx, dtype=np.float64)
    T, G, _ = q.shape
    codes = np.zeros(q.shape, dtype=np.uint8)
    ex = np.zeros((T, G), dtype=np.uint8)
    for t in range(T):
        for g in range(G):
            e = scale_exponent(np.abs(q[t, g]).max())
            codes[t, g] = quantize(q[t, g], e)
            ex[t, g] = e + E8M0_BIAS
    return codes, ex


def quantize_k_idx(k_idx, cu_seqlens_k, nb_max, block=BLOCK):
    """k_idx [total_k, d_idx] -> (codes uint8 [total_k, d_idx], E8M0 uint8 [batch, nb_max]).

    One scale per (sequence, 128-token block): block beta of sequence b is
    its key rows cu_k[b] + 128*beta .. min(cu_k[b] + 128*(beta+1), cu_k[b+1]) - 1.
    Blocks past a sequence's end get the neutral byte 127 (2^0).
    """
    k = np.asarray(k_idx, dtype=np.float64)
    cu_k = np.asarray(cu_seqlens_k, dtype=np.int64)
    B = len(cu_k) - 1
    codes = np.zeros(k.shape, dtype=np.uint8)
    ex = np.full((B, nb_max), E8M0_BIAS, dtype=np.uint8)
    for b in range(B):
        lo_b, hi_b = int(cu_k[b]), int(cu_k[b + 1])
        for beta in range(nb_max):
            lo = lo_b + beta * block
            hi = min(lo + block, hi_b)
            if lo >= hi:
                continue
            e = scale_exponent(np.abs(k[lo:hi]).max())
            codes[lo:hi] = quantize(k[lo:hi], e)
            ex[b, beta] = e + E8M0_BIAS
    return codes, ex


def dequantize_q_idx(codes, ex):
    """float64 [T, G, d_idx] values of quantised index queries."""
    vals = _TABLE[np.asarray(codes, dtype=np.int64)]
    return np.ldexp(vals, (np.asarray(ex, dtype=np.int64) - E8M0_BIAS)[..., None])


def dequantize_k_idx(codes, ex, cu_seqlens_k, block=BLOCK):
    """float64 [total_k, d_idx] values of quantised index keys."""
    cu_k = np.asarray(cu_seqlens_k, dtype=np.int64)
    vals = _TABLE[np.asarray(codes, dtype=np.int64)]
    out = np.empty(vals.shape, dtype=np.float64)
    ex = np.asarray(ex, dtype=np.int64)
    for b in range(len(cu_k) - 1):
        lo, hi = int(cu_k[b]), int(cu_k[b + 1])
        beta = np.arange(hi - lo) // block                 # block of each key of sequence b
        out[lo:hi] = np.ldexp(vals[lo:hi], (ex[b, beta] - E8M0_BIAS)[:, None])
    return out
