"""Quantised Main Branch oracle: 8-bit queries, keys and values ("Q8KV8").

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import or call this module.  It shares no
code, tables or helpers with the HIP library, and imports nothing from it.

Source: the dot-ai.myuuu.co.jp article on MiniMax M3.1 Flash, section
"MiniMax M3.1 Flashとは？428BのMoEモデルがウェイト公開" (the model card's
quantisation notes): the indexer and the Main Branch both run with 8-bit
queries and 8-bit keys/values.  The format readings of the quantised Index
Branch (oracle/fp8_index.py, Q1, Q2, Q4, Q5: OCP E4M3 codes, E8M0
power-of-two scales chosen as the smallest exponent that fits the largest
magnitude, round to nearest even) carry over; this module adds:

M1  scale granularity: one scale per (query row, query head) of q; one per
    (sequence, 128-token KV block, KV head) of k and of v (the unit the
    selection reads and the Main Branch stages), the neutral byte 127 for
    blocks past a sequence's end.
M2  the Main Branch then computes exactly what the bf16 path computes (softmax
    over the selected blocks' visible keys, shared selection per group) on
    the dequantised q, k and v; the selection itself comes from the Index
    Branch and is not changed by quantising the Main Branch's inputs.
M3  the pages name the storage format only: the arithmetic on the dequantised
    values (and so the tolerance) is that of the bf16 path.
"""
from __future__ import annotations

import numpy as np

from oracle import fp8_index as F

BLOCK = F.BLOCK


def quantize_q(q):
    """q [T, Hq, d] -> (codes uint8 [T, Hq, d], E8M0 bytes uint8 [T, Hq]); one scale per
    (query row, head) (M1)."""
    return F.quantize_q_idx(q)


def dequantize_q(codes, ex):
    """float64 [T, Hq, d] values of quantised queries."""
    return F.dequantize_q_idx(codes, ex)


def quantize_kv(x, cu_seqlens_k, nb_max, block=BLOCK):
    """k or v [total_k, G, d] -> (codes uint8 [total_k, G, d], E8M0 uint8 [batch, nb_max, G]).

    One scale per (sequence, 128-token block, KV head) (M1): block beta of
    sequence b is its rows cu_k[b] + 128*beta .. min(cu_k[b] + 128*(beta+1),
    cu_k[b+1]) - 1, and head g scales those rows' [:, g, :] entries alone.
    """
    x = np.asarray(x, dtype=np.float64)
    cu_k = np.asarray(cu_seqlens_k, dtype=np.int64)
    B, G = len(cu_k) - 1, x.shape[1]
    codes = np.zeros(x.shape, dtype=np.uint8)
    ex = np.full((B, nb_max, G), F.E8M0_BIAS, dtype=np.uint8)
    for b in range(B):
        lo_b, hi_b = int(cu_k[b]), int(cu_k[b + 1])
        for beta in range(nb_max):
            lo = lo_b + beta * block
            hi = min(lo + block, hi_b)
            if lo >= hi:
                continue
            for g in range(G):
                e = F.scale_exponent(np.abs(x[lo:hi, g]).max())
                codes[lo:hi, g] = F.quantize(x[lo:hi, g], e)
                ex[b, beta, g] = e + F.E8M0_BIAS
    return codes, ex


def dequantize_kv(codes, ex, cu_seqlens_k, block=BLOCK):
    """float64 [total_k, G, d] values of quantised keys or values."""
    cu_k = np.asarray(cu_seqlens_k, dtype=np.int64)
    vals = F.e4m3_table()[np.asarray(codes, dtype=np.int64)]
    out = np.empty(vals.shape, dtype=np.float64)
    ex = np.asarray(ex, dtype=np.int64)
    for b in range(len(cu_k) - 1):
        lo, hi = int(cu_k[b]), int(cu_k[b + 1])
        beta = np.arange(hi - lo) // block
        out[lo:hi] = np.ldexp(vals[lo:hi], (ex[b, beta, :] - F.E8M0_BIAS)[:, :, None])
    return out


class DequantizedRows:
    """Rows of a packed k or v cache [total_k, G, d] as they are after 8-bit
    quantisation, computed one (sequence block) at a time on first use: a
    (block, head) unit's codes and scale depend on that block alone (M1), so
    this equals quantize_kv + dequantize_kv on the whole cache.

    ``fetch(lo, hi)`` returns float64 rows lo .. hi-1 of the unquantised
    cache.  Supports the access patterns of the oracle: slices of rows
    (views sharing the cache), and x[rows, g] with an array of rows.
    """

    def __init__(self, fetch, n_rows, row_shape, cu_seqlens_k, lo=0, hi=None, cache=None):
        self.fetch, self.n = fetch, int(n_rows)
        self.row_shape = tuple(row_shape)
        self.cu = np.asarray(cu_seqlens_k, dtype=np.int64)
        self.lo, self.hi = lo, self.n if hi is None else hi
        self.shape = (self.hi - self.lo,) + self.row_shape
        self.cache = {} if cache is None else cache

    def __len__(self):
        return self.hi - self.lo

    def _block(self, b, beta):
        key = (b, beta)
        if key not in self.cache:
            lo = int(self.cu[b]) + BLOCK * beta
            hi = min(lo + BLOCK, int(self.cu[b + 1]))
            cu = np.array([0, hi - lo])
            self.cache[key] = dequantize_kv(*quantize_kv(self.fetch(lo, hi), cu, 1), cu)
        return self.cache[key]

    def __getitem__(self, idx):
        if isinstance(idx, slice):
            a, z, st = idx.indices(len(self))
            assert st == 1
            return DequantizedRows(self.fetch, self.n, self.row_shape, self.cu, self.lo + a,
                                   self.lo + z, self.cache)
        rows, col = idx
        rows = np.asarray(rows, dtype=np.int64) + self.lo
        out = np.empty((len(rows),) + self.row_shape[1:])
        for i, r in enumerate(rows):
            b = int(np.searchsorted(self.cu, r, side="right") - 1)
            j = int(r - self.cu[b])
            out[i] = self._block(b, j // BLOCK)[j % BLOCK, int(col)]
        return out
