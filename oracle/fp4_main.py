"""Main Branch with 4-bit keys and values ("Q8KV4"): oracle.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import or call this module.  It shares no
code, tables or helpers with the HIP library, and imports nothing from it.

Source: the dot-ai.myuuu.co.jp article on MiniMax M3.1 Flash, section
"MiniMax M3.1 Flashとは？428BのMoEモデルがウェイト公開" (the model card's
quantisation notes): the sparse-attention indexer and Main Branch move from
8-bit queries and keys/values to 8-bit queries and 4-bit keys/values.  The
8-bit queries are those of the 8-bit Main Branch (oracle/fp8_main.py, M1: one
E4M3 scale per (query row, head)); this module takes, for k and v:

M4  the 4-bit format of the 4-bit index keys (oracle/fp4_index.py, F1-F3):
    E2M1 codes with one E8M0 exponent per 32 consecutive elements, applied to
    every (key, KV head) row of d elements; the Main Branch then computes the
    bf16 path on the dequantised q, k and v (M2, M3).
"""
from __future__ import annotations

import numpy as np

from oracle import fp4_index as F4


def quantize_kv4(x):
    """k or v [total_k, G, d] -> (codes uint8 [total_k, G, d] in 0..15,
    E8M0 uint8 [total_k, G, d / 32]); each (key, head) row scaled per 32
    elements (M4)."""
    x = np.asarray(x, dtype=np.float64)
    T, G, d = x.shape
    codes, ex = F4.quantize_k_idx4(x.reshape(T * G, d))
    return codes.reshape(T, G, d), ex.reshape(T, G, d // F4.GROUP)


def dequantize_kv4(codes, ex):
    """float64 [total_k, G, d] values of 4-bit keys or values."""
    codes = np.asarray(codes)
    T, G, d = codes.shape
    return F4.dequantize_k_idx4(codes.reshape(T * G, d),
                                np.asarray(ex).reshape(T * G, d // F4.GROUP)).reshape(T, G, d)


class DequantizedRows4:
    """Rows of a k or v cache [total_k, G, d] as they are after 4-bit
    quantisation, computed a slice at a time on first use (every (key, head)
    row is scaled on its own, so any slice quantises as the whole cache does).

    ``fetch(lo, hi)`` returns float64 rows lo .. hi-1 of the unquantised
    cache.  Supports the oracle's access patterns: row slices (views sharing
    the cache) and x[rows, g] with an array of rows.
    """

    def __init__(self, fetch, n_rows, row_shape, lo=0, hi=None, cache=None):
        self.fetch, self.n = fetch, int(n_rows)
        self.row_shape = tuple(row_shape)
        self.lo, self.hi = lo, self.n if hi is None else hi
        self.shape = (self.hi - self.lo,) + self.row_shape
        self.cache = {} if cache is None else cache

    def __len__(self):
        return self.hi - self.lo

    _CHUNK = 128   # rows quantised together (any split gives the same values)

    def _chunk(self, c):
        if c not in self.cache:
            lo = c * self._CHUNK
            hi = min(lo + self._CHUNK, self.n)
            self.cache[c] = dequantize_kv4(*quantize_kv4(self.fetch(lo, hi)))
        return self.cache[c]

    def __getitem__(self, idx):
        if isinstance(idx, slice):
            a, z, st = idx.indices(len(self))
            assert st == 1
            return DequantizedRows4(self.fetch, self.n, self.row_shape, self.lo + a, self.lo + z,
                                    self.cache)
        rows, col = idx
        rows = np.asarray(rows, dtype=np.int64) + self.lo
        out = np.empty((len(rows),) + self.row_shape[1:])
        chunk = rows // self._CHUNK
        for c in np.unique(chunk):
            sel = chunk == c
            out[sel] = self._chunk(int(c))[rows[sel] % self._CHUNK, int(col)]
        return out
