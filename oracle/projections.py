"""Index projections oracle: the index queries and keys from the layer input.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import or call this module.  It shares no
code, tables or helpers with the HIP library, and imports nothing from it.

Source: the MSA guide (ai-tool-zukan.com/minimax-msa-guide), section
"Index BranchとMain Branchの役割分担": the Index Branch adds just two
projection matrices to a standard GQA layer, one index-query head per GQA
group and one shared index-key head.  The pages give neither the layer width
nor any detail of the projections; readings:

P1  q_idx[t, g, :] = x[t, :] . W_q[g * d_idx:(g + 1) * d_idx, :]^T and
    k_idx[t, :] = x[t, :] . W_k^T: plain linear maps without bias, the weights
    in the usual (out_features, in_features) layout.
P2  the layer width D is a parameter (the workloads use D = Hq * d).
P3  the projections' outputs are bf16 (the Index Branch's input format):
    round to nearest even of the exact product sum.
P4  x holds one row per new token, in query-row order; the token of query row
    r of sequence b sits at position Lk_b - Lq_b + i, so its index key goes to
    key row cu_k[b] + Lk_b - Lq_b + i (prefill fills every key row; decode
    appends each sequence's new keys after its cached ones).
"""
from __future__ import annotations

import numpy as np


def bf16_round(x):
    """Nearest bfloat16 value of each float64 (8 significant bits, the
    exponent range of float32), ties to even, overflow to +-inf; returned as
    float64.  Rounds the float64 value directly (no float32 step, which could
    round twice): |v| = m * 2^e with m in [0.5, 1), so bf16 values near v are
    the multiples of q = 2^(e - 8) (2^-133 below the float32 normal range)."""
    v = np.asarray(x, dtype=np.float64)
    a = np.abs(v)
    _, e = np.frexp(a)
    q = np.ldexp(1.0, np.maximum(e, -125) - 8)
    r = a / q                                   # exact: q is a power of two
    n = np.floor(r)
    frac = r - n
    n = n + ((frac > 0.5) | ((frac == 0.5) & (np.fmod(n, 2.0) == 1.0)))
    y = n * q
    y = np.where(y >= 2.0 ** 128, np.inf, y)
    y = np.copysign(y, v)
    return np.where((a == 0.0) | ~np.isfinite(v), v, y)


def project(x, w_q, w_k, cu_seqlens_q, cu_seqlens_k, total_k, G):
    """(q_idx [T_q, G, d_idx], k_idx rows) for the new tokens x [T_q, D].

    Returns q_idx (float64 holding bf16 values), and a dict {key row: k_idx
    row} for the key rows the new tokens own (reading P4); every other key
    row is left to the caller.
    """
    x = np.asarray(x, dtype=np.float64)
    w_q = np.asarray(w_q, dtype=np.float64)
    w_k = np.asarray(w_k, dtype=np.float64)
    T, D = x.shape
    d_idx = w_k.shape[0]
    assert w_q.shape == (G * d_idx, D) and w_k.shape == (d_idx, D)
    q = bf16_round(x @ w_q.T).reshape(T, G, d_idx)
    k_new = bf16_round(x @ w_k.T)
    cu_q = np.asarray(cu_seqlens_q, dtype=np.int64)
    cu_k = np.asarray(cu_seqlens_k, dtype=np.int64)
    rows = {}
    for b in range(len(cu_q) - 1):
        lq = int(cu_q[b + 1] - cu_q[b])
        lk = int(cu_k[b + 1] - cu_k[b])
        for i in range(lq):
            rows[int(cu_k[b]) + lk - lq + i] = k_new[int(cu_q[b]) + i]
    return q, rows
