"""GPU parity of the KL-alignment target (msa_attend_with_mass + msa_index_kl)
against the oracle (oracle/kl_target.py).

The selection is first checked against the oracle (as for the plain forward);
the target is then compared on that selection: the Main-Branch masses P, the
index log-probabilities log Q and KL(P || Q) per (query, group).

Tolerances, from the arithmetic: P comes from fp32 exponentials of Main-Branch
scores accumulated in fp32 from bf16 inputs, so its error is a few fp32 units
of the scores (|score| <= a few tens): |dP| <= 1e-5 + 1e-4 P.  log Q and the
local block's score come from fp32 index scores whose accumulation error is
at most d_idx * 2^-23 * sum |q_c k_c| (<= 3e-3 for these inputs, index dot
products of order 100), and log-softmax at most doubles it:
|d log Q| <= 2 * that bound + 1e-5.  KL then moves by at most
max |d log Q| + |dP| terms: checked with the same bound plus 1e-4.
"""
import numpy as np
import pytest
import torch

import block_sparse_long_index_amd as msa
from msa_inputs import custom, generate, workload
from oracle import kl_target as KL

pytestmark = pytest.mark.gpu

from gpu_helpers import check_selection, log, problem_from  # noqa: E402


def _run_kl(w, t):
    dev = torch.device("cuda:0")
    g = {k: v.to(dev) for k, v in t.items()}
    dims = msa.dims_for(w)
    bufs = msa.Buffers(dims, dev, want_scores=True)
    msa.index_select(dims, g["q_idx"], g["k_idx"], g["cu_seqlens_q"], g["cu_seqlens_k"], bufs.sel,
                     bufs.sel_score, bufs.workspace)
    msa.build_block_query_lists(dims, bufs.sel, g["cu_seqlens_q"], g["cu_seqlens_k"], bufs.offsets,
                                bufs.entries, bufs.workspace)
    mass = torch.full((w.total_q, w.num_kv_heads, w.top_k), -1.0, dtype=torch.float32, device=dev)
    msa.attend_with_mass(dims, g["q"], g["k"], g["v"], g["cu_seqlens_q"], g["cu_seqlens_k"], bufs.sel,
                         bufs.offsets, bufs.entries, bufs.out, mass, bufs.lse, bufs.workspace)
    kl = torch.full((w.total_q, w.num_kv_heads), -1.0, dtype=torch.float32, device=dev)
    logq = torch.zeros((w.total_q, w.num_kv_heads, w.top_k), dtype=torch.float32, device=dev)
    msa.index_kl(dims, g["q_idx"], g["k_idx"], g["cu_seqlens_q"], g["cu_seqlens_k"], bufs.sel,
                 bufs.sel_score, mass, kl, logq)
    torch.cuda.synchronize()
    return dims, bufs, mass, kl, logq


def _check(w, tag, rows=None):
    t = generate(w, "cpu")
    dims, bufs, mass, kl, logq = _run_kl(w, t)
    P = problem_from(t, w)
    rows = list(range(w.total_q)) if rows is None else rows
    ref = P.run(rows, want_scores=True)
    sel = bufs.sel.cpu().numpy()[rows]
    bad, ties = check_selection(P, rows, sel, bufs.sel_score.cpu().numpy()[rows], ref, w.index_dim)
    assert not bad, bad[:3]
    gm, gk, gq = mass.cpu().numpy()[rows], kl.cpu().numpy()[rows], logq.cpu().numpy()[rows]
    worst = dict(mass=0.0, logq=0.0, kl=0.0)
    for i, r in enumerate(rows):
        m, lq, kv = KL.row_target(P, r, sel[i])
        # accumulation bound of the index scores of this row
        b, p, ko = int(P.seq[r]), int(P.pos[r]), int(P.koff[r])
        lk = int(P.cu_k[b + 1] - P.cu_k[b])
        sabs = np.abs(P.q_idx[r]) @ np.abs(P.k_idx[ko:ko + p + 1]).T
        eps = w.index_dim * 2.0 ** -23 * sabs.max(axis=1)          # per group
        for gg in range(P.G):
            n = int((sel[i, gg] >= 0).sum())
            dm = np.abs(gm[i, gg] - m[gg])
            assert np.all(dm <= 1e-5 + 1e-4 * m[gg]), (r, gg, gm[i, gg], m[gg])
            assert np.all(gm[i, gg, n:] == 0.0)
            assert abs(gm[i, gg, :n].sum() - 1.0) <= 1e-5
            dq = np.abs(gq[i, gg, :n] - lq[gg, :n])
            assert np.all(dq <= 2 * eps[gg] + 1e-5), (r, gg, dq, eps[gg])
            assert np.all(np.isnan(gq[i, gg, n:]))
            dk = abs(gk[i, gg] - kv[gg])
            assert dk <= 2 * eps[gg] + 1e-4, (r, gg, gk[i, gg], kv[gg])
            worst["mass"] = max(worst["mass"], float(dm.max()))
            worst["logq"] = max(worst["logq"], float(dq.max()))
            worst["kl"] = max(worst["kl"], dk)
    log(f"[{tag}] rows {len(rows)}; near-ties {ties}; worst |d| {worst}")


def test_kl_target_tiny():
    _check(workload("tiny"), "kl-tiny")


def test_kl_target_ragged_gqa():
    w = custom([1500, 900, 130, 3000], [1500, 300, 130, 2000], num_q_heads=16, num_kv_heads=4,
               head_dim=64, index_dim=64, top_k=6, seed=61, qkv_std=1.0)
    _check(w, "kl-ragged", rows=list(range(0, 3930, 7)))


def test_kl_target_decode():
    w = custom([5000, 20000, 128, 300], [1, 1, 1, 1], num_q_heads=16, num_kv_heads=8,
               head_dim=128, index_dim=128, top_k=16, seed=62, qkv_std=1.0)
    _check(w, "kl-decode")


def test_kl_target_dense_selection():
    # top_k covers every block: P is the dense attention mass per block
    w = custom([700], [700], num_q_heads=8, num_kv_heads=2, head_dim=64, index_dim=32, top_k=8,
               seed=63, qkv_std=1.0)
    _check(w, "kl-dense")
