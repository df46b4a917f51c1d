"""GPU parity at full benchmark sizes for the later rows of the path: the
speculative-decoding verification shape (verify8), decode from a paged key
cache, and the KL-alignment target at 128K, each in the launch configuration
bench.py times, on sampled rows the oracle computes one by one."""
import numpy as np
import pytest
import torch

import block_sparse_long_index_amd as msa
from msa_inputs import generate, paged_layout, sample_rows, to_pages, workload
from oracle import kl_target as KL

pytestmark = pytest.mark.gpu

from gpu_helpers import check_out, check_selection, log, problem_from, run_gpu_inputs  # noqa: E402


def _check_rows(name, w, t, P, rows, bufs):
    ref = P.run(rows, want_scores=True)
    ridx = torch.as_tensor(rows, device="cuda:0", dtype=torch.long)
    sel = bufs.sel.index_select(0, ridx).cpu().numpy()
    score = bufs.sel_score.index_select(0, ridx).cpu().numpy()
    bad, ties = check_selection(P, rows, sel, score, ref, w.index_dim)
    log(f"[{name}] selection mismatches {len(bad)} near-ties {ties} of {len(rows) * P.G}")
    assert not bad, bad[:3]
    out = bufs.out.index_select(0, ridx).float().cpu().numpy()
    lse = bufs.lse.index_select(0, ridx).cpu().numpy()
    check_out(out, ref["out"], lse, ref["lse"], name)
    return sel


def test_verify8_sampled():
    w = workload("verify8")
    log(f"[verify8] generating {w.note}")
    t = generate(w, "cuda:0")
    dims, bufs = run_gpu_inputs(w, t)
    assert not msa.attend_reads_lists(dims)
    rows = sample_rows(w, 32)
    log(f"[verify8] forward done; oracle on {len(rows)} rows")
    _check_rows("verify8", w, t, problem_from(t, w, lazy=True), rows, bufs)


def test_paged_decode_full_size():
    # the decode workload's caches scattered into scrambled 128-row pages: every row
    # against the oracle on the contiguous inputs, and bit-equal to the contiguous run
    w = workload("decode")
    log(f"[paged-decode] generating {w.note}")
    t = generate(w, "cuda:0")
    dims_c, bufs_c = run_gpu_inputs(w, t)
    table, rows_k, pages = paged_layout(w, seed=w.seed)
    table_d, rows_d = table.to("cuda:0"), rows_k.to("cuda:0")
    kc, vc, kic = (to_pages(t[n], rows_d, pages) for n in ("k", "v", "k_idx"))
    dims = msa.make_dims(batch=w.batch, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                         head_dim=w.head_dim, index_dim=w.index_dim, top_k=w.top_k,
                         total_q=w.total_q, total_k=pages * 128, max_q_len=max(w.seq_q_lens),
                         max_k_len=max(w.seq_k_lens), block_table=table_d)
    bufs = msa.Buffers(dims, torch.device("cuda:0"), want_scores=True)
    msa.msa_forward(dims, t["q"], kc, vc, t["q_idx"], kic, t["cu_seqlens_q"], t["cu_seqlens_k"], bufs)
    torch.cuda.synchronize()
    log(f"[paged-decode] {pages} pages; oracle on all {w.total_q} rows")
    assert torch.equal(bufs.sel, bufs_c.sel) and torch.equal(bufs.out, bufs_c.out)
    assert torch.equal(bufs.lse, bufs_c.lse)
    _check_rows("paged-decode", w, t, problem_from(t, w, lazy=True), list(range(w.total_q)), bufs)


def test_kl_target_p128k_sampled():
    # the forward with the KL-alignment target as bench.py --kl runs it
    w = workload("p128k")
    log(f"[kl-p128k] generating {w.note}")
    t = generate(w, "cuda:0")
    dims = msa.dims_for(w)
    dev = torch.device("cuda:0")
    bufs = msa.Buffers(dims, dev, want_scores=True, want_lse=True)
    mass = torch.empty((w.total_q, w.num_kv_heads, w.top_k), dtype=torch.float32, device=dev)
    kl = torch.empty((w.total_q, w.num_kv_heads), dtype=torch.float32, device=dev)
    logq = torch.empty((w.total_q, w.num_kv_heads, w.top_k), dtype=torch.float32, device=dev)
    msa.index_select(dims, t["q_idx"], t["k_idx"], t["cu_seqlens_q"], t["cu_seqlens_k"], bufs.sel,
                     bufs.sel_score, bufs.workspace)
    msa.build_block_query_lists(dims, bufs.sel, t["cu_seqlens_q"], t["cu_seqlens_k"], bufs.offsets,
                                bufs.entries, bufs.workspace)
    msa.attend_with_mass(dims, t["q"], t["k"], t["v"], t["cu_seqlens_q"], t["cu_seqlens_k"], bufs.sel,
                         bufs.offsets, bufs.entries, bufs.out, mass, bufs.lse, bufs.workspace)
    msa.index_kl(dims, t["q_idx"], t["k_idx"], t["cu_seqlens_q"], t["cu_seqlens_k"], bufs.sel,
                 bufs.sel_score, mass, kl, logq)
    torch.cuda.synchronize()
    rows = sample_rows(w, 12)
    log(f"[kl-p128k] forward done; oracle on {len(rows)} rows")
    P = problem_from(t, w, lazy=True)
    sel = _check_rows("kl-p128k", w, t, P, rows, bufs)
    ridx = torch.as_tensor(rows, device=dev, dtype=torch.long)
    gm = mass.index_select(0, ridx).cpu().numpy()
    gk = kl.index_select(0, ridx).cpu().numpy()
    gq = logq.index_select(0, ridx).cpu().numpy()
    worst = dict(mass=0.0, logq=0.0, kl=0.0)
    for i, r in enumerate(rows):
        m, lq, kv = KL.row_target(P, r, sel[i])
        # the fp32 accumulation bound of this row's index scores (as in the small-case tests)
        ko, p = int(P.koff[r]), int(P.pos[r])
        sabs = np.abs(P.q_idx[r]) @ np.abs(P.k_idx[ko:ko + p + 1]).T
        eps = w.index_dim * 2.0 ** -23 * sabs.max(axis=1)
        for g in range(P.G):
            n = int((sel[i, g] >= 0).sum())
            dm = np.abs(gm[i, g] - m[g])
            assert np.all(dm <= 1e-5 + 1e-4 * m[g]), (r, g, gm[i, g], m[g])
            assert np.all(gm[i, g, n:] == 0.0)
            dq = np.abs(gq[i, g, :n] - lq[g, :n])
            assert np.all(dq <= 2 * eps[g] + 1e-5), (r, g, dq, eps[g])
            assert np.all(np.isnan(gq[i, g, n:]))
            dk = abs(gk[i, g] - kv[g])
            assert dk <= 2 * eps[g] + 1e-4, (r, g, gk[i, g], kv[g])
            worst["mass"] = max(worst["mass"], float(dm.max()))
            worst["logq"] = max(worst["logq"], float(dq.max()))
            worst["kl"] = max(worst["kl"], dk)
    log(f"[kl-p128k] worst |d| {worst}")
