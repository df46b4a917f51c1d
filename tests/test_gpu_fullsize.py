"""GPU parity at the benchmark workloads' full sizes, in the launch
configuration bench.py times (default query chunking), on sampled rows the
oracle computes one by one.  Inputs are generated on the GPU with the seeded
recipe; the oracle reads only the rows and blocks it needs."""
import numpy as np
import pytest
import torch

import block_sparse_long_index_amd as msa
from msa_inputs import generate, sample_rows, workload

pytestmark = pytest.mark.gpu

from gpu_helpers import check_out, check_selection, log, problem_from, run_gpu_inputs  # noqa: E402


def _sampled(name, n_random, max_rows=None, flags=0, pass_edges=False):
    w = workload(name)
    log(f"[{name}] generating {w.note}")
    t = generate(w, "cuda:0")
    dims, bufs = run_gpu_inputs(w, t, flags=flags)
    rows = sample_rows(w, n_random)
    if max_rows:
        rows = rows[:max_rows]
    if pass_edges:
        # the first and last rows of every attend pass
        step = msa.attend_pass_rows(dims)
        edges = [r for a in range(step, w.total_q, step) for r in (a - 1, a)]
        log(f"[{name}] attend passes of {step} rows; edge rows {edges}")
        rows = sorted(set(rows) | set(edges))
    log(f"[{name}] forward done; oracle on {len(rows)} rows")
    P = problem_from(t, w, lazy=True)
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
    return w, t, bufs


def test_p32k_sampled():
    _sampled("p32k", 48)


def test_p32k_peaky_sampled():
    _sampled("p32k_peaky", 24)


def test_p128k_sampled():
    _sampled("p128k", 24)


def test_decode_batch_all_rows():
    w, t, bufs = _sampled("decode", 0)
    assert len(sample_rows(w, 0)) == w.total_q


def test_p1m_sampled():
    # 64 random rows (top-k over up to 8191 earlier blocks), the first two
    # blocks' ends, the last block, and both sides of every attend pass boundary
    _sampled("p1m", 64, pass_edges=True)


def test_p128k_compact_partials_sampled():
    _sampled("p128k", 24, flags=msa.FLAG_COMPACT_PARTIALS, pass_edges=True)


def test_p32k_peaky_compact_partials_sampled():
    _sampled("p32k_peaky", 24, flags=msa.FLAG_COMPACT_PARTIALS)
