"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare it with the CPU oracle on the same seeded inputs."""
from __future__ import annotations

import numpy as np
import torch

import block_sparse_long_index_amd as msa
from oracle import msa_oracle as O

# the benchmark spec tolerances for bf16 I/O with fp32 accumulation
MAX_ABS = 2e-2
MEAN_ABS = 2e-3
REL_L2 = 1e-2
REL_MAX = 2e-2
LSE_ABS = 2e-3


def log(msg):
    print(msg, flush=True)


class LazyRows:
    """Row-sliceable view of a device tensor for the oracle: only the rows and
    columns the oracle indexes are copied to the host (as float64)."""

    def __init__(self, t, lo=0, hi=None):
        self.t, self.lo = t, lo
        self.hi = t.shape[0] if hi is None else hi
        self.shape = (self.hi - self.lo,) + tuple(t.shape[1:])

    def __len__(self):
        return self.hi - self.lo

    def __getitem__(self, idx):
        if isinstance(idx, slice):
            a, b, st = idx.indices(len(self))
            assert st == 1
            return LazyRows(self.t, self.lo + a, self.lo + b)
        if isinstance(idx, tuple):
            rows, rest = idx[0], idx[1:]
        else:
            rows, rest = idx, ()
        scalar_row = isinstance(rows, (int, np.integer))
        if scalar_row:
            x = self.t[self.lo + int(rows)]
        else:
            r = torch.as_tensor(np.asarray(rows, dtype=np.int64) + self.lo, device=self.t.device)
            x = self.t.index_select(0, r)
        assert len(rest) <= 1
        if rest:
            x = x[int(rest[0])] if scalar_row else x[:, int(rest[0])]
        return x.double().cpu().numpy()


def problem_from(t, w, lazy=False):
    """Oracle problem on the inputs t (any device)."""
    if lazy:
        q, k, v, qi = (LazyRows(t[n]) for n in ("q", "k", "v", "q_idx"))
        ki = t["k_idx"].float().cpu().numpy()
    else:
        f = lambda x: x.double().cpu().numpy()
        q, k, v, qi, ki = f(t["q"]), f(t["k"]), f(t["v"]), f(t["q_idx"]), f(t["k_idx"])
    return O.Problem(q, k, v, qi, ki, t["cu_seqlens_q"].cpu().numpy(),
                     t["cu_seqlens_k"].cpu().numpy(), w.top_k)


def run_gpu(w, t, q_chunk=0, want_scores=True, workspace_fill=None, flags=0):
    dev = torch.device("cuda:0")
    g = {k: v.to(dev) for k, v in t.items()}
    dims = msa.dims_for(w, q_chunk=q_chunk, flags=flags)
    bufs = msa.Buffers(dims, dev, want_scores=want_scores)
    if workspace_fill is not None:
        bufs.workspace.fill_(workspace_fill)
    msa.msa_forward(dims, g["q"], g["k"], g["v"], g["q_idx"], g["k_idx"], g["cu_seqlens_q"],
                    g["cu_seqlens_k"], bufs)
    torch.cuda.synchronize()
    return dims, bufs, g


def check_selection(P, rows, gpu_sel, gpu_score=None, ref=None, d_idx=None):
    """Selections must equal the oracle's except on near-ties, where the GPU's
    choice must still be a valid top-(k-1).  Returns (mismatches, near_ties)."""
    ref = ref if ref is not None else P.run(rows, want_scores=True)
    bad, ties = [], 0
    for i, r in enumerate(rows):
        beta_p = int(P.pos[r]) // P.block
        for g in range(P.G):
            S = ref["S"][i][g]
            tie = O.near_tie(S, beta_p, P.top_k)
            ties += int(tie)
            if not np.array_equal(gpu_sel[i, g], ref["sel"][i, g]):
                if not (tie and O.valid_selection(S, beta_p, P.top_k, gpu_sel[i, g])):
                    bad.append((r, g, list(gpu_sel[i, g]), list(ref["sel"][i, g])))
            if gpu_score is not None and np.array_equal(gpu_sel[i, g], ref["sel"][i, g]):
                sc = gpu_score[i, g]
                rs = ref["sel_score"][i, g]
                n = int((ref["sel"][i, g] >= 0).sum())
                assert np.isinf(sc[n - 1]) and sc[n - 1] > 0
                assert np.all(np.isnan(sc[n:]))
                if n > 1:
                    tol = (d_idx or 128) * 2.0 ** -23 * (np.abs(rs[:n - 1]) + 1.0) * 8
                    assert np.all(np.abs(sc[:n - 1] - rs[:n - 1]) <= tol), (r, g, sc, rs)
    return bad, ties


def check_out(gpu_out, ref_out, gpu_lse=None, ref_lse=None, what=""):
    d = np.abs(gpu_out - ref_out)
    mx, mean = float(d.max()), float(d.mean())
    rel2 = float(np.linalg.norm(d) / max(np.linalg.norm(ref_out), 1e-30))
    relmax = float(d.max() / max(np.abs(ref_out).max(), 1e-30))
    log(f"{what}: max|d| {mx:.3e} mean|d| {mean:.3e} relL2 {rel2:.3e} relmax {relmax:.3e}")
    assert mx <= MAX_ABS and mean <= MEAN_ABS, (mx, mean)
    assert rel2 <= REL_L2 and relmax <= REL_MAX, (rel2, relmax)
    if gpu_lse is not None:
        dl = float(np.abs(gpu_lse - ref_lse).max())
        log(f"{what}: max|d lse| {dl:.3e}")
        assert dl <= LSE_ABS


def run_gpu_inputs(w, t, q_chunk=0, want_scores=True, flags=0):
    """Forward on inputs already on the GPU (full-size workloads)."""
    dims = msa.dims_for(w, q_chunk=q_chunk, flags=flags)
    bufs = msa.Buffers(dims, t["q"].device, want_scores=want_scores)
    msa.msa_forward(dims, t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"], t["cu_seqlens_q"],
                    t["cu_seqlens_k"], bufs)
    torch.cuda.synchronize()
    return dims, bufs
