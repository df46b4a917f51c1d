#!/usr/bin/env python3
"""MSA hot-path benchmark on one MI355X.

One step = the whole hot path on one batch of synthetic input already in HBM:
msa_index_select -> msa_build_block_query_lists -> msa_attend, through the C
ABI on one stream.  Prints ONE JSON line on stdout; progress goes to stderr.

    python bench.py [--steps K] [--warmup W] [--workload p128k|p1m|p32k|decode|verify8|tiny]
                    [--index bf16|fp8|q8k4]

The default workload is the 128K-token single-layer prefill (64 query heads /
8 KV heads, head dim 128, index dim 128, top-k 16 incl. the local block).
After the timed region the oracle runs on a bounded random sample of query
rows on the host cores: its rate is the cpu_baseline, and the same rows gate
parity (selection bit-exact except near-ties; output within tolerance).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MSA prefill tokens/s + Main-Branch MFMA % at 128K/1M; decode HBM GB/s"
PEAK_BF16_FLOPS = 2.5e15      # MI355X dense bf16 MFMA
PEAK_FP8_FLOPS = 5.0e15       # MI355X dense fp8 MFMA
FP8_DOT_REL = 2.0 ** -10      # fp8 matrix-core dot product error bound, relative to sum |q_c k_c|
PEAK_HBM_BYTES = 8.0e12       # MI355X HBM3E
BLOCK = 128


def _decode_like(w):
    """Decode and speculative-verification steps: a few new tokens per sequence."""
    return w.name == "decode" or w.name.startswith("verify")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# algorithmic work model (what the method must touch, not what a kernel does)
# ---------------------------------------------------------------------------
def work_model(w) -> dict:
    """FLOPs and bytes per step implied by the method for workload w."""
    G, Hq, d, di, k = w.num_kv_heads, w.num_q_heads, w.head_dim, w.index_dim, w.top_k
    hpg = Hq // G
    idx_flops = main_flops = 0.0
    sel_total = 0.0            # sum over (row, group) of |Sel|
    scored_keys = 0.0          # sum over rows of 128 * beta(p)  (non-local keys)
    kv_blocks = 0.0            # (sequence, group, block) items read once
    dec_kidx_tokens = 0.0
    for lq, lk in zip(w.seq_q_lens, w.seq_k_lens):
        if lq == 0:
            continue
        p = np.arange(lk - lq, lk, dtype=np.int64)
        beta = p // BLOCK
        nsel = np.minimum(k, beta + 1)
        J = BLOCK * (nsel - 1) + (p % BLOCK) + 1
        idx_flops += float(G * 2 * di * BLOCK * beta.sum())
        main_flops += float(Hq * 4 * d * J.sum())
        sel_total += float(G * nsel.sum())
        scored_keys += float(BLOCK * beta.sum())
        kv_blocks += float(G * min((lk + BLOCK - 1) // BLOCK, int(nsel.sum())))
        dec_kidx_tokens += float(BLOCK * beta.max())
    T = w.total_q
    q_gather = sel_total * hpg * d * 2
    part_write = sel_total * hpg * (d * 4 + 8)
    kv_once = kv_blocks * BLOCK * d * 2 * 2
    attend_bytes = q_gather + part_write + kv_once
    merge_bytes = sel_total * hpg * (d * 4 + 8) + T * Hq * (d * 2 + 4)
    # compact partials (prefill-shaped steps): fp16 values + (w, E) per row
    part_compact = sel_total * hpg * (d * 2 + 8)
    attend_bytes_compact = q_gather + part_compact + kv_once
    merge_bytes_compact = part_compact + T * Hq * (d * 2 + 4)
    topk_bytes = scored_keys * G * 4 / BLOCK + T * G * k * 4
    # decode-shaped steps: index keys of every sequence's earlier blocks, read once for all
    # groups and new tokens, plus each selected (group, block) of K/V once, Q, index queries, O
    decode_bytes = (dec_kidx_tokens * di * 2 + kv_once
                    + T * (Hq * d * 2 * 2 + G * di * 2))
    # fp8 index branch: quantisation reads the bf16 projections and writes codes + exponents;
    # the decode scan then reads one byte per index-key element
    nblk = sum((lk + BLOCK - 1) // BLOCK for lk in w.seq_k_lens)
    quant_bytes = (T * G * di + w.total_k * di) * 3 + T * G + nblk
    if _decode_like(w):         # a decode step quantises only its new index queries
        quant_bytes = T * G * di * 3 + T * G
    decode_fp8_bytes = (dec_kidx_tokens * di + kv_once
                        + T * (Hq * d * 2 * 2 + G * (di + 1)))
    index_decode_fp8_bytes = dec_kidx_tokens * di + T * G * (di + 1)
    index_decode_bytes = dec_kidx_tokens * di * 2 + T * G * di * 2
    # 4-bit index keys: di / 2 code bytes + di / 32 exponent bytes per key
    k4_row = di / 2 + di / 32
    quant_q8k4_bytes = T * G * (di * 3 + 1) + w.total_k * (di * 2 + k4_row)
    if _decode_like(w):
        quant_q8k4_bytes = T * G * (di * 3 + 1)
    index_decode_q8k4_bytes = dec_kidx_tokens * k4_row + T * G * (di + 1)
    decode_q8k4_bytes = (dec_kidx_tokens * k4_row + kv_once
                         + T * (Hq * d * 2 * 2 + G * (di + 1)))
    # 8-bit Main Branch: one byte per q / k / v element (+ one exponent per (row, head) and
    # per (block, KV head)); the fp32 partials are unchanged
    kv_once_fp8 = kv_blocks * (BLOCK * d + 1) * 2
    attend_bytes_fp8 = sel_total * hpg * (d + 1) + part_write + kv_once_fp8
    main_quant_bytes = (T * Hq * d + 2 * w.total_k * G * d) * 3 + T * Hq + 2 * nblk * G
    if _decode_like(w):         # a decode step quantises only its new queries
        main_quant_bytes = T * Hq * d * 3 + T * Hq
    decode_kv_fp8_delta = kv_once_fp8 - kv_once + T * Hq * (d + 1 - 2 * d)
    # 8-bit q with 4-bit k and v: d / 2 code bytes + d / 32 exponent bytes per (key, head) row
    kv4_row = d / 2 + d / 32
    kv_once_kv4 = kv_blocks * BLOCK * kv4_row * 2
    attend_bytes_kv4 = sel_total * hpg * (d + 1) + part_write + kv_once_kv4
    main_quant_kv4_bytes = T * Hq * (d * 3 + 1) + 2 * w.total_k * G * (d * 2 + kv4_row)
    if _decode_like(w):
        main_quant_kv4_bytes = T * Hq * (d * 3 + 1)
    decode_kv4_delta = kv_once_kv4 - kv_once + T * Hq * (d + 1 - 2 * d)
    return dict(index_flops=idx_flops, main_flops=main_flops, sel_total=sel_total,
                attend_bytes_fp8=attend_bytes_fp8, main_quant_bytes=main_quant_bytes,
                decode_kv_fp8_delta=decode_kv_fp8_delta, attend_bytes_kv4=attend_bytes_kv4,
                main_quant_kv4_bytes=main_quant_kv4_bytes, decode_kv4_delta=decode_kv4_delta,
                attend_bytes=attend_bytes, merge_bytes=merge_bytes, topk_bytes=topk_bytes,
                attend_bytes_compact=attend_bytes_compact, merge_bytes_compact=merge_bytes_compact,
                decode_bytes=decode_bytes, kv_once_bytes=kv_once, quant_bytes=quant_bytes,
                decode_fp8_bytes=decode_fp8_bytes, index_decode_fp8_bytes=index_decode_fp8_bytes,
                index_decode_bytes=index_decode_bytes, quant_q8k4_bytes=quant_q8k4_bytes,
                index_decode_q8k4_bytes=index_decode_q8k4_bytes, decode_q8k4_bytes=decode_q8k4_bytes)


# ---------------------------------------------------------------------------
# oracle on sampled rows (host cores)
# ---------------------------------------------------------------------------
class _RowSubset:
    """Rows of a larger array, addressable by their global row index."""

    def __init__(self, rows, data):
        self.index = {int(r): i for i, r in enumerate(rows)}
        self.data = data
        self.shape = (None,) + tuple(data.shape[1:])

    def __getitem__(self, r):
        return self.data[self.index[int(r)]]


class _LazyDevRows:
    """Row-sliceable view of a device tensor; copies only what is indexed."""

    def __init__(self, t, lo=0, hi=None):
        self.t, self.lo = t, lo
        self.hi = t.shape[0] if hi is None else hi
        self.shape = (self.hi - self.lo,) + tuple(t.shape[1:])

    def __getitem__(self, idx):
        import torch
        if isinstance(idx, slice):
            a, b, _ = idx.indices(self.hi - self.lo)
            return _LazyDevRows(self.t, self.lo + a, self.lo + b)
        rows, rest = (idx[0], idx[1:]) if isinstance(idx, tuple) else (idx, ())
        if isinstance(rows, (int, np.integer)):
            x = self.t[self.lo + int(rows)]
            x = x[int(rest[0])] if rest else x
        else:
            r = torch.as_tensor(np.asarray(rows, dtype=np.int64) + self.lo, device=self.t.device)
            x = self.t.index_select(0, r)
            x = x[:, int(rest[0])] if rest else x
        return x.double().cpu().numpy()


class _SliceDequant4:
    """Index keys as the oracle sees them after 4-bit quantisation, one
    sequence slice at a time (keys scale per 32 elements of a row, so a slice
    quantises as the whole cache does).  prefetch() quantises the sequences of
    the given query rows before the oracle is timed: a decode step's key cache
    is stored quantised, outside the step."""

    def __init__(self, kidx, f4):
        self.kidx, self.f4, self.cache = kidx, f4, {}
        self.shape = kidx.shape

    def __getitem__(self, sl):
        assert isinstance(sl, slice) and (sl.step in (None, 1))
        key = (sl.start, sl.stop)
        if key not in self.cache:
            self.cache[key] = self.f4.dequantize_k_idx4(*self.f4.quantize_k_idx4(self.kidx[sl]))
        return self.cache[key]

    def prefetch(self, rows, cuq, cuk):
        for r in rows:
            b = int(np.searchsorted(cuq, r, side="right") - 1)
            self[int(cuk[b]):int(cuk[b + 1])]


_W = {}   # per-worker cache: attached shared arrays and the oracle problem


def _oracle_task(job):
    """Worker: oracle rows on inputs held in shared memory."""
    from multiprocessing import resource_tracker, shared_memory

    from threadpoolctl import threadpool_limits

    from oracle import msa_oracle as O
    spec, rows = job
    if _W.get("id") != spec["id"]:
        arrs = {}
        shms = []
        for name, (shm_name, shape, dtype) in spec["arrays"].items():
            shm = shared_memory.SharedMemory(name=shm_name)
            try:
                resource_tracker.unregister(shm._name, "shared_memory")
            except Exception:
                pass
            shms.append(shm)
            arrs[name] = np.ndarray(shape, dtype=dtype, buffer=shm.buf)
        q = _RowSubset(spec["rows"], arrs["q"])
        qi = _RowSubset(spec["rows"], arrs["q_idx"])
        _W.clear()
        _W.update(id=spec["id"], shms=shms,
                  P=O.Problem(q, arrs["k"], arrs["v"], qi, arrs["k_idx"], arrs["cu_q"], arrs["cu_k"],
                              spec["top_k"]))
    P = _W["P"]
    out = []
    with threadpool_limits(limits=1):
        for r in rows:
            out.append((int(r), P.row(int(r), want_scores=True)))
    return out


class OraclePool:
    """Worker processes forked before the GPU is touched; inputs reach them
    through shared memory, so no worker inherits GPU state."""

    def __init__(self, workers):
        import multiprocessing as mp
        self.workers = workers
        self.pool = mp.get_context("fork").Pool(workers) if workers > 1 else None
        self.shms = []

    def share(self, arrays):
        from multiprocessing import shared_memory
        spec = {}
        for name, a in arrays.items():
            a = np.ascontiguousarray(a)
            shm = shared_memory.SharedMemory(create=True, size=max(1, a.nbytes))
            np.ndarray(a.shape, dtype=a.dtype, buffer=shm.buf)[...] = a
            self.shms.append(shm)
            spec[name] = (shm.name, a.shape, a.dtype.str)
        return spec

    def run(self, spec, rows):
        jobs = [(spec, rows[i::self.workers * 4]) for i in range(self.workers * 4)]
        jobs = [j for j in jobs if len(j[1])]
        t0 = time.perf_counter()
        parts = self.pool.map(_oracle_task, jobs) if self.pool else [_oracle_task(j) for j in jobs]
        dt = time.perf_counter() - t0
        return {r: x for part in parts for r, x in part}, dt

    def close(self):
        if self.pool:
            self.pool.close()
            self.pool.join()
        for shm in self.shms:
            try:
                shm.close()
                shm.unlink()
            except Exception:
                pass
        self.shms = []


def _fp8_top_set_valid(P, r, g, S, sel):
    """fp8 index branch: a selection that differs from the oracle's is valid if
    every chosen block could still outrank every unchosen one after each block
    score moves by the matrix cores' error bound (FP8_DOT_REL * sum |q_c k_c|,
    maximised over the block's tokens)."""
    from oracle import msa_oracle as O
    b, p, ko = int(P.seq[r]), int(P.pos[r]), int(P.koff[r])
    lk = int(P.cu_k[b + 1] - P.cu_k[b])
    qa = np.abs(np.asarray(P.q_idx[r], dtype=np.float64))[g:g + 1]
    ka = np.abs(np.asarray(P.k_idx[ko:ko + lk][: p + 1], dtype=np.float64))
    B = FP8_DOT_REL * O.block_max_pool(qa @ ka.T, p, P.block)[0]
    beta_p = p // P.block
    mine = [int(x) for x in sel if x >= 0]
    if beta_p not in mine or len(set(mine)) != len(mine) or max(mine) > beta_p:
        return False
    chosen = [x for x in mine if x != beta_p]
    others = [z for z in range(beta_p) if z not in chosen]
    if len(mine) != min(P.top_k, beta_p + 1) or not chosen:
        return len(mine) == min(P.top_k, beta_p + 1)
    return min(S[x] + B[x] for x in chosen) >= max((S[z] - B[z] for z in others), default=-np.inf)


def projection_parity(proj, t, w, D, dev, k_store, key_rows=None, n_rows=64):
    """Index projections on sampled rows against the oracle's: each bf16 output
    equals the rounding of the exact sum, or (where the fp32-accumulated sum
    may cross a rounding boundary) lies within the accumulation bound plus one
    unit in the last place of it.  ``k_store`` is the index-key cache the step
    writes (``key_rows`` maps contiguous key rows to its rows when paged)."""
    import torch
    from oracle import projections as PR
    rng = np.random.Generator(np.random.PCG64(4321))
    rows = np.unique(rng.integers(0, w.total_q, n_rows))
    ridx = torch.as_tensor(rows, device=dev, dtype=torch.long)
    x = proj["x"].index_select(0, ridx).double().cpu().numpy()
    wq, wk = proj["w_q"].double().cpu().numpy(), proj["w_k"].double().cpu().numpy()
    cuq = t["cu_seqlens_q"].cpu().numpy()
    cuk = t["cu_seqlens_k"].cpu().numpy()
    b = np.searchsorted(cuq, rows, side="right") - 1
    krows = cuk[b] + (cuk[b + 1] - cuk[b]) - (cuq[b + 1] - cuq[b]) + (rows - cuq[b])
    got_q = t["q_idx"].index_select(0, ridx).double().cpu().numpy().reshape(len(rows), -1)
    kr = torch.as_tensor(krows, device=dev)
    if key_rows is not None:
        kr = key_rows.index_select(0, kr)
    got_k = k_store.index_select(0, kr).double().cpu().numpy()
    bad = n_diff = 0
    for got, W in ((got_q, wq), (got_k, wk)):
        y, sa = x @ W.T, np.abs(x) @ np.abs(W).T
        r = PR.bf16_round(y)
        _, e = np.frexp(np.abs(y))
        ulp = np.ldexp(1.0, np.maximum(e, -125) - 8)
        eps = D * 2.0 ** -24 * sa + 1e-300
        diff = got != r
        ok = ((ulp / 2 - np.abs(y - r)) <= eps) & (np.abs(got - y) <= eps + ulp)
        n_diff += int(diff.sum())
        bad += int((diff & ~ok).sum())
    return dict(ok=bad == 0, rows=int(len(rows)), outputs_differing_from_rounding=n_diff,
                outputs_outside_bound=bad)


def parity_on_rows(P, rows, ref, sel_gpu, out_gpu, lse_gpu, top_k, fp8=False):
    from oracle import msa_oracle as O
    bad = ties = 0
    fp8_differ = 0
    tie_differ = 0
    dmax = dsum = 0.0
    n = 0
    ref_abs_max = 0.0
    l2d = l2r = 0.0
    lse_max = 0.0
    for i, r in enumerate(rows):
        x = ref[r]
        beta_p = int(P.pos[r]) // BLOCK
        ref_out, ref_lse = x["out"], x["lse"]
        differs = False
        for g in range(P.G):
            tie = O.near_tie(x["S"][g], beta_p, top_k)
            ties += int(tie)
            if not np.array_equal(sel_gpu[i, g], x["sel"][g]):
                differs = True
                if fp8:
                    fp8_differ += 1
                    if not _fp8_top_set_valid(P, r, g, x["S"][g], sel_gpu[i, g]):
                        bad += 1
                elif not (tie and O.valid_selection(x["S"][g], beta_p, top_k, sel_gpu[i, g])):
                    bad += 1
                else:
                    tie_differ += 1
        if differs:
            # Main Branch checked on the selection the GPU made
            ref_out, ref_lse = P.attend_with_selection(r, sel_gpu[i])
        dd = np.abs(out_gpu[i] - ref_out)
        dmax = max(dmax, float(dd.max()))
        dsum += float(dd.sum())
        n += dd.size
        ref_abs_max = max(ref_abs_max, float(np.abs(ref_out).max()))
        l2d += float((dd ** 2).sum())
        l2r += float((ref_out ** 2).sum())
        lse_max = max(lse_max, float(np.abs(lse_gpu[i] - ref_lse).max()))
    mean = dsum / max(n, 1)
    rel2 = math.sqrt(l2d / max(l2r, 1e-300))
    relmax = dmax / max(ref_abs_max, 1e-300)
    ok = bad == 0 and dmax <= 2e-2 and mean <= 2e-3 and rel2 <= 1e-2 and relmax <= 2e-2 and lse_max <= 2e-3
    res = dict(ok=bool(ok), rows=len(rows), selection_mismatches=bad, near_ties=ties,
               near_ties_chosen_differently=tie_differ,
               max_abs=dmax, mean_abs=mean, rel_l2=rel2, rel_max=relmax, lse_max_abs=lse_max)
    if fp8:
        res["fp8_selections_differing_within_bound"] = fp8_differ
    return res


# ---------------------------------------------------------------------------
def source_code_hash(path: str) -> str:
    """sha256 of a kernel source and of the local headers it includes (recursively),
    with comments and whitespace removed: a traffic record stays valid while the
    code it was measured on is unchanged."""
    import hashlib
    import re
    seen, order = set(), []

    def visit(p):
        if p in seen or not os.path.exists(p):
            return
        seen.add(p)
        order.append(p)
        for inc in sorted(re.findall(r'#include\s+"([^"]+)"', open(p, encoding="utf-8").read())):
            visit(os.path.join(os.path.dirname(p), inc))

    visit(path)
    h = hashlib.sha256()
    for p in order:
        text = open(p, encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="p128k")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target host time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--q-chunk", type=int, default=0)
    ap.add_argument("--json-out", default="")
    ap.add_argument("--copy-gib", type=float, default=0.0,
                    help="before the workload, run three device copies of this many GiB (fp32): a "
                         "kernel of known traffic for scaling the FETCH_SIZE/WRITE_SIZE counters")
    ap.add_argument("--index", choices=["bf16", "fp8", "q8k4"], default="bf16",
                    help="Index Branch precision: bf16 projections; quantised in the step to "
                         "FP8 E4M3 with power-of-two scales and scored on the fp8 matrix cores "
                         "(fp8); or 8-bit queries with 4-bit E2M1 keys scaled per 32 elements, "
                         "scored on the microscaled matrix cores (q8k4).  A decode step's "
                         "index-key cache is stored quantised; only its new queries are quantised")
    ap.add_argument("--main", choices=["bf16", "fp8", "q8kv4"], default="bf16",
                    help="Main Branch inputs: bf16 q/k/v; FP8 E4M3 codes with power-of-two "
                         "scales (fp8); or E4M3 queries with 4-bit E2M1 keys and values scaled "
                         "per 32 elements (q8kv4).  Prefill quantises in the step; a decode "
                         "step's key/value cache is stored quantised and only its new queries "
                         "are quantised")
    ap.add_argument("--project-dim", type=int, default=0,
                    help="also run the index projections in the step: q_idx and the new tokens' "
                         "k_idx from a layer input of this width (0: off; the index projections "
                         "are then checked element-wise on the sampled rows instead of the whole path)")
    ap.add_argument("--kl", action="store_true",
                    help="also compute the Index Branch's KL-alignment target in the step "
                         "(Main-Branch block masses + index log-probabilities + KL per query and group)")
    ap.add_argument("--paged", action="store_true",
                    help="hold K, V and the index keys in a paged cache (128-row pages in a "
                         "scrambled order, found through a block table) instead of contiguous rows")
    ap.add_argument("--graph", choices=["auto", "on", "off"], default="auto",
                    help="replay the step as a captured HIP graph (auto: on for decode, whose "
                         "kernels are short enough for launch gaps to matter)")
    ap.add_argument("--partials", choices=["fp32", "both"], default=None,
                    help="Main-Branch partials: fp32 (the library default) only, or both: the step "
                         "is timed with fp32 partials for the headline and again with compact partials "
                         "(fp16 values with a log-sum-exp and a power-of-two exponent per row), whose "
                         "result goes under 'compact_partials' (default: both for prefill workloads "
                         "with the bf16 Main Branch and no KL target, else fp32)")
    ap.add_argument("--no-legs", action="store_true",
                    help="default workload only: skip the decode and 1M-prefill legs that the default "
                         "run measures in child processes and appends under 'legs'")
    ap.add_argument("--ceilings", action="store_true",
                    help="also measure the HBM rate of a plain streaming kernel at the read:write "
                         "mixes of the Main Branch's passes (on by default for the headline run)")
    ap.add_argument("--leg", action="store_true", help=argparse.SUPPRESS)
    return ap.parse_args(argv)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def kv_reread_schedule(msa, dims, bufs, w, lists):
    """K/V blocks staged by the Main Branch's work items beyond one per
    selected (sequence, group, block), relative to those unique blocks.

    Lists path: a (sequence, group, block) item is staged once per query pass
    whose rows it serves, so an item whose ascending list crosses a pass
    boundary is staged again.  Decode path: every (query, slot) stages its
    block, so blocks selected by several new tokens of a sequence repeat."""
    import torch
    if lists:
        off = bufs.offsets.long()
        n = int(off[-1])
        counts = off[1:] - off[:-1]
        unique = int((counts > 0).sum())
        if n == 0 or unique == 0:
            return dict(staged=0, unique=0, frac=0.0)
        bucket = torch.repeat_interleave(torch.arange(len(counts), device=off.device), counts)
        pass_id = (bufs.entries[:n].long() >> 5) // msa.attend_pass_rows(dims)
        extra = int(((pass_id[1:] != pass_id[:-1]) & (bucket[1:] == bucket[:-1])).sum())
        staged = unique + extra
    else:
        sel = bufs.sel.long()
        valid = sel >= 0
        staged = int(valid.sum())
        G = sel.shape[1]
        seq = torch.repeat_interleave(torch.arange(w.batch, device=sel.device),
                                      torch.as_tensor(w.seq_q_lens, device=sel.device))
        nb = msa.nb_max(dims)
        key = (seq[:, None, None] * G + torch.arange(G, device=sel.device)[None, :, None]) * nb + sel
        unique = int(torch.unique(key[valid]).numel())
    return dict(staged=staged, unique=unique, frac=(staged - unique) / max(unique, 1))


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this build has no "
              f"multi-GPU path. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    default_run = (not args.leg and not args.no_legs and args.workload == "p128k"
                   and args.index == "bf16" and args.main == "bf16" and not args.project_dim
                   and not args.kl and not args.paged and not args.q_chunk and not args.copy_gib)
    legs = {}
    if default_run:
        # the metric's other legs, each in a child process started before this process
        # touches the GPU; their progress goes to stderr, their JSON line to a file
        import subprocess
        import tempfile
        for name, opts, limit in (("decode", ["--steps", "200", "--warmup", "20"], 420),
                                  ("p1m", ["--steps", "3", "--warmup", "1", "--cpu-seconds", "12"], 900)):
            fd, path = tempfile.mkstemp(prefix=f"bench_{name}_", suffix=".json")
            os.close(fd)
            cmd = [sys.executable, os.path.abspath(__file__), "--leg", "--workload", name,
                   "--json-out", path, *opts]
            log(f"[bench] leg {name}: {' '.join(cmd[1:])}")
            t0 = time.perf_counter()
            try:
                rc = subprocess.run(cmd, stdout=sys.stderr, stderr=sys.stderr, timeout=limit).returncode
            except subprocess.TimeoutExpired:
                rc = "timeout"
            try:
                leg = json.load(open(path)) if os.path.getsize(path) else {}
            except (OSError, ValueError):
                leg = {}
            os.unlink(path)
            leg.pop("work", None)
            leg["exit_code"] = rc
            leg["wall_s"] = time.perf_counter() - t0
            legs[name] = leg
            log(f"[bench] leg {name} done: exit {rc}, {leg['wall_s']:.0f} s")
    args.ceilings = args.ceilings or default_run
    line, ok = run_leg(args)
    if legs:
        line["legs"] = legs
    s = json.dumps(line)
    print(s, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(s + "\n")
    if not ok:
        log("[bench] PARITY FAILED on sampled rows")
        sys.exit(1)


def run_leg(args):
    if args.kl and (args.index != "bf16" or args.main != "bf16"):
        print("--kl uses the bf16 index and Main branches", file=sys.stderr)
        sys.exit(2)
    from msa_inputs import workload as _wl
    w = _wl(args.workload)
    cores = min(16, len(os.sched_getaffinity(0)))
    host_bytes = w.total_k * w.num_kv_heads * w.head_dim * 4 * 2 + w.total_k * w.index_dim * 4
    pooled = (not args.no_cpu_baseline) and not args.project_dim and host_bytes <= (16 << 30) \
        and cores > 1
    pool = OraclePool(cores) if pooled else None   # forked before any GPU call

    import torch

    import block_sparse_long_index_amd as msa
    from msa_inputs import generate

    dev = torch.device("cuda:0")
    if args.copy_gib > 0:
        n = int(args.copy_gib * 2**30) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {args.copy_gib} GiB three times (counter calibration)")
        del src, dst
        torch.cuda.empty_cache()
    log(f"[bench] workload {w.name}: {w.note}; generating inputs on {dev}")
    t0 = time.perf_counter()
    t = generate(w, dev)
    torch.cuda.synchronize()
    log(f"[bench] inputs ready in {time.perf_counter() - t0:.1f}s")
    dims = msa.dims_for(w, q_chunk=args.q_chunk)
    # the step's key caches: the contiguous inputs, or the same rows scattered into pages
    kc, vc, kic, key_rows = t["k"], t["v"], t["k_idx"], None
    if args.paged:
        from msa_inputs import paged_layout, to_pages
        table, rows_h, pages = paged_layout(w, seed=w.seed)
        key_rows = rows_h.to(dev)
        table_d = table.to(dev)
        kc, vc, kic = (to_pages(t[n], key_rows, pages) for n in ("k", "v", "k_idx"))
        dims = msa.make_dims(batch=w.batch, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                             head_dim=w.head_dim, index_dim=w.index_dim, top_k=w.top_k,
                             total_q=w.total_q, total_k=pages * BLOCK, max_q_len=max(w.seq_q_lens),
                             max_k_len=max(w.seq_k_lens), q_chunk=args.q_chunk, block_table=table_d)
        torch.cuda.synchronize()
        log(f"[bench] paged key cache: {pages} pages of {BLOCK} rows, scrambled order")
    bufs = msa.Buffers(dims, dev, want_scores=args.kl, want_lse=True)
    # the compact-partial pass (measured after the headline) may hold more rows per pass,
    # i.e. need more workspace: one buffer serves both
    if (args.partials == "both" or (args.partials is None and not _decode_like(w) and args.main == "bf16"
                                    and not args.kl and not args.project_dim)):
        dims_probe = msa.Dims.from_buffer_copy(dims)
        dims_probe.flags = msa.FLAG_COMPACT_PARTIALS
        need_c = msa.workspace_size(dims_probe, msa.OP_ATTEND)
        if need_c > bufs.workspace.numel():
            bufs.workspace = torch.empty((need_c,), dtype=torch.uint8, device=dev)
    kl_out = None
    if args.kl:
        kl_out = dict(mass=torch.empty((w.total_q, w.num_kv_heads, w.top_k), dtype=torch.float32, device=dev),
                      kl=torch.empty((w.total_q, w.num_kv_heads), dtype=torch.float32, device=dev))
    fp8 = msa.Fp8Index(dims, dev) if args.index == "fp8" else None
    qk = msa.Q8K4Index(dims, dev) if args.index == "q8k4" else None
    log(f"[bench] workspace {bufs.workspace.numel() / 2**30:.2f} GiB; index branch {args.index}")
    # fp8 decode: the index-key cache is stored quantised (quantised once, outside the step);
    # each step quantises only its new index queries.  Prefill quantises both in the step.
    step_k_idx = kic
    if fp8 is not None and _decode_like(w):
        msa.index_quantize_fp8(dims, None, kic, t["cu_seqlens_k"], fp8)
        torch.cuda.synchronize()
        step_k_idx = None
    if qk is not None and _decode_like(w):
        msa.index_quantize_q8k4(dims, None, kic, t["cu_seqlens_k"], qk)
        torch.cuda.synchronize()
        step_k_idx = None

    # fp8 Main Branch: prefill quantises q, k, v in the step; decode keeps a quantised K/V
    # cache (quantised once, outside the step) and quantises its new queries
    f8m = (msa.Fp8Main(dims, dev) if args.main == "fp8" else
           msa.Q8KV4Main(dims, dev) if args.main == "q8kv4" else None)
    step_k, step_v = kc, vc
    if f8m is not None and _decode_like(w):
        (msa.main_quantize_fp8 if args.main == "fp8" else msa.main_quantize_q8kv4)(
            dims, None, kc, vc, t["cu_seqlens_k"], f8m)
        torch.cuda.synchronize()
        step_k = step_v = None

    proj = None
    if args.project_dim:
        from msa_inputs import generate_projection
        proj = generate_projection(w, args.project_dim, dev)
        torch.cuda.synchronize()
        log(f"[bench] index projections from a width-{args.project_dim} layer input")

    def step(d=None):
        d = dims if d is None else d
        if proj is not None:
            # q_idx and the new tokens' index keys come from the layer input
            msa.index_project(d, proj["x"], proj["w_q"], proj["w_k"], t["cu_seqlens_q"],
                              t["cu_seqlens_k"], t["q_idx"], kic, bufs.workspace)
        if kl_out is None:
            msa.msa_forward(d, t["q"], step_k, step_v, t["q_idx"], step_k_idx, t["cu_seqlens_q"],
                            t["cu_seqlens_k"], bufs, fp8=fp8, fp8_main=f8m, q8k4=qk)
            return
        # the forward with the KL-alignment target (bf16 index branch)
        msa.index_select(dims, t["q_idx"], kic, t["cu_seqlens_q"], t["cu_seqlens_k"],
                         bufs.sel, bufs.sel_score, bufs.workspace)
        msa.build_block_query_lists(dims, bufs.sel, t["cu_seqlens_q"], t["cu_seqlens_k"], bufs.offsets,
                                    bufs.entries, bufs.workspace)
        msa.attend_with_mass(dims, t["q"], kc, vc, t["cu_seqlens_q"], t["cu_seqlens_k"],
                             bufs.sel, bufs.offsets, bufs.entries, bufs.out, kl_out["mass"], bufs.lse,
                             bufs.workspace)
        msa.index_kl(dims, t["q_idx"], kic, t["cu_seqlens_q"], t["cu_seqlens_k"], bufs.sel,
                     bufs.sel_score, kl_out["mass"], kl_out["kl"])

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"[bench] warmup {i + 1}/{args.warmup} done")

    use_graph = args.graph == "on" or (args.graph == "auto" and _decode_like(w))
    run = step
    if use_graph:
        # capture the three calls once (no allocation, no memset, no host sync inside)
        cs = torch.cuda.Stream()
        cs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cs):
            step()
        torch.cuda.current_stream().wait_stream(cs)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=cs):
            step()
        torch.cuda.synchronize()
        run = graph.replay
        log("[bench] step captured as a graph")

    def timed(fn, n, profile):
        if profile:
            msa.profile_collect()             # drop anything recorded before
            msa.profile_enable(True)
        # one event between consecutive steps on the launch stream (no host wait inside)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev[0].record()
        for i in range(n):
            fn()
            ev[i + 1].record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        prof = None
        if profile:
            msa.profile_enable(False)
            prof = msa.profile_collect()
        per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(n))
        median = per[n // 2] if n % 2 else 0.5 * (per[n // 2 - 1] + per[n // 2])
        return (t1 - t0) * 1e3 / n, prof, median

    # timed region: exactly `steps` steps; stage times from library HIP events on the
    # launch stream (an eager pass of the same length when the timed steps are graph replays)
    ms_per_step, prof, ms_median = timed(run, args.steps, profile=not use_graph)
    if use_graph:
        _, prof, _ = timed(step, args.steps, profile=True)
    log(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms/step (median {ms_median:.3f})")

    wm = work_model(w)
    wm["project_flops"] = (2.0 * w.total_q * args.project_dim * (w.num_kv_heads + 1) * w.index_dim
                           if args.project_dim else 0.0)
    stage = {}
    for name, (ms, n) in prof.items():
        if n:
            stage[name] = dict(ms_per_step=ms / args.steps, launches_per_step=n / args.steps,
                               ms_per_launch=ms / n)
    per_step = {k_: v["ms_per_step"] for k_, v in stage.items()}
    log("[bench] stages (ms/step): " + ", ".join(f"{k_} {v:.3f}" for k_, v in per_step.items()))

    def traffic_record(name, compact=False, launches=None):
        """Measured HBM bytes per launch (FETCH_SIZE/WRITE_SIZE scaled by a copy of known
        size, profiles/<kernel>_<workload>[_compact]_traffic.json) if the kernel code is
        unchanged."""
        path = os.path.join(ROOT, "profiles",
                            f"{name}_{w.name}{'_compact' if compact else ''}_traffic.json")
        if not os.path.exists(path):
            return None
        rec = json.load(open(path))
        if source_code_hash(os.path.join(ROOT, rec["source"])) != rec.get("source_code_sha256") or \
                args.q_chunk or args.main != "bf16" or args.paged:
            return None
        # a launch's bytes depend on the pass size: the record must come from a run
        # that launched the kernel as often per step as this one does
        if "dispatches_per_step" in rec and rec["dispatches_per_step"] != launches:
            return None
        return rec["per_dispatch"]["total_bytes"] / 1e9

    def roof(name, st_=None, compact=False):
        """Roofline of one stage: algorithmic work per launch / average launch time."""
        s_ = (stage if st_ is None else st_).get(name)
        if not s_:
            return None
        n_launch = s_["launches_per_step"]
        sec = s_["ms_per_launch"] / 1e3
        if name == "index_project":
            a = wm["project_flops"] / n_launch / sec
            return dict(bound="mfma", achieved=a / 1e12, peak=PEAK_BF16_FLOPS / 1e12, unit="TFLOP/s",
                        frac=a / PEAK_BF16_FLOPS, traffic=traffic_record(name, launches=n_launch), dtype="bf16")
        if name in ("index_select_prefill", "index_select_prefill_fp8", "index_select_prefill_q8k4"):
            # E2M1 x E4M3 runs at the fp8 rate (an 8-bit operand sets the MFMA's cycle count)
            peak = PEAK_BF16_FLOPS if name == "index_select_prefill" else PEAK_FP8_FLOPS
            a = wm["index_flops"] / n_launch / sec
            return dict(bound="mfma", achieved=a / 1e12, peak=peak / 1e12, unit="TFLOP/s",
                        frac=a / peak, traffic=traffic_record(name, launches=n_launch),
                        dtype={"index_select_prefill": "bf16", "index_select_prefill_fp8": "fp8 e4m3",
                               "index_select_prefill_q8k4": "e2m1 keys x e4m3 queries"}[name])
        bytes_ = {"attend_blocks": wm[{"bf16": "attend_bytes", "fp8": "attend_bytes_fp8",
                                       "q8kv4": "attend_bytes_kv4"}[args.main]],
                  "merge_partials": wm["merge_bytes"],
                  "quantize_main_fp8": wm["main_quant_bytes"],
                  "quantize_main_q8kv4": wm["main_quant_kv4_bytes"],
                  "topk_select": wm["topk_bytes"],
                  "index_score_decode": wm["index_decode_bytes"],
                  "index_score_decode_fp8": wm["index_decode_fp8_bytes"],
                  "index_score_decode_q8k4": wm["index_decode_q8k4_bytes"],
                  "quantize_index_q8k4": wm["quant_q8k4_bytes"],
                  "quantize_index_fp8": wm["quant_bytes"]}
        if compact:
            bytes_["attend_blocks"] = wm["attend_bytes_compact"]
            bytes_["merge_partials"] = wm["merge_bytes_compact"]
        if name in bytes_:
            per_launch = bytes_[name] / n_launch
            a = per_launch / sec
            return dict(bound="hbm", achieved=a / 1e9, peak=PEAK_HBM_BYTES / 1e9, unit="GB/s",
                        frac=a / PEAK_HBM_BYTES, traffic=traffic_record(name, compact, n_launch),
                        traffic_unit="GB per launch (HBM, counters scaled by a copy of known size)",
                        algorithmic_per_launch=per_launch / 1e9)
        return None

    dominant = max(per_step, key=per_step.get) if per_step else None
    kernels = {k_: dict(stage[k_], roofline=roof(k_)) for k_ in stage}
    t_main = (per_step.get("attend_blocks", 0.0) + per_step.get("merge_partials", 0.0)) / 1e3
    main_mfma_frac = wm["main_flops"] / (t_main * PEAK_BF16_FLOPS) if t_main > 0 else None
    decode = _decode_like(w)
    value = w.total_q / (ms_per_step / 1e3)
    # K/V re-reads of the Main Branch: from its schedule (exact), and from the attend
    # kernel's FETCH_SIZE record where one matches this source (counters minus the
    # gathered Q, list entries and unique K/V bytes; calibration-limited when Q dominates)
    lists_path = bool(msa.attend_reads_lists(dims))
    reread = kv_reread_schedule(msa, dims, bufs, w, lists_path)
    kv_block_bytes = BLOCK * w.head_dim * 2 * 2
    reread["unique_kv_bytes"] = reread["unique"] * kv_block_bytes
    rec_name = "attend_blocks"
    rec_path = os.path.join(ROOT, "profiles", f"{rec_name}_{w.name}_traffic.json")
    if os.path.exists(rec_path) and args.main == "bf16" and not args.paged and not args.q_chunk:
        rec = json.load(open(rec_path))
        n_disp = stage.get("attend_blocks", {}).get("launches_per_step", 0)
        if source_code_hash(os.path.join(ROOT, rec["source"])) == rec.get("source_code_sha256") and \
                rec.get("dispatches_per_step", n_disp) == n_disp:
            fetch = rec["per_dispatch"]["read_gb"] * 1e9 * n_disp
            hpg = w.num_q_heads // w.num_kv_heads
            q_bytes = wm["sel_total"] * hpg * w.head_dim * 2
            list_bytes = wm["sel_total"] * 4 if lists_path else 0.0
            kv_read = fetch - q_bytes - list_bytes
            reread["counter_kv_read_bytes"] = kv_read
            # the estimate subtracts the gathered Q, assumed all from HBM (some comes
            # from the caches); when the unique K/V is a small share of the kernel's
            # reads that assumption's error exceeds the K/V term, and no fraction is given
            share = reread["unique_kv_bytes"] / fetch if fetch > 0 else 0.0
            reread["counter_kv_share_of_reads"] = share
            if share >= 0.05:
                reread["counter_frac"] = kv_read / reread["unique_kv_bytes"] - 1.0
            else:
                reread["counter_frac"] = None
                reread["counter_note"] = (f"unique K/V is {100 * share:.1f}% of the attend kernel's HBM "
                                          "reads, below what subtracting the gathered Q can resolve")
    log(f"[bench] K/V re-read fraction (schedule): {reread['frac']:.4f}")
    extra = {}
    if decode:
        dec_bytes = wm["decode_fp8_bytes" if fp8 is not None else
                       "decode_q8k4_bytes" if qk is not None else "decode_bytes"]
        if f8m is not None:
            dec_bytes += wm["decode_kv_fp8_delta" if args.main == "fp8" else "decode_kv4_delta"]
        gbs = dec_bytes / (ms_per_step / 1e3) / 1e9
        extra["decode_hbm_GBps"] = gbs
        extra["decode_hbm_frac"] = gbs * 1e9 / PEAK_HBM_BYTES

    # ---- oracle sample: parity gate + cpu baseline --------------------------------
    cpu = None
    parity = None
    oracle_ctx = None
    if proj is not None:
        parity = projection_parity(proj, t, w, args.project_dim, dev, kic, key_rows)
        log(f"[bench] projection parity on sampled rows: {parity}")
    elif not args.no_cpu_baseline:
        from oracle import msa_oracle as O
        rng = np.random.Generator(np.random.PCG64(12345))
        cuq = t["cu_seqlens_q"].cpu().numpy()
        cuk = t["cu_seqlens_k"].cpu().numpy()
        if pooled:
            kk = t["k"].float().cpu().numpy()
            vv = t["v"].float().cpu().numpy()
            kidx = t["k_idx"].float().cpu().numpy()
        else:
            kk, vv = _LazyDevRows(t["k"]), _LazyDevRows(t["v"])
            kidx = t["k_idx"].float().cpu().numpy()

        if fp8 is not None:
            # the oracle scores the dequantised codes it computes itself from the bf16 inputs
            from oracle import fp8_index as F
            nbk = int((np.diff(cuk).max() + BLOCK - 1) // BLOCK)
            kcodes, kexp = F.quantize_k_idx(kidx, cuk, nbk)
            kidx = F.dequantize_k_idx(kcodes, kexp, cuk)
            del kcodes
        if qk is not None:
            # 4-bit keys scale per 32 elements of a row: any slice of rows quantises alone
            from oracle import fp8_index as F
            from oracle import fp4_index as F4
            kidx = (F4.dequantize_k_idx4(*F4.quantize_k_idx4(kidx)) if pooled
                    else _SliceDequant4(kidx, F4))
        if f8m is not None and args.main == "q8kv4":
            # 8-bit q as in the fp8 Main Branch; k and v scale per 32 elements of a
            # (key, head) row, so any slice of rows quantises alone
            from oracle import fp4_main as M4
            from oracle import fp8_main as FM
            if pooled:
                kk = M4.dequantize_kv4(*M4.quantize_kv4(kk))
                vv = M4.dequantize_kv4(*M4.quantize_kv4(vv))
            else:
                def fetch(x):
                    return lambda lo, hi: x[lo:hi].double().cpu().numpy()
                kk = M4.DequantizedRows4(fetch(t["k"]), w.total_k, t["k"].shape[1:])
                vv = M4.DequantizedRows4(fetch(t["v"]), w.total_k, t["v"].shape[1:])
        elif f8m is not None:
            # the oracle attends on the dequantised q, k, v it computes itself from the bf16 inputs
            from oracle import fp8_main as FM
            if pooled:
                nbk = int((np.diff(cuk).max() + BLOCK - 1) // BLOCK)
                kk = FM.dequantize_kv(*FM.quantize_kv(kk, cuk, nbk), cuk)
                vv = FM.dequantize_kv(*FM.quantize_kv(vv, cuk, nbk), cuk)
            else:
                def fetch(x):
                    return lambda lo, hi: x[lo:hi].double().cpu().numpy()
                kk = FM.DequantizedRows(fetch(t["k"]), w.total_k, t["k"].shape[1:], cuk)
                vv = FM.DequantizedRows(fetch(t["v"]), w.total_k, t["v"].shape[1:], cuk)

        def host_rows(rows):
            ridx = torch.as_tensor(rows, device=dev, dtype=torch.long)
            qi = t["q_idx"].index_select(0, ridx).float().cpu().numpy()
            if fp8 is not None or qk is not None:
                qi = F.dequantize_q_idx(*F.quantize_q_idx(qi))
            qh = t["q"].index_select(0, ridx).float().cpu().numpy()
            if f8m is not None:
                qh = FM.dequantize_q(*FM.quantize_q(qh))
            return qh, qi

        # per-row cost on one core, then a sample sized to the time target
        pilot = sorted(set(int(x) for x in rng.integers(0, w.total_q, size=min(6, w.total_q))))
        qh, qih = host_rows(pilot)
        if isinstance(kidx, _SliceDequant4):     # a decode step's key cache is stored quantised
            kidx.prefetch(pilot, cuq, cuk)
        Pp = O.Problem(_RowSubset(pilot, qh), kk, vv, _RowSubset(pilot, qih), kidx, cuq, cuk, w.top_k)
        tp0 = time.perf_counter()
        for r in pilot:
            Pp.row(r)
        per_row = (time.perf_counter() - tp0) / len(pilot)
        used = cores if pooled else 1
        n_rows = int(max(16, min(w.total_q, args.cpu_seconds * used / max(per_row, 1e-6))))
        # a workload with fewer rows than the time budget allows (decode) is taken whole
        rows = (list(range(w.total_q)) if n_rows >= w.total_q else
                sorted(set(int(x) for x in rng.integers(0, w.total_q, size=n_rows))))
        log(f"[bench] oracle: {per_row * 1e3:.1f} ms/row on one core; sampling {len(rows)} rows "
            f"on {used} worker(s)")
        qh, qih = host_rows(rows)
        if isinstance(kidx, _SliceDequant4):
            kidx.prefetch(rows, cuq, cuk)
        P = O.Problem(_RowSubset(rows, qh), kk, vv, _RowSubset(rows, qih), kidx, cuq, cuk, w.top_k)
        if pooled:
            spec = dict(id=1, rows=rows, top_k=w.top_k,
                        arrays=pool.share(dict(q=qh, q_idx=qih, k=kk, v=vv, k_idx=kidx,
                                               cu_q=cuq, cu_k=cuk)))
            ref, dt = pool.run(spec, rows)
            pool.close()
        else:
            t1 = time.perf_counter()
            ref = {r: P.row(r, want_scores=True) for r in rows}
            dt = time.perf_counter() - t1
        log(f"[bench] oracle sample done in {dt:.1f}s")
        ridx = torch.as_tensor(rows, device=dev, dtype=torch.long)
        sel_g = bufs.sel.index_select(0, ridx).cpu().numpy()
        out_g = bufs.out.index_select(0, ridx).float().cpu().numpy()
        lse_g = bufs.lse.index_select(0, ridx).cpu().numpy()
        parity = parity_on_rows(P, rows, ref, sel_g, out_g, lse_g, w.top_k,
                                fp8=fp8 is not None or qk is not None)
        log(f"[bench] parity on sampled rows: {parity}")
        oracle_ctx = (P, rows, ref)
        cpu = dict(value=len(rows) / dt, unit="tokens/s", cores=used, kind="oracle",
                   cpu_model=cpu_model(),
                   # uniformly random rows sample the per-row cost (which grows with the
                   # row's position) without bias, so the whole workload on the same
                   # cores would take about total_q / value seconds
                   full_workload_s_extrapolated=w.total_q * dt / len(rows),
                   sample=(f"all {len(rows)} query rows" if len(rows) == w.total_q else
                           f"{len(rows)} uniformly random query rows") + f" of {w.name}, each through the "
                          f"full Index and Main Branch in fp64 numpy"
                          f"{' (on the dequantised fp8 index projections)' if fp8 is not None else ''}"
                          f"{' (on the dequantised 8-bit index queries and 4-bit index keys)' if qk is not None else ''}"
                          f"{' (on the dequantised fp8 q, k, v)' if args.main == 'fp8' else ''}"
                          f"{' (on the dequantised 8-bit q and 4-bit k, v)' if args.main == 'q8kv4' else ''}; "
                          f"{used} worker process(es), 1 BLAS thread each; {dt:.1f} s")
    elif pool:
        pool.close()

    # ---- the same step with compact Main-Branch partials (same inputs, same rows) ----
    compact = None
    want_compact = (args.partials == "both" or
                    (args.partials is None and not decode and args.main == "bf16" and kl_out is None
                     and proj is None))
    if want_compact and msa.attend_reads_lists(dims):
        dims_c = msa.Dims.from_buffer_copy(dims)
        dims_c.flags = msa.FLAG_COMPACT_PARTIALS
        dims_c._block_table = getattr(dims, "_block_table", None)
        step(dims_c)
        torch.cuda.synchronize()
        ms_c, prof_c, med_c = timed(lambda: step(dims_c), args.steps, profile=True)
        stage_c = {name: dict(ms_per_step=ms / args.steps, launches_per_step=n / args.steps,
                              ms_per_launch=ms / n) for name, (ms, n) in prof_c.items() if n}
        per_step_c = {k_: v["ms_per_step"] for k_, v in stage_c.items()}
        t_main_c = (per_step_c.get("attend_blocks", 0.0) + per_step_c.get("merge_partials", 0.0)) / 1e3
        compact = dict(
            ms_per_step=ms_c, ms_per_step_median=med_c, value=w.total_q / (ms_c / 1e3),
            unit="tokens/s",
            main_branch_mfma_frac=wm["main_flops"] / (t_main_c * PEAK_BF16_FLOPS) if t_main_c else None,
            stages_ms_per_step=per_step_c,
            kernels={k_: dict(stage_c[k_], roofline=roof(k_, stage_c, compact=True))
                     for k_ in ("attend_blocks", "merge_partials") if k_ in stage_c},
            pass_rows=msa.attend_pass_rows(dims_c))
        log(f"[bench] compact partials: {ms_c:.3f} ms/step (median {med_c:.3f}); stages "
            + ", ".join(f"{k_} {v:.3f}" for k_, v in per_step_c.items()))
        if oracle_ctx is not None:
            P_, rows_, ref_ = oracle_ctx
            ridx = torch.as_tensor(rows_, device=dev, dtype=torch.long)
            compact["parity"] = parity_on_rows(
                P_, rows_, ref_, bufs.sel.index_select(0, ridx).cpu().numpy(),
                bufs.out.index_select(0, ridx).float().cpu().numpy(),
                bufs.lse.index_select(0, ridx).cpu().numpy(), w.top_k,
                fp8=fp8 is not None or qk is not None)
            log(f"[bench] compact partials parity on the same rows: {compact['parity']}")
            if not compact["parity"]["ok"]:
                parity = dict(parity, ok=False, compact_partials_failed=True)

    # ---- streaming ceilings at the Main Branch's read:write mixes ---------------------
    ceilings = None
    if args.ceilings:
        gib = 4
        src = torch.randint(0, 255, (gib << 30,), dtype=torch.uint8, device=dev)
        dst = torch.empty((2 * (gib << 30),), dtype=torch.uint8, device=dev)
        sink = torch.empty((8192,), dtype=torch.uint8, device=dev)
        ceilings = {}
        for ratio, name in ((0, "read_only"), (1, "read1_write1"), (2, "read1_write2")):
            msa.hbm_stream(src, ratio, dst, sink)
            torch.cuda.synchronize()
            reps = 5
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                msa.hbm_stream(src, ratio, dst, sink)
            e1.record()
            torch.cuda.synchronize()
            sec = e0.elapsed_time(e1) / 1e3 / reps
            ceilings[name] = dict(GBps=(1 + ratio) * (gib << 30) / sec / 1e9, read_GiB=gib,
                                  write_GiB=gib * ratio)
        del src, dst, sink
        torch.cuda.empty_cache()
        log("[bench] streaming ceilings (GB/s): " + ", ".join(f"{k_} {v['GBps']:.0f}" for k_, v in ceilings.items()))
        mixes = [(kernels, "attend_blocks", "read1_write2"), (kernels, "merge_partials", "read_only")]
        if compact:
            mixes += [(compact["kernels"], "attend_blocks", "read1_write1"),
                      (compact["kernels"], "merge_partials", "read_only")]
        for ks_, k_, cname in mixes:
            r_ = ks_.get(k_, {}).get("roofline")
            if r_:
                r_["frac_of_stream_ceiling"] = r_["achieved"] / ceilings[cname]["GBps"]
                r_["stream_ceiling"] = cname

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s" if not decode else "tokens/s (new tokens)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16" if fp8 is None and f8m is None and qk is None else
                  ({"bf16": "bf16", "fp8": "fp8 e4m3 storage, bf16 MFMA",
                    "q8kv4": "e4m3 q, e2m1 k/v storage, bf16 MFMA"}[args.main] + " (Main Branch), "
                   + ("fp8 e4m3" if fp8 is not None else
                      "e4m3 queries, e2m1 keys" if qk is not None else "bf16") + " (Index Branch)")),
        "data": "synthetic",
        "graph": use_graph,
        "config": {"workload": w.name, "seq_k_lens": (w.seq_k_lens if len(w.seq_k_lens) <= 4 else
                                                       f"{len(w.seq_k_lens)} seqs, total {w.total_k}"),
                   "total_q": w.total_q, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "index_dim": w.index_dim, "block": BLOCK, "top_k": w.top_k,
                   "q_chunk": args.q_chunk, "index_branch": args.index, "main_branch": args.main,
                   "index_projection_dim": args.project_dim or None, "kl_target": bool(args.kl),
                   "kv_cache": "paged (128-row pages, scrambled)" if args.paged else "contiguous",
                   "parallelism": "single GPU"},
        "roofline": roof(dominant) if dominant else None,
        "dominant_kernel": dominant,
        "main_branch_mfma_frac": main_mfma_frac,
        "cpu_baseline": cpu,
        "parity": parity,
        "kernels": kernels,
        "kv_reread": reread,
        "compact_partials": compact,
        "stream_ceilings": ceilings,
        "work": {k_: v for k_, v in wm.items()},
        **extra,
    }
    line["ms_per_step_median"] = ms_median
    ok = parity is None or bool(parity["ok"])
    if args.leg and args.json_out:
        with open(args.json_out, "w") as f:
            f.write(json.dumps(line) + "\n")
    return line, ok


if __name__ == "__main__":
    main()
