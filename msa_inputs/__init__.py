"""Seeded synthetic inputs for the MSA hot path.

This module is shared by the oracle tests, the GPU parity tests and the
benchmark.  It holds random draws and the shape of the synthetic workloads
only: none of the method's arithmetic (scoring, pooling, selection,
attention) lives here.

Workload recipe (the pages measure no public suite for this path, so
nothing stands in for one; the shapes follow the pages' stated design,
MSA guide at ai-tool-zukan.com/minimax-msa-guide, table in section
"ブロック単位選択の数値設計": 128-token blocks, 16 blocks per query and group):

* Per sequence, one centroid per 128-token block, ``c_beta ~ N(0, I)`` of
  the index dimension.  Index key of token j: ``c_{beta(j)} + 0.5 * eps_j``.
* Index queries are either plain ``N(0, 1)`` (``planted_q=False``) or
  *planted*: for every (query, group) draw 16 blocks uniformly with
  replacement among the blocks strictly before the query's own block and
  set ``q_idx = 0.25 * sum(c) + 0.5 * eta`` (no draw when the query sits in
  block 0: then ``q_idx = 0.5 * eta``).
* Q, K, V ~ ``N(0, 1) * qkv_std`` then cast to bf16 (round to nearest even).

All draws go through one ``torch.Generator`` seeded with the workload seed,
in a fixed order and in fixed row chunks, so a (workload, seed, device,
torch version) tuple always gives the same tensors.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

BLOCK = 128
_ROW_CHUNK = 8192  # rows per draw; part of the recipe (changing it changes values)


@dataclass
class Workload:
    name: str
    seq_k_lens: list          # context length per sequence (keys)
    seq_q_lens: list          # queries per sequence (the last ones of its keys)
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    index_dim: int
    top_k: int
    seed: int
    qkv_std: float
    planted_q: bool
    n_planted: int = 16
    noise: float = 0.5
    block: int = BLOCK
    note: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return len(self.seq_k_lens)

    @property
    def total_q(self) -> int:
        return int(sum(self.seq_q_lens))

    @property
    def total_k(self) -> int:
        return int(sum(self.seq_k_lens))


def _decode_lengths(seed: int, batch: int, lo_blocks: int, hi_blocks: int) -> list:
    rng = np.random.Generator(np.random.PCG64(seed))
    nblk = rng.integers(lo_blocks, hi_blocks, size=batch, endpoint=True)
    return [int(BLOCK * n) for n in nblk]


def workload(name: str, **overrides) -> Workload:
    """The named synthetic workloads (sizes as the benchmark and tests use them)."""
    big = dict(num_q_heads=64, num_kv_heads=8, head_dim=128, index_dim=128, top_k=16,
               qkv_std=1.0 / math.sqrt(128.0), planted_q=True)
    if name == "tiny":
        w = Workload("tiny", [2048], [2048], 4, 1, 64, 32, 4, 1001, 1.0, False,
                     note="1 seq, L=2048, 4/1 heads, d=64, d_idx=32, top-k 4 incl. local")
    elif name == "p32k":
        w = Workload("p32k", [32768], [32768], seed=1002, **big,
                     note="1 seq, L=32768, 64/8 heads, d=128, d_idx=128, top-k 16")
    elif name == "p32k_peaky":
        b = dict(big, qkv_std=1.0)
        w = Workload("p32k_peaky", [32768], [32768], seed=1002, **b,
                     note="as p32k with Q/K/V ~ N(0,1) (peaked softmax)")
    elif name == "p128k":
        w = Workload("p128k", [131072], [131072], seed=1003, **big,
                     note="1 seq, L=131072, 64/8 heads, d=128, d_idx=128, top-k 16")
    elif name == "p1m":
        w = Workload("p1m", [1048576], [1048576], seed=1005, **big,
                     note="1 seq, L=1048576, 64/8 heads, d=128, d_idx=128, top-k 16")
    elif name == "decode":
        lens = _decode_lengths(1004, 32, 512, 2048)
        w = Workload("decode", lens, [1] * len(lens), seed=1004, **big,
                     note="32 seqs x 1 new token, contexts 128*U{512..2048}")
    elif name in ("verify2", "verify4", "verify8"):
        # speculative-decoding verification: the decode contexts, n new tokens each
        n = int(name[-1])
        lens = _decode_lengths(1004, 32, 512, 2048)
        w = Workload(name, lens, [n] * len(lens), seed=1006, **big,
                     note=f"32 seqs x {n} new tokens, contexts 128*U{{512..2048}}")
    else:
        raise KeyError(name)
    for k_, v_ in overrides.items():
        setattr(w, k_, v_)
    return w


def custom(seq_k_lens, seq_q_lens, num_q_heads, num_kv_heads, head_dim, index_dim, top_k,
           seed, qkv_std=1.0, planted_q=True, name="custom") -> Workload:
    return Workload(name, list(seq_k_lens), list(seq_q_lens), num_q_heads, num_kv_heads,
                    head_dim, index_dim, top_k, seed, qkv_std, planted_q)


def _randn(gen, shape, device, std=1.0):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * std


def generate(w: Workload, device="cpu") -> dict:
    """Draw every input tensor of workload ``w`` on ``device``.

    Returns a dict of contiguous tensors::

        q      bf16 [total_q, Hq, d]        k, v   bf16 [total_k, Hkv, d]
        q_idx  bf16 [total_q, Hkv, d_idx]   k_idx  bf16 [total_k, d_idx]
        cu_seqlens_q, cu_seqlens_k  int32 [batch + 1]

    Query i of sequence b sits at position ``Lk_b - Lq_b + i`` of that sequence.
    """
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(int(w.seed))
    G, Hq, d, di = w.num_kv_heads, w.num_q_heads, w.head_dim, w.index_dim
    for lq, lk in zip(w.seq_q_lens, w.seq_k_lens):
        if not (0 <= lq <= lk):
            raise ValueError("each sequence needs 0 <= Lq <= Lk")
    tq, tk = w.total_q, w.total_k
    bf = torch.bfloat16
    k_idx = torch.empty((tk, di), dtype=bf, device=device)
    q_idx = torch.empty((tq, G, di), dtype=bf, device=device)
    q = torch.empty((tq, Hq, d), dtype=bf, device=device)
    k = torch.empty((tk, G, d), dtype=bf, device=device)
    v = torch.empty((tk, G, d), dtype=bf, device=device)

    koff = 0
    qoff = 0
    for lq, lk in zip(w.seq_q_lens, w.seq_k_lens):
        nb = (lk + w.block - 1) // w.block
        cent = _randn(gen, (max(nb, 1), di), device)
        for r0 in range(0, lk, _ROW_CHUNK):
            r1 = min(lk, r0 + _ROW_CHUNK)
            blk = torch.arange(r0, r1, device=device) // w.block
            eps = _randn(gen, (r1 - r0, di), device)
            k_idx[koff + r0:koff + r1] = (cent[blk] + w.noise * eps).to(bf)
        first_pos = lk - lq
        for r0 in range(0, lq, _ROW_CHUNK):
            r1 = min(lq, r0 + _ROW_CHUNK)
            n = r1 - r0
            eta = _randn(gen, (n, G, di), device)
            if w.planted_q:
                pos = torch.arange(first_pos + r0, first_pos + r1, device=device)
                own = (pos // w.block).to(torch.float32)           # blocks strictly before own
                u = torch.rand((n, G, w.n_planted), generator=gen, device=device)
                pick = torch.floor(u * own[:, None, None]).to(torch.int64)
                pick = torch.minimum(pick, (own[:, None, None] - 1).clamp(min=0).to(torch.int64))
                acc = torch.zeros((n, G, di), dtype=torch.float32, device=device)
                for t in range(w.n_planted):
                    acc += cent[pick[:, :, t]]
                has = (own > 0).to(torch.float32)[:, None, None]
                qi = 0.25 * acc * has + w.noise * eta
            else:
                qi = eta
            q_idx[qoff + r0:qoff + r1] = qi.to(bf)
        koff += lk
        qoff += lq
    # main-branch tensors after all index tensors, in fixed row chunks
    for r0 in range(0, tq, _ROW_CHUNK):
        r1 = min(tq, r0 + _ROW_CHUNK)
        q[r0:r1] = _randn(gen, (r1 - r0, Hq, d), device, w.qkv_std).to(bf)
    for t in (k, v):
        for r0 in range(0, tk, _ROW_CHUNK):
            r1 = min(tk, r0 + _ROW_CHUNK)
            t[r0:r1] = _randn(gen, (r1 - r0, G, d), device, w.qkv_std).to(bf)

    cu_q = torch.zeros(w.batch + 1, dtype=torch.int32)
    cu_k = torch.zeros(w.batch + 1, dtype=torch.int32)
    cu_q[1:] = torch.tensor(np.cumsum(w.seq_q_lens), dtype=torch.int32)
    cu_k[1:] = torch.tensor(np.cumsum(w.seq_k_lens), dtype=torch.int32)
    return dict(q=q, k=k, v=v, q_idx=q_idx, k_idx=k_idx,
                cu_seqlens_q=cu_q.to(device), cu_seqlens_k=cu_k.to(device))


def sample_rows(w: Workload, n_random: int, seed: int = 7) -> list:
    """Global query rows for sampled checks: the first two blocks' ends, random
    rows, and the first/last row of every sequence's last block."""
    rng = np.random.Generator(np.random.PCG64(seed))
    rows = set()
    qoff = 0
    for lq in w.seq_q_lens:
        if lq == 0:
            continue
        for r in (0, min(lq - 1, 127), min(lq - 1, 128), min(lq - 1, 255)):
            rows.add(qoff + r)
        rows.add(qoff + lq - 1)
        rows.add(qoff + max(0, lq - 1 - ((lq - 1) % BLOCK)))
        qoff += lq
    tq = w.total_q
    if tq > 0 and n_random > 0:
        rows.update(int(x) for x in rng.integers(0, tq, size=n_random))
    return sorted(rows)


def generate_projection(w: Workload, model_dim: int, device="cpu", seed_offset: int = 100) -> dict:
    """Layer input and index-projection weights for workload ``w``.

    x: bf16 [total_q, model_dim] ~ N(0, 1) (one row per new token, query-row
    order); w_q: bf16 [num_kv_heads * index_dim, model_dim] and w_k: bf16
    [index_dim, model_dim] ~ N(0, 1/model_dim), so projected values are of
    order one.  Drawn with their own generator (seed + seed_offset) in fixed
    row chunks, so they do not disturb the other inputs of the workload.
    """
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(int(w.seed) + int(seed_offset))
    G, di, D = w.num_kv_heads, w.index_dim, int(model_dim)
    bf = torch.bfloat16
    sw = float(D) ** -0.5
    w_q = _randn(gen, (G * di, D), device, sw).to(bf)
    w_k = _randn(gen, (di, D), device, sw).to(bf)
    x = torch.empty((w.total_q, D), dtype=bf, device=device)
    for r0 in range(0, w.total_q, _ROW_CHUNK):
        r1 = min(w.total_q, r0 + _ROW_CHUNK)
        x[r0:r1] = _randn(gen, (r1 - r0, D), device).to(bf)
    return dict(x=x.contiguous(), w_q=w_q.contiguous(), w_k=w_k.contiguous())


def paged_layout(w: Workload, seed: int = 0, spare_pages: int = 7):
    """A scrambled paged placement of the workload's key rows (serving-style
    key cache): every sequence's 128-token blocks get distinct pages drawn as
    a random permutation (numpy PCG64(seed)) of ``sum(blocks) + spare_pages``
    pages.  Returns (block_table int32 [batch, max_blocks + 2], -1 past each
    sequence's blocks; cache row of every contiguous key row int64
    [total_k]; page count)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    nblk = [(int(n) + BLOCK - 1) // BLOCK for n in w.seq_k_lens]
    pages = sum(nblk) + int(spare_pages)
    perm = rng.permutation(pages).astype(np.int32)
    table = np.full((w.batch, max(nblk) + 2), -1, dtype=np.int32)
    rows = np.empty(w.total_k, dtype=np.int64)
    i = off = 0
    for b, n in enumerate(w.seq_k_lens):
        table[b, :nblk[b]] = perm[i:i + nblk[b]]
        i += nblk[b]
        j = np.arange(int(n))
        rows[off:off + int(n)] = table[b, j // BLOCK].astype(np.int64) * BLOCK + j % BLOCK
        off += int(n)
    return torch.from_numpy(table), torch.from_numpy(rows), pages


def to_pages(src: torch.Tensor, rows: torch.Tensor, pages: int, fill=0.0) -> torch.Tensor:
    """Copy contiguous key rows ``src`` [total_k, ...] into a paged cache of
    ``pages * 128`` rows at ``rows``; every other row holds ``fill``."""
    cache = torch.full((pages * BLOCK,) + tuple(src.shape[1:]), fill, dtype=src.dtype,
                       device=src.device)
    cache[rows.to(src.device)] = src
    return cache
