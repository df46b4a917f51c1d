"""Paged key cache (block_table in msa_dims_t): the same problem laid out in
128-row pages in scrambled order must give bit-for-bit the results of the
contiguous layout, which is itself checked against the oracle here.  Unused
pages and the unused tail rows of each sequence's last page hold NaN, so a
kernel that reads a row it should not would show up in the outputs."""
import numpy as np
import pytest
import torch

import block_sparse_long_index_amd as msa
from msa_inputs import custom, generate, generate_projection

pytestmark = pytest.mark.gpu

from gpu_helpers import check_out, check_selection, log, problem_from  # noqa: E402

SPARE_PAGES = 7


def _paged(w, t, seed=0):
    """Scatter the contiguous key rows of t into a scrambled page layout."""
    rng = np.random.default_rng(seed)
    cu_k = t["cu_seqlens_k"].numpy()
    nblk = [(int(cu_k[b + 1] - cu_k[b]) + 127) // 128 for b in range(w.batch)]
    pages = sum(nblk) + SPARE_PAGES
    perm = rng.permutation(pages)
    mb = max(nblk) + 2
    table = np.full((w.batch, mb), -1, dtype=np.int32)
    i = 0
    for b in range(w.batch):
        for beta in range(nblk[b]):
            table[b, beta] = perm[i]
            i += 1
    rows = np.array([int(table[b, j // 128]) * 128 + j % 128
                     for b in range(w.batch) for j in range(int(cu_k[b + 1] - cu_k[b]))],
                    dtype=np.int64)
    out = {}
    for name in ("k", "v", "k_idx"):
        src = t[name]
        cache = torch.full((pages * 128,) + tuple(src.shape[1:]), float("nan"), dtype=src.dtype)
        cache[torch.from_numpy(rows)] = src
        out[name] = cache
    return out, torch.from_numpy(table), pages, rows


def _dims(w, dev, table=None, pages=0):
    d = msa.dims_for(w)
    if table is None:
        return d
    return msa.make_dims(batch=w.batch, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                         head_dim=w.head_dim, index_dim=w.index_dim, top_k=w.top_k,
                         total_q=w.total_q, total_k=pages * 128, max_q_len=max(w.seq_q_lens),
                         max_k_len=max(w.seq_k_lens), block_table=table)


def _forward(dims, g, k, v, k_idx, fp8=False, want_kl=False):
    dev = g["q"].device
    bufs = msa.Buffers(dims, dev, want_scores=True)
    f8 = msa.Fp8Index(dims, dev) if fp8 else None
    if not want_kl:
        msa.msa_forward(dims, g["q"], k, v, g["q_idx"], k_idx, g["cu_seqlens_q"], g["cu_seqlens_k"],
                        bufs, fp8=f8)
        torch.cuda.synchronize()
        return bufs, f8, None
    msa.index_select(dims, g["q_idx"], k_idx, g["cu_seqlens_q"], g["cu_seqlens_k"], bufs.sel,
                     bufs.sel_score, bufs.workspace)
    msa.build_block_query_lists(dims, bufs.sel, g["cu_seqlens_q"], g["cu_seqlens_k"], bufs.offsets,
                                bufs.entries, bufs.workspace)
    mass = torch.empty((dims.total_q, dims.num_kv_heads, dims.top_k), dtype=torch.float32, device=dev)
    msa.attend_with_mass(dims, g["q"], k, v, g["cu_seqlens_q"], g["cu_seqlens_k"], bufs.sel,
                         bufs.offsets, bufs.entries, bufs.out, mass, bufs.lse, bufs.workspace)
    kl = torch.empty((dims.total_q, dims.num_kv_heads), dtype=torch.float32, device=dev)
    msa.index_kl(dims, g["q_idx"], k_idx, g["cu_seqlens_q"], g["cu_seqlens_k"], bufs.sel,
                 bufs.sel_score, mass, kl)
    torch.cuda.synchronize()
    return bufs, f8, (mass, kl)


def _check_paged(w, tag, fp8=False, want_kl=False, oracle=True):
    dev = torch.device("cuda:0")
    t = generate(w, "cpu")
    g = {k_: v_.to(dev) for k_, v_ in t.items()}
    cache, table, pages, rows = _paged(w, t, seed=w.seed)
    gc = {k_: v_.to(dev) for k_, v_ in cache.items()}
    table_d = table.to(dev)
    d_c = _dims(w, dev)
    d_p = _dims(w, dev, table_d, pages)
    a, fa, xa = _forward(d_c, g, g["k"], g["v"], g["k_idx"], fp8, want_kl)
    b, fb, xb = _forward(d_p, g, gc["k"], gc["v"], gc["k_idx"], fp8, want_kl)
    log(f"[{tag}] lens k={w.seq_k_lens} q={w.seq_q_lens} pages={pages} fp8={fp8} kl={want_kl}")
    if oracle and not fp8:
        P = problem_from(t, w)
        rr = list(range(0, w.total_q, max(1, w.total_q // 300)))
        ref = P.run(rr, want_scores=True)
        bad, _ = check_selection(P, rr, a.sel.cpu().numpy()[rr], a.sel_score.cpu().numpy()[rr], ref,
                                 w.index_dim)
        assert not bad, bad[:3]
        check_out(a.out.float().cpu().numpy()[rr], ref["out"], a.lse.cpu().numpy()[rr], ref["lse"], tag)
    assert torch.equal(a.sel, b.sel)
    assert torch.equal(a.sel_score.nan_to_num(), b.sel_score.nan_to_num())
    assert torch.equal(a.out, b.out) and torch.equal(a.lse, b.lse)
    assert not torch.isnan(b.out.float()).any()
    if fp8:
        assert torch.equal(fa.q_idx8, fb.q_idx8) and torch.equal(fa.q_exp, fb.q_exp)
        kr = torch.from_numpy(rows).to(dev)
        assert torch.equal(fa.k_idx8, fb.k_idx8.index_select(0, kr))
        tb = table.numpy()
        for bb in range(w.batch):
            nb = (w.seq_k_lens[bb] + 127) // 128
            assert torch.equal(fa.k_exp[bb, :nb].cpu(), fb.k_exp.cpu()[torch.from_numpy(tb[bb, :nb]).long()])
    if want_kl:
        assert torch.equal(xa[0], xb[0]) and torch.equal(xa[1], xb[1])


def test_dims_keep_the_block_table_alive():
    # the struct stores only the table's device address: the dims hold the tensor
    import gc
    import weakref
    t = torch.zeros((2, 4), dtype=torch.int32, device="cuda:0")
    ref, addr = weakref.ref(t), t.data_ptr()
    d = msa.make_dims(batch=2, num_q_heads=4, num_kv_heads=2, head_dim=64, index_dim=64, top_k=4,
                      total_q=2, total_k=8 * 128, max_q_len=1, max_k_len=500, block_table=t)
    del t
    gc.collect()
    assert ref() is not None and d.block_table == addr and d.kv_pages == 8


def test_paged_prefill_bf16():
    w = custom([1500, 900, 130, 3000], [1500, 300, 130, 2000], num_q_heads=16, num_kv_heads=4,
               head_dim=128, index_dim=64, top_k=6, seed=71, qkv_std=1.0)
    _check_paged(w, "paged-prefill")


def test_paged_decode_and_verify_bf16():
    w = custom([5000, 20000, 128, 300, 4100], [1, 1, 1, 1, 1], num_q_heads=16, num_kv_heads=8,
               head_dim=128, index_dim=128, top_k=16, seed=72, qkv_std=1.0)
    _check_paged(w, "paged-decode")
    w = custom([7000, 4100, 300, 2049], [8, 8, 5, 8], num_q_heads=32, num_kv_heads=8, head_dim=64,
               index_dim=128, top_k=8, seed=73, qkv_std=1.0)
    _check_paged(w, "paged-verify8")


def test_paged_fp8_prefill_and_decode():
    w = custom([1500, 900, 2000], [1500, 300, 2000], num_q_heads=16, num_kv_heads=4, head_dim=64,
               index_dim=128, top_k=6, seed=74, qkv_std=1.0)
    _check_paged(w, "paged-fp8-prefill", fp8=True)
    w = custom([5000, 20000, 300], [1, 2, 1], num_q_heads=16, num_kv_heads=8, head_dim=128,
               index_dim=64, top_k=16, seed=75, qkv_std=1.0)
    _check_paged(w, "paged-fp8-decode", fp8=True)


def test_paged_kl_target():
    w = custom([1500, 900], [1500, 900], num_q_heads=16, num_kv_heads=4, head_dim=64, index_dim=64,
               top_k=5, seed=76, qkv_std=1.0)
    _check_paged(w, "paged-kl", want_kl=True, oracle=False)


# model width 256: the large-tile kernel writes the keys; 2048: K is split over
# 4 workgroup slices (12 tiles), and the reduce kernel writes them through the table
@pytest.mark.parametrize("D", [256, 2048])
def test_paged_projection_writes_the_pages(D):
    w = custom([700, 2000, 130], [1, 2000, 3], num_q_heads=16, num_kv_heads=4, head_dim=64,
               index_dim=64, top_k=5, seed=77, qkv_std=1.0)
    dev = torch.device("cuda:0")
    t = generate(w, "cpu")
    p = generate_projection(w, D, "cpu")
    cache, table, pages, rows = _paged(w, t)
    g = {k_: v_.to(dev) for k_, v_ in t.items()}
    gp = {k_: v_.to(dev) for k_, v_ in p.items()}
    table_d = table.to(dev)
    d_c, d_p = _dims(w, dev), _dims(w, dev, table_d, pages)
    qa = torch.empty((w.total_q, w.num_kv_heads, w.index_dim), dtype=torch.bfloat16, device=dev)
    qb = torch.empty_like(qa)
    ka = g["k_idx"].clone()
    kb = cache["k_idx"].to(dev)
    msa.index_project(d_c, gp["x"], gp["w_q"], gp["w_k"], g["cu_seqlens_q"], g["cu_seqlens_k"], qa, ka)
    msa.index_project(d_p, gp["x"], gp["w_q"], gp["w_k"], g["cu_seqlens_q"], g["cu_seqlens_k"], qb, kb)
    torch.cuda.synchronize()
    assert torch.equal(qa, qb)
    kr = torch.from_numpy(rows).to(dev)
    assert torch.equal(ka, kb.index_select(0, kr))
    used = np.zeros(pages * 128, dtype=bool)
    used[rows] = True
    assert torch.isnan(kb[torch.from_numpy(~used).to(dev)].float()).all()
