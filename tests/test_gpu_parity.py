"""GPU parity of the MSA hot path against the CPU oracle (small and ragged cases).

Every call goes through the C ABI (libmsa.so) via the Python binding.  Sizes
are small enough for the oracle to check every row while spanning several
tiles, ragged tails, Lq < Lk, single-query sequences and the degenerate
selections (top_k = 1; top_k covering every block).
"""
import numpy as np
import pytest
import torch

import block_sparse_long_index_amd as msa
from msa_inputs import custom, generate, workload
from oracle import msa_oracle as O

pytestmark = pytest.mark.gpu

from gpu_helpers import check_out, check_selection, log, problem_from, run_gpu  # noqa: E402


def _full_check(w, q_chunk=0, tag=""):
    log(f"[{tag or w.name}] lens k={w.seq_k_lens} q={w.seq_q_lens} Hq={w.num_q_heads} G={w.num_kv_heads} "
        f"d={w.head_dim} di={w.index_dim} k={w.top_k} chunk={q_chunk}")
    t = generate(w, "cpu")
    dims, bufs, _ = run_gpu(w, t, q_chunk=q_chunk)
    P = problem_from(t, w)
    rows = list(range(w.total_q))
    ref = P.run(rows, want_scores=True)
    sel = bufs.sel.cpu().numpy()
    bad, ties = check_selection(P, rows, sel, bufs.sel_score.cpu().numpy(), ref, w.index_dim)
    log(f"[{tag or w.name}] selection mismatches {len(bad)} near-ties {ties}")
    assert not bad, bad[:5]
    check_out(bufs.out.float().cpu().numpy(), ref["out"], bufs.lse.cpu().numpy(), ref["lse"],
              tag or w.name)
    # Main Branch on the oracle's own selection (same rows)
    return t, dims, bufs, P, ref


def test_tiny_full():
    _full_check(workload("tiny"))


def test_ragged_batch_prefill():
    w = custom([1500, 900, 130, 128, 3000, 257], [1500, 300, 130, 1, 2000, 200], num_q_heads=8,
               num_kv_heads=2, head_dim=64, index_dim=64, top_k=5, seed=21, qkv_std=1.0)
    _full_check(w)


def test_gqa8_d128_prefill():
    w = custom([2200], [2200], num_q_heads=64, num_kv_heads=8, head_dim=128, index_dim=128,
               top_k=16, seed=22, qkv_std=1.0)
    _full_check(w)


def test_decode_path_small():
    w = custom([5000, 20000, 128, 300, 129], [1, 1, 1, 1, 1], num_q_heads=16, num_kv_heads=8,
               head_dim=128, index_dim=128, top_k=16, seed=23, qkv_std=1.0)
    _full_check(w)


@pytest.mark.parametrize("d,hq,g", [(64, 8, 8), (64, 64, 8), (128, 16, 1), (128, 64, 4),
                                     (128, 128, 4), (64, 32, 1)],
                         ids=["d64-hpg1", "d64-hpg8", "d128-hpg16", "d128-hpg16-g4",
                              "d128-hpg32", "d64-hpg32"])
def test_decode_attend_head_layouts(d, hq, g):
    """The decode Main Branch across head dims and heads per group: contexts
    shorter than a block, exactly one block, a ragged last block, and long."""
    w = custom([100, 128, 1300, 9000, 257], [1, 1, 1, 1, 1], num_q_heads=hq, num_kv_heads=g,
               head_dim=d, index_dim=64, top_k=8, seed=27 + d + hq + g, qkv_std=1.0)
    _full_check(w, tag=f"decode-d{d}-hpg{hq // g}")


def test_decode_attend_more_rows_than_one_launch():
    """8200 sequences x 8 new tokens = 65600 rows, one pass: the decode
    attention's rows sit in a grid dimension limited to 65535, so the pass
    takes two launches; rows on both sides of the split are checked."""
    rng = np.random.default_rng(36)
    n = 8200
    lk = [int(x) for x in rng.integers(129, 260, size=n)]
    w = custom(lk, [8] * n, num_q_heads=2, num_kv_heads=1, head_dim=64, index_dim=32, top_k=2,
               seed=36, qkv_std=1.0)
    t = generate(w, "cpu")
    dims, bufs, _ = run_gpu(w, t)
    assert w.total_q > 65535 and not msa.attend_reads_lists(dims)
    P = problem_from(t, w, lazy=True)
    rows = sorted(set(list(range(8)) + list(range(65520, 65560)) + list(range(w.total_q - 8, w.total_q))
                      + [int(x) for x in rng.integers(0, w.total_q, size=32)]))
    ref = P.run(rows, want_scores=True)
    idx = torch.as_tensor(rows)
    bad, ties = check_selection(P, rows, bufs.sel.cpu()[idx].numpy(), bufs.sel_score.cpu()[idx].numpy(),
                                ref, w.index_dim)
    log(f"[rows>65535] selection mismatches {len(bad)} near-ties {ties}")
    assert not bad, bad[:3]
    check_out(bufs.out.cpu()[idx].float().numpy(), ref["out"], bufs.lse.cpu()[idx].numpy(), ref["lse"],
              "rows>65535")


def test_lists_path_more_sequence_groups_than_a_grid_dimension():
    """4100 sequences x 16 KV heads = 65600 (sequence, group) pairs on the
    lists path (400 tokens each, so max_q_len > 8): the list builder runs one
    workgroup per pair, more than a grid's y or z dimension holds.  The lists
    must be the exact inverse of the selection, and sampled rows match the
    oracle."""
    n, L = 4100, 400
    w = custom([L] * n, [L] * n, num_q_heads=16, num_kv_heads=16, head_dim=64, index_dim=32,
               top_k=2, seed=37, qkv_std=1.0)
    dev = torch.device("cuda:0")
    t = generate(w, dev)
    dims = msa.dims_for(w)
    assert msa.attend_reads_lists(dims) and w.batch * w.num_kv_heads > 65535
    bufs = msa.Buffers(dims, dev, want_scores=True)
    msa.msa_forward(dims, t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"], t["cu_seqlens_q"],
                    t["cu_seqlens_k"], bufs)
    torch.cuda.synchronize()
    sel = bufs.sel.cpu().numpy()
    P = problem_from(t, w, lazy=True)
    off, ent = O.build_block_query_lists(sel, P.seq, w.batch, w.num_kv_heads, msa.nb_max(dims))
    assert np.array_equal(bufs.offsets.cpu().numpy(), off)
    assert np.array_equal(bufs.entries.cpu().numpy()[:len(ent)], ent)
    rng = np.random.default_rng(37)
    rows = sorted(set([0, 399, 400, w.total_q - 1] + [int(x) for x in rng.integers(0, w.total_q, 40)]
                      + list(range(65535 // 16 * L, 65535 // 16 * L + 3))))
    ref = P.run(rows, want_scores=True)
    idx = torch.as_tensor(rows)
    bad, ties = check_selection(P, rows, sel[rows], bufs.sel_score.cpu()[idx].numpy(), ref, w.index_dim)
    log(f"[pairs>65535] selection mismatches {len(bad)} near-ties {ties}")
    assert not bad, bad[:3]
    check_out(bufs.out.cpu()[idx].float().numpy(), ref["out"], bufs.lse.cpu()[idx].numpy(), ref["lse"],
              "pairs>65535")


def test_multi_token_decode_path():
    # 4 new tokens x 8 groups = 32 rows: still the split-scan index path
    w = custom([9000, 4100], [4, 3], num_q_heads=32, num_kv_heads=8, head_dim=64, index_dim=32,
               top_k=6, seed=24, qkv_std=1.0)
    _full_check(w)


def test_top_k_one_is_block_local():
    w = custom([1000, 333], [1000, 333], num_q_heads=4, num_kv_heads=2, head_dim=64, index_dim=32,
               top_k=1, seed=25, qkv_std=1.0)
    _full_check(w)


def test_top_k_covering_everything_is_dense():
    w = custom([700, 1100], [700, 1100], num_q_heads=8, num_kv_heads=1, head_dim=128, index_dim=64,
               top_k=9, seed=26, qkv_std=1.0)
    _full_check(w)


def test_top_k_32_and_hpg_32():
    w = custom([6000], [6000], num_q_heads=32, num_kv_heads=1, head_dim=64, index_dim=32,
               top_k=32, seed=27, qkv_std=1.0)
    _full_check(w)


def test_three_groups_non_power_of_two():
    # G = 3: a prefill tile holds 170 queries x 3 groups = 510 of its 512 rows
    w = custom([1900, 700], [1900, 700], num_q_heads=12, num_kv_heads=3, head_dim=64,
               index_dim=64, top_k=5, seed=34, qkv_std=1.0)
    _full_check(w)


def test_six_groups_hpg_16_offset_queries():
    # Lq < Lk with an offset that is not a multiple of the tile: tiles span blocks
    w = custom([2500, 1333], [1111, 1333], num_q_heads=96, num_kv_heads=6, head_dim=128,
               index_dim=32, top_k=7, seed=35, qkv_std=1.0)
    _full_check(w)


def test_hpg_1():
    w = custom([2000], [2000], num_q_heads=4, num_kv_heads=4, head_dim=64, index_dim=32,
               top_k=3, seed=28, qkv_std=1.0)
    _full_check(w)


def test_chunking_is_bitwise_invisible():
    w = custom([3000, 1000], [3000, 1000], num_q_heads=8, num_kv_heads=2, head_dim=128,
               index_dim=64, top_k=4, seed=29, qkv_std=1.0)
    t = generate(w, "cpu")
    _, a, _ = run_gpu(w, t, q_chunk=0)
    _, b, _ = run_gpu(w, t, q_chunk=333)
    _, c, _ = run_gpu(w, t, q_chunk=1)
    for x in (b, c):
        assert torch.equal(a.sel, x.sel)
        assert torch.equal(a.offsets, x.offsets)
        assert torch.equal(a.out, x.out)
        assert torch.equal(a.lse, x.lse)


def test_prefill_split_into_query_chunks_is_bitwise_the_whole():
    """A prefill cut into query-row sub-problems, each with the keys up to its
    last query (the queries are the last Lq of Lk; chunked prefill as a serving
    engine runs it), selects and attends bitwise as the whole prefill does:
    every row's scores, selection and partials depend only on its own
    position.  Chunk edges fall inside 128-token blocks; every chunk keeps
    more than 128 / G rows, so all of them take the prefill kernels."""
    w = custom([2600], [2600], num_q_heads=16, num_kv_heads=2, head_dim=128, index_dim=64,
               top_k=6, seed=31, qkv_std=1.0)
    t = generate(w, "cpu")
    _, whole, g = run_gpu(w, t)
    dev = g["q"].device
    G, K = w.num_kv_heads, w.top_k
    sel = torch.full_like(whole.sel, -7)
    out = torch.zeros_like(whole.out)
    lse = torch.zeros_like(whole.lse)
    edges = [0, 700, 1301, 2048, 2600]
    log(f"[split] chunk edges {edges}")
    for a, z in zip(edges[:-1], edges[1:]):
        d = msa.make_dims(batch=1, num_q_heads=w.num_q_heads, num_kv_heads=G, head_dim=w.head_dim,
                          index_dim=w.index_dim, top_k=K, total_q=z - a, total_k=z,
                          max_q_len=z - a, max_k_len=z)
        assert (z - a) * G > 128 and msa.attend_reads_lists(d)
        cq = torch.tensor([0, z - a], dtype=torch.int32, device=dev)
        ck = torch.tensor([0, z], dtype=torch.int32, device=dev)
        b = msa.Buffers(d, dev)
        msa.index_select(d, g["q_idx"][a:z], g["k_idx"][:z], cq, ck, sel[a:z], workspace=b.workspace)
        msa.build_block_query_lists(d, sel[a:z], cq, ck, b.offsets, b.entries, b.workspace)
        msa.attend(d, g["q"][a:z], g["k"][:z], g["v"][:z], cq, ck, sel[a:z], b.offsets, b.entries,
                   out[a:z], lse[a:z], b.workspace)
    torch.cuda.synchronize()
    assert torch.equal(sel, whole.sel)
    assert torch.equal(out, whole.out)
    assert torch.equal(lse, whole.lse)


def test_deterministic_and_workspace_poison_proof():
    w = custom([2500], [2500], num_q_heads=16, num_kv_heads=2, head_dim=128, index_dim=128,
               top_k=8, seed=30, qkv_std=1.0)
    t = generate(w, "cpu")
    _, a, _ = run_gpu(w, t)
    _, b, _ = run_gpu(w, t, workspace_fill=0xFF)   # all-NaN float workspace
    _, c, _ = run_gpu(w, t, workspace_fill=0x00)
    for x in (b, c):
        assert torch.equal(a.sel, x.sel) and torch.equal(a.sel_score.nan_to_num(), x.sel_score.nan_to_num())
        assert torch.equal(a.entries[: int(a.offsets[-1])], x.entries[: int(x.offsets[-1])])
        assert torch.equal(a.out, x.out) and torch.equal(a.lse, x.lse)


def test_lists_are_exact_inverse():
    w = custom([1500, 900, 4000], [1500, 300, 4000], num_q_heads=8, num_kv_heads=2, head_dim=64,
               index_dim=32, top_k=6, seed=31, qkv_std=1.0)
    t = generate(w, "cpu")
    dims, bufs, _ = run_gpu(w, t)
    P = problem_from(t, w)
    sel = bufs.sel.cpu().numpy()
    off, ent = O.build_block_query_lists(sel, P.seq, P.batch, P.G, P.nb_max)
    n = int(off[-1])
    assert np.array_equal(bufs.offsets.cpu().numpy().astype(np.int64), off)
    assert np.array_equal(bufs.entries[:n].cpu().numpy().astype(np.int64), ent)


@pytest.mark.parametrize("top_k", [2, 4])
def test_lists_when_tiles_reach_more_blocks_than_they_select(top_k):
    """Late query tiles of a long context can select from more blocks than they
    hold selections (128 rows x top_k); the list builder then looks up the
    first position of the selected blocks only.  Lists must still be the exact
    inverse of the selection, and the outputs those of the oracle."""
    w = custom([40000, 9000], [300, 70], num_q_heads=4, num_kv_heads=1, head_dim=64, index_dim=32,
               top_k=top_k, seed=37, qkv_std=1.0)
    t, dims, bufs, P, ref = _full_check(w, tag=f"lists-long-k{top_k}")
    sel = bufs.sel.cpu().numpy()
    off, ent = O.build_block_query_lists(sel, P.seq, P.batch, P.G, P.nb_max)
    n = int(off[-1])
    assert np.array_equal(bufs.offsets.cpu().numpy().astype(np.int64), off)
    assert np.array_equal(bufs.entries[:n].cpu().numpy().astype(np.int64), ent)


def test_attend_on_oracle_selection():
    """Main Branch checked on the oracle's own selection (lists built on GPU)."""
    import block_sparse_long_index_amd as msa
    w = custom([3000, 700], [3000, 700], num_q_heads=16, num_kv_heads=4, head_dim=128,
               index_dim=64, top_k=7, seed=32, qkv_std=1.0)
    t = generate(w, "cpu")
    P = problem_from(t, w)
    ref = P.run()
    dev = torch.device("cuda:0")
    g = {k: v.to(dev) for k, v in t.items()}
    dims = msa.dims_for(w)
    bufs = msa.Buffers(dims, dev)
    bufs.sel.copy_(torch.from_numpy(ref["sel"].astype(np.int32)))
    msa.build_block_query_lists(dims, bufs.sel, g["cu_seqlens_q"], g["cu_seqlens_k"], bufs.offsets,
                                bufs.entries, bufs.workspace)
    msa.attend(dims, g["q"], g["k"], g["v"], g["cu_seqlens_q"], g["cu_seqlens_k"], bufs.sel,
               bufs.offsets, bufs.entries, bufs.out, bufs.lse, bufs.workspace)
    torch.cuda.synchronize()
    check_out(bufs.out.float().cpu().numpy(), ref["out"], bufs.lse.cpu().numpy(), ref["lse"],
              "oracle-selection")


def test_decode_equals_prefill_last_row():
    L = 3333
    wp = custom([L], [L], num_q_heads=16, num_kv_heads=8, head_dim=128, index_dim=128, top_k=16,
                seed=33, qkv_std=1.0)
    t = generate(wp, "cpu")
    _, pre, _ = run_gpu(wp, t)
    td = dict(t)
    td["q"] = t["q"][L - 1:L].clone()
    td["q_idx"] = t["q_idx"][L - 1:L].clone()
    td["cu_seqlens_q"] = torch.tensor([0, 1], dtype=torch.int32)
    wd = custom([L], [1], 16, 8, 128, 128, 16, 33)
    _, dec, _ = run_gpu(wd, td)
    assert torch.equal(dec.sel[0], pre.sel[L - 1])
    d = (dec.out[0].float() - pre.out[L - 1].float()).abs().max().item()
    assert d <= 1e-2, d


def test_empty_query_set():
    import block_sparse_long_index_amd as msa
    dims = msa.make_dims(batch=1, num_q_heads=4, num_kv_heads=1, head_dim=64, index_dim=32, top_k=4,
                         total_q=0, total_k=256, max_q_len=0, max_k_len=256)
    dev = torch.device("cuda:0")
    q = torch.zeros((0, 4, 64), dtype=torch.bfloat16, device=dev)
    kv = torch.zeros((256, 1, 64), dtype=torch.bfloat16, device=dev)
    qi = torch.zeros((0, 1, 32), dtype=torch.bfloat16, device=dev)
    ki = torch.zeros((256, 32), dtype=torch.bfloat16, device=dev)
    cuq = torch.tensor([0, 0], dtype=torch.int32, device=dev)
    cuk = torch.tensor([0, 256], dtype=torch.int32, device=dev)
    bufs = msa.msa_forward(dims, q, kv, kv, qi, ki, cuq, cuk)
    # a decode-shaped step: the forward does not build the lists; built on their own
    # for no queries they are all empty
    assert not msa.attend_reads_lists(dims)
    msa.build_block_query_lists(dims, bufs.sel, cuq, cuk, bufs.offsets, bufs.entries, bufs.workspace)
    torch.cuda.synchronize()
    assert int(bufs.offsets[-1]) == 0


def test_verification_shapes_two_and_four_row_tiles():
    # speculative-decoding verification: 8 and 16 new tokens x 8 groups = 64 / 128 rows per
    # sequence (two / four row tiles of the split-scan index kernel), ragged contexts, tokens
    # that straddle a block boundary; attention through the per-(query, slot) kernel (<= 8
    # queries) and the list-based kernel (16 queries)
    for lq, seed in ((8, 36), (16, 37)):
        w = custom([7000, 4100, 300, 2049], [lq, lq, 5, lq], num_q_heads=32, num_kv_heads=8,
                   head_dim=128, index_dim=128, top_k=8, seed=seed, qkv_std=1.0)
        _full_check(w, tag=f"verify{lq}")


def test_decode_topk_long_rows_and_many_survivors():
    # decode selection from the block-score buffer: a row with exactly 2048 earlier blocks
    # whose scores make more candidates reach the selection threshold than LDS gathers
    # (in every wave, the blocks of lanes 0..13 tie at 2048, lane 14's at 1024, the rest 1:
    # each wave's threshold is a 1024 key, so 449 keys reach the row's: the list-merge
    # fallback), and a row with 3000 earlier blocks (candidates beyond the 8 per thread, 2048
    # per row, held in registers)
    lk = [2048 * 128 + 100, 3000 * 128 + 5, 777]
    w = custom(lk, [1, 1, 1], num_q_heads=2, num_kv_heads=1, head_dim=64, index_dim=32,
               top_k=16, seed=38, qkv_std=1.0)
    t = generate(w, "cpu")
    n0 = lk[0]
    beta = np.arange(n0) // 128
    lane = beta % 64
    c = np.where(lane < 14, 2048.0, np.where(lane == 14, 1024.0, 1.0))
    ki = torch.zeros((n0, 32), dtype=torch.float32)
    ki[:, 0] = torch.from_numpy(c)
    t["k_idx"][:n0] = ki.to(torch.bfloat16)
    qi = torch.zeros((1, 1, 32), dtype=torch.bfloat16)
    qi[0, 0, 0] = 1.0
    t["q_idx"][0:1] = qi
    dims, bufs, _ = run_gpu(w, t)
    P = problem_from(t, w)
    rows = [0, 1, 2]
    ref = P.run(rows, want_scores=True)
    sel = bufs.sel.cpu().numpy()
    # ties broken by the lower block id: blocks 0..13 and 64, then the local block 2048
    assert list(ref["sel"][0][0]) == list(range(14)) + [64, 2048]
    bad, ties = check_selection(P, rows, sel, bufs.sel_score.cpu().numpy(), ref, w.index_dim)
    log(f"[long-rows] selection mismatches {len(bad)} near-ties {ties}")
    assert np.array_equal(sel[0], ref["sel"][0])
    assert not bad, bad[:3]
    check_out(bufs.out.float().cpu().numpy(), ref["out"], bufs.lse.cpu().numpy(), ref["lse"],
              "long-rows")
