"""msa_attend_noalloc: the Main Branch with its partials in the library's own
per-GPU scratch, for callers that cannot allocate.

It runs msa_attend's kernels, so its outputs must equal msa_attend's bit for
bit.  Two calls in a row, the second with a smaller input (and on another
stream) over the scratch the first one left behind; a size beyond the
scratch is rejected on the host before anything is enqueued.
"""
import ctypes

import numpy as np
import pytest
import torch

import block_sparse_long_index_amd as msa
from msa_inputs import custom, generate


def _reference(w, dev, q_chunk=0):
    """Selection, lists and msa_attend's output through the C ABI."""
    t = generate(w, dev)
    dims = msa.dims_for(w, q_chunk=q_chunk)
    bufs = msa.Buffers(dims, dev, want_scores=False)
    msa.index_select(dims, t["q_idx"], t["k_idx"], t["cu_seqlens_q"], t["cu_seqlens_k"], bufs.sel,
                     None, bufs.workspace)
    if msa.attend_reads_lists(dims):
        msa.build_block_query_lists(dims, bufs.sel, t["cu_seqlens_q"], t["cu_seqlens_k"],
                                    bufs.offsets, bufs.entries, bufs.workspace)
    msa.attend(dims, t["q"], t["k"], t["v"], t["cu_seqlens_q"], t["cu_seqlens_k"], bufs.sel,
               bufs.offsets, bufs.entries, bufs.out, bufs.lse, bufs.workspace)
    return t, dims, bufs


def _noalloc(t, dims, bufs, stream=None):
    out = torch.full_like(bufs.out, float("nan"))
    lse = torch.full_like(bufs.lse, float("nan"))
    msa.attend_noalloc(dims, t["q"], t["k"], t["v"], t["cu_seqlens_q"], t["cu_seqlens_k"], bufs.sel,
                       bufs.offsets, bufs.entries, out, lse, stream=stream)
    return out, lse


@pytest.mark.gpu
def test_noalloc_equals_attend_on_two_calls():
    dev = torch.device("cuda:0")
    # a ragged prefill on the lists path, then a smaller decode step on the per-slot path
    big = custom([1500, 900, 700], [1500, 300, 700], num_q_heads=8, num_kv_heads=2, head_dim=64,
                 index_dim=64, top_k=5, seed=71, qkv_std=1.0)
    small = custom([5000, 300, 129], [1, 1, 1], num_q_heads=16, num_kv_heads=8, head_dim=128,
                   index_dim=128, top_k=16, seed=72, qkv_std=1.0)
    tb, db, bb = _reference(big, dev)
    ts, ds, bs = _reference(small, dev)
    assert msa.attend_reads_lists(db) and not msa.attend_reads_lists(ds)
    for d in (db, ds):
        assert msa.workspace_size(d, msa.OP_ATTEND) <= msa.NOALLOC_SCRATCH_BYTES
    torch.cuda.synchronize()
    print(f"[noalloc] big {big.total_q} rows, small {small.total_q} rows", flush=True)
    out1, lse1 = _noalloc(tb, db, bb)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        out2, lse2 = _noalloc(ts, ds, bs, stream=side)
    torch.cuda.synchronize()
    assert torch.equal(out1, bb.out) and torch.equal(lse1, bb.lse)
    assert torch.equal(out2, bs.out) and torch.equal(lse2, bs.lse)
    # once more on the first input, after the smaller call left its partials behind
    out3, lse3 = _noalloc(tb, db, bb)
    torch.cuda.synchronize()
    assert torch.equal(out3, bb.out) and torch.equal(lse3, bb.lse)


@pytest.mark.gpu
def test_noalloc_with_passes_equals_attend():
    """A problem whose partials exceed the scratch runs in several passes once
    q_chunk brings one pass under it; the result is msa_attend's."""
    dev = torch.device("cuda:0")
    w = custom([4000], [4000], num_q_heads=64, num_kv_heads=8, head_dim=128, index_dim=128,
               top_k=16, seed=73, qkv_std=1.0)
    full = msa.dims_for(w)
    assert msa.workspace_size(full, msa.OP_ATTEND) > msa.NOALLOC_SCRATCH_BYTES
    t, dims, bufs = _reference(w, dev, q_chunk=100)
    assert msa.workspace_size(dims, msa.OP_ATTEND) <= msa.NOALLOC_SCRATCH_BYTES
    out, lse = _noalloc(t, dims, bufs)
    torch.cuda.synchronize()
    assert torch.equal(out, bufs.out) and torch.equal(lse, bufs.lse)


def test_noalloc_rejects_sizes_beyond_the_scratch():
    """Checked on the host before any device call (runs without a GPU)."""
    lib = msa.load_library()
    d = msa.make_dims(batch=1, num_q_heads=64, num_kv_heads=8, head_dim=128, index_dim=128, top_k=16,
                      total_q=32768, total_k=32768, max_q_len=32768, max_k_len=32768)
    assert msa.workspace_size(d, msa.OP_ATTEND) > msa.NOALLOC_SCRATCH_BYTES
    st = lib.msa_attend_noalloc(ctypes.byref(d), *([None] * 11))
    assert st == 5                                       # MSA_ERR_WORKSPACE_TOO_SMALL
    assert b"q_chunk" in lib.msa_last_error()
    assert msa.NOALLOC_SCRATCH_BYTES == 64 << 20
