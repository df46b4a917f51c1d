"""Writes stay inside their buffers, and the debug mode changes nothing but timing.

Guard bands: every output and the workspace are views into larger tensors
whose first and last 256 bytes hold a canary pattern; after the calls the
canaries must be intact (a write past either end of any buffer shows).  Run
for the prefill (lists) and decode paths, the 8-bit index branch, the 4-bit
Main Branch, compact partials and the allocation-free Main Branch.

MSA_DEBUG_SYNC=1 (a host-blocking debugging aid: every stage is followed by a
wait and an error check, and cu_seqlens are validated on the host before any
launch) must give bit-identical outputs, and malformed cu_seqlens must be
rejected before anything runs.
"""
import os

import numpy as np
import pytest
import torch

import block_sparse_long_index_amd as msa
from msa_inputs import custom, generate

pytestmark = pytest.mark.gpu

from gpu_helpers import log  # noqa: E402

GUARD = 256          # bytes of canary on each side
CANARY = 0xA5


def _guarded(shape, dtype, dev):
    """(view, backing tensor): a contiguous view with GUARD canary bytes on each side."""
    n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
    raw = torch.full((GUARD + n + GUARD,), CANARY, dtype=torch.uint8, device=dev)
    view = raw[GUARD:GUARD + n].view(dtype).view(*shape)
    return view, raw


def _intact(raw, name):
    head = raw[:GUARD].cpu().numpy()
    tail = raw[-GUARD:].cpu().numpy()
    assert (head == CANARY).all(), f"{name}: bytes before the buffer were written"
    assert (tail == CANARY).all(), f"{name}: bytes after the buffer were written"


class GuardedBuffers(msa.Buffers):
    """msa.Buffers with every buffer placed between canary bands."""

    def __init__(self, dims, dev, flags_note=""):
        T, G, k = dims.total_q, dims.num_kv_heads, dims.top_k
        U = dims.batch * G * msa.nb_max(dims)
        self.raws = {}
        def g(name, shape, dtype):
            v, raw = _guarded(shape, dtype, dev)
            self.raws[name] = raw
            return v
        self.sel = g("sel", (T, G, k), torch.int32)
        self.sel_score = g("sel_score", (T, G, k), torch.float32)
        self.offsets = g("offsets", (U + 1,), torch.int32)
        self.entries = g("entries", (max(1, T * G * k),), torch.int32)
        self.out = g("out", (T, dims.num_q_heads, dims.head_dim), torch.bfloat16)
        self.lse = g("lse", (T, dims.num_q_heads), torch.float32)
        need = max(msa.workspace_size(dims, op) for op in
                   (msa.OP_INDEX_SELECT, msa.OP_BUILD_LISTS, msa.OP_ATTEND, msa.OP_INDEX_PROJECT))
        self.workspace = g("workspace", (need,), torch.uint8)

    def check(self, tag):
        torch.cuda.synchronize()
        for name, raw in self.raws.items():
            _intact(raw, f"{tag}/{name}")


def _guarded_obj(obj, dev, raws, prefix):
    """Replace every tensor attribute of a quantised-input holder by a guarded copy."""
    for name, t in list(vars(obj).items()):
        if isinstance(t, torch.Tensor):
            v, raw = _guarded(tuple(t.shape), t.dtype, dev)
            setattr(obj, name, v)
            raws[f"{prefix}.{name}"] = raw


CASES = {
    "prefill": custom([1500, 900, 130, 128, 3000, 257], [1500, 300, 130, 1, 2000, 200], num_q_heads=16,
                      num_kv_heads=4, head_dim=128, index_dim=64, top_k=5, seed=141, qkv_std=1.0),
    "decode": custom([5000, 20000, 128, 300, 129], [1, 3, 1, 2, 1], num_q_heads=16, num_kv_heads=8,
                     head_dim=128, index_dim=128, top_k=16, seed=142, qkv_std=1.0),
}


@pytest.mark.parametrize("kind", ["bf16", "compact", "fp8_index", "q8k4_q8kv4", "noalloc"])
@pytest.mark.parametrize("shape", sorted(CASES))
def test_writes_stay_inside_buffers(shape, kind):
    w = CASES[shape]
    dev = torch.device("cuda:0")
    t = generate(w, dev)
    # the allocation-free call needs one pass's partials within its 64 MiB scratch
    dims = msa.dims_for(w, flags=msa.FLAG_COMPACT_PARTIALS if kind == "compact" else 0,
                        q_chunk=500 if kind == "noalloc" else 0)
    if kind == "noalloc":
        assert msa.workspace_size(dims, msa.OP_ATTEND) <= msa.NOALLOC_SCRATCH_BYTES
    bufs = GuardedBuffers(dims, dev)
    log(f"[guards] {shape} {kind}")
    if kind == "noalloc":
        msa.index_select(dims, t["q_idx"], t["k_idx"], t["cu_seqlens_q"], t["cu_seqlens_k"], bufs.sel,
                         bufs.sel_score, bufs.workspace)
        if msa.attend_reads_lists(dims):
            msa.build_block_query_lists(dims, bufs.sel, t["cu_seqlens_q"], t["cu_seqlens_k"],
                                        bufs.offsets, bufs.entries, bufs.workspace)
        msa.attend_noalloc(dims, t["q"], t["k"], t["v"], t["cu_seqlens_q"], t["cu_seqlens_k"], bufs.sel,
                           bufs.offsets, bufs.entries, bufs.out, bufs.lse)
    else:
        fp8 = q8k4 = main = None
        if kind == "fp8_index":
            fp8 = msa.Fp8Index(dims, dev)
            _guarded_obj(fp8, dev, bufs.raws, "fp8")
        if kind == "q8k4_q8kv4":
            q8k4 = msa.Q8K4Index(dims, dev)
            main = msa.Q8KV4Main(dims, dev)
            _guarded_obj(q8k4, dev, bufs.raws, "q8k4")
            _guarded_obj(main, dev, bufs.raws, "q8kv4")
        msa.msa_forward(dims, t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"], t["cu_seqlens_q"],
                        t["cu_seqlens_k"], bufs, fp8=fp8, q8k4=q8k4, fp8_main=main)
    bufs.check(f"{shape}-{kind}")
    assert torch.isfinite(bufs.out.float()).all()


def test_debug_sync_is_bit_identical_and_rejects_bad_seqlens(monkeypatch):
    dev = torch.device("cuda:0")
    for shape, w in sorted(CASES.items()):
        t = generate(w, dev)
        dims = msa.dims_for(w)
        ref = msa.Buffers(dims, dev, want_scores=True)
        msa.msa_forward(dims, t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"], t["cu_seqlens_q"],
                        t["cu_seqlens_k"], ref)
        torch.cuda.synchronize()
        monkeypatch.setenv("MSA_DEBUG_SYNC", "1")
        dbg = msa.Buffers(dims, dev, want_scores=True)
        msa.msa_forward(dims, t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"], t["cu_seqlens_q"],
                        t["cu_seqlens_k"], dbg)
        torch.cuda.synchronize()
        for name in ("sel", "sel_score", "out", "lse"):
            a, b = getattr(ref, name), getattr(dbg, name)
            if a.is_floating_point():    # NaN padding of sel_score compares unequal to itself
                assert torch.equal(torch.isnan(a), torch.isnan(b)), (shape, name)
                a, b = a.nan_to_num(), b.nan_to_num()
            assert torch.equal(a, b), (shape, name)
        # malformed sequence offsets: caught on the host, nothing launched
        bad_q = t["cu_seqlens_q"].clone()
        bad_q[-1] += 1                                   # does not end at total_q
        bad_k = t["cu_seqlens_k"].clone()
        bad_k[1] = bad_k[2] + 1                          # decreases
        for cq, ck in ((bad_q, t["cu_seqlens_k"]), (t["cu_seqlens_q"], bad_k)):
            with pytest.raises(msa.MSAError) as ei:
                msa.index_select(dims, t["q_idx"], t["k_idx"], cq, ck, dbg.sel, None, dbg.workspace)
            assert ei.value.status == 2 and "MSA_DEBUG_SYNC" in str(ei.value)
            with pytest.raises(msa.MSAError):
                msa.attend(dims, t["q"], t["k"], t["v"], cq, ck, dbg.sel, dbg.offsets, dbg.entries,
                           dbg.out, dbg.lse, dbg.workspace)
        monkeypatch.delenv("MSA_DEBUG_SYNC")
        torch.cuda.synchronize()
