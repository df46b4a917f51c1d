"""GPU parity of the Index Branch with 4-bit index keys (Q8KV4) against the oracle.

The oracle quantises the same bf16 inputs itself (oracle/fp8_index.py for the
queries, oracle/fp4_index.py for the keys) and runs the unquantised oracle on
the dequantised values; nothing it uses comes from the GPU.  Checked: query
codes and exponents, packed key codes and per-32 exponents, bit for bit; the
selection against the exact scores of the dequantised values, allowing only
the choices the matrix cores' error bound leaves open (the E2M1 x E4M3
microscaled MFMA sums products as the fp8 one does: within 2^-10 of
sum_c |q_c k_c| per token score), with the reported block scores inside that
bound; the output of the whole forward against the oracle's Main Branch on
the selection made.  Small cases check every row; the full-size workloads
check sampled rows in the configuration the benchmark times.
"""
import numpy as np
import pytest
import torch

import block_sparse_long_index_amd as msa
from msa_inputs import custom, generate, paged_layout, sample_rows, to_pages, workload
from oracle import fp4_index as F4
from oracle import fp8_index as F8
from oracle import msa_oracle as O

pytestmark = pytest.mark.gpu

from gpu_helpers import LazyRows, log  # noqa: E402
from test_gpu_fp8 import _DeqQ, check_rows_fp8  # noqa: E402


def _run(w, t, q_chunk=0, dims=None, k_idx=None):
    dev = torch.device("cuda:0")
    g = {k: v.to(dev) for k, v in t.items()}
    dims = dims or msa.dims_for(w, q_chunk=q_chunk)
    bufs = msa.Buffers(dims, dev, want_scores=True)
    qk = msa.Q8K4Index(dims, dev)
    qk.k_idx4.fill_(0x77)          # rows no sequence owns: codes of 6.0 at 2^127
    qk.k_exp4.fill_(254)
    msa.msa_forward(dims, g["q"], g["k"] if k_idx is None else k_idx[1],
                    g["v"] if k_idx is None else k_idx[2], g["q_idx"],
                    g["k_idx"] if k_idx is None else k_idx[0], g["cu_seqlens_q"],
                    g["cu_seqlens_k"], bufs, q8k4=qk)
    torch.cuda.synchronize()
    return dims, bufs, qk


def _oracle_codes(t):
    qc, qe = F8.quantize_q_idx(t["q_idx"].double().numpy())
    kc, ke = F4.quantize_k_idx4(t["k_idx"].double().numpy())
    return qc, qe, kc, ke


def _check_codes(qk, qc, qe, kc, ke, tag, rows=None):
    gk, gke = qk.k_idx4.cpu().numpy(), qk.k_exp4.cpu().numpy()
    if rows is not None:
        gk, gke = gk[rows], gke[rows]
    nq = int((qk.q_idx8.cpu().numpy() != qc).sum())
    nk = int((gk != F4.pack(kc)).sum())
    log(f"[{tag}] code mismatches q {nq}/{qc.size} k {nk}/{gk.size}")
    assert np.array_equal(qk.q_exp.cpu().numpy(), qe)
    assert np.array_equal(gke, ke)
    assert nq == 0 and nk == 0


def _full_check(w, tag, q_chunk=0, plant=None):
    log(f"[{tag}] lens k={w.seq_k_lens} q={w.seq_q_lens} Hq={w.num_q_heads} G={w.num_kv_heads} "
        f"d={w.head_dim} di={w.index_dim} k={w.top_k} chunk={q_chunk}")
    t = generate(w, "cpu")
    if plant:
        plant(t)
    dims, bufs, qk = _run(w, t, q_chunk)
    qc, qe, kc, ke = _oracle_codes(t)
    _check_codes(qk, qc, qe, kc, ke, tag)
    f = lambda x: x.double().numpy()
    P = O.Problem(f(t["q"]), f(t["k"]), f(t["v"]), F8.dequantize_q_idx(qc, qe),
                  F4.dequantize_k_idx4(kc, ke), t["cu_seqlens_q"].numpy(),
                  t["cu_seqlens_k"].numpy(), w.top_k)
    rows = list(range(w.total_q))
    ref = P.run(rows, want_scores=True)
    check_rows_fp8(P, rows, bufs.sel.cpu().numpy(), bufs.sel_score.cpu().numpy(), ref,
                   bufs.out.float().cpu().numpy(), bufs.lse.cpu().numpy(), tag)
    return t, bufs, qk


def test_q8k4_tiny():
    _full_check(workload("tiny"), "q8k4-tiny")


def test_q8k4_ragged_prefill_di64():
    w = custom([1500, 900, 130, 128, 3000, 257], [1500, 300, 130, 1, 2000, 200], num_q_heads=8,
               num_kv_heads=2, head_dim=64, index_dim=64, top_k=5, seed=61, qkv_std=1.0)
    _full_check(w, "q8k4-ragged")


def test_q8k4_gqa8_di128():
    w = custom([2200, 700], [2200, 700], num_q_heads=64, num_kv_heads=8, head_dim=128,
               index_dim=128, top_k=16, seed=62, qkv_std=1.0)
    _full_check(w, "q8k4-gqa8")


def test_q8k4_three_groups_di32_k32():
    w = custom([5000], [5000], num_q_heads=12, num_kv_heads=3, head_dim=64, index_dim=32,
               top_k=32, seed=63, qkv_std=1.0)
    _full_check(w, "q8k4-g3")


def test_q8k4_decode_path():
    w = custom([5000, 20000, 128, 300, 129], [1, 1, 1, 1, 1], num_q_heads=16, num_kv_heads=8,
               head_dim=128, index_dim=128, top_k=16, seed=64, qkv_std=1.0)
    _full_check(w, "q8k4-decode")


def test_q8k4_decode_di64_and_di32():
    for di, seed in ((64, 70), (32, 71)):
        w = custom([3000, 9000, 129], [1, 1, 1], num_q_heads=16, num_kv_heads=8, head_dim=64,
                   index_dim=di, top_k=8, seed=seed, qkv_std=1.0)
        _full_check(w, f"q8k4-decode-di{di}")


def test_q8k4_multi_token_decode_di32():
    w = custom([9000, 4100], [4, 3], num_q_heads=32, num_kv_heads=8, head_dim=64, index_dim=32,
               top_k=6, seed=65, qkv_std=1.0)
    _full_check(w, "q8k4-mtd")


def test_q8k4_degenerate_rows_and_groups():
    """All-zero, tiny and huge index rows, an all-zero key block, one key with
    a huge 32-element group next to ordinary ones, signed zeros."""
    w = custom([1300, 700], [1300, 700], num_q_heads=8, num_kv_heads=2, head_dim=64, index_dim=64,
               top_k=4, seed=66, qkv_std=1.0)

    def plant(t):
        qi, ki = t["q_idx"], t["k_idx"]
        qi[5, 0] = 0.0
        qi[6, 1] = -0.0
        qi[700, 0] *= 1e-20
        qi[701, 1] *= 1e20
        qi[702, 0, ::2] = 0.0
        ki[128 * 3:128 * 4] = 0.0                  # sequence 0, block 3: all zero
        ki[1300 + 128 * 2:1300 + 128 * 3] *= 1e-12  # sequence 1, block 2: tiny
        ki[1300 + 5, :32] *= 1e15                   # one huge group in sequence 1, block 0
        ki[200, 32:] = -0.0
        t["q_idx"], t["k_idx"] = qi, ki

    _full_check(w, "q8k4-degenerate", plant=plant)


def test_q8k4_chunking_is_bitwise_invisible():
    w = custom([3000, 1000], [1, 1], num_q_heads=8, num_kv_heads=2, head_dim=128, index_dim=64,
               top_k=4, seed=67, qkv_std=1.0)
    t = generate(w, "cpu")
    _, a, _ = _run(w, t, q_chunk=0)
    _, b, _ = _run(w, t, q_chunk=1)
    assert torch.equal(a.sel, b.sel) and torch.equal(a.out, b.out)


def test_q8k4_decode_on_a_quantised_key_cache():
    """Keys quantised once (queries left out), then steps that quantise only
    their queries: the same selection and output as quantising both."""
    w = custom([7000, 3000, 12000], [1, 1, 1], num_q_heads=16, num_kv_heads=8, head_dim=128,
               index_dim=128, top_k=16, seed=69, qkv_std=1.0)
    t = generate(w, "cpu")
    dims, ref, ref4 = _run(w, t)
    dev = torch.device("cuda:0")
    g = {k: v.to(dev) for k, v in t.items()}
    qk = msa.Q8K4Index(dims, dev)
    qk.q_idx8.fill_(0x7F)      # NaN codes: must be overwritten by the query-only calls
    msa.index_quantize_q8k4(dims, None, g["k_idx"], g["cu_seqlens_k"], qk)
    torch.cuda.synchronize()
    assert torch.equal(qk.k_idx4, ref4.k_idx4) and torch.equal(qk.k_exp4, ref4.k_exp4)
    assert int((qk.q_idx8 == 0x7F).sum()) == qk.q_idx8.numel()   # queries untouched
    bufs = msa.Buffers(dims, dev, want_scores=True)
    for _ in range(2):
        msa.msa_forward(dims, g["q"], g["k"], g["v"], g["q_idx"], None, g["cu_seqlens_q"],
                        g["cu_seqlens_k"], bufs, q8k4=qk)
        torch.cuda.synchronize()
        assert torch.equal(qk.q_idx8, ref4.q_idx8) and torch.equal(qk.q_exp, ref4.q_exp)
        assert torch.equal(bufs.sel, ref.sel) and torch.equal(bufs.out, ref.out)


def test_q8k4_on_exact_values_agrees_with_bf16_path():
    """Index queries already on the E4M3 grid and keys on the E2M1 grid with
    power-of-two group scales: quantising is then the identity, so the 4-bit
    path and the bf16 path score the same exact values, each within its own
    error bound; their selections must agree wherever the oracle's scores
    leave one choice, and any row where they differ must be a near-tie that
    the 4-bit path resolved validly."""
    w = custom([2600, 900], [2600, 900], num_q_heads=16, num_kv_heads=4, head_dim=64,
               index_dim=128, top_k=8, seed=68, qkv_std=1.0)
    t = generate(w, "cpu")
    qc, qe, kc, ke = _oracle_codes(t)
    t["q_idx"] = torch.from_numpy(F8.dequantize_q_idx(qc, qe)).to(torch.bfloat16)
    t["k_idx"] = torch.from_numpy(F4.dequantize_k_idx4(kc, ke)).to(torch.bfloat16)
    dev = torch.device("cuda:0")
    g = {k: v.to(dev) for k, v in t.items()}
    dims = msa.dims_for(w)
    a = msa.Buffers(dims, dev, want_scores=True)
    msa.msa_forward(dims, g["q"], g["k"], g["v"], g["q_idx"], g["k_idx"], g["cu_seqlens_q"],
                    g["cu_seqlens_k"], a)
    _, b, qk = _run(w, t)
    torch.cuda.synchronize()
    # grid values come back as themselves (codes may move a binade: 224 * 2^e = 448 * 2^(e-1))
    qc2, qe2, kc2, ke2 = _oracle_codes(t)
    assert np.array_equal(F8.dequantize_q_idx(qc2, qe2), t["q_idx"].double().numpy())
    assert np.array_equal(F4.dequantize_k_idx4(kc2, ke2), t["k_idx"].double().numpy())
    _check_codes(qk, qc2, qe2, kc2, ke2, "q8k4-exact")
    rows = [int(r) for r in torch.nonzero((a.sel != b.sel).any(dim=-1).any(dim=-1)).flatten()]
    log(f"[q8k4-exact] rows whose selection differs from the bf16 path: {len(rows)}")
    if rows:
        f = lambda x: x.double().numpy()
        P = O.Problem(f(t["q"]), f(t["k"]), f(t["v"]), f(t["q_idx"]), f(t["k_idx"]),
                      t["cu_seqlens_q"].numpy(), t["cu_seqlens_k"].numpy(), w.top_k)
        ref = P.run(rows, want_scores=True)
        ridx = torch.as_tensor(rows)
        check_rows_fp8(P, rows, b.sel.cpu()[ridx].numpy(), b.sel_score.cpu()[ridx].numpy(), ref,
                       b.out.float().cpu()[ridx].numpy(), b.lse.cpu()[ridx].numpy(), "q8k4-exact")


@pytest.mark.parametrize("lens", [([3000, 700, 9000], [3000, 700, 1]), ([5000, 12000, 300], [1, 1, 1])],
                         ids=["prefill", "decode"])
def test_q8k4_paged_cache_matches_contiguous(lens):
    """The 4-bit key cache in scrambled 128-row pages (NaN keys and poisoned
    codes in every row no sequence owns): codes land on the pages' rows and
    selection and output equal the contiguous layout's bit for bit."""
    w = custom(lens[0], lens[1], num_q_heads=16, num_kv_heads=4, head_dim=64, index_dim=128,
               top_k=8, seed=72, qkv_std=1.0)
    t = generate(w, "cpu")
    _, a, a4 = _run(w, t)
    table, rows, pages = paged_layout(w, seed=3)
    dev = torch.device("cuda:0")
    ki = to_pages(t["k_idx"], rows, pages, float("nan")).to(dev)
    k = to_pages(t["k"], rows, pages, float("nan")).to(dev)
    v = to_pages(t["v"], rows, pages, float("nan")).to(dev)
    dims = msa.make_dims(batch=w.batch, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                         head_dim=w.head_dim, index_dim=w.index_dim, top_k=w.top_k,
                         total_q=w.total_q, total_k=pages * 128, max_q_len=max(w.seq_q_lens),
                         max_k_len=max(w.seq_k_lens), block_table=table.to(dev))
    _, b, b4 = _run(w, t, dims=dims, k_idx=(ki, k, v))
    r = rows.to(dev)
    assert torch.equal(b4.k_idx4.index_select(0, r), a4.k_idx4)
    assert torch.equal(b4.k_exp4.index_select(0, r), a4.k_exp4)
    assert torch.equal(a.sel, b.sel) and torch.equal(a.out, b.out)


def test_q8k4_verification_shape():
    w = custom([7000, 4100, 300, 2049], [8, 8, 5, 8], num_q_heads=32, num_kv_heads=8,
               head_dim=128, index_dim=128, top_k=8, seed=73, qkv_std=1.0)
    _full_check(w, "q8k4-verify8")


# ---------------------------------------------------------------------------
# full sizes: sampled rows; the oracle quantises only what it reads
# ---------------------------------------------------------------------------
class _DeqK4:
    """Index keys quantised to 4 bits and dequantised on demand, a slice at a
    time (keys are scaled per 32 elements of each row, so any slice of rows
    quantises as the whole cache does)."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)
        self.cache = {}

    def __getitem__(self, sl):
        assert isinstance(sl, slice)
        key = (sl.start, sl.stop)
        if key not in self.cache:
            x = self.t[sl].double().cpu().numpy()
            self.cache[key] = F4.dequantize_k_idx4(*F4.quantize_k_idx4(x))
        return self.cache[key]


def _sampled(name, rows_fn):
    w = workload(name)
    log(f"[q8k4-{name}] generating {w.note}")
    t = generate(w, "cuda:0")
    dims = msa.dims_for(w)
    bufs = msa.Buffers(dims, t["q"].device, want_scores=True)
    qk = msa.Q8K4Index(dims, t["q"].device)
    msa.msa_forward(dims, t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"], t["cu_seqlens_q"],
                    t["cu_seqlens_k"], bufs, q8k4=qk)
    torch.cuda.synchronize()
    rows = rows_fn(w)
    log(f"[q8k4-{name}] forward done; oracle on {len(rows)} rows")
    ridx = torch.as_tensor(rows, device="cuda:0", dtype=torch.long)
    qc, qe = F8.quantize_q_idx(t["q_idx"].index_select(0, ridx).double().cpu().numpy())
    assert np.array_equal(qk.q_idx8.index_select(0, ridx).cpu().numpy(), qc)
    assert np.array_equal(qk.q_exp.index_select(0, ridx).cpu().numpy(), qe)
    n0 = min(int(w.seq_k_lens[0]), 128 * 64)
    kc, ke = F4.quantize_k_idx4(t["k_idx"][:n0].double().cpu().numpy())
    assert np.array_equal(qk.k_idx4[:n0].cpu().numpy(), F4.pack(kc))
    assert np.array_equal(qk.k_exp4[:n0].cpu().numpy(), ke)
    P = O.Problem(LazyRows(t["q"]), LazyRows(t["k"]), LazyRows(t["v"]), _DeqQ(t["q_idx"]),
                  _DeqK4(t["k_idx"]), t["cu_seqlens_q"].cpu().numpy(),
                  t["cu_seqlens_k"].cpu().numpy(), w.top_k)
    ref = P.run(rows, want_scores=True)
    sel = bufs.sel.index_select(0, ridx).cpu().numpy()
    score = bufs.sel_score.index_select(0, ridx).cpu().numpy()
    out = bufs.out.index_select(0, ridx).float().cpu().numpy()
    lse = bufs.lse.index_select(0, ridx).cpu().numpy()
    check_rows_fp8(P, rows, sel, score, ref, out, lse, f"q8k4-{name}")


def test_q8k4_p128k_sampled():
    _sampled("p128k", lambda w: sample_rows(w, 24))


def test_q8k4_decode_sampled():
    _sampled("decode", lambda w: list(range(0, w.total_q, 4)))
