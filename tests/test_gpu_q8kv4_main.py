"""GPU parity of the Main Branch with 8-bit queries and 4-bit keys and values
(msa_main_quantize_q8kv4 and msa_attend_q8kv4) against the oracle
(oracle/fp4_main.py for k and v, oracle/fp8_main.py for q).

Codes and exponents must equal the oracle's bit for bit.  The Main Branch is
then checked against the fp64 oracle run on the dequantised q, k and v (the
selection comes from the unchanged bf16 index inputs, as for the bf16 path),
with the bf16 path's tolerances: the kernels dequantise exactly into bf16
operands, so their arithmetic is that of the bf16 path.  A paged cache must
give bit-for-bit the contiguous results.
"""
import numpy as np
import pytest
import torch

import block_sparse_long_index_amd as msa
from msa_inputs import custom, generate, paged_layout, sample_rows, to_pages, workload
from oracle import fp4_index as F4
from oracle import fp4_main as M4
from oracle import fp8_main as M8
from oracle import msa_oracle as O

pytestmark = pytest.mark.gpu

from gpu_helpers import LazyRows, check_out, check_selection, log  # noqa: E402


def _f64(x):
    return x.double().cpu().numpy()


def _oracle_problem(t, w):
    """Oracle on the dequantised q, k, v (quantised by the oracle from the bf16 inputs)."""
    qd = M8.dequantize_q(*M8.quantize_q(_f64(t["q"])))
    kd = M4.dequantize_kv4(*M4.quantize_kv4(_f64(t["k"])))
    vd = M4.dequantize_kv4(*M4.quantize_kv4(_f64(t["v"])))
    return O.Problem(qd, kd, vd, _f64(t["q_idx"]), _f64(t["k_idx"]), t["cu_seqlens_q"].cpu().numpy(),
                     t["cu_seqlens_k"].cpu().numpy(), w.top_k)


def _run(w, g, dims=None, k=None, v=None, k_idx=None, m=None):
    dims = dims or msa.dims_for(w)
    dev = g["q"].device
    bufs = msa.Buffers(dims, dev, want_scores=True)
    if m is None:
        m = msa.Q8KV4Main(dims, dev)
    msa.msa_forward(dims, g["q"], g["k"] if k is None else k, g["v"] if v is None else v, g["q_idx"],
                    g["k_idx"] if k_idx is None else k_idx, g["cu_seqlens_q"], g["cu_seqlens_k"], bufs,
                    fp8_main=m)
    torch.cuda.synchronize()
    return dims, bufs, m


def _packed(codes):
    T, G, d = codes.shape
    return F4.pack(codes.reshape(T * G, d)).reshape(T, G, d // 2)


def _check_codes(t, m, tag):
    cq, eq = M8.quantize_q(_f64(t["q"]))
    ck, ek = M4.quantize_kv4(_f64(t["k"]))
    cv, ev = M4.quantize_kv4(_f64(t["v"]))
    nk = int((m.k4.cpu().numpy() != _packed(ck)).sum())
    nv = int((m.v4.cpu().numpy() != _packed(cv)).sum())
    log(f"[{tag}] code mismatches k {nk} v {nv} of {ck.size // 2}")
    assert np.array_equal(m.q8.cpu().numpy(), cq) and np.array_equal(m.q_exp.cpu().numpy(), eq)
    assert np.array_equal(m.k_exp4.cpu().numpy(), ek) and np.array_equal(m.v_exp4.cpu().numpy(), ev)
    assert nk == 0 and nv == 0


def _check(w, tag):
    t = generate(w, "cpu")
    g = {k_: v_.to("cuda:0") for k_, v_ in t.items()}
    log(f"[{tag}] lens k={w.seq_k_lens} q={w.seq_q_lens} Hq={w.num_q_heads} G={w.num_kv_heads} d={w.head_dim}")
    dims, bufs, m = _run(w, g)
    _check_codes(t, m, tag)
    P = _oracle_problem(t, w)
    rows = list(range(w.total_q))
    ref = P.run(rows, want_scores=True)
    bad, ties = check_selection(P, rows, bufs.sel.cpu().numpy(), bufs.sel_score.cpu().numpy(), ref,
                                w.index_dim)
    log(f"[{tag}] selection mismatches {len(bad)} near-ties {ties}")
    assert not bad, bad[:3]
    check_out(bufs.out.float().cpu().numpy(), ref["out"], bufs.lse.cpu().numpy(), ref["lse"], tag)
    return t, g, dims, bufs, m


def test_q8kv4_main_prefill_ragged_gqa():
    w = custom([1500, 900, 130, 3000, 257], [1500, 300, 130, 2000, 200], num_q_heads=16,
               num_kv_heads=4, head_dim=128, index_dim=64, top_k=6, seed=91, qkv_std=1.0)
    _check(w, "q8kv4-prefill")


def test_q8kv4_main_head_dim_64_and_hpg_1():
    w = custom([1200, 700], [1200, 700], num_q_heads=4, num_kv_heads=4, head_dim=64, index_dim=32,
               top_k=4, seed=92, qkv_std=1.0)
    _check(w, "q8kv4-d64")


def test_q8kv4_main_decode_and_verify():
    w = custom([5000, 20000, 128, 300, 4100], [1, 1, 1, 1, 1], num_q_heads=16, num_kv_heads=8,
               head_dim=128, index_dim=128, top_k=16, seed=93, qkv_std=1.0)
    _check(w, "q8kv4-decode")
    w = custom([7000, 4100, 300, 2049], [8, 8, 5, 8], num_q_heads=32, num_kv_heads=8, head_dim=128,
               index_dim=128, top_k=8, seed=94, qkv_std=1.0)
    _check(w, "q8kv4-verify8")


@pytest.mark.parametrize("d,hq,g", [(64, 8, 8), (64, 128, 8), (128, 8, 8), (128, 256, 8),
                                    (128, 32, 2)])
def test_q8kv4_main_decode_head_layouts(d, hq, g):
    """Decode across head dims and heads per group (1, 16, 32): the P tile
    keeps the group's head columns only, so every layout is checked."""
    w = custom([100, 128, 1300, 9000, 257], [1, 1, 1, 1, 1], num_q_heads=hq, num_kv_heads=g,
               head_dim=d, index_dim=64, top_k=8, seed=111 + d + hq + g, qkv_std=1.0)
    _check(w, f"q8kv4-decode-d{d}-hpg{hq // g}")


def test_q8kv4_main_decode_head_dim_64():
    w = custom([100, 128, 1300, 9000, 257], [1, 1, 1, 1, 1], num_q_heads=64, num_kv_heads=8,
               head_dim=64, index_dim=64, top_k=8, seed=95, qkv_std=1.0)
    _check(w, "q8kv4-decode-d64")


def test_q8kv4_main_wide_magnitudes():
    # exponents that differ per (key, head, 32-element group): values scaled by 2^-6 .. 2^6
    w = custom([1100, 600], [1100, 600], num_q_heads=8, num_kv_heads=2, head_dim=64, index_dim=32,
               top_k=4, seed=96, qkv_std=1.0)
    t = generate(w, "cpu")
    rng = np.random.default_rng(96)
    Tq, Hq, D = t["q"].shape
    Tk, G = t["k"].shape[:2]
    sq = torch.from_numpy(np.ldexp(1.0, rng.integers(-6, 7, size=(Tq, Hq, 1))))
    t["q"] = (t["q"].double() * sq).to(torch.bfloat16)
    sk = torch.from_numpy(np.repeat(np.ldexp(1.0, rng.integers(-6, 7, size=(Tk, G, D // 32))), 32, axis=2))
    t["k"] = (t["k"].double() * sk).to(torch.bfloat16)
    t["v"] = (t["v"].double() * sk.flip(2)).to(torch.bfloat16)
    g = {k_: v_.to("cuda:0") for k_, v_ in t.items()}
    dims, bufs, m = _run(w, g)
    _check_codes(t, m, "q8kv4-wide")
    P = _oracle_problem(t, w)
    rows = list(range(0, w.total_q, 3))
    ref = P.run(rows, want_scores=True)
    bad, _ = check_selection(P, rows, bufs.sel.cpu().numpy()[rows], bufs.sel_score.cpu().numpy()[rows],
                             ref, w.index_dim)
    assert not bad, bad[:3]
    # outputs reach magnitudes where one bf16 unit exceeds the absolute bounds of
    # unit-scale inputs: the bounds here are the relative ones (and lse's)
    out = bufs.out.float().cpu().numpy()[rows]
    d = np.abs(out - ref["out"])
    rel2 = float(np.linalg.norm(d) / np.linalg.norm(ref["out"]))
    relmax = float(d.max() / np.abs(ref["out"]).max())
    dl = float(np.abs(bufs.lse.cpu().numpy()[rows] - ref["lse"]).max())
    log(f"[q8kv4-wide] relL2 {rel2:.3e} relmax {relmax:.3e} max|d lse| {dl:.3e}")
    assert rel2 <= 1e-2 and relmax <= 2e-2 and dl <= 2e-3, (rel2, relmax, dl)


def test_q8kv4_main_paged_equals_contiguous():
    for lq, seed in ((None, 97), (1, 98)):
        lens = [1500, 900, 2000, 300]
        w = custom(lens, lens if lq is None else [lq] * 4, num_q_heads=16, num_kv_heads=4,
                   head_dim=128, index_dim=64, top_k=6, seed=seed, qkv_std=1.0)
        t = generate(w, "cpu")
        g = {k_: v_.to("cuda:0") for k_, v_ in t.items()}
        _, a, ma = _run(w, g)
        table, rows_k, pages = paged_layout(w, seed=seed)
        rows_d, table_d = rows_k.to("cuda:0"), table.to("cuda:0")
        kc, vc, kic = (to_pages(g[n], rows_d, pages, float("nan")) for n in ("k", "v", "k_idx"))
        dims = msa.make_dims(batch=w.batch, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                             head_dim=w.head_dim, index_dim=w.index_dim, top_k=w.top_k,
                             total_q=w.total_q, total_k=pages * 128, max_q_len=max(w.seq_q_lens),
                             max_k_len=max(w.seq_k_lens), block_table=table_d)
        _, b, mb = _run(w, g, dims=dims, k=kc, v=vc, k_idx=kic)
        log(f"[q8kv4-paged lq={lq}] {pages} pages")
        assert torch.equal(a.sel, b.sel) and torch.equal(a.out, b.out) and torch.equal(a.lse, b.lse)
        for name in ("k4", "v4", "k_exp4", "v_exp4"):
            assert torch.equal(getattr(ma, name), getattr(mb, name).index_select(0, rows_d)), name


def test_q8kv4_main_decode_on_a_quantised_cache():
    """k and v quantised once; steps that quantise only their queries give the
    outputs of quantising everything."""
    w = custom([7000, 3000, 12000], [1, 1, 1], num_q_heads=16, num_kv_heads=8, head_dim=128,
               index_dim=128, top_k=16, seed=99, qkv_std=1.0)
    t = generate(w, "cpu")
    g = {k_: v_.to("cuda:0") for k_, v_ in t.items()}
    dims, ref, mref = _run(w, g)
    m = msa.Q8KV4Main(dims, g["q"].device)
    msa.main_quantize_q8kv4(dims, None, g["k"], g["v"], g["cu_seqlens_k"], m)
    torch.cuda.synchronize()
    for name in ("k4", "v4", "k_exp4", "v_exp4"):
        assert torch.equal(getattr(m, name), getattr(mref, name)), name
    bufs = msa.Buffers(dims, g["q"].device, want_scores=True)
    for _ in range(2):
        msa.msa_forward(dims, g["q"], None, None, g["q_idx"], g["k_idx"], g["cu_seqlens_q"],
                        g["cu_seqlens_k"], bufs, fp8_main=m)
        torch.cuda.synchronize()
        assert torch.equal(bufs.out, ref.out) and torch.equal(bufs.lse, ref.lse)


class _LazyQuantQ(LazyRows):
    """Dequantised query rows (one scale per (row, head)) of a device tensor."""

    def __getitem__(self, idx):
        x = super().__getitem__(idx)
        if x.ndim == 2:
            return M8.dequantize_q(*M8.quantize_q(x[None]))[0]
        return M8.dequantize_q(*M8.quantize_q(x))


def _sampled_full(name, n_random):
    w = workload(name)
    log(f"[{name}-q8kv4] generating {w.note}")
    t = generate(w, "cuda:0")
    dims, bufs, m = _run(w, t)
    rows = sample_rows(w, n_random)
    def rows_of(x):
        return lambda lo, hi: _f64(x[lo:hi])
    kq = M4.DequantizedRows4(rows_of(t["k"]), t["k"].shape[0], t["k"].shape[1:])
    vq = M4.DequantizedRows4(rows_of(t["v"]), t["v"].shape[0], t["v"].shape[1:])
    P = O.Problem(_LazyQuantQ(t["q"]), kq, vq, LazyRows(t["q_idx"]), t["k_idx"].float().cpu().numpy(),
                  t["cu_seqlens_q"].cpu().numpy(), t["cu_seqlens_k"].cpu().numpy(), w.top_k)
    log(f"[{name}-q8kv4] forward done; oracle on {len(rows)} rows")
    ref = P.run(rows, want_scores=True)
    ridx = torch.as_tensor(rows, device="cuda:0", dtype=torch.long)
    sel = bufs.sel.index_select(0, ridx).cpu().numpy()
    bad, ties = check_selection(P, rows, sel, bufs.sel_score.index_select(0, ridx).cpu().numpy(), ref,
                                w.index_dim)
    log(f"[{name}-q8kv4] selection mismatches {len(bad)} near-ties {ties}")
    assert not bad, bad[:3]
    check_out(bufs.out.index_select(0, ridx).float().cpu().numpy(), ref["out"],
              bufs.lse.index_select(0, ridx).cpu().numpy(), ref["lse"], f"{name}-q8kv4")


def test_q8kv4_main_p128k_sampled():
    _sampled_full("p128k", 16)


def test_q8kv4_main_decode_all_rows():
    _sampled_full("decode", 0)


def test_q8k4_index_q8kv4_main_p1m_sampled():
    """Both branches quantised as in production (8-bit queries, 4-bit keys
    and values; the pages' "Q8KV4") at 1M tokens, in the launch configuration
    bench.py times: index codes checked on the sampled rows and on the first
    key blocks, the selection against the oracle on the dequantised index
    projections within the fp8 matrix cores' bound, the Main Branch against
    the oracle on the dequantised q, k, v."""
    from test_gpu_fp8 import _DeqQ, check_rows_fp8
    from test_gpu_q8k4 import _DeqK4
    from oracle import fp8_index as F8
    w = workload("p1m")
    log(f"[p1m-q8k4-q8kv4] generating {w.note}")
    t = generate(w, "cuda:0")
    dims = msa.dims_for(w)
    dev = t["q"].device
    bufs = msa.Buffers(dims, dev, want_scores=True)
    qk = msa.Q8K4Index(dims, dev)
    m = msa.Q8KV4Main(dims, dev)
    msa.msa_forward(dims, t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"], t["cu_seqlens_q"],
                    t["cu_seqlens_k"], bufs, q8k4=qk, fp8_main=m)
    torch.cuda.synchronize()
    rows = sample_rows(w, 48)
    log(f"[p1m-q8k4-q8kv4] forward done; oracle on {len(rows)} rows")
    ridx = torch.as_tensor(rows, device=dev, dtype=torch.long)
    qc, qe = F8.quantize_q_idx(t["q_idx"].index_select(0, ridx).double().cpu().numpy())
    assert np.array_equal(qk.q_idx8.index_select(0, ridx).cpu().numpy(), qc)
    assert np.array_equal(qk.q_exp.index_select(0, ridx).cpu().numpy(), qe)
    n0 = 128 * 64
    kc, ke = F4.quantize_k_idx4(t["k_idx"][:n0].double().cpu().numpy())
    assert np.array_equal(qk.k_idx4[:n0].cpu().numpy(), F4.pack(kc))
    assert np.array_equal(qk.k_exp4[:n0].cpu().numpy(), ke)

    def rows_of(x):
        return lambda lo, hi: _f64(x[lo:hi])
    kq = M4.DequantizedRows4(rows_of(t["k"]), t["k"].shape[0], t["k"].shape[1:])
    vq = M4.DequantizedRows4(rows_of(t["v"]), t["v"].shape[0], t["v"].shape[1:])
    P = O.Problem(_LazyQuantQ(t["q"]), kq, vq, _DeqQ(t["q_idx"]), _DeqK4(t["k_idx"]),
                  t["cu_seqlens_q"].cpu().numpy(), t["cu_seqlens_k"].cpu().numpy(), w.top_k)
    ref = P.run(rows, want_scores=True)
    sel = bufs.sel.index_select(0, ridx).cpu().numpy()
    score = bufs.sel_score.index_select(0, ridx).cpu().numpy()
    out = bufs.out.index_select(0, ridx).float().cpu().numpy()
    lse = bufs.lse.index_select(0, ridx).cpu().numpy()
    check_rows_fp8(P, rows, sel, score, ref, out, lse, "p1m-q8k4-q8kv4")
