"""GPU parity of the quantised Main Branch (8-bit q, k, v: msa_main_quantize_fp8
and msa_attend_fp8) against the oracle (oracle/fp8_main.py).

Codes and exponents must equal the oracle's bit for bit.  The Main Branch is
then checked against the fp64 oracle run on the dequantised q, k and v (the
selection, from the unchanged bf16 index inputs, as for the bf16 path), with
the bf16 path's tolerances: the kernels dequantise exactly into bf16
operands, so their arithmetic is that of the bf16 path.  A paged cache must
give bit-for-bit the contiguous results.
"""
import numpy as np
import pytest
import torch

import block_sparse_long_index_amd as msa
from msa_inputs import custom, generate, paged_layout, sample_rows, to_pages, workload
from oracle import fp8_main as M
from oracle import msa_oracle as O

pytestmark = pytest.mark.gpu

from gpu_helpers import LazyRows, check_out, check_selection, log  # noqa: E402


def _f64(x):
    return x.double().cpu().numpy()


def _oracle_problem(t, w):
    """Oracle on the dequantised q, k, v (quantised by the oracle from the bf16 inputs)."""
    cu_k = t["cu_seqlens_k"].cpu().numpy()
    nbm = (max(w.seq_k_lens) + 127) // 128
    qd = M.dequantize_q(*M.quantize_q(_f64(t["q"])))
    kd = M.dequantize_kv(*M.quantize_kv(_f64(t["k"]), cu_k, nbm), cu_k)
    vd = M.dequantize_kv(*M.quantize_kv(_f64(t["v"]), cu_k, nbm), cu_k)
    return O.Problem(qd, kd, vd, _f64(t["q_idx"]), _f64(t["k_idx"]), t["cu_seqlens_q"].cpu().numpy(),
                     cu_k, w.top_k)


def _run(w, g, dims=None, k=None, v=None, k_idx=None):
    dims = dims or msa.dims_for(w)
    dev = g["q"].device
    bufs = msa.Buffers(dims, dev, want_scores=True)
    f8 = msa.Fp8Main(dims, dev)
    msa.msa_forward(dims, g["q"], g["k"] if k is None else k, g["v"] if v is None else v, g["q_idx"],
                    g["k_idx"] if k_idx is None else k_idx, g["cu_seqlens_q"], g["cu_seqlens_k"], bufs,
                    fp8_main=f8)
    torch.cuda.synchronize()
    return dims, bufs, f8


def _check(w, tag):
    t = generate(w, "cpu")
    g = {k_: v_.to("cuda:0") for k_, v_ in t.items()}
    log(f"[{tag}] lens k={w.seq_k_lens} q={w.seq_q_lens} Hq={w.num_q_heads} G={w.num_kv_heads} d={w.head_dim}")
    dims, bufs, f8 = _run(w, g)
    # codes and exponents: bit-exact
    cu_k = t["cu_seqlens_k"].numpy()
    nbm = (max(w.seq_k_lens) + 127) // 128
    cq, eq = M.quantize_q(_f64(t["q"]))
    ck, ek = M.quantize_kv(_f64(t["k"]), cu_k, nbm)
    cv, ev = M.quantize_kv(_f64(t["v"]), cu_k, nbm)
    assert np.array_equal(f8.q8.cpu().numpy(), cq) and np.array_equal(f8.q_exp.cpu().numpy(), eq)
    assert np.array_equal(f8.k8.cpu().numpy(), ck) and np.array_equal(f8.k_exp.cpu().numpy(), ek)
    assert np.array_equal(f8.v8.cpu().numpy(), cv) and np.array_equal(f8.v_exp.cpu().numpy(), ev)
    # the Main Branch on the dequantised values
    P = _oracle_problem(t, w)
    rows = list(range(w.total_q))
    ref = P.run(rows, want_scores=True)
    bad, ties = check_selection(P, rows, bufs.sel.cpu().numpy(), bufs.sel_score.cpu().numpy(), ref,
                                w.index_dim)
    log(f"[{tag}] selection mismatches {len(bad)} near-ties {ties}")
    assert not bad, bad[:3]
    check_out(bufs.out.float().cpu().numpy(), ref["out"], bufs.lse.cpu().numpy(), ref["lse"], tag)
    return t, g, dims, bufs, f8


def test_fp8_main_prefill_ragged_gqa():
    w = custom([1500, 900, 130, 3000, 257], [1500, 300, 130, 2000, 200], num_q_heads=16,
               num_kv_heads=4, head_dim=128, index_dim=64, top_k=6, seed=81, qkv_std=1.0)
    _check(w, "fp8-main-prefill")


def test_fp8_main_head_dim_64_and_hpg_1():
    w = custom([1200, 700], [1200, 700], num_q_heads=4, num_kv_heads=4, head_dim=64, index_dim=32,
               top_k=4, seed=82, qkv_std=1.0)
    _check(w, "fp8-main-d64")


def test_fp8_main_decode_and_verify():
    w = custom([5000, 20000, 128, 300, 4100], [1, 1, 1, 1, 1], num_q_heads=16, num_kv_heads=8,
               head_dim=128, index_dim=128, top_k=16, seed=83, qkv_std=1.0)
    _check(w, "fp8-main-decode")
    w = custom([7000, 4100, 300, 2049], [8, 8, 5, 8], num_q_heads=32, num_kv_heads=8, head_dim=128,
               index_dim=128, top_k=8, seed=84, qkv_std=1.0)
    _check(w, "fp8-main-verify8")


@pytest.mark.parametrize("d,hq,g", [(64, 8, 8), (64, 128, 8), (128, 8, 8), (128, 256, 8),
                                    (128, 32, 2)])
def test_fp8_main_decode_head_layouts(d, hq, g):
    """Decode across head dims and heads per group (1, 16, 32): the P tile
    keeps the group's head columns only, so every layout is checked."""
    w = custom([100, 128, 1300, 9000, 257], [1, 1, 1, 1, 1], num_q_heads=hq, num_kv_heads=g,
               head_dim=d, index_dim=64, top_k=8, seed=101 + d + hq + g, qkv_std=1.0)
    _check(w, f"fp8-main-decode-d{d}-hpg{hq // g}")


def test_fp8_main_wide_magnitudes():
    # per-head and per-block exponents that differ widely: values scaled by 2^-6 .. 2^6
    w = custom([1100, 600], [1100, 600], num_q_heads=8, num_kv_heads=2, head_dim=64, index_dim=32,
               top_k=4, seed=85, qkv_std=1.0)
    t = generate(w, "cpu")
    rng = np.random.default_rng(85)
    Tq, Hq = t["q"].shape[:2]
    Tk, G = t["k"].shape[:2]
    sq = torch.from_numpy(np.ldexp(1.0, rng.integers(-6, 7, size=(Tq, Hq, 1))))
    t["q"] = (t["q"].double() * sq).to(torch.bfloat16)
    # one power of two per (128 packed rows, head): blocks of both sequences see
    # different exponents per head, and some blocks two of them
    sk = torch.from_numpy(np.ldexp(1.0, rng.integers(-6, 7, size=(Tk // 128 + 1, G, 1))))
    idx = torch.arange(Tk) // 128
    t["k"] = (t["k"].double() * sk[idx]).to(torch.bfloat16)
    t["v"] = (t["v"].double() * sk[idx].flip(1)).to(torch.bfloat16)
    g = {k_: v_.to("cuda:0") for k_, v_ in t.items()}
    dims, bufs, f8 = _run(w, g)
    cu_k = t["cu_seqlens_k"].numpy()
    ck, ek = M.quantize_kv(_f64(t["k"]), cu_k, (max(w.seq_k_lens) + 127) // 128)
    assert np.array_equal(f8.k8.cpu().numpy(), ck) and np.array_equal(f8.k_exp.cpu().numpy(), ek)
    P = _oracle_problem(t, w)
    rows = list(range(0, w.total_q, 3))
    ref = P.run(rows, want_scores=True)
    sel = bufs.sel.cpu().numpy()[rows]
    bad, _ = check_selection(P, rows, sel, bufs.sel_score.cpu().numpy()[rows], ref, w.index_dim)
    assert not bad, bad[:3]
    # outputs reach magnitudes where one bf16 unit exceeds the absolute bounds of
    # unit-scale inputs: the bounds here are the relative ones (and lse's)
    out = bufs.out.float().cpu().numpy()[rows]
    d = np.abs(out - ref["out"])
    rel2 = float(np.linalg.norm(d) / np.linalg.norm(ref["out"]))
    relmax = float(d.max() / np.abs(ref["out"]).max())
    dl = float(np.abs(bufs.lse.cpu().numpy()[rows] - ref["lse"]).max())
    log(f"[fp8-main-wide] relL2 {rel2:.3e} relmax {relmax:.3e} max|d lse| {dl:.3e}")
    assert rel2 <= 1e-2 and relmax <= 2e-2 and dl <= 2e-3, (rel2, relmax, dl)


def test_fp8_main_paged_equals_contiguous():
    for lq, seed in ((None, 86), (1, 87)):
        lens = [1500, 900, 2000, 300]
        w = custom(lens, lens if lq is None else [lq] * 4, num_q_heads=16, num_kv_heads=4,
                   head_dim=128, index_dim=64, top_k=6, seed=seed, qkv_std=1.0)
        t = generate(w, "cpu")
        g = {k_: v_.to("cuda:0") for k_, v_ in t.items()}
        _, a, fa = _run(w, g)
        table, rows_k, pages = paged_layout(w, seed=seed)
        rows_d, table_d = rows_k.to("cuda:0"), table.to("cuda:0")
        kc, vc, kic = (to_pages(g[n], rows_d, pages, float("nan")) for n in ("k", "v", "k_idx"))
        dims = msa.make_dims(batch=w.batch, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                             head_dim=w.head_dim, index_dim=w.index_dim, top_k=w.top_k,
                             total_q=w.total_q, total_k=pages * 128, max_q_len=max(w.seq_q_lens),
                             max_k_len=max(w.seq_k_lens), block_table=table_d)
        _, b, fb = _run(w, g, dims=dims, k=kc, v=vc, k_idx=kic)
        log(f"[fp8-main-paged lq={lq}] {pages} pages")
        assert torch.equal(a.sel, b.sel) and torch.equal(a.out, b.out) and torch.equal(a.lse, b.lse)
        assert torch.equal(fa.k8, fb.k8.index_select(0, rows_d))
        tb = table.numpy()
        for bb in range(w.batch):
            nb = (w.seq_k_lens[bb] + 127) // 128
            pg = torch.from_numpy(tb[bb, :nb]).long()
            assert torch.equal(fa.k_exp[bb, :nb].cpu(), fb.k_exp.cpu()[pg])
            assert torch.equal(fa.v_exp[bb, :nb].cpu(), fb.v_exp.cpu()[pg])


class _LazyQuantQ(LazyRows):
    """Dequantised query rows (one scale per (row, head)) of a device tensor."""

    def __getitem__(self, idx):
        x = super().__getitem__(idx)
        if x.ndim == 2:
            return M.dequantize_q(*M.quantize_q(x[None]))[0]
        return M.dequantize_q(*M.quantize_q(x))


def _sampled_full(name, n_random):
    w = workload(name)
    log(f"[{name}-fp8-main] generating {w.note}")
    t = generate(w, "cuda:0")
    dims, bufs, f8 = _run(w, t)
    rows = sample_rows(w, n_random)
    cu_k = t["cu_seqlens_k"].cpu().numpy()
    def rows_of(x):
        return lambda lo, hi: _f64(x[lo:hi])
    kq = M.DequantizedRows(rows_of(t["k"]), t["k"].shape[0], t["k"].shape[1:], cu_k)
    vq = M.DequantizedRows(rows_of(t["v"]), t["v"].shape[0], t["v"].shape[1:], cu_k)
    P = O.Problem(_LazyQuantQ(t["q"]), kq, vq,
                  LazyRows(t["q_idx"]), t["k_idx"].float().cpu().numpy(), t["cu_seqlens_q"].cpu().numpy(),
                  cu_k, w.top_k)
    log(f"[{name}-fp8-main] forward done; oracle on {len(rows)} rows")
    ref = P.run(rows, want_scores=True)
    ridx = torch.as_tensor(rows, device="cuda:0", dtype=torch.long)
    sel = bufs.sel.index_select(0, ridx).cpu().numpy()
    bad, ties = check_selection(P, rows, sel, bufs.sel_score.index_select(0, ridx).cpu().numpy(), ref,
                                w.index_dim)
    log(f"[{name}-fp8-main] selection mismatches {len(bad)} near-ties {ties}")
    assert not bad, bad[:3]
    check_out(bufs.out.index_select(0, ridx).float().cpu().numpy(), ref["out"],
              bufs.lse.index_select(0, ridx).cpu().numpy(), ref["lse"], f"{name}-fp8-main")


def test_fp8_main_p128k_sampled():
    _sampled_full("p128k", 16)


def test_fp8_main_decode_all_rows():
    _sampled_full("decode", 0)
