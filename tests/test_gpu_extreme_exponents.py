"""The quantised Main Branch at the ends of the power-of-two scale range.

Queries near 2^120, keys near 2^-118 (some blocks or 32-element groups small
enough that their exponent clamps at -127, where the smallest codes fall
below bf16's subnormal resolution), values near 2^100 and some near 2^-110:
the codes must still equal the oracle's bit for bit, and the Main Branch on
both the lists path (prefill) and the decode path must match the oracle on
the dequantised values.  Outputs sit near 2^100, far beyond the absolute
bounds of unit-scale inputs, so the bounds here are the relative ones and
lse's.
"""
import numpy as np
import pytest
import torch

from msa_inputs import custom, generate
from oracle import fp8_main as M8

pytestmark = pytest.mark.gpu

from gpu_helpers import check_selection, log  # noqa: E402
import test_gpu_fp8_main as T8  # noqa: E402
import test_gpu_q8kv4_main as T4  # noqa: E402


def _pow2(rng, lo, hi, shape):
    return torch.from_numpy(np.ldexp(1.0, rng.integers(lo, hi + 1, size=shape)))


def _extreme_inputs(w, seed, kv4):
    t = generate(w, "cpu")
    rng = np.random.default_rng(seed)
    Tq, Hq = t["q"].shape[:2]
    Tk, G, D = t["k"].shape
    t["q"] = (t["q"].double() * _pow2(rng, 110, 120, (Tq, Hq, 1))).to(torch.bfloat16)
    chunk = torch.arange(Tk) // 128
    nch = Tk // 128 + 1
    sk = _pow2(rng, -120, -116, (nch, G, 1))
    sv = _pow2(rng, 90, 100, (nch, G, 1))
    # every fourth chunk: keys small enough that the exponent clamps at -127;
    # every fifth: tiny values
    sk[::4] = 2.0 ** -127
    sv[::5] = 2.0 ** -110
    k = t["k"].double() * sk[chunk]
    v = t["v"].double() * sv[chunk]
    if kv4:
        # 32-element groups of single rows pushed further down, to the clamp
        rows = torch.from_numpy(rng.integers(0, Tk, size=64))
        k[rows, :, :32] *= 2.0 ** -9
    t["k"] = k.to(torch.bfloat16)
    t["v"] = v.to(torch.bfloat16)
    return t


def _relative_check(bufs, ref, rows, tag):
    out = bufs.out.float().cpu().numpy()[rows]
    assert np.isfinite(out).all()
    d = np.abs(out - ref["out"])
    rel2 = float(np.linalg.norm(d) / np.linalg.norm(ref["out"]))
    relmax = float(d.max() / np.abs(ref["out"]).max())
    dl = float(np.abs(bufs.lse.cpu().numpy()[rows] - ref["lse"]).max())
    log(f"[{tag}] relL2 {rel2:.3e} relmax {relmax:.3e} max|d lse| {dl:.3e}")
    assert rel2 <= 1e-2 and relmax <= 2e-2 and dl <= 2e-3, (rel2, relmax, dl)


CASES = {
    "lists": ([1100, 600], [1100, 600]),
    "decode": ([1100, 600, 333, 128], [1, 1, 1, 1]),
}


@pytest.mark.parametrize("path", sorted(CASES))
def test_fp8_main_extreme_exponents(path):
    kl, ql = CASES[path]
    w = custom(kl, ql, num_q_heads=8, num_kv_heads=2, head_dim=64, index_dim=32, top_k=4,
               seed=91, qkv_std=1.0)
    t = _extreme_inputs(w, 91, kv4=False)
    g = {k_: v_.to("cuda:0") for k_, v_ in t.items()}
    dims, bufs, f8 = T8._run(w, g)
    cu_k = t["cu_seqlens_k"].numpy()
    nbm = (max(w.seq_k_lens) + 127) // 128
    for name, codes, exps in (("k", f8.k8, f8.k_exp), ("v", f8.v8, f8.v_exp)):
        c, e = M8.quantize_kv(T8._f64(t[name]), cu_k, nbm)
        assert np.array_equal(codes.cpu().numpy(), c) and np.array_equal(exps.cpu().numpy(), e), name
    assert (f8.k_exp.cpu().numpy() == 0).any()          # some blocks clamp at 2^-127
    cq, eq = M8.quantize_q(T8._f64(t["q"]))
    assert np.array_equal(f8.q8.cpu().numpy(), cq) and np.array_equal(f8.q_exp.cpu().numpy(), eq)
    P = T8._oracle_problem(t, w)
    rows = list(range(w.total_q)) if path == "decode" else list(range(0, w.total_q, 3))
    ref = P.run(rows, want_scores=True)
    bad, _ = check_selection(P, rows, bufs.sel.cpu().numpy()[rows], bufs.sel_score.cpu().numpy()[rows],
                             ref, w.index_dim)
    assert not bad, bad[:3]
    _relative_check(bufs, ref, rows, f"fp8-extreme-{path}")


@pytest.mark.parametrize("path", sorted(CASES))
def test_q8kv4_main_extreme_exponents(path):
    kl, ql = CASES[path]
    w = custom(kl, ql, num_q_heads=8, num_kv_heads=2, head_dim=64, index_dim=32, top_k=4,
               seed=92, qkv_std=1.0)
    t = _extreme_inputs(w, 92, kv4=True)
    g = {k_: v_.to("cuda:0") for k_, v_ in t.items()}
    dims, bufs, m = T4._run(w, g)
    T4._check_codes(t, m, f"q8kv4-extreme-{path}")
    assert (m.k_exp4.cpu().numpy() == 0).any()          # some groups clamp at 2^-127
    P = T4._oracle_problem(t, w)
    rows = list(range(w.total_q)) if path == "decode" else list(range(0, w.total_q, 3))
    ref = P.run(rows, want_scores=True)
    bad, _ = check_selection(P, rows, bufs.sel.cpu().numpy()[rows], bufs.sel_score.cpu().numpy()[rows],
                             ref, w.index_dim)
    assert not bad, bad[:3]
    _relative_check(bufs, ref, rows, f"q8kv4-extreme-{path}")
