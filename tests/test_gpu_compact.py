"""GPU parity of the Main Branch with compact partials (MSA_FLAG_COMPACT_PARTIALS:
the per-(query, head, block) softmax partials kept as a log-sum-exp, a
power-of-two exponent and fp16 values instead of fp32) against the oracle,
at the same tolerances as the fp32 partials, on the paths that use them
(prefill-shaped steps, bf16 and quantised inputs, several passes) and the
ones that must not (decode-shaped steps: bit-identical to fp32 partials).
"""
import numpy as np
import pytest
import torch

import block_sparse_long_index_amd as msa
from msa_inputs import custom, generate

pytestmark = pytest.mark.gpu

from gpu_helpers import check_out, check_selection, log, problem_from, run_gpu  # noqa: E402

C = msa.FLAG_COMPACT_PARTIALS


def _full_check(w, tag, q_chunk=0):
    log(f"[{tag}] lens k={w.seq_k_lens} q={w.seq_q_lens} Hq={w.num_q_heads} G={w.num_kv_heads} "
        f"d={w.head_dim} k={w.top_k} chunk={q_chunk}")
    t = generate(w, "cpu")
    dims, bufs, g = run_gpu(w, t, q_chunk=q_chunk, flags=C)
    assert msa.attend_reads_lists(dims)
    P = problem_from(t, w)
    rows = list(range(w.total_q))
    ref = P.run(rows, want_scores=True)
    bad, ties = check_selection(P, rows, bufs.sel.cpu().numpy(), bufs.sel_score.cpu().numpy(), ref,
                                w.index_dim)
    assert not bad, bad[:3]
    check_out(bufs.out.float().cpu().numpy(), ref["out"], bufs.lse.cpu().numpy(), ref["lse"], tag)
    return t, dims, bufs, g


def test_compact_ragged_prefill():
    w = custom([1500, 900, 130, 128, 3000, 257], [1500, 300, 130, 1, 2000, 200], num_q_heads=8,
               num_kv_heads=2, head_dim=64, index_dim=64, top_k=5, seed=121, qkv_std=1.0)
    _full_check(w, "compact-ragged")


def test_compact_gqa8_d128_k16():
    w = custom([2200], [2200], num_q_heads=64, num_kv_heads=8, head_dim=128, index_dim=128,
               top_k=16, seed=122, qkv_std=1.0)
    _full_check(w, "compact-gqa8")


def test_compact_hpg32_k32_and_hpg1():
    w = custom([5000], [5000], num_q_heads=32, num_kv_heads=1, head_dim=64, index_dim=32,
               top_k=32, seed=123, qkv_std=1.0)
    _full_check(w, "compact-hpg32")
    w = custom([2000], [2000], num_q_heads=4, num_kv_heads=4, head_dim=128, index_dim=32,
               top_k=3, seed=124, qkv_std=1.0)
    _full_check(w, "compact-hpg1")


def test_compact_passes_are_invisible_and_close_to_fp32():
    """Several query passes give the one-pass result bit for bit; the compact
    result stays within fp16 rounding of the fp32-partial result."""
    w = custom([3000, 1000], [3000, 1000], num_q_heads=16, num_kv_heads=4, head_dim=128,
               index_dim=64, top_k=6, seed=125, qkv_std=1.0)
    t, dims, bufs, g = _full_check(w, "compact-passes", q_chunk=0)
    _, bufs2, _ = run_gpu(w, t, q_chunk=333, flags=C)
    assert torch.equal(bufs.out, bufs2.out) and torch.equal(bufs.lse, bufs2.lse)
    _, b32, _ = run_gpu(w, t)
    d = (bufs.out.float() - b32.out.float()).abs()
    vmax = float(g["v"].float().abs().max())
    log(f"[compact-passes] max |compact - fp32| {float(d.max()):.3e} (bound 2^-11 * {vmax:.2f} + bf16 ulp)")
    assert float(d.max()) <= 2.0 ** -11 * vmax + 2.0 ** -8 * float(b32.out.float().abs().max())
    assert float((bufs.lse - b32.lse).abs().max()) <= 1e-5


def test_compact_decode_shaped_steps_keep_fp32():
    w = custom([5000, 20000, 128, 300], [1, 4, 1, 2], num_q_heads=16, num_kv_heads=8, head_dim=128,
               index_dim=128, top_k=16, seed=126, qkv_std=1.0)
    t = generate(w, "cpu")
    dims, bufs, _ = run_gpu(w, t, flags=C)
    assert not msa.attend_reads_lists(dims)
    _, b32, _ = run_gpu(w, t)
    assert torch.equal(bufs.out, b32.out) and torch.equal(bufs.lse, b32.lse)


def test_compact_extreme_magnitudes():
    """Values near 2^100 and 2^-110 in different blocks, queries near 2^120,
    keys near 2^-118: the per-row exponents carry the range (relative bounds,
    as the outputs sit far above the unit-scale absolute bounds)."""
    from test_gpu_extreme_exponents import _extreme_inputs
    w = custom([1100, 600], [1100, 600], num_q_heads=8, num_kv_heads=2, head_dim=64, index_dim=32,
               top_k=4, seed=127, qkv_std=1.0)
    t = _extreme_inputs(w, 127, kv4=False)
    dims, bufs, _ = run_gpu(w, t, flags=C)
    P = problem_from(t, w)
    rows = list(range(0, w.total_q, 3))
    ref = P.run(rows, want_scores=True)
    bad, _ = check_selection(P, rows, bufs.sel.cpu().numpy()[rows], bufs.sel_score.cpu().numpy()[rows],
                             ref, w.index_dim)
    assert not bad, bad[:3]
    out = bufs.out.float().cpu().numpy()[rows]
    assert np.isfinite(out).all()
    d = np.abs(out - ref["out"])
    rel2 = float(np.linalg.norm(d) / np.linalg.norm(ref["out"]))
    relmax = float(d.max() / np.abs(ref["out"]).max())
    dl = float(np.abs(bufs.lse.cpu().numpy()[rows] - ref["lse"]).max())
    log(f"[compact-extreme] relL2 {rel2:.3e} relmax {relmax:.3e} max|d lse| {dl:.3e}")
    assert rel2 <= 1e-2 and relmax <= 2e-2 and dl <= 2e-3


@pytest.mark.parametrize("kind", ["fp8", "q8kv4"])
def test_compact_quantised_main_branch(kind):
    """8-bit and 4-bit Main-Branch inputs with compact partials against the
    oracle on the dequantised q, k, v."""
    import test_gpu_fp8_main as T8
    import test_gpu_q8kv4_main as T4
    T = T8 if kind == "fp8" else T4
    w = custom([1500, 900, 700], [1500, 300, 700], num_q_heads=16, num_kv_heads=2, head_dim=128,
               index_dim=64, top_k=5, seed=128, qkv_std=1.0)
    t = generate(w, "cpu")
    g = {k_: v_.to("cuda:0") for k_, v_ in t.items()}
    dims, bufs, _ = T._run(w, g, dims=msa.dims_for(w, flags=C))
    P = T._oracle_problem(t, w)
    rows = list(range(w.total_q))
    ref = P.run(rows, want_scores=True)
    bad, _ = check_selection(P, rows, bufs.sel.cpu().numpy(), bufs.sel_score.cpu().numpy(), ref,
                             w.index_dim)
    assert not bad, bad[:3]
    check_out(bufs.out.float().cpu().numpy(), ref["out"], bufs.lse.cpu().numpy(), ref["lse"],
              f"compact-{kind}")
