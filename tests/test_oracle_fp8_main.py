"""Pins of the quantised Main Branch oracle (oracle/fp8_main.py), CPU only.

What fixes the answers: the scale granularity through power-of-two
equivariance (scaling one (row, head) of q, or one (block, head) of k/v, by
2^t moves only that unit's exponent, by t, and leaves every code unchanged);
blocks counted from each sequence's start; the neutral exponent past a
sequence's end; exact round trips of values on the E4M3 grid; the E4M3
half-unit error bound; and, with a selection that covers every block, the
Main Branch on the dequantised values against torch's float64
scaled_dot_product_attention (a library routine).
"""
import numpy as np
import torch

from oracle import fp8_index as F
from oracle import fp8_main as M
from oracle import msa_oracle as O


def _kv(seed, lens=(300, 130), G=3, d=8):
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return rng.standard_normal((int(cu[-1]), G, d)), cu


def test_q_scale_is_per_row_and_head():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((5, 4, 16))
    c0, e0 = M.quantize_q(q)
    q2 = q.copy()
    q2[2, 1] *= 2.0 ** 5
    q2[3] *= 2.0 ** -3
    c1, e1 = M.quantize_q(q2)
    assert np.array_equal(c0, c1)
    d = e1.astype(int) - e0.astype(int)
    want = np.zeros_like(d)
    want[2, 1] = 5
    want[3, :] = -3
    assert np.array_equal(d, want)


def test_kv_scale_is_per_block_and_head():
    k, cu = _kv(2)
    c0, e0 = M.quantize_kv(k, cu, 3)
    k2 = k.copy()
    k2[128:256, 2] *= 2.0 ** 4            # sequence 0, block 1, head 2
    c1, e1 = M.quantize_kv(k2, cu, 3)
    assert np.array_equal(c0, c1)
    d = e1.astype(int) - e0.astype(int)
    want = np.zeros_like(d)
    want[0, 1, 2] = 4
    assert np.array_equal(d, want)


def test_kv_blocks_start_at_each_sequence():
    k, cu = _kv(3)
    _, e0 = M.quantize_kv(k, cu, 3)
    k2 = k.copy()
    k2[300:428, 0] *= 2.0 ** -6            # sequence 1, its block 0, head 0
    _, e1 = M.quantize_kv(k2, cu, 3)
    d = e1.astype(int) - e0.astype(int)
    want = np.zeros_like(d)
    want[1, 0, 0] = -6
    assert np.array_equal(d, want)
    # sequence 1 has 130 keys: 2 blocks; its third is past the end
    assert np.all(e0[1, 2] == 127)


def test_values_on_the_grid_round_trip_exactly():
    rng = np.random.default_rng(4)
    table = F.e4m3_table()
    finite = np.array([c for c in range(256) if np.isfinite(table[c])], dtype=np.uint8)
    lens, G, d = (300, 130), 2, 8
    cu = np.array([0, 300, 430])
    k = np.empty((430, G, d))
    for b in range(2):
        for beta in range((lens[b] + 127) // 128):
            lo = cu[b] + 128 * beta
            hi = min(lo + 128, cu[b + 1])
            for g in range(G):
                e = int(rng.integers(-20, 20))
                codes = rng.choice(finite, size=(hi - lo, d))
                codes[0, 0] = 0x7E                  # 448: the block's scale is exactly 2^e
                k[lo:hi, g] = np.ldexp(table[codes], e)
    c, ex = M.quantize_kv(k, cu, 3)
    assert np.array_equal(M.dequantize_kv(c, ex, cu), k)
    q = np.ldexp(table[rng.choice(finite, size=(7, 4, 16))], 3)
    q[:, :, 0] = 448.0 * 8
    cq, eq = M.quantize_q(q)
    assert np.array_equal(M.dequantize_q(cq, eq), q)


def test_error_bound_of_half_a_unit():
    k, cu = _kv(5, lens=(700, 200), G=2, d=32)
    k *= np.exp(np.random.default_rng(6).uniform(-8, 8, size=k.shape))   # wide magnitudes
    c, ex = M.quantize_kv(k, cu, 6)
    deq = M.dequantize_kv(c, ex, cu)
    for b in range(2):
        for beta in range(6):
            lo = cu[b] + 128 * beta
            hi = min(lo + 128, cu[b + 1])
            if lo >= hi:
                continue
            for g in range(2):
                e = int(ex[b, beta, g]) - 127
                err = np.abs(deq[lo:hi, g] - k[lo:hi, g])
                bound = 2.0 ** -4 * np.abs(k[lo:hi, g]) + 2.0 ** (e - 10)
                assert np.all(err <= bound)


def test_main_branch_on_dequantised_values_is_dense_attention():
    rng = np.random.default_rng(7)
    L, Hq, G, d, di = 500, 4, 2, 32, 16
    cu = np.array([0, L])
    q, k, v = rng.standard_normal((L, Hq, d)), rng.standard_normal((L, G, d)), rng.standard_normal((L, G, d))
    cq, eq = M.quantize_q(q)
    ck, ek = M.quantize_kv(k, cu, 4)
    cv, ev = M.quantize_kv(v, cu, 4)
    qd, kd, vd = M.dequantize_q(cq, eq), M.dequantize_kv(ck, ek, cu), M.dequantize_kv(cv, ev, cu)
    P = O.Problem(qd, kd, vd, rng.standard_normal((L, G, di)), rng.standard_normal((L, di)), cu, cu, 8)
    rows = [3, 130, 499]
    res = P.run(rows)
    for i, r in enumerate(rows):
        for h in range(Hq):
            g = h // (Hq // G)
            Q = torch.from_numpy(qd[r, h])[None, None, None]
            K = torch.from_numpy(kd[:r + 1, g])[None, None]
            V = torch.from_numpy(vd[:r + 1, g])[None, None]
            want = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=d ** -0.5)[0, 0, 0]
            assert np.allclose(res["out"][i, h], want.numpy(), atol=1e-12, rtol=0)


def test_lazy_dequantized_rows_equal_the_whole_cache():
    k, cu = _kv(8, lens=(700, 300, 5), G=2, d=8)
    whole = M.dequantize_kv(*M.quantize_kv(k, cu, 6), cu)
    lazy = M.DequantizedRows(lambda lo, hi: k[lo:hi], k.shape[0], k.shape[1:], cu)
    J = np.array([0, 5, 130, 699, 700, 850, 999, 1004])
    assert np.array_equal(lazy[J, 1], whole[J, 1])
    view = lazy[700:1000]
    assert np.array_equal(view[np.array([0, 150, 299]), 0], whole[[700, 850, 999], 0])
