"""Pins of the 4-bit Main Branch oracle (oracle/fp4_main.py), CPU only.

What fixes the answers: the scale granularity through power-of-two
equivariance (scaling one 32-element group of one (key, head) row by 2^t
moves only that group's exponent, by t, and leaves every code unchanged);
exact round trips of values on the E2M1 grid; the E2M1 error bound; and, with
a selection that covers every block, the Main Branch on the dequantised
values against torch's float64 scaled_dot_product_attention (a library
routine).  The element format itself is pinned in test_oracle_fp4.py.
"""
import numpy as np
import torch

from oracle import fp4_index as F4
from oracle import fp4_main as M4
from oracle import fp8_main as M8
from oracle import msa_oracle as O


def test_scale_is_per_row_head_and_32_elements():
    rng = np.random.default_rng(41)
    x = rng.standard_normal((50, 3, 64))
    c0, e0 = M4.quantize_kv4(x)
    assert c0.shape == (50, 3, 64) and e0.shape == (50, 3, 2)
    for j, g, grp, t in [(0, 0, 0, 5), (17, 2, 1, -3), (49, 1, 0, 8)]:
        x2 = x.copy()
        x2[j, g, 32 * grp:32 * grp + 32] *= 2.0 ** t
        c1, e1 = M4.quantize_kv4(x2)
        assert np.array_equal(c0, c1)
        d = e1.astype(int) - e0.astype(int)
        want = np.zeros_like(d)
        want[j, g, grp] = t
        assert np.array_equal(d, want)


def test_values_on_the_grid_round_trip_exactly():
    rng = np.random.default_rng(42)
    tab = F4.e2m1_table()
    codes = rng.integers(0, 16, size=(40, 2, 64)).astype(np.uint8)
    codes[:, :, 0] = 7                     # 6.0 in every first group: its scale is exactly 2^e
    codes[:, :, 32] = 15                   # -6.0 in every second group
    ex = rng.integers(-20, 10, size=(40, 2, 2))
    x = np.ldexp(tab[codes], np.repeat(ex, 32, axis=2))
    c, e = M4.quantize_kv4(x)
    assert np.array_equal(e.astype(int) - 127, ex)
    assert np.array_equal(M4.dequantize_kv4(c, e), x)


def test_error_bound():
    rng = np.random.default_rng(43)
    x = rng.standard_normal((64, 2, 128)) * np.exp(rng.uniform(-6, 6, (64, 2, 1)))
    c, e = M4.quantize_kv4(x)
    deq = M4.dequantize_kv4(c, e)
    ee = np.repeat(e.astype(np.int64) - 127, 32, axis=2)
    y = np.abs(x) * 2.0 ** -ee.astype(np.float64)
    bound = np.where(y >= 1.0, np.abs(x) / 4, 2.0 ** (ee - 2).astype(np.float64))
    assert np.all(np.abs(deq - x) <= bound)


def test_main_branch_on_dequantised_values_is_dense_attention():
    rng = np.random.default_rng(44)
    L, Hq, G, d, di = 500, 4, 2, 64, 16
    cu = np.array([0, L])
    q, k, v = rng.standard_normal((L, Hq, d)), rng.standard_normal((L, G, d)), rng.standard_normal((L, G, d))
    qd = M8.dequantize_q(*M8.quantize_q(q))
    kd = M4.dequantize_kv4(*M4.quantize_kv4(k))
    vd = M4.dequantize_kv4(*M4.quantize_kv4(v))
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


def test_lazy_rows_equal_the_whole_cache():
    rng = np.random.default_rng(45)
    x = rng.standard_normal((9000, 2, 64))
    whole = M4.dequantize_kv4(*M4.quantize_kv4(x))
    lazy = M4.DequantizedRows4(lambda lo, hi: x[lo:hi], x.shape[0], x.shape[1:])
    J = np.array([0, 5, 127, 128, 4095, 4096, 8191, 8999, 5])
    assert np.array_equal(lazy[J, 1], whole[J, 1])
    view = lazy[4000:9000]
    assert np.array_equal(view[np.array([0, 96, 4999, 1]), 0], whole[[4000, 4096, 8999, 4001], 0])
