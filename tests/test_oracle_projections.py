"""Pins of the index-projection oracle (oracle/projections.py), CPU only.

What fixes the answers: torch's bfloat16 conversion (a library routine) on
float32-exact values; a value where a float32 intermediate would round twice;
identity and one-hot weights (the output is the input / a weight column);
power-of-two scaling commuting with the projection and its rounding; where
the new tokens' index keys land (prefill: every key row; decode: after the
cached keys); a float64 library product (torch.nn.functional.linear) for
general inputs.  Six planted mistakes must each fail a pin.
"""
import numpy as np
import pytest
import torch

from oracle import projections as PR


def test_bf16_round_matches_library_on_float32_values():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(50000) * np.exp(rng.uniform(-40, 40, 50000))
    x = np.concatenate([x, [0.0, -0.0, 3.3e38, -3.3e38, 1e-40, -1e-42]])
    x32 = x.astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).double().numpy()
    got = PR.bf16_round(x32.astype(np.float64))
    assert np.array_equal(np.isinf(got), np.isinf(ref))
    ok = np.isfinite(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got), np.signbit(ref))


def test_bf16_round_no_double_rounding():
    # midpoint of 1 and 1 + 2^-7 plus a tail below float32 precision: rounds up
    v = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert PR.bf16_round(np.array([v]))[0] == 1.0 + 2.0 ** -7
    assert PR.bf16_round(np.array([-v]))[0] == -(1.0 + 2.0 ** -7)
    # exact midpoints go to the even neighbour
    assert PR.bf16_round(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    assert PR.bf16_round(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    # largest bf16 and the overflow boundary
    big = (2.0 - 2.0 ** -7) * 2.0 ** 127
    assert PR.bf16_round(np.array([big]))[0] == big
    assert np.isinf(PR.bf16_round(np.array([big + 2.0 ** 119]))[0])


def _bf16_values(rng, shape, scale=1.0):
    return torch.from_numpy(rng.standard_normal(shape).astype(np.float32) * scale) \
        .to(torch.bfloat16).double().numpy()


def test_identity_weights_return_the_input():
    rng = np.random.default_rng(2)
    G, di, T = 2, 32, 50
    D = G * di
    x = _bf16_values(rng, (T, D))
    w_q = np.eye(D)
    w_k = np.eye(D)[di:2 * di]                     # picks columns di .. 2di-1
    cu = np.array([0, T])
    q, rows = PR.project(x, w_q, w_k, cu, cu, T, G)
    assert np.array_equal(q.reshape(T, D), x)
    assert np.array_equal(q[:, 1, :], x[:, di:])   # group 1 = features di .. 2di-1
    assert sorted(rows) == list(range(T))
    assert all(np.array_equal(rows[t], x[t, di:2 * di]) for t in range(T))


def test_one_hot_inputs_pick_weight_columns():
    rng = np.random.default_rng(3)
    G, di, D = 3, 32, 96
    w_q = _bf16_values(rng, (G * di, D))
    w_k = _bf16_values(rng, (di, D))
    x = np.zeros((D, D))
    x[np.arange(D), np.arange(D)] = 1.0
    cu = np.array([0, D])
    q, rows = PR.project(x, w_q, w_k, cu, cu, D, G)
    for t in range(D):
        assert np.array_equal(q[t].reshape(-1), w_q[:, t])
        assert np.array_equal(rows[t], w_k[:, t])


def test_power_of_two_scaling_commutes():
    rng = np.random.default_rng(4)
    G, di, D, T = 2, 64, 128, 40
    x = _bf16_values(rng, (T, D))
    w_q = _bf16_values(rng, (G * di, D), 0.1)
    w_k = _bf16_values(rng, (di, D), 0.1)
    cu = np.array([0, T])
    q1, r1 = PR.project(x, w_q, w_k, cu, cu, T, G)
    q2, r2 = PR.project(x * 2.0 ** 7, w_q, w_k, cu, cu, T, G)
    assert np.array_equal(q2, q1 * 2.0 ** 7)
    assert all(np.array_equal(r2[k], r1[k] * 2.0 ** 7) for k in r1)


def test_new_keys_land_after_the_cached_ones():
    rng = np.random.default_rng(5)
    G, di, D = 1, 32, 64
    lq, lk = [1, 3, 2], [500, 3, 130]
    cu_q, cu_k = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    T = cu_q[-1]
    x = _bf16_values(rng, (T, D))
    w_q = _bf16_values(rng, (G * di, D))
    w_k = _bf16_values(rng, (di, D))
    _, rows = PR.project(x, w_q, w_k, cu_q, cu_k, cu_k[-1], G)
    assert sorted(rows) == [499, 500, 501, 502, 631, 632]
    ref = PR.bf16_round(x @ w_k.T)
    assert np.array_equal(rows[499], ref[0])       # sequence 0's one new token
    assert np.array_equal(rows[502], ref[3])       # sequence 2's first of two


def test_general_inputs_against_library_product():
    rng = np.random.default_rng(6)
    G, di, D, T = 4, 32, 256, 70
    x = _bf16_values(rng, (T, D))
    w_q = _bf16_values(rng, (G * di, D), D ** -0.5)
    w_k = _bf16_values(rng, (di, D), D ** -0.5)
    cu = np.array([0, T])
    q, rows = PR.project(x, w_q, w_k, cu, cu, T, G)
    lin_q = torch.nn.functional.linear(torch.from_numpy(x), torch.from_numpy(w_q)).numpy()
    lin_k = torch.nn.functional.linear(torch.from_numpy(x), torch.from_numpy(w_k)).numpy()
    # bf16 outputs: within half a unit in the last place (8 significant bits)
    assert np.all(np.abs(q.reshape(T, -1) - lin_q) <= 2.0 ** -8 * np.abs(lin_q) + 1e-300)
    kk = np.stack([rows[t] for t in range(T)])
    assert np.all(np.abs(kk - lin_k) <= 2.0 ** -8 * np.abs(lin_k) + 1e-300)
    # and each output is a bf16 value
    assert np.array_equal(PR.bf16_round(q), q)
