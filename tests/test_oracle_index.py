"""Pins of the oracle's Index Branch (scores, block max-pool, selection).

Every expected value here comes from the pages' constants, from inputs built
so that the answer is known by construction, from hand-worked cases, or from
brute force over all subsets -- never from the oracle itself.
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import msa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_constants_match_pages():
    c = json.load(open(os.path.join(GOLDEN, "msa_constants.json")))
    assert O.BLOCK == c["block_size"] == 128
    assert O.TOP_K == c["top_k"] == 16
    assert O.BLOCK * O.TOP_K == c["budget_tokens"] == 2048


def test_hand_worked_selections():
    cases = json.load(open(os.path.join(GOLDEN, "hand_selection.json")))["cases"]
    for c in cases:
        got = O.select_blocks(np.asarray(c["scores"]), c["beta_p"], c["top_k"])
        assert got == c["expected"], c["name"]


def _is_valid_topk(S, beta_p, chosen):
    """Defining property of the top-(k-1): every chosen earlier block beats
    every unchosen earlier block under (higher score, then lower id)."""
    unchosen = [b for b in range(beta_p) if b not in chosen]
    for c in chosen:
        for u in unchosen:
            if not (S[c] > S[u] or (S[c] == S[u] and c < u)):
                return False
    return True


@pytest.mark.parametrize("seed", range(40))
def test_selection_brute_force(seed):
    rng = np.random.default_rng(seed)
    nb = int(rng.integers(1, 9))
    beta_p = nb - 1
    top_k = int(rng.integers(1, nb + 2))
    # small integer scores force many exact ties
    S = rng.integers(-3, 4, size=nb).astype(np.float64)
    got = O.select_blocks(S, beta_p, top_k)
    m = min(top_k - 1, beta_p)
    valid = [set(c) for c in itertools.combinations(range(beta_p), m)
             if _is_valid_topk(S, beta_p, set(c))]
    assert len(valid) == 1                     # the tie rule makes it unique
    assert got == sorted(valid[0] | {beta_p})


def _one_hot_problem(L=1024, G=3, d_idx=8, planted=None, beta_p_rows=None):
    """Index inputs whose block scores are known by construction.

    Token j's index key is w_j * e_{beta(j) mod d_idx}; group g's index query
    is e_{m_g}.  So s[g, j] = w_j when beta(j) = m_g (mod d_idx), else 0, and
    S[g, beta] = max w over the block's visible tokens for the matching blocks.
    """
    nb = L // O.BLOCK
    k_idx = np.zeros((L, d_idx))
    w = np.full(L, 1.0)
    planted = planted or {}
    for beta, val in planted.items():
        w[beta * O.BLOCK + 37] = val          # one strong token inside the block
    for j in range(L):
        k_idx[j, (j // O.BLOCK) % d_idx] = w[j]
    m = [g % d_idx for g in range(G)]
    q_idx = np.zeros((G, d_idx))
    for g in range(G):
        q_idx[g, m[g]] = 1.0
    return k_idx, q_idx, m, nb


def test_scores_and_pool_constructed():
    d_idx = 4
    planted = {0: 50.0, 4: 20.0, 5: 90.0, 1: 7.0, 6: 3.0}
    k_idx, q_idx, m, nb = _one_hot_problem(L=1024, G=2, d_idx=d_idx, planted=planted)
    p = 1023
    s = O.index_token_scores(q_idx, k_idx, p)
    S = O.block_max_pool(s, p)
    assert S.shape == (2, nb)
    # group 0 reads dim 0 -> blocks 0, 4 (50, 20); group 1 reads dim 1 -> 1, 5 (7, 90)
    assert S[0, 0] == 50.0 and S[0, 4] == 20.0
    assert S[1, 1] == 7.0 and S[1, 5] == 90.0
    assert S[0, 1] == 0.0 and S[1, 0] == 0.0 and S[0, 2] == 0.0
    # selection, k = 3: group 0 -> {0, 4} + local 7; group 1 -> {5, 1} + local 7
    assert O.select_blocks(S[0], 7, 3) == [0, 4, 7]
    assert O.select_blocks(S[1], 7, 3) == [1, 5, 7]


def test_pool_ignores_invisible_tokens_of_local_block():
    d_idx = 2
    L = 512
    k_idx = np.zeros((L, d_idx))
    k_idx[:, 0] = 1.0
    k_idx[300, 0] = 5.0        # visible for p >= 300
    k_idx[400, 0] = 1000.0     # future for p < 400
    q_idx = np.array([[1.0, 0.0]])
    p = 350                     # block 2 covers 256..383
    S = O.block_max_pool(O.index_token_scores(q_idx, k_idx, p), p)
    assert S.shape == (1, 3)
    assert S[0, 2] == 5.0
    p = 399
    S = O.block_max_pool(O.index_token_scores(q_idx, k_idx, p), p)
    assert S[0, 3] == 1.0      # block 3 covers 384..399 visible; 400 is not
    p = 400
    S = O.block_max_pool(O.index_token_scores(q_idx, k_idx, p), p)
    assert S[0, 3] == 1000.0


def test_score_is_a_dot_product_closed_form():
    # k_idx rows = j * u (u fixed) -> s_j = j * (q . u); block max at the block's last visible token
    d_idx = 4
    L = 640
    u = np.array([1.0, -2.0, 0.5, 3.0])
    q = np.array([[0.25, 1.0, -4.0, 2.0]])          # q . u = 0.25 - 2 - 2 + 6 = 2.25
    k_idx = np.arange(L, dtype=np.float64)[:, None] * u[None, :]
    p = 600
    S = O.block_max_pool(O.index_token_scores(q, k_idx, p), p)
    for beta in range(p // 128 + 1):
        last = min(beta * 128 + 127, p)
        assert S[0, beta] == 2.25 * last


def test_special_cases_k1_and_k_ge_nb():
    rng = np.random.default_rng(3)
    for beta_p in range(0, 12):
        S = rng.normal(size=beta_p + 1)
        assert O.select_blocks(S, beta_p, 1) == [beta_p]
        assert O.select_blocks(S, beta_p, beta_p + 1) == list(range(beta_p + 1))
        assert O.select_blocks(S, beta_p, beta_p + 7) == list(range(beta_p + 1))


def test_power_of_two_scaling_keeps_selection():
    from msa_inputs import generate, workload
    w = workload("tiny")
    t = generate(w, "cpu")
    f32 = lambda x: x.float().numpy()
    P1 = O.Problem(f32(t["q"]), f32(t["k"]), f32(t["v"]), f32(t["q_idx"]), f32(t["k_idx"]),
                   t["cu_seqlens_q"].numpy(), t["cu_seqlens_k"].numpy(), w.top_k)
    P2 = O.Problem(f32(t["q"]), f32(t["k"]), f32(t["v"]), 4.0 * f32(t["q_idx"]), f32(t["k_idx"]),
                   t["cu_seqlens_q"].numpy(), t["cu_seqlens_k"].numpy(), w.top_k)
    rows = list(range(0, 2048, 97)) + [2047]
    a = P1.run(rows)["sel"]
    b = P2.run(rows)["sel"]
    assert np.array_equal(a, b)


def test_selection_invariants_tiny():
    from msa_inputs import generate, workload
    w = workload("tiny")
    t = generate(w, "cpu")
    f32 = lambda x: x.float().numpy()
    P = O.Problem(f32(t["q"]), f32(t["k"]), f32(t["v"]), f32(t["q_idx"]), f32(t["k_idx"]),
                  t["cu_seqlens_q"].numpy(), t["cu_seqlens_k"].numpy(), w.top_k)
    rows = list(range(0, 2048, 13))
    res = P.run(rows, want_scores=True)
    for i, r in enumerate(rows):
        beta_p = r // 128
        for g in range(P.G):
            s = res["sel"][i, g]
            chosen = [int(x) for x in s if x >= 0]
            assert beta_p in chosen
            assert len(chosen) == min(w.top_k, beta_p + 1)
            assert chosen == sorted(set(chosen))
            assert max(chosen) == beta_p
            assert all(x == -1 for x in s[len(chosen):])
            assert _is_valid_topk(res["S"][i][g], beta_p, set(chosen) - {beta_p})
            sc = res["sel_score"][i, g]
            assert sc[len(chosen) - 1] == np.inf
