"""Pins of the KL-alignment target oracle (oracle/kl_target.py), CPU only.

What fixes the answers: closed forms (uniform attention when the query is
zero; two-point log-softmax and KL values), invariants (masses sum to one;
KL(P || P) = 0 and KL >= 0; log Q unchanged by a common shift of the scores;
the local block's score ignores its invisible tokens; Q only sees the
selected blocks), and, for a selection that covers every block, the dense
attention weights from torch.softmax (a library routine) summed per block.
"""
import math

import numpy as np
import torch

from oracle import kl_target as KL
from oracle import msa_oracle as O


def _problem(seed, L=700, Hq=4, G=2, d=32, di=32, top_k=3, scale_q=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((L, Hq, d)) * scale_q
    k = rng.standard_normal((L, G, d))
    v = rng.standard_normal((L, G, d))
    qi = rng.standard_normal((L, G, di))
    ki = rng.standard_normal((L, di))
    cu = np.array([0, L])
    return O.Problem(q, k, v, qi, ki, cu, cu, top_k)


def test_mass_sums_to_one_and_is_a_distribution():
    P = _problem(1)
    for r in (0, 130, 255, 256, 699):
        res = P.row(r)
        m, lq, kl = KL.row_target(P, r, res["sel"])
        for g in range(P.G):
            n = int((res["sel"][g] >= 0).sum())
            assert abs(m[g, :n].sum() - 1.0) < 1e-12
            assert np.all(m[g, :n] >= 0) and np.all(m[g, n:] == 0)
            assert abs(np.exp(lq[g, :n]).sum() - 1.0) < 1e-12
            assert kl[g] >= -1e-15


def test_zero_query_gives_uniform_mass():
    P = _problem(2, scale_q=0.0)
    r = 600
    res = P.row(r)
    m, _, _ = KL.row_target(P, r, res["sel"])
    p = int(P.pos[r])
    for g in range(P.G):
        blocks = [int(x) for x in res["sel"][g] if x >= 0]
        J = O.selected_keys(blocks, p)
        for i, beta in enumerate(blocks):
            assert abs(m[g, i] - np.sum(J // 128 == beta) / len(J)) < 1e-12


def test_dense_selection_matches_library_softmax():
    P = _problem(3, L=500, top_k=8)                # 4 blocks: the selection is everything
    r = 450
    res = P.row(r)
    m, _, _ = KL.row_target(P, r, res["sel"])
    p = int(P.pos[r])
    for g in range(P.G):
        K = torch.from_numpy(P.k[:p + 1, g])
        want = np.zeros(4)
        for h in range(g * 2, g * 2 + 2):
            w = torch.softmax(P.scale * (K @ torch.from_numpy(P.q[r, h])), dim=0).numpy()
            for beta in range(4):
                want[beta] += w[beta * 128:(beta + 1) * 128].sum() / 2
        assert np.allclose(m[g, :4], want, atol=1e-13, rtol=0)


def test_log_softmax_and_kl_closed_forms():
    lq = KL.index_log_probs([2.0, 1.0])
    z = math.log(math.e ** 2 + math.e)
    assert np.allclose(lq, [2.0 - z, 1.0 - z], atol=1e-15)
    assert np.allclose(KL.index_log_probs([2.0 + 37.0, 1.0 + 37.0]), lq, atol=1e-13)
    got = KL.kl([0.5, 0.5], np.log([0.25, 0.75]))
    assert abs(got - (0.5 * math.log(2.0) + 0.5 * math.log(2.0 / 3.0))) < 1e-15
    p = np.array([0.2, 0.0, 0.8])
    assert KL.kl(p, np.log([0.2, 0.3, 0.8])) == 0.0 + 0.0   # zero-mass term ignored, rest equal
    rng = np.random.default_rng(4)
    for _ in range(50):
        a = rng.dirichlet(np.ones(5))
        b = rng.dirichlet(np.ones(5))
        assert KL.kl(a, np.log(b)) >= 0 and abs(KL.kl(a, np.log(a))) < 1e-15


def test_local_block_score_ignores_invisible_tokens():
    rng = np.random.default_rng(5)
    ki = rng.standard_normal((400, 16))
    qv = rng.standard_normal(16)
    p = 300                                    # local block 2: tokens 256..383, visible 256..300
    ki[350] = qv * 100                         # invisible, would dominate
    want = max(float(ki[j] @ qv) for j in range(256, 301))
    assert KL.local_block_score(qv, ki, p) == want


def test_index_distribution_sees_only_the_selection():
    P = _problem(6, L=900, top_k=3)
    r = 800
    b_p = int(P.pos[r]) // 128
    res = P.row(r, want_scores=True)
    # a hand-made selection that leaves out the best-scoring earlier block
    S = res["S"]
    g = 0
    order = np.argsort(-S[g, :b_p])
    sel = np.array(res["sel"])
    sel[g] = sorted([int(order[1]), int(order[2]), b_p])
    _, lq, _ = KL.row_target(P, r, sel)
    want = KL.index_log_probs([S[g, x] for x in sel[g]])
    assert np.allclose(lq[g], want, atol=1e-13)
    # the left-out block must not appear in the normaliser
    full = S[g, :b_p + 1]
    wrong = np.array([S[g, x] for x in sel[g]]) - (full.max() + math.log(np.exp(full - full.max()).sum()))
    assert not np.allclose(lq[g], wrong, atol=1e-6)
