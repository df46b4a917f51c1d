"""Pins of the oracle's near-tie rule, its selection-validity check and its
default softmax scale.

near_tie and valid_selection decide which GPU selections the parity tests
accept, so each is pinned by hand-worked cases at, just below and just above
the tolerance (tests/golden/near_tie.json) and by brute force over every
subset on small rows.  The brute force states validity differently from the
oracle: a selection is valid when it is the exact top-(k-1) of some scores
that differ from the given ones by at most half the tolerance each.
default_scale is pinned by a library routine that applies its own default.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from msa_inputs import custom, generate
from oracle import msa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
REL = 1e-4


def _golden():
    return json.load(open(os.path.join(GOLDEN, "near_tie.json")))


def test_near_tie_hand_worked():
    for c in _golden()["near_tie"]:
        got = O.near_tie(np.asarray(c["scores"]), c["beta_p"], c["top_k"])
        assert got == c["expected"], c["name"]


def test_valid_selection_hand_worked():
    for c in _golden()["valid_selection"]:
        got = O.valid_selection(np.asarray(c["scores"]), c["beta_p"], c["top_k"], c["chosen"])
        assert got == c["expected"], c["name"]


def _top_of_perturbed(S, beta_p, m, C, half_tol):
    """Top-m earlier blocks after raising the blocks of C by half_tol and
    lowering the others by half_tol; equal perturbed scores favour C."""
    Sp = [(S[b] + half_tol, 0) if b in C else (S[b] - half_tol, 1) for b in range(beta_p)]
    order = sorted(range(beta_p), key=lambda b: (-Sp[b][0], Sp[b][1]))
    return set(order[:m])


def _tolerance_by_hand(S, beta_p, top_k):
    v = sorted((float(x) for x in S[:beta_p]), reverse=True)
    return REL * max(abs(v[top_k - 2]), abs(v[top_k - 1]), 1e-30)


@pytest.mark.parametrize("seed", range(60))
def test_valid_selection_brute_force(seed):
    """Every (k-1)-subset of up to 7 earlier blocks: valid exactly when it is
    the top-(k-1) of scores moved by at most tol/2 each."""
    rng = np.random.default_rng(seed)
    nb = int(rng.integers(3, 9))
    beta_p = nb - 1
    top_k = int(rng.integers(2, beta_p + 3))
    # quarter-offset integers near 10^4: gaps of 1 sit near the tolerance (about 1.0), gaps of
    # 2 beyond it; the tolerance is never an integer, so no case lands on it exactly
    S = (10000.25 + rng.integers(-3, 4, size=nb)).astype(np.float64)
    S[beta_p] = rng.integers(-50, 50)                   # the local block's score is irrelevant
    m = min(top_k - 1, beta_p)
    if beta_p <= top_k - 1:
        sets = [set(range(beta_p))]
        tol = 0.0
    else:
        sets = [set(c) for c in itertools.combinations(range(beta_p), m)]
        tol = _tolerance_by_hand(S, beta_p, top_k)
        assert abs(tol - round(tol)) > 1e-6
    n_valid = 0
    for C in sets:
        expect = _top_of_perturbed(S, beta_p, m, C, tol / 2) == C
        got = O.valid_selection(S, beta_p, top_k, sorted(C | {beta_p}))
        assert got == expect, (S.tolist(), beta_p, top_k, sorted(C))
        n_valid += int(expect)
        # the same set without the local block, or with one block too many, never passes
        assert not O.valid_selection(S, beta_p, top_k, sorted(C))
        extra = [b for b in range(beta_p) if b not in C]
        if extra:
            assert not O.valid_selection(S, beta_p, top_k, sorted(C | {beta_p, extra[0]}))
    # the oracle's own selection is always valid, and it is the only one off a near-tie
    assert O.valid_selection(S, beta_p, top_k, O.select_blocks(S, beta_p, top_k))
    if not O.near_tie(S, beta_p, top_k):
        assert n_valid == 1


@pytest.mark.parametrize("seed", range(30))
def test_near_tie_brute_force(seed):
    """A row is a near-tie exactly when more than one selection is valid
    (the perturbation characterisation above) -- for rows with a choice."""
    rng = np.random.default_rng(1000 + seed)
    nb = int(rng.integers(4, 9))
    beta_p = nb - 1
    top_k = int(rng.integers(2, beta_p + 1))
    S = (10000.25 + rng.integers(-3, 4, size=nb)).astype(np.float64)
    m = top_k - 1
    tol = _tolerance_by_hand(S, beta_p, top_k)
    n_valid = sum(_top_of_perturbed(S, beta_p, m, set(C), tol / 2) == set(C)
                  for C in itertools.combinations(range(beta_p), m))
    assert O.near_tie(S, beta_p, top_k) == (n_valid > 1), (S.tolist(), beta_p, top_k)


def test_default_scale_against_library_default():
    """With no scale given, the Main Branch must use the library's own default
    softmax scale (torch's scaled_dot_product_attention without `scale=`,
    which applies 1/sqrt(head_dim)): top_k covering every block makes MSA
    dense causal GQA, so the two must agree."""
    for d in (16, 64):
        w = custom([300], [300], num_q_heads=4, num_kv_heads=2, head_dim=d, index_dim=8,
                   top_k=4, seed=21 + d, qkv_std=1.0)
        t = generate(w, "cpu")
        c = lambda x: x.double().numpy()
        P = O.Problem(c(t["q"]), c(t["k"]), c(t["v"]), c(t["q_idx"]), c(t["k_idx"]),
                      t["cu_seqlens_q"].numpy(), t["cu_seqlens_k"].numpy(), w.top_k)
        res = P.run()
        q = torch.from_numpy(c(t["q"])).permute(1, 0, 2)
        k = torch.from_numpy(c(t["k"])).permute(1, 0, 2).repeat_interleave(2, dim=0).contiguous()
        v = torch.from_numpy(c(t["v"])).permute(1, 0, 2).repeat_interleave(2, dim=0).contiguous()
        ref = F.scaled_dot_product_attention(q, k, v, is_causal=True).permute(1, 0, 2).numpy()
        np.testing.assert_allclose(res["out"], ref, rtol=0, atol=1e-12)
