"""Pins of the oracle's Main Branch, log-sum-exp merge, decode and lists.

Independent references: torch's scaled_dot_product_attention in float64 on
the CPU (a library routine, not the oracle's numpy code), closed forms, and
structural properties.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from msa_inputs import custom, generate, workload
from oracle import msa_oracle as O


def _problem(w, dtype=np.float64, top_k=None, t=None):
    t = t or generate(w, "cpu")
    c = lambda x: x.double().numpy().astype(dtype)
    P = O.Problem(c(t["q"]), c(t["k"]), c(t["v"]), c(t["q_idx"]), c(t["k_idx"]),
                  t["cu_seqlens_q"].numpy(), t["cu_seqlens_k"].numpy(),
                  w.top_k if top_k is None else top_k)
    return P, t


def _sdpa_rows(P, b, mask_fn):
    """Library attention for every query of sequence b: float64 SDPA with an
    explicit boolean mask [Hkv, Lq, Lk] expanded over the group's heads."""
    q0, q1 = int(P.cu_q[b]), int(P.cu_q[b + 1])
    k0, k1 = int(P.cu_k[b]), int(P.cu_k[b + 1])
    q = torch.from_numpy(np.asarray(P.q[q0:q1], np.float64)).permute(1, 0, 2)      # [Hq, Lq, d]
    k = torch.from_numpy(np.asarray(P.k[k0:k1], np.float64)).permute(1, 0, 2)      # [G, Lk, d]
    v = torch.from_numpy(np.asarray(P.v[k0:k1], np.float64)).permute(1, 0, 2)
    hpg = P.Hq // P.G
    k = k.repeat_interleave(hpg, dim=0).contiguous()
    v = v.repeat_interleave(hpg, dim=0).contiguous()
    mask = mask_fn(q1 - q0, k1 - k0)                                               # [G, Lq, Lk] bool
    mask = torch.from_numpy(mask).repeat_interleave(hpg, dim=0)
    out = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=P.scale)
    return out.permute(1, 0, 2).numpy()


def test_dense_when_k_covers_everything():
    """top_k >= number of blocks: MSA equals dense causal GQA."""
    w = custom([600, 333], [600, 333], num_q_heads=6, num_kv_heads=2, head_dim=32,
               index_dim=16, top_k=8, seed=11, qkv_std=1.0)
    P, _ = _problem(w)
    res = P.run()
    for b in range(P.batch):
        q0, q1 = int(P.cu_q[b]), int(P.cu_q[b + 1])
        lq = q1 - q0
        lk = int(P.cu_k[b + 1] - P.cu_k[b])
        causal = lambda lq_, lk_: np.broadcast_to(
            np.tril(np.ones((lq_, lk_), bool), k=lk_ - lq_), (P.G, lq_, lk_)).copy()
        ref = _sdpa_rows(P, b, causal)
        np.testing.assert_allclose(res["out"][q0:q1], ref, rtol=0, atol=1e-12)


def test_k1_is_block_diagonal_causal():
    w = custom([700], [700], num_q_heads=4, num_kv_heads=2, head_dim=16, index_dim=8,
               top_k=1, seed=12, qkv_std=1.0)
    P, _ = _problem(w)
    res = P.run()

    def mask(lq, lk):
        i = np.arange(lq)[:, None] + (lk - lq)
        j = np.arange(lk)[None, :]
        m = (j <= i) & (j // 128 == i // 128)
        return np.broadcast_to(m, (P.G, lq, lk)).copy()

    ref = _sdpa_rows(P, 0, mask)
    np.testing.assert_allclose(res["out"], ref, rtol=0, atol=1e-12)


def test_general_selection_against_library_attention():
    w = custom([1500, 900], [1500, 300], num_q_heads=4, num_kv_heads=2, head_dim=32,
               index_dim=16, top_k=4, seed=13, qkv_std=1.0)
    P, _ = _problem(w)
    res = P.run()
    for b in range(P.batch):
        q0, q1 = int(P.cu_q[b]), int(P.cu_q[b + 1])
        sel = res["sel"][q0:q1]                                   # [Lq, G, k]

        def mask(lq, lk, sel=sel):
            i = np.arange(lq) + (lk - lq)
            blk = np.arange(lk) // 128
            m = np.zeros((P.G, lq, lk), bool)
            for g in range(P.G):
                for r in range(lq):
                    ok = np.isin(blk, sel[r, g][sel[r, g] >= 0])
                    m[g, r] = ok & (np.arange(lk) <= i[r])
            return m

        ref = _sdpa_rows(P, b, mask)
        np.testing.assert_allclose(res["out"][q0:q1], ref, rtol=0, atol=1e-12)


def test_zero_query_closed_form():
    """q = 0: all logits equal, so out = mean of V over J and lse = log |J|."""
    w = custom([1000], [1000], num_q_heads=2, num_kv_heads=1, head_dim=8, index_dim=8,
               top_k=3, seed=14)
    P, _ = _problem(w)
    P.q = np.zeros_like(P.q)
    for r in (0, 127, 128, 500, 999):
        res = P.row(r)
        chosen = [int(x) for x in res["sel"][0] if x >= 0]
        J = [j for j in range(r + 1) if j // 128 in chosen]
        np.testing.assert_allclose(res["out"][0], P.v[J, 0].mean(axis=0), atol=1e-13)
        assert abs(res["lse"][0] - math.log(len(J))) < 1e-13
        assert len(J) == sum(min(128, r + 1 - 128 * c) for c in chosen)


def test_merge_identity():
    w = workload("tiny")
    P, _ = _problem(w)
    for r in (5, 300, 1100, 2047):
        res = P.row(r)
        for h in range(P.Hq):
            g = h // (P.Hq // P.G)
            parts = [O.block_partial(P.q[r, h], P.k, P.v, r, int(beta), g, P.scale)
                     for beta in res["sel"][g] if beta >= 0]
            out, lse = O.merge_partials(parts)
            np.testing.assert_allclose(out, res["out"][h], atol=1e-12)
            assert abs(lse - res["lse"][h]) < 1e-12


def test_lse_against_logsumexp_of_library_scores():
    w = custom([400], [400], num_q_heads=2, num_kv_heads=1, head_dim=16, index_dim=8,
               top_k=2, seed=15, qkv_std=1.0)
    P, _ = _problem(w)
    for r in (10, 200, 399):
        res = P.row(r)
        chosen = [int(x) for x in res["sel"][0] if x >= 0]
        keep = torch.tensor([j // 128 in chosen and j <= r for j in range(400)])
        z = (torch.from_numpy(P.k[:, 0]) @ torch.from_numpy(P.q[r, 1])) * P.scale
        ref = torch.logsumexp(z[keep], dim=0).item()
        assert abs(res["lse"][1] - ref) < 1e-12


def test_decode_row_equals_prefill_last_row():
    """One new token at position N-1 (decode) gives the prefill's last row."""
    L = 777
    wp = custom([L], [L], num_q_heads=4, num_kv_heads=2, head_dim=16, index_dim=8,
                top_k=3, seed=16, qkv_std=1.0)
    Pp, t = _problem(wp)
    last = Pp.row(L - 1)
    td = dict(t)
    td["q"] = t["q"][L - 1:L].clone()
    td["q_idx"] = t["q_idx"][L - 1:L].clone()
    td["cu_seqlens_q"] = torch.tensor([0, 1], dtype=torch.int32)
    wd = custom([L], [1], 4, 2, 16, 8, 3, 16)
    Pd, _ = _problem(wd, t=td)
    dec = Pd.row(0)
    assert np.array_equal(dec["sel"], last["sel"])
    np.testing.assert_array_equal(dec["out"], last["out"])


def test_group_heads_share_selection_groups_independent():
    w = custom([1024], [1024], num_q_heads=8, num_kv_heads=2, head_dim=16, index_dim=8,
               top_k=3, seed=17, qkv_std=1.0)
    P, _ = _problem(w)
    # make group 1's index queries the negation of group 0's: different picks expected
    P.q_idx = P.q_idx.copy()
    P.q_idx[:, 1] = -P.q_idx[:, 0]
    diffs = 0
    for r in range(600, 1024, 17):
        res = P.row(r)
        diffs += int(not np.array_equal(res["sel"][0], res["sel"][1]))
        # heads of one group attend over the same keys: swapping the queries of
        # two heads in a group swaps their outputs exactly
        q2 = P.q.copy()
        q2[r, [0, 1]] = q2[r, [1, 0]]
        P2 = O.Problem(q2, P.k, P.v, P.q_idx, P.k_idx, P.cu_q, P.cu_k, P.top_k)
        res2 = P2.row(r)
        np.testing.assert_array_equal(res2["out"][0], res["out"][1])
    assert diffs > 0


def test_lists_are_exact_inverse_of_selection():
    w = custom([1500, 900], [1500, 300], num_q_heads=4, num_kv_heads=2, head_dim=16,
               index_dim=8, top_k=4, seed=18, qkv_std=1.0)
    P, _ = _problem(w)
    sel = P.run()["sel"]
    off, ent = O.build_block_query_lists(sel, P.seq, P.batch, P.G, P.nb_max)
    # independent construction with plain loops
    expect = {}
    for r in range(sel.shape[0]):
        for g in range(P.G):
            for s in range(P.top_k):
                beta = sel[r, g, s]
                if beta >= 0:
                    u = (int(P.seq[r]) * P.G + g) * P.nb_max + int(beta)
                    expect.setdefault(u, []).append(r * 32 + s)
    U = P.batch * P.G * P.nb_max
    assert len(off) == U + 1 and off[0] == 0 and off[-1] == len(ent)
    for u in range(U):
        got = list(ent[off[u]:off[u + 1]])
        assert got == expect.get(u, []), u
        rows = [e >> 5 for e in got]
        assert rows == sorted(rows)
