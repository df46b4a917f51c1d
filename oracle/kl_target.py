"""KL-alignment target of the Index Branch (forward only): oracle.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import or call this module.  It shares no
code, tables or helpers with the HIP library, and imports nothing from it.

Source: the MSA guide (ai-tool-zukan.com/minimax-msa-guide), sections
"非微分的な選択をどう学習させるか（KLダイバージェンス）" and "選択を学習可能にするKL損失":
the top-k choice is not differentiable, so the Index Branch is trained by
pulling the distribution of its per-block scores towards the distribution of
which blocks the Main Branch's exact attention actually relied on, measured by
a KL divergence.  The pages give no formula; readings:

K1  target P(beta) = the Main Branch's attention mass on selected block beta
    for (query, group): the softmax weights of the visible keys of beta,
    averaged over the group's query heads (each head's weights sum to 1 over
    the selected keys, so P sums to 1 over the selection).
K2  index distribution Q(beta) = softmax, over the selected blocks, of their
    block scores S(beta) (max-pooled index scores, no temperature); the local
    block's score is the max over its visible tokens.  Restricting Q to the
    blocks the Main Branch saw keeps both distributions on one support.
K3  divergence KL(P || Q) = sum over the selection of P (log P - log Q), per
    (query, group); terms with P = 0 contribute 0.  Forward pass only.
"""
from __future__ import annotations

import math

import numpy as np

from oracle import msa_oracle as O


def block_mass(q_row, k_seq, v_seq, p, sel_by_group, scale, block=O.BLOCK):
    """P[g][i] for the i-th selected block of group g (reading K1), fp64.

    Per head: softmax over J(p, g) of scale * q . k; summed over the block's
    visible keys; averaged over the group's heads.
    """
    q = np.asarray(q_row, dtype=np.float64)
    Hq = q.shape[0]
    G = len(sel_by_group)
    hpg = Hq // G
    out = []
    for g in range(G):
        blocks = sorted(sel_by_group[g])
        J = O.selected_keys(blocks, p, block)
        K = np.asarray(k_seq[J, g], dtype=np.float64)
        owner = J // block
        mass = np.zeros(len(blocks))
        for h in range(g * hpg, (g + 1) * hpg):
            z = scale * (K @ q[h])
            w = np.exp(z - z.max())
            w /= w.sum()
            for i, beta in enumerate(blocks):
                mass[i] += w[owner == beta].sum()
        out.append(mass / hpg)
    return out


def local_block_score(q_idx_row_g, k_idx_seq, p, block=O.BLOCK):
    """S of the query's own block: max of q_idx . k_idx over its visible tokens."""
    lo = (p // block) * block
    k = np.asarray(k_idx_seq[lo:p + 1], dtype=np.float64)
    return float((k @ np.asarray(q_idx_row_g, dtype=np.float64)).max())


def index_log_probs(scores):
    """log Q over the selection: log-softmax of the selected blocks' scores (K2)."""
    s = np.asarray(scores, dtype=np.float64)
    m = s.max()
    return s - (m + math.log(np.exp(s - m).sum()))


def kl(p_mass, log_q):
    """KL(P || Q) = sum P (log P - log Q), with 0 log 0 = 0 (K3)."""
    p_mass = np.asarray(p_mass, dtype=np.float64)
    log_q = np.asarray(log_q, dtype=np.float64)
    nz = p_mass > 0
    return float((p_mass[nz] * (np.log(p_mass[nz]) - log_q[nz])).sum())


def row_target(P, r, sel_row):
    """For query row r of problem P (msa_oracle.Problem) and a selection
    sel_row [G, top_k] (ascending, -1 padded): (mass [G, top_k],
    log_q [G, top_k], kl [G]); padding slots hold 0 mass and NaN log Q."""
    b, p, ko = int(P.seq[r]), int(P.pos[r]), int(P.koff[r])
    lk = int(P.cu_k[b + 1] - P.cu_k[b])
    groups = [[int(x) for x in sel_row[g] if x >= 0] for g in range(P.G)]
    mass = block_mass(P.q[r], P.k[ko:ko + lk], P.v[ko:ko + lk], p, groups, P.scale, P.block)
    kidx = P.k_idx[ko:ko + lk]
    s_tok = O.index_token_scores(P.q_idx[r], kidx, p)
    S = O.block_max_pool(s_tok, p, P.block)
    k = sel_row.shape[1]
    out_m = np.zeros((P.G, k))
    out_q = np.full((P.G, k), np.nan)
    out_kl = np.zeros(P.G)
    for g in range(P.G):
        blocks = groups[g]
        sc = [S[g, beta] for beta in blocks]            # the local block's S is its own max
        lq = index_log_probs(sc)
        out_m[g, :len(blocks)] = mass[g]
        out_q[g, :len(blocks)] = lq
        out_kl[g] = kl(mass[g], lq)
    return out_m, out_q, out_kl
