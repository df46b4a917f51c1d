"""The KL-target pins must catch plausible mistakes: each case plants one
mistake in the oracle (CPU only, via monkeypatch) and checks that some pin
then fails."""
import math

import numpy as np
import pytest

from oracle import kl_target as KL
from oracle import msa_oracle as O
import test_oracle_kl as TK

PINS = [TK.test_mass_sums_to_one_and_is_a_distribution,
        TK.test_zero_query_gives_uniform_mass,
        TK.test_dense_selection_matches_library_softmax,
        TK.test_log_softmax_and_kl_closed_forms,
        TK.test_local_block_score_ignores_invisible_tokens,
        TK.test_index_distribution_sees_only_the_selection]


def _some_pin_fails():
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            return True
    return False


ORIG_MASS = KL.block_mass
ORIG_ROW = KL.row_target


def _mass_summed(*a, **k):
    hpg = np.asarray(a[0]).shape[0] // len(a[4])
    return [m * hpg for m in ORIG_MASS(*a, **k)]


def _mass_first_head(q_row, k_seq, v_seq, p, sel_by_group, scale, block=O.BLOCK):
    q = np.asarray(q_row, dtype=np.float64).copy()
    G = len(sel_by_group)
    hpg = q.shape[0] // G
    for g in range(G):
        q[g * hpg:(g + 1) * hpg] = q[g * hpg]
    return ORIG_MASS(q, k_seq, v_seq, p, sel_by_group, scale, block)


def _row_q_over_all_visible(P, r, sel_row):
    m, _, _ = ORIG_ROW(P, r, sel_row)
    b, p, ko = int(P.seq[r]), int(P.pos[r]), int(P.koff[r])
    lk = int(P.cu_k[b + 1] - P.cu_k[b])
    S = O.block_max_pool(O.index_token_scores(P.q_idx[r], P.k_idx[ko:ko + lk], p), p)
    k = sel_row.shape[1]
    lq = np.full((P.G, k), np.nan)
    klv = np.zeros(P.G)
    for g in range(P.G):
        blocks = [int(x) for x in sel_row[g] if x >= 0]
        full = S[g]
        lse = full.max() + math.log(np.exp(full - full.max()).sum())
        lq[g, :len(blocks)] = [S[g, x] - lse for x in blocks]
        klv[g] = KL.kl(m[g, :len(blocks)], lq[g, :len(blocks)])
    return m, lq, klv


def _local_whole_block(q_idx_row_g, k_idx_seq, p, block=O.BLOCK):
    lo = (p // block) * block
    k = np.asarray(k_idx_seq[lo:lo + block], dtype=np.float64)
    return float((k @ np.asarray(q_idx_row_g, dtype=np.float64)).max())


def _kl_reversed(p_mass, log_q):
    p_mass = np.asarray(p_mass, dtype=np.float64)
    q = np.exp(np.asarray(log_q, dtype=np.float64))
    nz = p_mass > 0
    return float((q[nz] * (np.log(q[nz]) - np.log(p_mass[nz]))).sum())


def test_pins_pass_unmutated():
    assert not _some_pin_fails()


@pytest.mark.parametrize("name", ["mass_summed", "mass_first_head", "q_over_all_visible",
                                  "local_whole_block", "kl_reversed"])
def test_mutation_is_caught(monkeypatch, name):
    if name == "mass_summed":
        monkeypatch.setattr(KL, "block_mass", _mass_summed)
    elif name == "mass_first_head":
        monkeypatch.setattr(KL, "block_mass", _mass_first_head)
    elif name == "q_over_all_visible":
        monkeypatch.setattr(KL, "row_target", _row_q_over_all_visible)
    elif name == "local_whole_block":
        monkeypatch.setattr(KL, "local_block_score", _local_whole_block)
    elif name == "kl_reversed":
        monkeypatch.setattr(KL, "kl", _kl_reversed)
    assert _some_pin_fails(), name
