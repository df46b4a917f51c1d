"""The pins must catch plausible mistakes: each case plants one mistake in the
oracle (CPU only, via monkeypatch) and checks that some pin then fails."""
import math

import numpy as np
import pytest

from oracle import msa_oracle as O
import test_oracle_index as TI
import test_oracle_main as TM
import test_oracle_ties as TT


def _attend_variant(scale_mul=1.0, group_of=None, causal=True):
    def attend_row(q_row, k_seq, v_seq, p, sel_by_group, scale, block=O.BLOCK):
        q = np.asarray(q_row, dtype=np.float64)
        Hq, d = q.shape
        G = len(sel_by_group)
        hpg = Hq // G
        out = np.empty((Hq, d))
        lse = np.empty((Hq,))
        for h in range(Hq):
            g = group_of(h, Hq, G) if group_of else h // hpg
            J = []
            for beta in sorted(sel_by_group[g]):
                hi = min((beta + 1) * block, p + 1) if causal else (beta + 1) * block
                hi = min(hi, len(k_seq))
                J.extend(range(beta * block, hi))
            K = np.asarray(k_seq[J, g], np.float64)
            V = np.asarray(v_seq[J, g], np.float64)
            z = scale * scale_mul * (K @ q[h])
            m = z.max()
            wts = np.exp(z - m)
            out[h] = wts @ V / wts.sum()
            lse[h] = m + math.log(wts.sum())
        return out, lse
    return attend_row


def _select_no_local(S_g, beta_p, top_k):
    order = sorted(range(beta_p + 1), key=lambda b: (-float(S_g[b]), b))
    return sorted(order[:min(top_k, beta_p + 1)])


def _select_high_id_ties(S_g, beta_p, top_k):
    others = list(range(beta_p))
    if len(others) > top_k - 1:
        others = sorted(others, key=lambda b: (-float(S_g[b]), -b))[: top_k - 1]
    return sorted(others + [beta_p])


def _pool_min(s, p, block=O.BLOCK):
    nbv = p // block + 1
    return np.stack([s[:, b * block:min((b + 1) * block, p + 1)].min(axis=1) for b in range(nbv)], 1)


def _scores_drop_last(q_idx_row, k_idx_seq, p):
    q = np.asarray(q_idx_row, np.float64)
    k = np.asarray(k_idx_seq[: p + 1], np.float64).copy()
    k[p] = 0.0
    return q @ k.T


def _lists_unstable(sel, seq_of_row, batch, G, nb_max):
    off, ent = ORIG_LISTS(sel, seq_of_row, batch, G, nb_max)
    ent = ent.copy()
    for u in range(len(off) - 1):
        ent[off[u]:off[u + 1]] = ent[off[u]:off[u + 1]][::-1]
    return off, ent


ORIG_LISTS = O.build_block_query_lists


def _near_tie_off_by_one(S_g, beta_p, top_k, rel=1e-4):
    # compares S_(k-2) with S_(k-1) instead of S_(k-1) with S_(k)
    if beta_p <= top_k - 1 or top_k < 3:
        return False
    v = np.sort(np.asarray(S_g[:beta_p], dtype=np.float64))[::-1]
    a, b = v[top_k - 3], v[top_k - 2]
    return (a - b) <= rel * max(abs(a), abs(b), 1e-30)


def _near_tie_absolute(S_g, beta_p, top_k, rel=1e-4):
    if beta_p <= top_k - 1 or top_k < 2:
        return False
    v = np.sort(np.asarray(S_g[:beta_p], dtype=np.float64))[::-1]
    return (v[top_k - 2] - v[top_k - 1]) <= rel


def _near_tie_signed_scale(S_g, beta_p, top_k, rel=1e-4):
    if beta_p <= top_k - 1 or top_k < 2:
        return False
    v = np.sort(np.asarray(S_g[:beta_p], dtype=np.float64))[::-1]
    a, b = v[top_k - 2], v[top_k - 1]
    return (a - b) <= rel * max(a, b, 1e-30)


def _near_tie_with_local(S_g, beta_p, top_k, rel=1e-4):
    if beta_p <= top_k - 1 or top_k < 2:
        return False
    v = np.sort(np.asarray(S_g[:beta_p + 1], dtype=np.float64))[::-1]
    a, b = v[top_k - 2], v[top_k - 1]
    return (a - b) <= rel * max(abs(a), abs(b), 1e-30)


def _valid_floor_only(S_g, beta_p, top_k, chosen, rel=1e-4):
    # every chosen block above S_(k) - tol, with no check against the unchosen blocks
    chosen = [int(x) for x in chosen if x >= 0]
    if beta_p not in chosen or len(chosen) != min(top_k, beta_p + 1):
        return False
    if len(set(chosen)) != len(chosen) or max(chosen) > beta_p:
        return False
    if beta_p <= top_k - 1:
        return True
    v = np.sort(np.asarray(S_g[:beta_p], dtype=np.float64))[::-1]
    kth, nxt = v[top_k - 2], v[top_k - 1]
    floor_ = nxt - rel * max(abs(kth), abs(nxt), 1e-30)
    return all(S_g[c] >= floor_ for c in chosen if c != beta_p)


def _valid_variant(check_size=True, check_local=True, check_future=True, absolute=False):
    def valid_selection(S_g, beta_p, top_k, chosen, rel=1e-4):
        chosen = [int(x) for x in chosen if x >= 0]
        if check_local and beta_p not in chosen:
            return False
        if check_size and len(chosen) != min(top_k, beta_p + 1):
            return False
        if len(set(chosen)) != len(chosen) or (check_future and max(chosen) > beta_p):
            return False
        if beta_p <= top_k - 1:
            return True
        v = np.sort(np.asarray(S_g[:beta_p], dtype=np.float64))[::-1]
        tol = rel if absolute else rel * max(abs(v[top_k - 2]), abs(v[top_k - 1]), 1e-30)
        mine = [c for c in chosen if c != beta_p]
        rest = [u for u in range(beta_p) if u not in mine]
        if not mine or not rest:
            return True
        return max(S_g[u] for u in rest) - min(S_g[c] for c in mine) <= tol
    return valid_selection

PINS = [TI.test_hand_worked_selections,
        lambda: [TI.test_selection_brute_force(s) for s in range(40)],
        TI.test_scores_and_pool_constructed,
        TI.test_pool_ignores_invisible_tokens_of_local_block,
        TI.test_score_is_a_dot_product_closed_form,
        TI.test_selection_invariants_tiny,
        TM.test_dense_when_k_covers_everything,
        TM.test_k1_is_block_diagonal_causal,
        TM.test_general_selection_against_library_attention,
        TM.test_zero_query_closed_form,
        TM.test_lists_are_exact_inverse_of_selection,
        TT.test_near_tie_hand_worked,
        TT.test_valid_selection_hand_worked,
        lambda: [TT.test_valid_selection_brute_force(s) for s in range(60)],
        lambda: [TT.test_near_tie_brute_force(s) for s in range(30)],
        TT.test_default_scale_against_library_default]

MUTATIONS = {
    "pool_uses_min": ("block_max_pool", _pool_min),
    "score_drops_last_visible_token": ("index_token_scores", _scores_drop_last),
    "local_block_not_forced": ("select_blocks", _select_no_local),
    "ties_prefer_high_id": ("select_blocks", _select_high_id_ties),
    "scale_off_by_sqrt_d": ("attend_row", _attend_variant(scale_mul=2.0)),
    "head_to_group_interleaved": ("attend_row", _attend_variant(group_of=lambda h, Hq, G: h % G)),
    "local_block_not_causal": ("attend_row", _attend_variant(causal=False)),
    "lists_not_ascending": ("build_block_query_lists", _lists_unstable),
    "near_tie_off_by_one_order_statistic": ("near_tie", _near_tie_off_by_one),
    "near_tie_absolute_tolerance": ("near_tie", _near_tie_absolute),
    "near_tie_signed_scale": ("near_tie", _near_tie_signed_scale),
    "near_tie_counts_local_block": ("near_tie", _near_tie_with_local),
    "valid_selection_floor_only": ("valid_selection", _valid_floor_only),
    "valid_selection_no_size_check": ("valid_selection", _valid_variant(check_size=False)),
    "valid_selection_no_local_check": ("valid_selection", _valid_variant(check_local=False)),
    "valid_selection_allows_future_block": ("valid_selection", _valid_variant(check_future=False)),
    "valid_selection_absolute_tolerance": ("valid_selection", _valid_variant(absolute=True)),
    "default_scale_one_over_d": ("default_scale", lambda d: 1.0 / d),
    "default_scale_sqrt_d": ("default_scale", lambda d: math.sqrt(d)),
    "default_scale_one_over_sqrt_index_dim_guess": ("default_scale", lambda d: 1.0 / math.sqrt(2 * d)),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_some_pin_catches(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    failed = 0
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed += 1
    assert failed > 0, f"no pin caught mutation {name}"
