"""The projection pins must catch plausible mistakes: each case plants one
mistake in the projection oracle (CPU only, via monkeypatch) and checks that
some pin then fails."""
import numpy as np
import pytest

from oracle import projections as PR
import test_oracle_projections as TP

PINS = [
    TP.test_bf16_round_matches_library_on_float32_values,
    TP.test_bf16_round_no_double_rounding,
    TP.test_identity_weights_return_the_input,
    TP.test_one_hot_inputs_pick_weight_columns,
    TP.test_power_of_two_scaling_commutes,
    TP.test_new_keys_land_after_the_cached_ones,
    TP.test_general_inputs_against_library_product,
]


def _some_pin_fails():
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError, KeyError):
            return True
    return False


ORIG_ROUND = PR.bf16_round
ORIG_PROJECT = PR.project


def _round_truncate(x):
    v = np.asarray(x, dtype=np.float64)
    a = np.abs(v)
    _, e = np.frexp(a)
    q = np.ldexp(1.0, np.maximum(e, -125) - 8)
    y = np.copysign(np.floor(a / q) * q, v)
    return np.where((a == 0.0) | ~np.isfinite(v), v, y)


def _round_via_float32(x):
    v = np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    return ORIG_ROUND(v)


def _project_group_minor(x, w_q, w_k, cu_q, cu_k, total_k, G):
    q, rows = ORIG_PROJECT(x, w_q, w_k, cu_q, cu_k, total_k, G)
    T, _, di = q.shape
    return q.reshape(T, di, G).transpose(0, 2, 1).copy(), rows


def _project_keys_at_front(x, w_q, w_k, cu_q, cu_k, total_k, G):
    q, _ = ORIG_PROJECT(x, w_q, w_k, cu_q, cu_k, total_k, G)
    k_new = PR.bf16_round(np.asarray(x, np.float64) @ np.asarray(w_k, np.float64).T)
    rows = {}
    for b in range(len(cu_q) - 1):
        for i in range(int(cu_q[b + 1] - cu_q[b])):
            rows[int(cu_k[b]) + i] = k_new[int(cu_q[b]) + i]      # mistake: first positions
    return q, rows


def _project_no_rounding(x, w_q, w_k, cu_q, cu_k, total_k, G):
    x = np.asarray(x, np.float64)
    T = x.shape[0]
    q = (x @ np.asarray(w_q, np.float64).T).reshape(T, G, -1)
    _, rows = ORIG_PROJECT(x, w_q, w_k, cu_q, cu_k, total_k, G)
    return q, rows


def _project_wrong_weight_half(x, w_q, w_k, cu_q, cu_k, total_k, G):
    # mistake: k from the first d_idx rows of W_q instead of W_k
    q, rows = ORIG_PROJECT(x, w_q, w_k, cu_q, cu_k, total_k, G)
    di = np.asarray(w_k).shape[0]
    _, rows2 = ORIG_PROJECT(x, w_q, np.asarray(w_q)[:di], cu_q, cu_k, total_k, G)
    return q, rows2


def test_pins_pass_unmutated():
    assert not _some_pin_fails()


@pytest.mark.parametrize("name", ["truncate", "via_float32", "group_minor", "keys_at_front",
                                  "no_rounding", "wrong_weight"])
def test_mutation_is_caught(monkeypatch, name):
    if name == "truncate":
        monkeypatch.setattr(PR, "bf16_round", _round_truncate)
    elif name == "via_float32":
        monkeypatch.setattr(PR, "bf16_round", _round_via_float32)
    elif name == "group_minor":
        monkeypatch.setattr(PR, "project", _project_group_minor)
    elif name == "keys_at_front":
        monkeypatch.setattr(PR, "project", _project_keys_at_front)
    elif name == "no_rounding":
        monkeypatch.setattr(PR, "project", _project_no_rounding)
    elif name == "wrong_weight":
        monkeypatch.setattr(PR, "project", _project_wrong_weight_half)
    assert _some_pin_fails(), name
