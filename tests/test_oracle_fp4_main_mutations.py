"""The 4-bit Main Branch pins must catch plausible mistakes: each case plants
one mistake in oracle/fp4_main.py (CPU only, via monkeypatch) and checks that
some pin then fails."""
import numpy as np
import pytest

from oracle import fp4_index as F4
from oracle import fp4_main as M4
import test_oracle_fp4_main as TP

PINS = [
    TP.test_scale_is_per_row_head_and_32_elements,
    TP.test_values_on_the_grid_round_trip_exactly,
    TP.test_error_bound,
    TP.test_main_branch_on_dequantised_values_is_dense_attention,
]

ORIG_Q = M4.quantize_kv4


def _some_pin_fails():
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            return True
    return False


def _one_scale_per_row(x):
    x = np.asarray(x, dtype=np.float64)
    T, G, d = x.shape
    codes, ex = F4.quantize_k_idx4(x.reshape(T * G, d), group=d)
    return codes.reshape(T, G, d), np.repeat(ex.reshape(T, G, 1), d // 32, axis=2)


def _truncating_codes(x):
    codes, ex = ORIG_Q(x)
    vals = M4.dequantize_kv4(codes, ex)
    x = np.asarray(x, dtype=np.float64)
    # round toward zero: step down one grid point wherever rounding went up in magnitude
    up = np.abs(vals) > np.abs(x)
    c = codes.copy()
    low = (c & 7) > 0
    c[up & low] = (c[up & low] & 8) | ((c[up & low] & 7) - 1)
    return c, ex


MUTATIONS = {
    "one_scale_per_row": _one_scale_per_row,
    "truncating_codes": _truncating_codes,
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    monkeypatch.setattr(M4, "quantize_kv4", MUTATIONS[name])
    assert _some_pin_fails(), f"mutation {name} not caught by any pin"


def test_unmutated_oracle_passes_every_pin():
    assert not _some_pin_fails()
