"""The 4-bit pins must catch plausible mistakes: each case plants one mistake
in the 4-bit index-key oracle (CPU only, via monkeypatch) and checks that some
pin then fails."""
import math

import numpy as np
import pytest

from oracle import fp4_index as F4
import test_oracle_fp4 as TF

PINS = [
    TF.test_decode_matches_library_for_all_codes,
    TF.test_encode_matches_library_rne,
    TF.test_encode_midpoints_round_to_even,
    TF.test_encode_roundtrip_every_code,
    TF.test_scale_exponent_closed_forms,
    TF.test_scale_exponent_is_smallest,
    TF.test_group_scale_is_per_32_elements,
    TF.test_group_exponent_follows_group_maximum,
    TF.test_quantisation_error_bound,
    TF.test_representable_values_quantise_to_themselves,
    TF.test_pack_matches_library,
    TF.test_selection_on_representable_inputs_equals_unquantised_oracle,
]


def _some_pin_fails():
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            return True
    return False


POS = F4.e2m1_table()[:8]


def _encode_ties_away(x):
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    i = np.clip(np.searchsorted(POS, a, side="right") - 1, 0, 7)
    j = np.minimum(i + 1, 7)
    code = np.where((POS[j] - a) <= (a - POS[i]), j, i).astype(np.uint8)
    return np.where(np.signbit(x), code | 0x8, code).astype(np.uint8)


def _encode_truncate(x):
    x = np.asarray(x, dtype=np.float64)
    i = np.clip(np.searchsorted(POS, np.abs(x), side="right") - 1, 0, 7).astype(np.uint8)
    return np.where(np.signbit(x), i | 0x8, i).astype(np.uint8)


def _decode_subnormal_quarter(code):
    code = int(code) & 0xF
    sign = -1.0 if code & 0x8 else 1.0
    e, m = (code >> 1) & 3, code & 1
    if e == 0:
        return sign * m * 0.25
    return sign * (1.0 + m / 2.0) * 2.0 ** (e - 1)


def _scale_floor_log2(amax):
    # the saturating alternative: floor(log2 amax) - 2, values above 6 clamped
    if amax == 0:
        return 0
    _, E = math.frexp(float(amax))
    return max(-127, min(127, E - 1 - 2))


def _scale_off_by_one(amax):
    if amax == 0:
        return 0
    f, E = math.frexp(float(amax))
    return max(-127, min(127, (E - 3 if f < 0.75 else E - 2)))


def _scales_floor_log2(amax):
    a = np.asarray(amax, dtype=np.float64)
    _, E = np.frexp(a)
    return np.clip(np.where(a == 0, 0, E - 3), -127, 127).astype(np.int64)


def _quantize_per_row(k_idx, group=F4.GROUP):
    k = np.asarray(k_idx, dtype=np.float64)
    T, D = k.shape
    codes = np.zeros((T, D), dtype=np.uint8)
    ex = np.zeros((T, D // group), dtype=np.uint8)
    for t in range(T):
        e = F4.scale_exponent4(np.abs(k[t]).max())
        codes[t] = F4.e2m1_encode(np.ldexp(k[t], -e))
        ex[t, :] = e + 127
    return codes, ex


def _pack_high_first(codes):
    c = np.asarray(codes, dtype=np.uint8)
    return ((c[:, 0::2] << 4) | c[:, 1::2]).astype(np.uint8)


MUTATIONS = {
    "ties_away": [("e2m1_encode", _encode_ties_away)],
    "truncate": [("e2m1_encode", _encode_truncate)],
    "subnormal_quarter": [("e2m1_decode", _decode_subnormal_quarter)],
    "scale_floor_log2": [("scale_exponent4", _scale_floor_log2)],
    "scale_off_by_one": [("scale_exponent4", _scale_off_by_one)],
    "scale_per_row": [("quantize_k_idx4", _quantize_per_row)],
    "vector_scale_floor_log2": [("scale_exponents4", _scales_floor_log2)],
    "pack_high_first": [("pack", _pack_high_first)],
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    for attr, fn in MUTATIONS[name]:
        monkeypatch.setattr(F4, attr, fn)
    if name == "subnormal_quarter":
        table = np.array([_decode_subnormal_quarter(c) for c in range(16)])
        monkeypatch.setattr(F4, "_TABLE", table)
        monkeypatch.setattr(F4, "_POS", table[:8])
    assert _some_pin_fails(), f"mutation {name} not caught by any pin"


def test_unmutated_oracle_passes_every_pin():
    assert not _some_pin_fails()
