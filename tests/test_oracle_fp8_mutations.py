"""The fp8 pins must catch plausible mistakes: each case plants one mistake in
the quantised-index oracle (CPU only, via monkeypatch) and checks that some pin
then fails."""
import math

import numpy as np
import pytest

from oracle import fp8_index as F
import test_oracle_fp8 as TF

PINS = [
    TF.test_decode_matches_library_for_all_codes,
    TF.test_encode_matches_library_rne,
    TF.test_encode_midpoints_round_to_even,
    TF.test_encode_roundtrip_every_finite_code,
    TF.test_scale_exponent_closed_forms,
    TF.test_scale_exponent_is_smallest,
    TF.test_quantisation_error_bound,
    TF.test_representable_values_quantise_to_themselves,
    TF.test_k_block_scale_is_per_sequence_block,
    TF.test_k_block_exponent_follows_block_maximum,
    TF.test_selection_on_representable_inputs_equals_bf16_path,
    TF.test_query_power_of_two_scaling_leaves_selection,
]


def _some_pin_fails():
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            return True
    return False


ORIG_ENCODE = F.e4m3_encode
ORIG_TABLE = F._TABLE


def _encode_ties_away(x):
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    pos = ORIG_TABLE[:127]
    i = np.clip(np.searchsorted(pos, a, side="right") - 1, 0, 126)
    j = np.minimum(i + 1, 126)
    pick_hi = (pos[j] - a) <= (a - pos[i])
    code = np.where(pick_hi, j, i).astype(np.uint8)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


def _encode_truncate(x):
    x = np.asarray(x, dtype=np.float64)
    i = np.clip(np.searchsorted(ORIG_TABLE[:127], np.abs(x), side="right") - 1, 0, 126).astype(np.uint8)
    return np.where(np.signbit(x), i | 0x80, i).astype(np.uint8)


def _decode_bias8(code):
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 7
    if e == 15 and m == 7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -7
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 8)


def _scale_off_by_one(amax):
    if amax == 0:
        return 0
    f, E = math.frexp(float(amax))
    return max(-127, min(127, E - 8))


def _quantize_k_global_blocks(k_idx, cu_seqlens_k, nb_max, block=F.BLOCK):
    k = np.asarray(k_idx, dtype=np.float64)
    cu_k = np.asarray(cu_seqlens_k, dtype=np.int64)
    codes = np.zeros(k.shape, dtype=np.uint8)
    ex = np.full((len(cu_k) - 1, nb_max), 127, dtype=np.uint8)
    for b in range(len(cu_k) - 1):
        for beta in range(nb_max):
            lo = beta * block                    # mistake: blocks counted from row 0
            hi = min(lo + block, int(cu_k[-1]))
            if lo >= hi:
                continue
            e = F.scale_exponent(np.abs(k[lo:hi]).max())
            codes[lo:hi] = F.quantize(k[lo:hi], e)
            ex[b, beta] = e + 127
    return codes, ex


def _quantize_q_shared_over_groups(q_idx):
    q = np.asarray(q_idx, dtype=np.float64)
    T, G, _ = q.shape
    codes = np.zeros(q.shape, dtype=np.uint8)
    ex = np.zeros((T, G), dtype=np.uint8)
    for t in range(T):
        e = F.scale_exponent(np.abs(q[t]).max())  # mistake: one scale per token
        for g in range(G):
            codes[t, g] = F.quantize(q[t, g], e)
            ex[t, g] = e + 127
    return codes, ex


def test_pins_pass_unmutated():
    assert not _some_pin_fails()


@pytest.mark.parametrize("name", ["ties_away", "truncate", "bias8", "scale_off_by_one",
                                  "k_global_blocks", "q_shared_over_groups"])
def test_mutation_is_caught(monkeypatch, name):
    if name == "ties_away":
        monkeypatch.setattr(F, "e4m3_encode", _encode_ties_away)
    elif name == "truncate":
        monkeypatch.setattr(F, "e4m3_encode", _encode_truncate)
    elif name == "bias8":
        monkeypatch.setattr(F, "e4m3_decode", _decode_bias8)
        monkeypatch.setattr(F, "_TABLE", np.array([_decode_bias8(c) for c in range(256)]))
        monkeypatch.setattr(F, "_POS", np.array([_decode_bias8(c) for c in range(127)]))
    elif name == "scale_off_by_one":
        monkeypatch.setattr(F, "scale_exponent", _scale_off_by_one)
    elif name == "k_global_blocks":
        monkeypatch.setattr(F, "quantize_k_idx", _quantize_k_global_blocks)
    elif name == "q_shared_over_groups":
        monkeypatch.setattr(F, "quantize_q_idx", _quantize_q_shared_over_groups)
    assert _some_pin_fails(), name
