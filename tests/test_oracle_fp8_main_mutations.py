"""The quantised Main Branch pins must catch plausible mistakes: each case
plants one mistake in the oracle (CPU only, via monkeypatch) and checks that
some pin then fails."""
import numpy as np
import pytest

from oracle import fp8_index as F
from oracle import fp8_main as M
import test_oracle_fp8_main as TM

PINS = [TM.test_q_scale_is_per_row_and_head, TM.test_kv_scale_is_per_block_and_head,
        TM.test_kv_blocks_start_at_each_sequence, TM.test_values_on_the_grid_round_trip_exactly,
        TM.test_error_bound_of_half_a_unit, TM.test_main_branch_on_dequantised_values_is_dense_attention]


def _some_pin_fails():
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            return True
    return False


ORIG_Q = M.quantize_q
ORIG_KV = M.quantize_kv
ORIG_QUANT = F.quantize


def _q_per_row(q):
    # mistake: one scale per query row, shared by its heads
    q = np.asarray(q, dtype=np.float64)
    T, H, _ = q.shape
    codes = np.zeros(q.shape, dtype=np.uint8)
    ex = np.zeros((T, H), dtype=np.uint8)
    for t in range(T):
        e = F.scale_exponent(np.abs(q[t]).max())
        codes[t] = F.quantize(q[t], e)
        ex[t, :] = e + F.E8M0_BIAS
    return codes, ex


def _kv_shared_heads(x, cu, nb_max, block=M.BLOCK):
    # mistake: one scale per block, shared by the KV heads
    x = np.asarray(x, dtype=np.float64)
    codes = np.zeros(x.shape, dtype=np.uint8)
    ex = np.full((len(cu) - 1, nb_max, x.shape[1]), F.E8M0_BIAS, dtype=np.uint8)
    for b in range(len(cu) - 1):
        for beta in range(nb_max):
            lo = int(cu[b]) + beta * block
            hi = min(lo + block, int(cu[b + 1]))
            if lo >= hi:
                continue
            e = F.scale_exponent(np.abs(x[lo:hi]).max())
            codes[lo:hi] = F.quantize(x[lo:hi], e)
            ex[b, beta, :] = e + F.E8M0_BIAS
    return codes, ex


def _kv_global_blocks(x, cu, nb_max, block=M.BLOCK):
    # mistake: 128-row blocks counted from row 0 of the packed cache, not per sequence
    x = np.asarray(x, dtype=np.float64)
    codes = np.zeros(x.shape, dtype=np.uint8)
    ex = np.full((len(cu) - 1, nb_max, x.shape[1]), F.E8M0_BIAS, dtype=np.uint8)
    for lo in range(0, x.shape[0], block):
        hi = min(lo + block, x.shape[0])
        b = int(np.searchsorted(cu, lo, side="right") - 1)
        beta = (lo - int(cu[b])) // block
        for g in range(x.shape[1]):
            e = F.scale_exponent(np.abs(x[lo:hi, g]).max())
            codes[lo:hi, g] = F.quantize(x[lo:hi, g], e)
            if beta < nb_max:
                ex[b, beta, g] = e + F.E8M0_BIAS
    return codes, ex


def _quantize_truncating(x, e):
    # mistake: codes truncated towards zero instead of rounded to nearest
    y = np.ldexp(np.asarray(x, dtype=np.float64), -int(e))
    table = F.e4m3_table()[:127]
    i = np.clip(np.searchsorted(table, np.abs(y), side="right") - 1, 0, 126).astype(np.uint8)
    return np.where(np.signbit(y), i | 0x80, i).astype(np.uint8)


def test_pins_pass_unmutated():
    assert not _some_pin_fails()


@pytest.mark.parametrize("name", ["q_per_row", "kv_shared_heads", "kv_global_blocks", "truncation"])
def test_mutation_is_caught(monkeypatch, name):
    if name == "q_per_row":
        monkeypatch.setattr(M, "quantize_q", _q_per_row)
    elif name == "kv_shared_heads":
        monkeypatch.setattr(M, "quantize_kv", _kv_shared_heads)
    elif name == "kv_global_blocks":
        monkeypatch.setattr(M, "quantize_kv", _kv_global_blocks)
    elif name == "truncation":
        monkeypatch.setattr(F, "quantize", _quantize_truncating)
    assert _some_pin_fails(), name
