"""Pins of the quantised Index Branch oracle (oracle/fp8_index.py), CPU only.

What fixes the answers:
* the OCP FP8 E4M3 format, through torch's own float8_e4m3fn dtype (a library
  routine): decoding of all 256 codes, and round-to-nearest-even encoding of
  float32 values, exact midpoints included;
* closed forms of the power-of-two scale rule (amax = 448 * 2^t gives e = t);
* invariants: the scaled row maximum lies in (224, 448]; codes that are
  already representable come back unchanged; multiplying one KV block's index
  keys by 2^t moves only that block's exponent, by t; multiplying an index
  query by 2^t leaves the selection unchanged;
* the E4M3 error bound (half a unit in the last place of a 3-bit mantissa);
* the Index Branch on dequantised values equals the bf16-path oracle run on
  the same (exactly representable) values.
"""
import math

import numpy as np
import pytest
import torch

from oracle import fp8_index as F
from oracle import msa_oracle as O


def _torch_decode_all():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_encode(x32):
    t = torch.from_numpy(np.asarray(x32, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_matches_library_for_all_codes():
    mine = F.e4m3_table()
    ref = _torch_decode_all()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    # the format's landmarks (OFP8 E4M3): two NaN codes, largest finite 448,
    # smallest normal 2^-6, smallest subnormal 2^-9, one = 0x38
    assert np.isnan(mine[0x7F]) and np.isnan(mine[0xFF]) and np.isnan(mine).sum() == 2
    assert mine[0x7E] == 448.0 and mine[0xFE] == -448.0
    assert mine[0x08] == 2.0 ** -6 and mine[0x01] == 2.0 ** -9 and mine[0x38] == 1.0


def test_encode_matches_library_rne():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.uniform(-448, 448, 20000),
        rng.standard_normal(20000) * 3.0,
        rng.standard_normal(5000) * 2.0 ** -7,            # subnormal range
        np.ldexp(rng.uniform(-1, 1, 5000), rng.integers(-12, 9, 5000)),
    ]).astype(np.float32)
    x = np.clip(x, -448, 448)
    assert np.array_equal(F.e4m3_encode(x), _torch_encode(x))


def test_encode_midpoints_round_to_even():
    vals = F.e4m3_table()[:127]
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)   # exact in float32
    assert np.array_equal(mids.astype(np.float64), (vals[:-1] + vals[1:]) / 2)
    got = F.e4m3_encode(mids)
    assert np.array_equal(got, _torch_encode(mids))
    assert np.all(got % 2 == 0)                                # the even neighbour
    assert np.array_equal(F.e4m3_encode(-mids), _torch_encode(-mids))


def test_encode_roundtrip_every_finite_code():
    tab = F.e4m3_table()
    codes = np.array([c for c in range(256) if not math.isnan(tab[c])], dtype=np.uint8)
    assert np.array_equal(F.e4m3_encode(tab[codes]), codes)


def test_scale_exponent_closed_forms():
    for t in range(-100, 100, 7):
        assert F.scale_exponent(448.0 * 2.0 ** t) == t
        assert F.scale_exponent(np.nextafter(448.0, 1e9) * 2.0 ** t) == t + 1
        assert F.scale_exponent(256.0 * 2.0 ** t) == t          # 256 * 2^t * 2^-t <= 448
    assert F.scale_exponent(1.0) == -8
    assert F.scale_exponent(1.75) == -8
    assert F.scale_exponent(np.nextafter(1.75, 2.0)) == -7
    assert F.scale_exponent(0.0) == 0
    assert F.scale_exponent(2.0 ** -140) == -127                # clamped
    assert F.scale_exponent(3.0e38) == 120


def test_scale_exponent_is_smallest():
    rng = np.random.default_rng(8)
    for a in np.ldexp(rng.uniform(0.5, 1.0, 3000), rng.integers(-100, 120, 3000)):
        e = F.scale_exponent(a)
        assert a * 2.0 ** -e <= 448.0 < a * 2.0 ** -(e - 1)
        assert 224.0 < a * 2.0 ** -e


def test_quantisation_error_bound():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((64, 128)) * np.exp(rng.uniform(-8, 8, (64, 1)))
    for row in x:
        e = F.scale_exponent(np.abs(row).max())
        deq = F.dequantize(F.quantize(row, e), e)
        y = np.abs(row) * 2.0 ** -e
        bound = np.where(y >= 2.0 ** -6, 2.0 ** -4 * np.abs(row), 2.0 ** -10 * 2.0 ** e)
        assert np.all(np.abs(deq - row) <= bound)


def _representable_rows(rng, n, d):
    """Rows of exact E4M3 values times 2^e whose maximum code is in (224, 448]."""
    tab = F.e4m3_table()
    finite = np.array([c for c in range(256) if not math.isnan(tab[c])])
    codes = rng.choice(finite, size=(n, d))
    big = np.array([c for c in finite if 224 < abs(tab[c]) <= 448])
    codes[np.arange(n), rng.integers(0, d, n)] = rng.choice(big, n)
    ex = rng.integers(-20, 10, n)
    return np.ldexp(tab[codes], ex[:, None]), codes.astype(np.uint8), ex


def test_representable_values_quantise_to_themselves():
    rng = np.random.default_rng(10)
    x, codes, ex = _representable_rows(rng, 200, 64)
    q, qe = F.quantize_q_idx(x.reshape(100, 2, 64))
    assert np.array_equal(qe.reshape(-1).astype(np.int64) - 127, ex)
    # -0.0 vs +0.0 codes differ only in the sign bit; compare values
    assert np.array_equal(F.e4m3_table()[q.reshape(200, 64)], F.e4m3_table()[codes])
    assert np.array_equal(F.dequantize_q_idx(q, qe).reshape(200, 64), x)


def _k_setup(seed=11):
    rng = np.random.default_rng(seed)
    lk = [300, 128, 517]
    cu = np.concatenate([[0], np.cumsum(lk)])
    k = rng.standard_normal((cu[-1], 32)).astype(np.float32)
    nb = (max(lk) + 127) // 128
    return k, cu, nb


def test_k_block_scale_is_per_sequence_block():
    k, cu, nb = _k_setup()
    codes, ex = F.quantize_k_idx(k, cu, nb)
    base = F.dequantize_k_idx(codes, ex, cu)
    # blocks past each sequence's end hold the neutral exponent
    for b in range(3):
        nblk = (cu[b + 1] - cu[b] + 127) // 128
        assert np.all(ex[b, nblk:] == 127)
    for b, beta, t in [(0, 2, 5), (2, 1, -3), (1, 0, 7), (2, 4, 2)]:
        lo = cu[b] + 128 * beta
        hi = min(lo + 128, cu[b + 1])
        k2 = k.astype(np.float64).copy()
        k2[lo:hi] *= 2.0 ** t
        c2, e2 = F.quantize_k_idx(k2, cu, nb)
        assert np.array_equal(c2, codes)
        de = e2.astype(np.int64) - ex.astype(np.int64)
        expect = np.zeros_like(de)
        expect[b, beta] = t
        assert np.array_equal(de, expect)
        d2 = F.dequantize_k_idx(c2, e2, cu)
        scale = np.ones(len(k))
        scale[lo:hi] = 2.0 ** t
        assert np.array_equal(d2, base * scale[:, None])


def test_k_block_exponent_follows_block_maximum():
    k, cu, nb = _k_setup(12)
    _, ex = F.quantize_k_idx(k, cu, nb)
    for b in range(3):
        for beta in range((cu[b + 1] - cu[b] + 127) // 128):
            lo = cu[b] + 128 * beta
            hi = min(lo + 128, cu[b + 1])
            a = np.abs(k[lo:hi]).max()
            e = int(ex[b, beta]) - 127
            assert a * 2.0 ** -e <= 448 < a * 2.0 ** -(e - 1)


def _fp8_problem(rng, lens, G=2, d_idx=64, top_k=4):
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    q = rng.standard_normal((T, 2 * G, 64)).astype(np.float32)
    kv = rng.standard_normal((T, G, 64)).astype(np.float32)
    qi = rng.standard_normal((T, G, d_idx)).astype(np.float32)
    ki = rng.standard_normal((T, d_idx)).astype(np.float32)
    return q, kv, qi, ki, cu, top_k


def test_selection_on_representable_inputs_equals_bf16_path():
    """Already-representable index inputs: the quantised branch selects exactly
    what the unquantised oracle selects on the same values."""
    rng = np.random.default_rng(13)
    lens = [700, 260]
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    qrows, _, _ = _representable_rows(rng, T * 2, 64)
    qi = qrows.reshape(T, 2, 64)
    # keys: per block, representable values with one common exponent
    tab = F.e4m3_table()
    finite = np.array([c for c in range(127) if not math.isnan(tab[c])])
    ki = np.zeros((T, 64))
    for b in range(2):
        for lo in range(int(cu[b]), int(cu[b + 1]), 128):
            hi = min(lo + 128, int(cu[b + 1]))
            c = rng.choice(finite, size=(hi - lo, 64)) * rng.choice([-1, 1], size=(hi - lo, 64))
            c = np.abs(c).astype(np.int64) | np.where(c < 0, 0x80, 0)
            vals = tab[c]
            vals[0, 0] = 448.0
            ki[lo:hi] = np.ldexp(vals, int(rng.integers(-10, 5)))
    nb = (max(lens) + 127) // 128
    qc, qe = F.quantize_q_idx(qi)
    kc, ke = F.quantize_k_idx(ki, cu, nb)
    assert np.array_equal(F.dequantize_q_idx(qc, qe), qi)
    assert np.array_equal(F.dequantize_k_idx(kc, ke, cu), ki)
    q = rng.standard_normal((T, 4, 64))
    kv = rng.standard_normal((T, 2, 64))
    rows = list(range(0, T, 37))
    a = O.Problem(q, kv, kv, F.dequantize_q_idx(qc, qe), F.dequantize_k_idx(kc, ke, cu), cu, cu, 4)
    b = O.Problem(q, kv, kv, qi, ki, cu, cu, 4)
    for r in rows:
        assert np.array_equal(a.row(r)["sel"], b.row(r)["sel"])


def test_query_power_of_two_scaling_leaves_selection():
    rng = np.random.default_rng(14)
    q, kv, qi, ki, cu, top_k = _fp8_problem(rng, [900])
    nb = 8
    kc, ke = F.quantize_k_idx(ki, cu, nb)
    kd = F.dequantize_k_idx(kc, ke, cu)
    qc, qe = F.quantize_q_idx(qi)
    qc2, qe2 = F.quantize_q_idx(qi * 2.0 ** 9)
    assert np.array_equal(qc, qc2) and np.array_equal(qe2.astype(int) - qe.astype(int), np.full(qe.shape, 9))
    a = O.Problem(q, kv, kv, F.dequantize_q_idx(qc, qe), kd, cu, cu, top_k)
    b = O.Problem(q, kv, kv, F.dequantize_q_idx(qc2, qe2), kd, cu, cu, top_k)
    for r in range(0, 900, 29):
        assert np.array_equal(a.row(r)["sel"], b.row(r)["sel"])


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        F.e4m3_encode(np.array([449.0]))
    with pytest.raises(ValueError):
        F.e4m3_encode(np.array([np.nan]))
