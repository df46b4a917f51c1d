"""Pins of the 4-bit index-key oracle (oracle/fp4_index.py), CPU only.

What fixes the answers:
* the OCP FP4 E2M1 format, through torch's own sub-byte conversion routines
  (the code torch uses for float4_e2m1fn_x2, a library routine): decoding of
  all 16 codes, round-to-nearest-even encoding, exact midpoints included, and
  torch's packing of two codes per byte;
* closed forms of the power-of-two scale rule (amax = 6 * 2^t gives e = t,
  amax = 3 * 2^t gives e = t - 1);
* invariants: the scaled group maximum lies in (3, 6]; codes that are
  already representable come back unchanged; multiplying one 32-element group
  of one key by 2^t moves only that group's exponent, by t;
* the E2M1 error bound (half the spacing of the grid: a quarter of |x| in the
  normal range, a quarter of the scale below it);
* the Index Branch on dequantised values equals the unquantised oracle run on
  the same (exactly representable) values.
"""
import numpy as np
import pytest
import torch

from oracle import fp4_index as F4
from oracle import fp8_index as F8
from oracle import msa_oracle as O
import torch_floatx as TX


def _lib_encode(x):
    return TX.f32_to_e2m1(torch.from_numpy(np.asarray(x, dtype=np.float32))).numpy()


def test_decode_matches_library_for_all_codes():
    mine = F4.e2m1_table()
    ref = TX.e2m1_to_f32(torch.arange(16, dtype=torch.uint8)).double().numpy()
    assert np.array_equal(mine, ref)
    assert np.array_equal(np.signbit(mine), np.signbit(ref))
    # the format's landmarks: largest value 6, smallest subnormal 0.5, one = 0x2,
    # 0x8 is negative zero
    assert mine[0x7] == 6.0 and mine[0xF] == -6.0 and mine[0x1] == 0.5 and mine[0x2] == 1.0
    assert mine[0x8] == 0.0 and np.signbit(mine[0x8])
    assert list(mine[:8]) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_encode_matches_library_rne():
    rng = np.random.default_rng(21)
    x = np.concatenate([
        rng.uniform(-6, 6, 40000),
        rng.standard_normal(20000),
        rng.uniform(-0.3, 0.3, 5000),
    ]).astype(np.float32)
    x = np.clip(x, -6, 6)
    assert np.array_equal(F4.e2m1_encode(x), _lib_encode(x))


def test_encode_midpoints_round_to_even():
    vals = F4.e2m1_table()[:8]
    mids = (vals[:-1] + vals[1:]) / 2
    assert list(mids) == [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    got = F4.e2m1_encode(mids)
    assert list(got) == [0, 2, 2, 4, 4, 6, 6]             # the even neighbour each time
    assert np.array_equal(got, _lib_encode(mids))
    assert np.array_equal(F4.e2m1_encode(-mids), _lib_encode(-mids))
    assert np.array_equal(F4.e2m1_encode(-mids), got | 0x8)


def test_encode_roundtrip_every_code():
    codes = np.arange(16, dtype=np.uint8)
    assert np.array_equal(F4.e2m1_encode(F4.e2m1_table()[codes]), codes)


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        F4.e2m1_encode(np.array([6.01]))
    with pytest.raises(ValueError):
        F4.e2m1_encode(np.array([np.inf]))


def test_scale_exponent_closed_forms():
    for t in range(-100, 100, 7):
        assert F4.scale_exponent4(6.0 * 2.0 ** t) == t
        assert F4.scale_exponent4(np.nextafter(6.0, 7.0) * 2.0 ** t) == t + 1
        assert F4.scale_exponent4(4.0 * 2.0 ** t) == t          # 4 <= 6 < 8
        assert F4.scale_exponent4(3.0 * 2.0 ** t) == t - 1      # 3 * 2 = 6 still fits
        assert F4.scale_exponent4(np.nextafter(3.0, 4.0) * 2.0 ** t) == t
    assert F4.scale_exponent4(1.0) == -2
    assert F4.scale_exponent4(0.0) == 0
    assert F4.scale_exponent4(2.0 ** -140) == -127              # clamped
    assert F4.scale_exponent4(3.0e38) == 126


def test_scale_exponent_is_smallest():
    rng = np.random.default_rng(22)
    for a in np.ldexp(rng.uniform(0.5, 1.0, 3000), rng.integers(-100, 120, 3000)):
        e = F4.scale_exponent4(a)
        assert a * 2.0 ** -e <= 6.0 < a * 2.0 ** -(e - 1)
        assert 3.0 < a * 2.0 ** -e


def test_group_scale_is_per_32_elements():
    rng = np.random.default_rng(23)
    k = rng.standard_normal((40, 128))
    codes, ex = F4.quantize_k_idx4(k)
    assert codes.shape == (40, 128) and ex.shape == (40, 4)
    base = F4.dequantize_k_idx4(codes, ex)
    for r, grp, t in [(0, 0, 5), (7, 3, -4), (39, 1, 9), (20, 2, -11)]:
        k2 = k.copy()
        k2[r, 32 * grp:32 * grp + 32] *= 2.0 ** t
        c2, e2 = F4.quantize_k_idx4(k2)
        assert np.array_equal(c2, codes)
        de = e2.astype(np.int64) - ex.astype(np.int64)
        want = np.zeros_like(de)
        want[r, grp] = t
        assert np.array_equal(de, want)
        scale = np.ones_like(k)
        scale[r, 32 * grp:32 * grp + 32] = 2.0 ** t
        assert np.array_equal(F4.dequantize_k_idx4(c2, e2), base * scale)


def test_group_exponent_follows_group_maximum():
    rng = np.random.default_rng(24)
    k = rng.standard_normal((50, 64)) * np.exp(rng.uniform(-6, 6, (50, 1)))
    _, ex = F4.quantize_k_idx4(k)
    for r in range(50):
        for g in range(2):
            a = np.abs(k[r, 32 * g:32 * g + 32]).max()
            e = int(ex[r, g]) - 127
            assert a * 2.0 ** -e <= 6.0 < a * 2.0 ** -(e - 1)


def test_quantisation_error_bound():
    rng = np.random.default_rng(25)
    k = rng.standard_normal((64, 128)) * np.exp(rng.uniform(-8, 8, (64, 1)))
    codes, ex = F4.quantize_k_idx4(k)
    deq = F4.dequantize_k_idx4(codes, ex)
    e = np.repeat(ex.astype(np.int64) - 127, 32, axis=1)
    y = np.abs(k) * 2.0 ** -e.astype(np.float64)
    bound = np.where(y >= 1.0, np.abs(k) / 4, 2.0 ** (e - 2).astype(np.float64))
    assert np.all(np.abs(deq - k) <= bound)
    # the bound is reached: the coarsest gap (4 .. 6) at its midpoint
    one = np.full((1, 32), 5.0)
    one[0, 0] = 6.0
    c1, e1 = F4.quantize_k_idx4(one)
    assert F4.dequantize_k_idx4(c1, e1)[0, 1] == 4.0


def _representable_keys(rng, n, d):
    """Key rows of exact E2M1 values times 2^e per 32-group whose largest
    magnitude is 4 or 6 (so e is the group's own exponent)."""
    tab = F4.e2m1_table()
    codes = rng.integers(0, 16, size=(n, d)).astype(np.uint8)
    for g in range(d // 32):
        codes[np.arange(n), 32 * g + rng.integers(0, 32, n)] = rng.choice([6, 7, 14, 15], n)
    ex = rng.integers(-20, 10, (n, d // 32))
    return np.ldexp(tab[codes], np.repeat(ex, 32, axis=1)), codes, ex


def test_representable_values_quantise_to_themselves():
    rng = np.random.default_rng(26)
    x, codes, ex = _representable_keys(rng, 100, 128)
    c, e = F4.quantize_k_idx4(x)
    assert np.array_equal(e.astype(np.int64) - 127, ex)
    # -0.0 vs +0.0 codes differ only in the sign bit; compare values
    assert np.array_equal(F4.e2m1_table()[c], F4.e2m1_table()[codes])
    assert np.array_equal(F4.dequantize_k_idx4(c, e), x)


def test_pack_matches_library():
    rng = np.random.default_rng(27)
    codes = rng.integers(0, 16, size=(33, 64)).astype(np.uint8)
    p = F4.pack(codes)
    assert p.shape == (33, 32)
    assert np.array_equal(p, TX.pack_uint4(torch.from_numpy(codes)).numpy())
    assert np.array_equal(F4.unpack(p), codes)
    assert F4.pack(np.array([[1, 2]], dtype=np.uint8))[0, 0] == 0x21   # element 0 low


def test_selection_on_representable_inputs_equals_unquantised_oracle():
    """Index queries on the 8-bit grid and index keys on the 4-bit grid: the
    Q8KV4 branch selects exactly what the unquantised oracle selects on the
    same values."""
    rng = np.random.default_rng(28)
    lens = [700, 260]
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    tab8 = F8.e4m3_table()
    qcodes = rng.integers(0, 0x7F, size=(T * 2, 64))
    qcodes[np.arange(T * 2), rng.integers(0, 64, T * 2)] = 0x7E        # 448: exponent as built
    qi = np.ldexp(tab8[qcodes], rng.integers(-12, 4, (T * 2, 1))).reshape(T, 2, 64)
    ki, _, _ = _representable_keys(rng, T, 64)
    qc, qe = F8.quantize_q_idx(qi)
    kc, ke = F4.quantize_k_idx4(ki)
    assert np.array_equal(F8.dequantize_q_idx(qc, qe), qi)
    assert np.array_equal(F4.dequantize_k_idx4(kc, ke), ki)
    q = rng.standard_normal((T, 4, 64))
    kv = rng.standard_normal((T, 2, 64))
    a = O.Problem(q, kv, kv, F8.dequantize_q_idx(qc, qe), F4.dequantize_k_idx4(kc, ke), cu, cu, 4)
    b = O.Problem(q, kv, kv, qi, ki, cu, cu, 4)
    for r in range(0, T, 37):
        assert np.array_equal(a.row(r)["sel"], b.row(r)["sel"])

