"""Pins for oracle.fp4limb against the facts the AWE page prints (golden fixture) and
exhaustive brute force."""
import json
import os

import numpy as np

import ozk_inputs
from oracle import fp4limb

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "awe_fp4_digits.json")


def _golden():
    with open(GOLDEN) as fh:
        return json.load(fh)


def test_fp4_times_two_is_printed_set():
    g = _golden()
    assert fp4limb.fp4_times_two() == sorted(g["S"])


def test_set_covers_every_residue_mod_13():
    g = _golden()
    assert {d % g["modulus"] for d in g["S"]} == set(range(13))


def test_limb_sums_leave_the_set():
    g = _golden()
    s = set(g["S"])
    sums = {x + y for x in s for y in s}
    assert max(abs(v) for v in sums) == g["limb_sum_reach"]
    assert not sums <= s


def test_digit_table_least_magnitude():
    t = fp4limb.digit_table()
    s = fp4limb.fp4_times_two()
    for rho, d in enumerate(t):
        assert d in s and d % 13 == rho
        assert all(abs(d) <= abs(c) for c in s if c % 13 == rho)
    assert t[1] == 1 and t[12] == -1 and t[5] == -8


def test_split3_exhaustive_int8():
    g = _golden()
    s = set(g["S"])
    w = g["weights"]
    for x in range(-128, 128):
        d = fp4limb.split3(x)
        assert all(v in s for v in d)
        assert d[0] * w[0] + d[1] * w[1] + d[2] * w[2] == x
        assert abs(d[0]) <= 8 and abs(d[1]) <= 8 and d[2] in (-1, 0, 1)


def test_nine_products_exhaustive_pairs():
    g = _golden()
    w = g["weights"]
    digits = {x: fp4limb.split3(x) for x in range(-128, 128)}
    count = 0
    for x in range(-128, 128):
        dx = digits[x]
        for y in range(-128, 128):
            dy = digits[y]
            total = 0
            terms = 0
            for ia in range(3):
                for ib in range(3):
                    total += w[ia] * w[ib] * dx[ia] * dy[ib]
                    terms += 1
            assert total == x * y
            count += 1
    assert terms == g["fp4_gemms_per_int8_product"] and count == 65536


def test_e2m1_codes_roundtrip():
    for d in fp4limb.fp4_times_two():
        c = fp4limb.encode_digit(d)
        assert 0 <= c < 16 and 2 * fp4limb.e2m1_value(c) == d
    assert fp4limb.encode_digit(0) == 0
    # OCP e2m1 magnitudes for codes 0..7
    assert [fp4limb.e2m1_value(c) for c in range(8)] == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert fp4limb.e2m1_value(0b1111) == -6.0


def test_pack_codes_nibble_order():
    codes = np.array([[1, 2, 3, 4, 5]], dtype=np.uint8)
    packed = fp4limb.pack_codes(codes, 8)
    assert packed.tolist() == [[0x21, 0x43, 0x05, 0x00]]


def test_limb_gemm_equals_int64_matmul():
    a, b = ozk_inputs.int8_operands(33, 29, 70, seed=5)
    want = a.astype(np.int64) @ b.astype(np.int64)
    np.testing.assert_array_equal(fp4limb.int8_gemm(a, b), want)
    p = fp4limb.limb_products(a, b)
    assert p.shape == (3, 3, 33, 29)
    assert np.max(np.abs(p)) <= 64 * 70


def test_limb_codes_decode_to_digits():
    a, _ = ozk_inputs.int8_operands(7, 1, 19, seed=2)
    codes = fp4limb.limb_codes(a)
    digits = fp4limb.limb_digits(a)
    dec = np.vectorize(lambda c: int(2 * fp4limb.e2m1_value(int(c))))(codes)
    np.testing.assert_array_equal(dec, digits)
