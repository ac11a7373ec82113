"""Pins of the 4-product INT4 x INT8 FP4 oracle (oracle/fp4awe4.py) against facts other
than itself: the product count the [AWE] abstract prints (golden fixture), the exact
integer product of every int4 x int8 pair (all 4,096), interpolation of an arbitrary cubic
form, the definition of S through the e2m1 code, the limb-choice rule by brute force over
limb ranges, the fp32 exactness bound, int64 matrix products, and the packed layout
decoded back."""
import itertools
import json
import os

import numpy as np

from oracle import fp4awe4, fp4limb

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "awe_six_products.json")


def test_product_count_is_the_pages():
    with open(GOLDEN) as fh:
        g = json.load(fh)
    assert len(fp4awe4.coefficients()) == fp4awe4.N_PRODUCTS == g["int4_x_int8_fp4_products"]


def test_interpolation_of_any_cubic_form():
    """For any cubic form C(p, q) = sum_d c_d p^d q^(3-d), sum_t coef_t C(p_t, q_t) equals
    C(W, 1): the coefficients interpolate, independently of the limbs."""
    rng = np.random.default_rng(0)
    coef = fp4awe4.coefficients()
    for _ in range(50):
        c = [int(v) for v in rng.integers(-1000, 1000, 4)]
        form = lambda p, q: sum(c[d] * p ** d * q ** (3 - d) for d in range(4))
        assert sum(k * form(p, q) for k, (p, q) in zip(coef, fp4awe4.POINTS)) == \
            form(fp4awe4.W, 1)
    assert coef == (36, 90, 45, -10)


def test_every_value_is_encoded_with_fp4_planes():
    s = set(fp4limb.fp4_times_two())
    w = fp4awe4.W
    xt, yt = fp4awe4.x_table(), fp4awe4.y_table()
    assert sorted(xt) == list(range(-8, 8)) and sorted(yt) == list(range(-128, 128))
    for x, a in xt.items():
        assert a[0] + w * a[1] == x
        assert fp4awe4.x_planes(a) == (a[0], a[1], a[0] + a[1], 2 * a[0] + a[1])
        assert all(v in s for v in fp4awe4.x_planes(a))
    for y, b in yt.items():
        assert b[0] + w * b[1] + w * w * b[2] == y
        assert fp4awe4.y_planes(b) == (b[0], b[2], b[0] + b[1] + b[2],
                                       4 * b[0] + 2 * b[1] + b[2])
        assert all(v in s for v in fp4awe4.y_planes(b))


def test_identity_over_every_int4_int8_pair():
    """sum_t coef_t u_t(x) v_t(y) == x y for all 4,096 pairs (a dropped product, a wrong
    coefficient, a wrong point or a wrong plane fails here)."""
    xs, ys = np.arange(-8, 8), np.arange(-128, 128)
    u = fp4awe4.planes_x(xs[None, :])[:, 0, :].astype(np.int64)     # [4][16]
    v = fp4awe4.planes_y(ys[None, :])[:, 0, :].astype(np.int64)     # [4][256]
    coef = np.array(fp4awe4.coefficients(), dtype=np.int64)
    got = (u * coef[:, None]).T @ v
    np.testing.assert_array_equal(got, np.outer(xs, ys))


def test_limb_choice_by_brute_force():
    """The chosen limbs are the minimum of the rule over every limb tuple found by plain
    enumeration of bounded limb ranges (not through the plane-value solve)."""
    s = set(fp4limb.fp4_times_two())
    w = fp4awe4.W

    def key(planes, limbs):
        return (max(abs(t) for t in planes), sum(t * t for t in planes), limbs)

    for x in range(-8, 8):
        cands = [(key(fp4awe4.x_planes((x - w * a1, a1)), (x - w * a1, a1)), (x - w * a1, a1))
                 for a1 in range(-30, 31)
                 if all(t in s for t in fp4awe4.x_planes((x - w * a1, a1)))]
        assert min(cands)[1] == fp4awe4.x_table()[x]
    for y in (-128, -127, -64, -1, 0, 1, 5, 25, 63, 100, 126, 127):
        cands = []
        for b2, b1 in itertools.product(range(-12, 13), range(-200, 201)):
            b = (y - w * b1 - w * w * b2, b1, b2)
            pl = fp4awe4.y_planes(b)
            if all(t in s for t in pl):
                cands.append((key(pl, b), b))
        assert min(cands)[1] == fp4awe4.y_table()[y]


def test_search_finds_the_two_encodings():
    hits = fp4awe4.search_encodings()
    assert hits == [(5, ((0, 1), (1, 0), (1, 1), (1, 2))),
                    (4, ((0, 1), (1, 0), (-1, 1), (-1, 2)))]
    assert hits[0] == (fp4awe4.W, fp4awe4.POINTS)


def test_magnitudes_keep_fp32_exact():
    """A planes are at most 4 and B planes at most 12 in magnitude, so an elementary
    product is at most 48 and 48 K < 2^24 for K up to 349525 (beyond the library's
    131071)."""
    ax = max(max(abs(v) for v in fp4awe4.x_planes(a)) for a in fp4awe4.x_table().values())
    by = max(max(abs(v) for v in fp4awe4.y_planes(b)) for b in fp4awe4.y_table().values())
    assert (ax, by) == (4, 12)
    assert 48 * 349525 < 2**24 <= 48 * 349526
    assert 349525 >= 131071


def test_gemm_equals_int64_product():
    rng = np.random.default_rng(4)
    for m, n, k in ((7, 5, 1), (16, 33, 257), (40, 24, 1000)):
        a = rng.integers(-8, 8, (m, k))
        b = rng.integers(-128, 128, (k, n))
        np.testing.assert_array_equal(fp4awe4.int4_int8_gemm(a, b), a @ b)
    a = np.full((3, 300), -8)
    b = np.full((300, 2), -128)
    np.testing.assert_array_equal(fp4awe4.int4_int8_gemm(a, b), a @ b)


def test_int4_input_reads_the_low_nibble():
    raw = np.array([[0x17, -0x7f, 0x08, -9, 7]], dtype=np.int64)     # bytes
    vals = np.array([[fp4awe4.int4_value(v) for v in raw[0]]])
    assert vals.tolist() == [[7, 1, -8, 7, 7]]
    b = np.arange(-10, 15).reshape(5, 5)
    np.testing.assert_array_equal(fp4awe4.int4_int8_gemm(raw, b), vals @ b)


def test_packed_layout_decodes_back():
    rng = np.random.default_rng(6)
    y = rng.integers(-128, 128, (3, 100))
    planes = fp4awe4.planes_y(y)
    packed = fp4awe4.pack_lines(planes, 128)
    assert packed.shape == (3, 2 * 128)
    lut = {fp4limb.encode_digit(d): d for d in fp4limb.fp4_times_two()}
    for line in range(3):
        for h in range(128):
            s, c = divmod(h, 64)
            for t in range(4):
                byte = packed[line, 128 * s + 32 * t + c // 2]
                code = (byte >> 4) if c % 2 else (byte & 15)
                want = planes[t, line, h] if h < 100 else 0
                assert lut[int(code)] == want


def test_products_one_and_two_can_share_an_fp32_sum():
    """The coefficients of products 1 and 2 stand in the ratio 2 : 1, so a block scale of 2
    on product 1 lets both add into one fp32 sum 2 P1 + P2; per K value that sum is at most
    27 in magnitude over all int4 x int8 pairs, so it stays an exact integer below 2^24 for
    K up to 621378 (beyond the library's 131071).  The other pairs of coefficients are not
    power-of-two multiples of each other."""
    coef = fp4awe4.coefficients()
    assert coef[1] == 2 * coef[2]
    for i in range(4):
        for j in range(i + 1, 4):
            if (i, j) == (1, 2):
                continue
            ratio = abs(coef[i] / coef[j])
            assert not any(ratio == 2.0 ** e for e in range(-8, 9))
    us = [fp4awe4.x_planes(a) for a in fp4awe4.x_table().values()]
    vs = [fp4awe4.y_planes(b) for b in fp4awe4.y_table().values()]
    bound = max(abs(2 * u[1] * v[1] + u[2] * v[2]) for u in us for v in vs)
    assert bound == 27
    assert 27 * 621378 < 2**24 <= 27 * 621379
    # and the combination reproduces x y for every pair
    xs, ys = np.arange(-8, 8), np.arange(-128, 128)
    u = fp4awe4.planes_x(xs[None, :])[:, 0, :].astype(np.int64)
    v = fp4awe4.planes_y(ys[None, :])[:, 0, :].astype(np.int64)
    shared = 2 * np.outer(u[1], v[1]) + np.outer(u[2], v[2])
    got = coef[0] * np.outer(u[0], v[0]) + coef[2] * shared + coef[3] * np.outer(u[3], v[3])
    np.testing.assert_array_equal(got, np.outer(xs, ys))
