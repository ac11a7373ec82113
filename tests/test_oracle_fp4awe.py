"""Pins of the 6-product FP4 oracle (oracle/fp4awe.py) against facts other than itself:
the product count the [AWE] abstract prints (golden fixture), the exact integer product
of every pair of int8 values (all 65,536), the definition of S through the e2m1 code, the
fp32 exactness bound, int64 matrix products, and the packed layout decoded back."""
import json
import os

import numpy as np
import pytest

from oracle import fp4awe, fp4limb

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "awe_six_products.json")


def _golden():
    with open(GOLDEN) as fh:
        return json.load(fh)


def test_product_count_is_the_pages():
    g = _golden()
    assert len(fp4awe.coefficients()) == fp4awe.N_PRODUCTS == g["int8_x_int8_fp4_products"]
    assert g["prior_int8_x_int8_fp4_products"] == len(fp4limb.WEIGHTS) ** 2


def test_every_int8_value_is_encoded_with_fp4_planes():
    s = set(fp4limb.fp4_times_two())
    tab = fp4awe.limb_table()
    assert sorted(tab) == list(range(-128, 128))
    for x, a in tab.items():
        assert a[0] + 29 * a[1] + 37 * a[2] == x
        for v in fp4awe.plane_values(a):
            assert v in s, (x, a)


def test_identity_over_every_pair_of_int8_values():
    """sum_t coef_t u_t(x) v_t(y) == x y for all 65,536 pairs (a dropped product, a wrong
    coefficient or a wrong pair fails here)."""
    xs = np.arange(-128, 128)
    u = fp4awe.planes(xs[None, :])[:, 0, :].astype(np.int64)     # [6][256]
    coef = np.array(fp4awe.coefficients(), dtype=np.int64)
    got = (u * coef[:, None]).T @ u                              # [256][256]
    np.testing.assert_array_equal(got, np.outer(xs, xs))


def test_coefficients_closed_form():
    # c_i = w_i^2 - w_i (sum of the other weights); pair weights w_i w_j
    assert fp4awe.coefficients() == (1 - 66, 841 - 29 * 38, 1369 - 37 * 30, 29, 37, 29 * 37)


def test_magnitudes_keep_fp32_exact():
    """Every plane value is at most 6 in magnitude, so each elementary product is at most
    36 and 36 K < 2^24 for K up to 466033 (beyond the library's 131071)."""
    tab = fp4awe.limb_table()
    top = max(max(abs(v) for v in fp4awe.plane_values(a)) for a in tab.values())
    assert top == 6
    assert 36 * 466033 < 2**24 <= 36 * 466034
    assert 466033 >= 131071


def test_limb_choice_rule_on_a_tie():
    """Where several triples encode x, the chosen one minimises (largest magnitude, sum of
    squares, limbs): compare against every candidate by brute force."""
    tab = fp4awe.limb_table()
    for x in (-128, -1, 0, 1, 29, 37, 66, 127):
        cands = list(fp4awe.valid_triples(x))
        best = tab[x]

        def key(a):
            v = fp4awe.plane_values(a)
            return (max(abs(t) for t in v), sum(t * t for t in v), a)

        assert all(key(best) <= key(c) for c in cands)
    assert tab[0] == (0, 0, 0)


def test_search_finds_the_weights():
    hits = fp4awe.search_weights()
    assert len(hits) == 11
    sums_only = [w for w, sg in hits if sg == (1, 1, 1)]
    assert sums_only == [(1, 11, 39), (1, 29, 37)]
    assert fp4awe.WEIGHTS in sums_only


@pytest.mark.parametrize("m,n,k,seed", [(1, 1, 1, 0), (7, 5, 33, 1), (40, 30, 300, 2)])
def test_int8_gemm_equals_int64_product(m, n, k, seed):
    rng = np.random.default_rng(seed)
    a = rng.integers(-128, 128, size=(m, k), dtype=np.int8)
    b = rng.integers(-128, 128, size=(k, n), dtype=np.int8)
    a[0, 0] = b[0, 0] = -128
    want = a.astype(np.int64) @ b.astype(np.int64)
    np.testing.assert_array_equal(fp4awe.int8_gemm(a, b), want)
    p = fp4awe.plane_products(a, b)
    assert np.abs(p).max() <= 36 * k


def test_pack_layout_decodes_back():
    rng = np.random.default_rng(4)
    x = rng.integers(-128, 128, size=(3, 130), dtype=np.int8)
    packed = fp4awe.pack_lines(x, 192)
    assert packed.shape == (3, 3 * 192)
    vals = fp4awe.planes(x)
    for i in range(3):
        for h in range(192):
            s, r = divmod(h, 64)
            for t in range(6):
                byte = packed[i, 192 * s + 32 * t + r // 2]
                code = (byte >> 4) if r % 2 else (byte & 15)
                want = vals[t, i, h] if h < 130 else 0
                assert 2 * fp4limb.e2m1_value(int(code)) == want
