"""Pins for oracle.ozaki2: exponents, scaled integers, residue planes, modular
products, reconstruction, and the whole emulated product.

Pins: the scaling invariant, exact big-integer definitions, brute force, the exact
rational product with the a-priori bound, and small-integer matrices whose fp64
product is exact (so the emulation must equal numpy's matmul bit for bit)."""
import math
from fractions import Fraction

import numpy as np
import pytest

import ozk_inputs
from oracle import ozaki2, reference, rns


def _ilogb(t):
    return math.frexp(t)[1] - 1


def test_exponents_invariant():
    rng = np.random.default_rng(11)
    x = ozk_inputs.phi_matrix(rng, (40, 33), 4.0)
    x[3] = 0.0
    x[5, :] = 5e-324          # subnormal row
    x[6, 7] = -2.0**1000      # huge entry
    for p in (1, 20, 51, 52, 53, 71):
        e = ozaki2.scale_exponents(x, p, axis=0)
        for i in range(x.shape[0]):
            t = float(np.max(np.abs(x[i])))
            if t == 0:
                assert e[i] == 0
                continue
            scaled = Fraction(t) * Fraction(2) ** int(e[i])
            assert Fraction(2) ** (p - 1) <= scaled < Fraction(2) ** p
            assert e[i] == p - 1 - _ilogb(t)
        f = ozaki2.scale_exponents(x.T, p, axis=1)
        np.testing.assert_array_equal(e, f)


def test_exponents_nonfinite():
    x = np.ones((3, 4))
    x[1, 2] = np.nan
    x[2, 0] = -np.inf
    e = ozaki2.scale_exponents(x, 50, axis=0)
    assert e[0] == 50 - 1 and e[1] == ozaki2.NONFINITE and e[2] == ozaki2.NONFINITE


def test_scaled_integer_definition_ties():
    # RNE(a 2^e): 2.5 -> 2, 3.5 -> 4, -2.5 -> -2, and large values stay exact.
    assert ozaki2.scaled_integer(1.25, 1) == 2
    assert ozaki2.scaled_integer(1.75, 1) == 4
    assert ozaki2.scaled_integer(-1.25, 1) == -2
    assert ozaki2.scaled_integer(0.5, 0) == 0
    assert ozaki2.scaled_integer(1.5, 0) == 2
    big = 1.0 + 2.0**-52
    assert ozaki2.scaled_integer(big, 70) == 2**70 + 2**18


def _planes_by_definition(x, e, r):
    ms = rns.moduli(r)
    out = np.zeros((r,) + x.shape, dtype=np.int64)
    for i in range(x.shape[0]):
        for h in range(x.shape[1]):
            v = ozaki2.scaled_integer(float(x[i, h]), int(e[i]))
            for l, m in enumerate(ms):
                out[l, i, h] = rns.smod(v, m)
    return out


@pytest.mark.parametrize("p", [3, 24, 47, 51, 52, 53, 60, 71])
def test_residue_planes_match_definition(p):
    rng = np.random.default_rng(p)
    x = ozk_inputs.phi_matrix(rng, (9, 37), 4.0)
    x[0, :4] = [0.5, 1.5, -2.5, 3.5]      # exact ties once scaled by 2^0
    x[1, :3] = [5e-324, -1e-310, 0.0]
    e = ozaki2.scale_exponents(x, p, axis=0)
    e[0] = 0                              # force the tie row to scale by 1
    r = 20
    got = ozaki2.residue_planes(x, e, r, axis=0)
    want = _planes_by_definition(x, e, r)
    np.testing.assert_array_equal(got.astype(np.int64), want)
    got_t = ozaki2.residue_planes(x.T, e, r, axis=1)
    np.testing.assert_array_equal(got_t, got)


def test_residue_planes_nonfinite_line_is_zero():
    x = np.ones((2, 5))
    x[1, 1] = np.inf
    e = ozaki2.scale_exponents(x, 40, axis=0)
    pl = ozaki2.residue_planes(x, e, 4, axis=0)
    assert np.all(pl[:, 1, :] == 0) and np.any(pl[:, 0, :] != 0)


def test_modular_products_match_int64_matmul():
    rng = np.random.default_rng(5)
    pa = rng.integers(-128, 128, size=(3, 7, 300), dtype=np.int8)
    pb = rng.integers(-128, 128, size=(3, 5, 300), dtype=np.int8)
    got = ozaki2.modular_products(pa, pb)
    for l in range(3):
        want = pa[l].astype(np.int64) @ pb[l].astype(np.int64).T
        np.testing.assert_array_equal(got[l], want)
    extreme = np.full((1, 2, 4096), -128, dtype=np.int8)
    assert ozaki2.modular_products(extreme, extreme)[0, 0, 0] == 4096 * 2**14


@pytest.mark.parametrize("r,dist", [(14, "uniform"), (8, "uniform"), (20, "phi"), (5, "phi")])
def test_dgemm_equals_exact_scaled_definition(r, dist):
    """Residues + modular products + CRT reproduce the plain big-integer definition."""
    a, b = ozk_inputs.gemm_operands(6, 5, 9, seed=r, dist=dist, phi=4.0)
    got = ozaki2.dgemm(a, b, r)
    want = ozaki2.exact_scaled_product(a, b, r)
    np.testing.assert_array_equal(got, want)


def test_dgemm_small_integers_bitwise_equal_numpy():
    """|a|,|b| <= 2^10, k = 64: the fp64 product is exact, so is the emulation."""
    rng = np.random.default_rng(3)
    a = ozk_inputs.small_int_matrix(rng, (17, 64), 1024)
    b = ozk_inputs.small_int_matrix(rng, (64, 13), 1024)
    np.testing.assert_array_equal(ozaki2.dgemm(a, b, 14), a @ b)
    np.testing.assert_array_equal(ozaki2.dgemm(a * 2.0**-600, b * 2.0**300, 14),
                                  (a @ b) * 2.0**-300)


@pytest.mark.parametrize("r,dist", [(14, "uniform"), (12, "uniform"), (16, "phi"), (9, "phi")])
def test_dgemm_within_apriori_bound_of_exact(r, dist):
    a, b = ozk_inputs.gemm_operands(8, 7, 24, seed=100 + r, dist=dist, phi=4.0)
    got = ozaki2.dgemm(a, b, r)
    exact = reference.exact_matmul(a, b)
    bound = reference.elementwise_bound(a, b, r)
    u = 2.0**-53
    err = np.abs(got - exact)
    assert np.all(err <= bound + 2 * u * np.abs(exact)), np.max(err / (bound + 1e-300))


def test_dgemm_sampled_block_equals_full():
    a, b = ozk_inputs.gemm_operands(20, 18, 40, seed=7, dist="phi", phi=0.5)
    full = ozaki2.dgemm(a, b, 12)
    rows, cols = np.array([0, 5, 19]), np.array([2, 17])
    np.testing.assert_array_equal(ozaki2.dgemm(a, b, 12, rows=rows, cols=cols),
                                  full[np.ix_(rows, cols)])


def test_dgemm_nonfinite_rows_and_columns():
    a, b = ozk_inputs.gemm_operands(4, 3, 6, seed=9)
    a[2, 1] = np.nan
    b[0, 1] = np.inf
    c = ozaki2.dgemm(a, b, 14)
    assert np.all(np.isnan(c[2])) and np.all(np.isnan(c[:, 1]))
    mask = np.ones_like(c, dtype=bool)
    mask[2] = False
    mask[:, 1] = False
    assert np.all(np.isfinite(c[mask]))


def test_dgemm_zero_rows_give_positive_zero():
    a, b = ozk_inputs.gemm_operands(3, 4, 5, seed=1)
    a[1] = 0.0
    c = ozaki2.dgemm(a, b, 14)
    assert np.all(c[1] == 0) and not np.any(np.signbit(c[1]))


def test_round_scaled_single_rounding():
    tiny = 2.0**-1074
    assert ozaki2.round_scaled(3, 1075) == 2 * tiny          # 1.5 ulp -> 2 ulp (even)
    assert ozaki2.round_scaled(5, 1075) == 2 * tiny          # 2.5 ulp -> 2 ulp (even)
    assert ozaki2.round_scaled(7, 1075) == 4 * tiny          # 3.5 ulp -> 4 ulp (even)
    assert ozaki2.round_scaled(-3, 1075) == -2 * tiny
    assert ozaki2.round_scaled(2**53 + 1, 0) == 2.0**53      # tie to even
    assert ozaki2.round_scaled(2**53 + 3, 0) == 2.0**53 + 4
    assert ozaki2.round_scaled(1, -1024) == math.inf
    assert ozaki2.round_scaled(-1, -1024) == -math.inf
    assert ozaki2.round_scaled(2**52 - 1, -971) == (2.0**52 - 1) * 2.0**971


def test_cfg_tiny_normwise_accuracy_vs_dot2_and_exact():
    """The tiny 64^3 case at r = 14: normwise error below 1e-15 against both the
    double-double reference and the exact product."""
    a, b = ozk_inputs.gemm_operands(64, 64, 64, seed=1, dist="uniform")
    c = ozaki2.dgemm(a, b, 14)
    dd = reference.dot2_matmul(a, b)
    assert np.linalg.norm(c - dd) / np.linalg.norm(dd) <= 1e-15
    rows = np.arange(0, 64, 9)
    exact = reference.exact_matmul(a[rows], b)
    assert np.linalg.norm(c[rows] - exact) / np.linalg.norm(exact) <= 1e-15


# ---------------------------------------------------------------- norm scaling rule
def _exact_norm2(row):
    return sum(Fraction(float(v)) ** 2 for v in row)


def test_norm_bracket_bounds_the_exact_sum():
    """s_up >= the exact sum of squares of x 2^-T on rows mixing large and tiny entries
    (float summation alone falls below the exact sum on about half of them)."""
    rng = np.random.default_rng(21)
    below = 0
    for trial in range(300):
        k = int(rng.integers(2, 400))
        row = ozk_inputs.phi_matrix(rng, (1, k), float(rng.uniform(0.1, 6.0)))[0]
        if trial % 3 == 0:
            row[rng.integers(k)] = 2.0 - 2.0**-52     # square just below 4
        big_t, s_up = ozaki2.norm_bracket(row)
        exact = sum((Fraction(float(v)) * Fraction(2) ** -big_t) ** 2 for v in row)
        assert Fraction(s_up) >= exact
        scaled = np.ldexp(row, -big_t)
        below += Fraction(float(np.sum(scaled * scaled))) < exact
    assert below > 30    # the safety factor is doing work on this data


def test_norm_exponents_invariant():
    """2^(aA-1) <= 2^e ||a||_2 < 2^aA with exact rationals (the rule never overshoots and
    loses at most one bit to its power-of-two bracket), except that a sum of squares
    within 2^-30 below a power of two may lose one more."""
    rng = np.random.default_rng(12)
    x = ozk_inputs.phi_matrix(rng, (40, 33), 4.0)
    x[3] = 0.0
    x[5, :] = 5e-324
    x[6, 7] = -2.0**1000
    x[8, :] = 3.0              # all-equal row: ||a|| = sqrt(k) max|a|
    x[9, :] = 0.0
    x[9, 4] = 1.0 - 2.0**-53   # one-hot row just below a power of two
    for alpha in (2, 20, 46, 54, 61, 76):
        e = ozaki2.scale_exponents_norm(x, alpha, axis=0)
        for i in range(x.shape[0]):
            n2 = _exact_norm2(x[i])
            if n2 == 0:
                assert e[i] == 0
                continue
            scaled2 = n2 * Fraction(4) ** int(e[i])
            assert scaled2 < Fraction(4) ** alpha
            assert scaled2 >= Fraction(4) ** (alpha - 2)
            big_t = math.frexp(float(np.max(np.abs(x[i]))))[1] - 1
            s_exact = n2 * Fraction(4) ** -big_t
            j = s_exact.numerator.bit_length() - s_exact.denominator.bit_length() + 1
            near = Fraction(2) ** j * (1 - Fraction(2) ** -30) <= s_exact < Fraction(2) ** j
            if not near:
                assert scaled2 >= Fraction(4) ** (alpha - 1)
        f = ozaki2.scale_exponents_norm(x.T, alpha, axis=1)
        np.testing.assert_array_equal(e, f)


def test_norm_exponents_nonfinite():
    x = np.ones((3, 4))
    x[1, 2] = np.nan
    x[2, 0] = -np.inf
    e = ozaki2.scale_exponents_norm(x, 50, axis=0)
    assert e[0] == 50 - 1 - 1 and e[1] == ozaki2.NONFINITE and e[2] == ozaki2.NONFINITE


@pytest.mark.parametrize("r,k", [(2, 64), (2, 200), (3, 64), (3, 257), (4, 500), (14, 64)])
def test_norm_rule_keeps_every_dot_product_inside_the_crt_range(r, k):
    """Exact sum_h |a'||b'| <= (M-1)/2 on adversarial lines: all-equal entries (the
    Cauchy-Schwarz worst case), entries that round up by almost 1/2 after scaling, one-hot
    lines, and random wide-range lines."""
    rng = np.random.default_rng(r * 1000 + k)
    aa, ab = rns.scaling_bits_norm(r, k)
    rows = [np.full(k, 1.0), np.full(k, 1.0 + 2.0**-3), np.full(k, -0.75)]
    # entries that land on x.5 - tiny after scaling: rounding adds almost 1/2 each
    e_guess = aa - 1 - (math.frexp(math.sqrt(k))[1] - 1)
    rows.append(np.full(k, (2.49999) * 2.0 ** -e_guess))
    one = np.zeros(k)
    one[k // 2] = 1.0
    rows.append(one)
    rows.append(ozk_inputs.phi_matrix(rng, (1, k), 2.0)[0])
    a = np.array(rows)
    b = np.array(rows).T.copy()
    e = ozaki2.exponents(a, r, k, 0, "a", "norm")
    f = ozaki2.exponents(b, r, k, 1, "b", "norm")
    assert ozaki2.exact_sum_bound_ok(a, b, e, f, r)


@pytest.mark.parametrize("r,dist", [(8, "phi"), (14, "uniform"), (16, "phi")])
def test_norm_rule_dgemm_equals_exact_scaled_definition(r, dist):
    rng = np.random.default_rng(r + 5)
    shape_k = 37
    if dist == "phi":
        a = ozk_inputs.phi_matrix(rng, (9, shape_k), 3.0)
        b = ozk_inputs.phi_matrix(rng, (shape_k, 7), 3.0)
    else:
        a = ozk_inputs.uniform_matrix(rng, (9, shape_k))
        b = ozk_inputs.uniform_matrix(rng, (shape_k, 7))
    got = ozaki2.dgemm(a, b, r, scaling="norm")
    want = ozaki2.exact_scaled_product(a, b, r, scaling="norm")
    np.testing.assert_array_equal(got, want)
    e = ozaki2.exponents(a, r, shape_k, 0, "a", "norm")
    f = ozaki2.exponents(b, r, shape_k, 1, "b", "norm")
    np.testing.assert_array_equal(ozaki2.dgemm(a, b, r, exps=(e, f)), got)


def test_norm_rule_more_accurate_on_wide_range_data():
    """On (U - 0.5) exp(4 N) entries (a few large entries per line) the norm rule keeps
    more bits than the max rule: its error against the exact product is smaller at every
    r tried (by 2.4x to 14x on this draw)."""
    rng = np.random.default_rng(3)
    k = 256
    a = ozk_inputs.phi_matrix(rng, (6, k), 4.0)
    b = ozk_inputs.phi_matrix(rng, (k, 5), 4.0)
    exact = [Fraction(int(v), 2**2148) for v in reference.exact_matmul_ints(a, b).reshape(-1)]
    norm_exact = math.sqrt(sum(float(v) ** 2 for v in exact))
    errs = {}
    for rule in ("max", "norm"):
        for r in (8, 10, 12):
            c = ozaki2.dgemm(a, b, r, scaling=rule).reshape(-1)
            d = [float(Fraction(float(c[i])) - exact[i]) for i in range(c.size)]
            errs[rule, r] = math.sqrt(sum(v * v for v in d)) / norm_exact
    for r in (8, 10, 12):
        assert errs["norm", r] <= errs["max", r]
    assert errs["norm", 8] < errs["max", 8] / 4 and errs["norm", 12] < errs["max", 12] / 4
