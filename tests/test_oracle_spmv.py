"""Pins of the emulated-SpMV oracle (oracle/spmv.py) against what the mathematics fixes:
the plain definition with exact integer sums, a closed form of the 7-point operator, the
exactness bound of the budget, the dense emulation of the same product, and the special
rows the reading defines."""
import math
from fractions import Fraction

import numpy as np
import pytest

import ozk_inputs
from oracle import ozaki2, rns, spmv


def _dense(row_ptr, col_idx, vals, cols):
    a = np.zeros((len(row_ptr) - 1, cols))
    for i in range(len(row_ptr) - 1):
        for p in range(row_ptr[i], row_ptr[i + 1]):
            a[i, col_idx[p]] = vals[p]
    return a


@pytest.mark.parametrize("r,kmax,phi", [(5, 6, 0.0), (8, 6, 2.0), (14, 9, 4.0), (20, 9, 4.0)])
def test_spmv_equals_exact_definition(r, kmax, phi):
    rp, ci, v = ozk_inputs.random_csr(60, 40, kmax, seed=r + kmax, phi=phi)
    x = ozk_inputs.phi_matrix(np.random.default_rng(3), (40, 1), 2.0)[:, 0]
    got = spmv.spmv_csr(rp, ci, v, x, r, kmax)
    want = spmv.spmv_exact_definition(rp, ci, v, x, r, kmax)
    np.testing.assert_array_equal(got, want)


def test_row_exponents_bracket_the_row_maximum():
    rp, ci, v = ozk_inputs.random_csr(80, 30, 7, seed=5, phi=4.0)
    pa, _ = rns.scaling_bits(14, 7)
    e = spmv.row_exponents(rp, v, pa)
    for i in range(80):
        seg = v[rp[i]:rp[i + 1]]
        if not seg.size:
            assert e[i] == 0
            continue
        t = Fraction(float(np.max(np.abs(seg)))) * Fraction(2) ** int(e[i])
        assert Fraction(2) ** (pa - 1) <= t < Fraction(2) ** pa


def test_poisson_quadratic_closed_form():
    """6 u_p - sum of neighbours of u = i^2 + j^2 + k^2 is exactly -6 at every interior
    point; small integer data is scaled exactly, so the emulation returns it exactly."""
    n = 6
    rp, ci, v = ozk_inputs.poisson_7pt_csr(n)
    g = np.arange(n)
    u = (g[:, None, None] ** 2 + g[None, :, None] ** 2 + g[None, None, :] ** 2).astype(float)
    y = spmv.spmv_csr(rp, ci, v, u.reshape(-1), 10, 7)
    interior = np.zeros((n, n, n), dtype=bool)
    interior[1:-1, 1:-1, 1:-1] = True
    np.testing.assert_array_equal(y.reshape(n, n, n)[interior], -6.0)
    exact = _dense(rp, ci, v, n ** 3) @ u.reshape(-1)      # small integers: exact in fp64
    np.testing.assert_array_equal(y, exact)


def test_budget_keeps_every_row_sum_inside_the_crt_range():
    r, kmax = 6, 9
    rp, ci, v = ozk_inputs.random_csr(50, 30, kmax, seed=8, phi=3.0)
    x = ozk_inputs.phi_matrix(np.random.default_rng(9), (30, 1), 3.0)[:, 0]
    pa, pb = rns.scaling_bits(r, kmax)
    e = spmv.row_exponents(rp, v, pa)
    f = int(ozaki2.scale_exponents(x[:, None], pb, 1)[0])
    a = _dense(rp, ci, v, 30)
    assert ozaki2.exact_sum_bound_ok(a, x[:, None], e, np.array([f]), r)
    # and the budget is tight enough to matter: a wider budget breaks it somewhere
    assert (pa + pb + math.ceil(math.log2(kmax))) <= rns.budget_q(r)


def test_spmv_equals_dense_emulation_with_its_exponents():
    r, kmax = 14, 8
    rp, ci, v = ozk_inputs.random_csr(70, 45, kmax, seed=11, phi=2.0)
    x = ozk_inputs.uniform_matrix(np.random.default_rng(12), (45, 1))[:, 0]
    pa, pb = rns.scaling_bits(r, kmax)
    e = spmv.row_exponents(rp, v, pa)
    f = ozaki2.scale_exponents(x[:, None], pb, 1)
    dense = ozaki2.dgemm(_dense(rp, ci, v, 45), x[:, None], r, exps=(e, f))[:, 0]
    np.testing.assert_array_equal(spmv.spmv_csr(rp, ci, v, x, r, kmax), dense)


def test_special_rows():
    rp = np.array([0, 0, 2, 4, 7, 9], dtype=np.int32)        # row 0 empty
    ci = np.array([0, 3, 1, 2, 0, 1, 2, 1, 9], dtype=np.int32)
    v = np.array([1.0, 2.0, np.inf, 1.0, 1.0, 1.0, 1.0, 3.0, 4.0])
    x = np.array([1.0, -2.0, 0.5, 0.25])
    y = spmv.spmv_csr(rp, ci, v, x, 8, 2)
    assert y[0] == 0.0 and not math.copysign(1.0, y[0]) < 0     # +0
    assert y[1] == 1.0 + 2.0 * 0.25
    assert math.isnan(y[2])                                      # Inf in the row
    assert math.isnan(y[3])                                      # 3 > kmax = 2 nonzeros
    assert math.isnan(y[4])                                      # column 9 >= 4
    xs = x.copy()
    xs[2] = np.nan
    assert np.all(np.isnan(spmv.spmv_csr(rp, ci, v, xs, 8, 3)))


def test_sampled_rows_equal_the_full_result():
    rp, ci, v = ozk_inputs.random_csr(120, 60, 7, seed=21, phi=1.0)
    x = ozk_inputs.uniform_matrix(np.random.default_rng(22), (60, 1))[:, 0]
    full = spmv.spmv_csr(rp, ci, v, x, 16, 7)
    rows = np.array([0, 5, 17, 63, 119])
    np.testing.assert_array_equal(spmv.spmv_csr(rp, ci, v, x, 16, 7, rows=rows), full[rows])
