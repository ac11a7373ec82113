"""GPU parity of the norm (Cauchy-Schwarz) scaling rule against the CPU oracle.

Exponents: equal to the oracle's, except where the two fixed summation orders put the
bracketed sum of squares on different sides of a power of two (then off by one, and
the oracle's bracket sits within 2^-40 of that power); every GPU exponent is also
checked, in exact rational arithmetic, to keep 2^e ||line||_2 below 2^alpha.  Planes:
bit-exact against the oracle's residues for the GPU exponents.  DGEMM: <= 2 ulp of the
oracle fed the same exponents (expected bit-exact), sampled at 4096^3."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import fp64_gemm_emulation_ozk_amd as ozk
import ozk_inputs
from oracle import ozaki2, reference, rns

from gpu_common import announce, assert_within_ulps, to_dev

pytestmark = pytest.mark.gpu


def _special_lines(x: np.ndarray, axis: int) -> np.ndarray:
    """A zero line, a subnormal line, a tiny line, one huge entry among tiny ones, and a
    line whose entries span the whole exponent range."""
    x = x.copy()
    lines = x.shape[0] if axis == 0 else x.shape[1]
    if lines >= 5:
        sel = (lambda i: (i, slice(None))) if axis == 0 else (lambda i: (slice(None), i))
        x[sel(0)] = 0.0
        x[sel(1)] = x[sel(1)] * 1e-310
        x[sel(2)] = x[sel(2)] * 1e-300
        v = x[sel(3)] * 1e-200
        v[-1] = 2.0**900
        x[sel(3)] = v
        v = x[sel(4)]
        sign = np.where(v < 0, -1.0, 1.0)
        x[sel(4)] = np.ldexp(sign, np.linspace(-1070, 1020, v.shape[0]).astype(int))
    return x


def _exact_norm_ok(x: np.ndarray, e: np.ndarray, alpha: int, axis: int) -> None:
    """2^e_i ||line_i||_2 < 2^alpha in exact arithmetic, for every finite nonzero line."""
    lines = x if axis == 0 else x.T
    for i, line in enumerate(lines):
        if not np.all(np.isfinite(line)) or not np.any(line):
            continue
        ss = sum(Fraction(float(v)) ** 2 for v in line if v != 0.0)
        assert ss * Fraction(2) ** (2 * int(e[i])) < Fraction(2) ** (2 * alpha), i


def _check_exponents(got: np.ndarray, x: np.ndarray, alpha: int, axis: int,
                     exact: bool = True) -> None:
    want = ozaki2.scale_exponents_norm(x, alpha, axis)
    lines = x if axis == 0 else x.T
    for i in np.nonzero(got != want)[0]:
        assert abs(int(got[i]) - int(want[i])) == 1, (i, got[i], want[i])
        _, s_up = ozaki2.norm_bracket(lines[i])
        frac, _ = np.frexp(s_up)
        assert abs(frac - 0.5) < 2.0**-40 or abs(frac - 1.0) < 2.0**-40, (i, s_up)
    if exact:
        _exact_norm_ok(x, got, alpha, axis)


NORM_DECON_CASES = [
    # rows, cols, axis, r, dist
    (1, 1, 0, 14, "uniform"),
    (37, 100, 0, 14, "uniform"),
    (300, 257, 0, 16, "phi"),
    (130, 4100, 0, 20, "phi"),
    (6, 40000, 0, 14, "phi"),        # long rows: chunk partials of 2048 columns
    (100, 37, 1, 14, "uniform"),
    (257, 300, 1, 16, "phi"),
    (4100, 70, 1, 20, "phi"),        # 33 chunks of 128 rows, ragged last chunk and piece
    (600, 300, 1, 14, "phi"),        # 5 chunks: the last one has 2 pieces of 32 rows, ragged
    (64, 64, 1, 8, "uniform"),
    (33, 5, 1, 12, "phi"),           # a single ragged chunk
    (5000, 20, 1, 16, "phi"),        # 40 chunks: more than the 16 parts of the combine
]


@pytest.mark.parametrize("rows,cols,axis,r,dist", NORM_DECON_CASES)
def test_norm_deconstruct(rows, cols, axis, r, dist):
    announce(f"norm deconstruct rows={rows} cols={cols} axis={axis} r={r} {dist}")
    rng = np.random.default_rng(rows * 11 + cols)
    x = (ozk_inputs.phi_matrix(rng, (rows, cols), 4.0) if dist == "phi"
         else ozk_inputs.uniform_matrix(rng, (rows, cols)))
    x = _special_lines(x, axis)
    kdim = cols if axis == 0 else rows
    planes, exps = ozk.ozk_deconstruct_ex(to_dev(x), axis, r, "norm")
    torch.cuda.synchronize()
    aa, ab = rns.scaling_bits_norm(r, kdim)
    alpha = aa if axis == 0 else ab
    got_e = exps.cpu().numpy().astype(np.int64)
    _check_exponents(got_e, x, alpha, axis, exact=rows * cols <= 40000)
    want_pl = ozaki2.residue_planes(x, got_e, r, axis)
    got = planes.cpu().numpy()
    np.testing.assert_array_equal(got[:, :, :kdim], want_pl)
    assert not np.any(got[:, :, kdim:]), "K padding must be zero"


def test_norm_deconstruct_nonfinite_lines():
    announce("norm deconstruct nonfinite")
    x = ozk_inputs.uniform_matrix(np.random.default_rng(5), (6, 70))
    x[2, 5] = np.nan
    x[4, 0] = -np.inf
    planes, exps = ozk.ozk_deconstruct_ex(to_dev(x), 0, 14, "norm")
    planes_t, exps_t = ozk.ozk_deconstruct_ex(to_dev(x.T.copy()), 1, 14, "norm")
    torch.cuda.synchronize()
    e = exps.cpu().numpy()
    assert e[2] == ozaki2.NONFINITE and e[4] == ozaki2.NONFINITE
    np.testing.assert_array_equal(exps_t.cpu().numpy(), e)
    assert not np.any(planes.cpu().numpy()[:, [2, 4], :])
    np.testing.assert_array_equal(planes_t.cpu().numpy(), planes.cpu().numpy())


def test_norm_rows_and_columns_agree():
    """A row of A and the same vector as a column of B give the same exponent (the
    rows and columns paths sum in different orders; both must bracket the same norm)."""
    announce("norm rows vs columns")
    x = ozk_inputs.phi_matrix(np.random.default_rng(8), (200, 3000), 4.0)
    _, e_rows = ozk.ozk_deconstruct_ex(to_dev(x), 0, 16, "norm", k_budget=3000)
    _, e_cols = ozk.ozk_deconstruct_ex(to_dev(x.T.copy()), 1, 16, "norm", k_budget=3000)
    torch.cuda.synchronize()
    aa, ab = rns.scaling_bits_norm(16, 3000)
    er = e_rows.cpu().numpy().astype(np.int64) - aa
    ec = e_cols.cpu().numpy().astype(np.int64) - ab
    assert np.count_nonzero(er != ec) <= 1
    _check_exponents(e_rows.cpu().numpy().astype(np.int64), x, aa, 0, exact=False)


def _gpu_exps(a: np.ndarray, b: np.ndarray, r: int):
    k = a.shape[1]
    _, e = ozk.ozk_deconstruct_ex(to_dev(a), 0, r, "norm", k_budget=k)
    _, f = ozk.ozk_deconstruct_ex(to_dev(b), 1, r, "norm", k_budget=k)
    torch.cuda.synchronize()
    return e.cpu().numpy().astype(np.int64), f.cpu().numpy().astype(np.int64)


NORM_DGEMM_CASES = [
    (64, 64, 64, 14, "uniform"),
    (1, 1, 1, 5, "uniform"),
    (300, 200, 257, 16, "phi"),
    (257, 129, 100, 12, "phi"),
    (513, 260, 70, 20, "phi"),
    (100, 300, 1000, 18, "uniform"),
    (40, 50, 40000, 14, "phi"),      # long rows of A: unfused norm path
]


@pytest.mark.parametrize("m,n,k,r,dist", NORM_DGEMM_CASES)
def test_norm_dgemm_matches_oracle(m, n, k, r, dist):
    announce(f"norm dgemm m={m} n={n} k={k} r={r} {dist}")
    a, b = ozk_inputs.gemm_operands(m, n, k, seed=m + 5 * n + 3 * k, dist=dist, phi=4.0)
    got = ozk.ozk_dgemm_ex(to_dev(a), to_dev(b), r, "norm")
    e, f = _gpu_exps(a, b, r)
    aa, ab = rns.scaling_bits_norm(r, k)
    _check_exponents(e, a, aa, 0, exact=False)
    _check_exponents(f, b, ab, 1, exact=False)
    want = ozaki2.dgemm(a, b, r, exps=(e, f))
    assert assert_within_ulps(got.cpu().numpy(), want, 2) == 0


def test_norm_dgemm_exact_definition_small():
    """Tiny case against the plain definition (Python-integer sums) of the norm rule."""
    announce("norm dgemm exact definition")
    a, b = ozk_inputs.gemm_operands(9, 7, 33, seed=12, dist="phi", phi=4.0)
    got = ozk.ozk_dgemm_ex(to_dev(a), to_dev(b), 12, "norm").cpu().numpy()
    want = ozaki2.exact_scaled_product(a, b, 12, scaling="norm")
    assert assert_within_ulps(got, want, 0) == 0


def test_norm_dgemm_special_lines():
    announce("norm dgemm special lines")
    a, b = ozk_inputs.gemm_operands(70, 65, 90, seed=19, dist="phi", phi=4.0)
    a = _special_lines(a, 0)
    b = _special_lines(b, 1)
    a[10, 3] = np.nan
    b[7, 20] = np.inf
    got = ozk.ozk_dgemm_ex(to_dev(a), to_dev(b), 16, "norm")
    e, f = _gpu_exps(a, b, 16)
    want = ozaki2.dgemm(a, b, 16, exps=(e, f))
    assert assert_within_ulps(got.cpu().numpy(), want, 2) == 0


def test_norm_dgemm_deterministic_and_max_rule_unchanged():
    announce("norm dgemm determinism")
    a, b = ozk_inputs.gemm_operands(300, 300, 300, seed=2, dist="phi", phi=2.0)
    da, db = to_dev(a), to_dev(b)
    c1 = ozk.ozk_dgemm_ex(da, db, 16, "norm")
    c2 = ozk.ozk_dgemm_ex(da, db, 16, "norm")
    m1 = ozk.ozk_dgemm_ex(da, db, 16, "max")
    m2 = ozk.ozk_dgemm(da, db, 16)
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int64), c2.view(torch.int64))
    assert torch.equal(m1.view(torch.int64), m2.view(torch.int64))


@pytest.mark.parametrize("r", [10, 12, 14])
def test_norm_rule_more_accurate_on_wide_range(r):
    """On rows and columns whose entries span many binades (phi = 4), the norm rule keeps
    more bits per line: its error against the double-double product is no larger."""
    announce(f"norm vs max accuracy r={r}")
    a, b = ozk_inputs.gemm_operands(128, 128, 512, seed=31, dist="phi", phi=4.0)
    da, db = to_dev(a), to_dev(b)
    cn = ozk.ozk_dgemm_ex(da, db, r, "norm").cpu().numpy()
    cm = ozk.ozk_dgemm_ex(da, db, r, "max").cpu().numpy()
    dd = reference.dot2_matmul(a, b)
    err_n = np.linalg.norm(cn - dd) / np.linalg.norm(dd)
    err_m = np.linalg.norm(cm - dd) / np.linalg.norm(dd)
    assert err_n <= err_m


def test_norm_dgemm_square_4096_sampled():
    """The 4096^3 configuration at r = 16, entries (U-0.5) exp(0.5 N), sampled outputs
    against the oracle fed the GPU exponents, which are checked against the oracle's."""
    announce("norm dgemm 4096^3 r=16 sampled")
    a, b = ozk_inputs.gemm_operands(4096, 4096, 4096, seed=2, dist="phi", phi=0.5)
    da, db = to_dev(a), to_dev(b)
    got = ozk.ozk_dgemm_ex(da, db, 16, "norm")
    _, e_all = ozk.ozk_deconstruct_ex(da, 0, 16, "norm", k_budget=4096)
    _, f_all = ozk.ozk_deconstruct_ex(db, 1, 16, "norm", k_budget=4096)
    torch.cuda.synchronize()
    rng = np.random.default_rng(77)
    rows = np.sort(rng.choice(4096, 12, replace=False))
    cols = np.sort(rng.choice(4096, 40, replace=False))
    rows[-1], cols[-1] = 4095, 4095
    e = e_all.cpu().numpy().astype(np.int64)[rows]
    f = f_all.cpu().numpy().astype(np.int64)[cols]
    aa, ab = rns.scaling_bits_norm(16, 4096)
    _check_exponents(e, a[rows], aa, 0, exact=False)
    _check_exponents(f, b[:, cols], ab, 1, exact=False)
    want = ozaki2.dgemm(a, b, 16, rows=rows, cols=cols, exps=(e, f))
    sub = got[torch.as_tensor(rows, device=got.device)][:, torch.as_tensor(cols, device=got.device)]
    assert assert_within_ulps(sub.cpu().numpy(), want, 2) == 0
