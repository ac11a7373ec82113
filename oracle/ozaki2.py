"""Ozaki scheme II fp64 matrix product, written out step by step on the CPU (oracle).

Test infrastructure only (see the package docstring).  Follows [TME4], abstract: each
fp64 operand is scaled, rounded and reduced modulo each of r moduli ("deconstruction");
one integer matrix product per modulus (the tensor term); a per-output reconstruction
returns fp64.  [AWE], English abstract: each product of the scheme is an error-free
integer matrix product times a scale factor.

Readings of what the pages leave open (see also ``oracle.rns``):

* Scaling: a power of two per row of A and per column of B (and of X for the GEMV),
  set by the max rule e_i = P_A - 1 - ilogb(max_h |a_ih|) (0 for an all-zero row),
  so that 2^(P_A-1) <= max_h |a_ih| 2^e_i < 2^P_A.  A row or column holding Inf or NaN
  gets the exponent NONFINITE and its residues are 0; the outputs it touches are NaN.
* Norm rule (optional, ``scaling="norm"``): e_i = alpha_A - 1 - E_i with E_i an upper
  bound of floor(log2 ||a_i||_2): T = ilogb(max_h |a_ih|), s = sum_h (a_ih 2^-T)^2 in
  float64 (any order: its relative error is below 2^-35 for k <= 2^17), u = ilogb(RN(s
  (1 + 2^-32))), E_i = T + floor(u/2).  Then 2^e_i ||a_i||_2 < 2^alpha_A, and with the
  norm budget of ``rns.scaling_bits_norm`` the CRT lift stays exact (Cauchy-Schwarz).
  The bound follows each line's 2-norm instead of k times its largest entry, so lines
  with a few large entries keep more bits of the rest.
* Rounding: a'_ih = RNE(a_ih 2^e_i), round half to even, held as an exact integer
  (it may be wider than 53 bits).
* Output: C_ij = RN(X_ij 2^-(e_i + f_j)), one round-to-nearest-even of the exact value,
  where X_ij is the CRT lift of the r modular products; X_ij equals sum_h a'_ih b'_hj
  exactly because the bit budget keeps that sum inside (-(M-1)/2, (M-1)/2).

Functions take and return numpy arrays; the "plane" layout is the one the library
uses: A's planes are [r][m][k] (row-major, K contiguous) and B's planes are
[r][n][k] (B transposed, K contiguous).
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

from . import rns

NONFINITE = -(2**31)


# --------------------------------------------------------------------------- step 1
def scale_exponents(x: np.ndarray, p: int, axis: int) -> np.ndarray:
    """Per-row (axis 0) or per-column (axis 1) power-of-two exponents by the max rule.

    Returns int64 e with 2^(p-1) <= max|x| 2^e < 2^p, 0 for an all-zero line and
    NONFINITE for a line holding Inf or NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    red = 1 if axis == 0 else 0
    with np.errstate(invalid="ignore"):
        t = np.max(np.abs(x), axis=red)
    finite = np.all(np.isfinite(x), axis=red)
    _, ex = np.frexp(np.where(finite, t, 0.0))  # t = frac * 2^ex, ilogb(t) = ex - 1
    e = np.where(t > 0, p - ex.astype(np.int64), 0)
    return np.where(finite, e, NONFINITE).astype(np.int64)


def norm_bracket(row: np.ndarray) -> tuple[int, float]:
    """(T, s_up) for a finite, nonzero line: T = ilogb(max |x|) and s_up =
    RN(s (1 + 2^-32)) with s = sum (x 2^-T)^2 in float64, an upper bound of the exact
    sum of squares of x 2^-T whatever order s is summed in."""
    t = float(np.max(np.abs(row)))
    big_t = math.frexp(t)[1] - 1
    scaled = np.ldexp(row, -big_t)
    s = float(np.sum(scaled * scaled))
    return big_t, s * (1.0 + 2.0**-32)


def scale_exponents_norm(x: np.ndarray, alpha: int, axis: int) -> np.ndarray:
    """Per-row (axis 0) or per-column (axis 1) exponents by the norm rule: int64 e with
    2^e ||x_line||_2 < 2^alpha; 0 for an all-zero line, NONFINITE for a line holding Inf
    or NaN."""
    x = np.asarray(x, dtype=np.float64)
    lines = x if axis == 0 else x.T
    out = np.empty(lines.shape[0], dtype=np.int64)
    for i, row in enumerate(lines):
        if not np.all(np.isfinite(row)):
            out[i] = NONFINITE
            continue
        if not row.size or float(np.max(np.abs(row))) == 0.0:
            out[i] = 0
            continue
        big_t, s_up = norm_bracket(row)
        u = math.frexp(s_up)[1] - 1                        # ilogb(s_up)
        out[i] = alpha - 1 - (big_t + u // 2)
    return out


def exponents(x: np.ndarray, r: int, k: int, axis: int, operand: str,
              scaling: str = "max") -> np.ndarray:
    """Exponents of A's rows (operand "a") or B's columns (operand "b") by the given
    scaling rule, with the matching bit budget for r moduli and dot length k."""
    if scaling == "max":
        pa, pb = rns.scaling_bits(r, k)
        return scale_exponents(x, pa if operand == "a" else pb, axis)
    if scaling == "norm":
        aa, ab = rns.scaling_bits_norm(r, k)
        return scale_exponents_norm(x, aa if operand == "a" else ab, axis)
    raise ValueError(f"unknown scaling {scaling!r}")


def exact_sum_bound_ok(a: np.ndarray, b: np.ndarray, e, f, r: int) -> bool:
    """Whether sum_h |a'_ih| |b'_hj| <= (M-1)/2 for every output, in exact integers (the
    condition for the CRT lift to recover every dot product); small inputs only."""
    big_m, _ = rns.crt_basis(r)
    half = (big_m - 1) // 2
    m, k = a.shape
    n = b.shape[1]
    ai = [[abs(scaled_integer(float(a[i, h]), int(e[i]))) if e[i] != NONFINITE else 0
           for h in range(k)] for i in range(m)]
    bj = [[abs(scaled_integer(float(b[h, j]), int(f[j]))) if f[j] != NONFINITE else 0
           for h in range(k)] for j in range(n)]
    return all(sum(x * y for x, y in zip(ai[i], bj[j])) <= half
               for i in range(m) for j in range(n))


# --------------------------------------------------------------------------- step 2
def scaled_integer(a: float, e: int) -> int:
    """RNE(a * 2^e) as an exact Python integer (definition, one scalar)."""
    return round(Fraction(a) * (Fraction(2) ** e))


def _scaled_mantissa(x: np.ndarray, e: np.ndarray):
    """Write RNE(x 2^e) as mant * 2^sh with int64 mant (|mant| < 2^53) and sh >= -52.

    np.ldexp is exact here except where the result underflows below 2^-1022, and there
    both the exact value and the underflowed one round to the integer 0.  np.rint
    rounds half to even.  An integer-valued double is mant * 2^sh exactly.
    """
    xr = np.rint(np.ldexp(x, e))
    frac, ex = np.frexp(xr)
    mant = np.ldexp(frac, 53).astype(np.int64)
    sh = ex.astype(np.int64) - 53
    return mant, sh


def residue_planes(x: np.ndarray, exps: np.ndarray, r: int, axis: int) -> np.ndarray:
    """Symmetric residues smod(RNE(x 2^e), m_l) for l = 1..r, as int8 planes.

    axis 0: x is (rows, k), exps per row, result [r][rows][k].
    axis 1: x is (k, cols), exps per column, result [r][cols][k] (transposed so K is
    contiguous, as the matrix products consume it).
    Lines whose exponent is NONFINITE give all-zero residues.
    """
    x = np.asarray(x, dtype=np.float64)
    if axis == 1:
        x = x.T
    exps = np.asarray(exps, dtype=np.int64)
    bad = exps == NONFINITE
    e = np.where(bad, 0, exps)[:, None]
    xs = np.where(bad[:, None], 0.0, x)
    mant, sh = _scaled_mantissa(xs, np.broadcast_to(e, xs.shape))
    out = np.empty((r,) + xs.shape, dtype=np.int8)
    max_sh = int(max(sh.max(initial=0), 0))
    for l, m in enumerate(rns.moduli(r)):
        pow2 = np.array([pow(2, s, m) for s in range(max_sh + 1)], dtype=np.int64)
        big = (mant % m) * pow2[np.clip(sh, 0, max_sh)] % m     # sh >= 0: mant * 2^sh
        small = (mant >> np.clip(-sh, 0, 62)) % m                # sh < 0: exact shift
        res = np.where(sh >= 0, big, small)
        half = m // 2
        out[l] = ((res + half) % m - half).astype(np.int8)
    return out


# --------------------------------------------------------------------------- step 3
def modular_products(planes_a: np.ndarray, planes_b: np.ndarray) -> np.ndarray:
    """P_l = A~_l B~_l^T for every modulus, exact, int64 [r][m][n].

    The float64 matmul is exact: every product is an integer of magnitude <= 2^14 and
    every partial sum stays below k 2^14 < 2^53, whatever order the library sums in.
    """
    r, m, k = planes_a.shape
    if k >= 2**39:
        raise ValueError("k too large for an exact float64 residue product")
    out = np.empty((r, m, planes_b.shape[1]), dtype=np.int64)
    for l in range(r):
        out[l] = (planes_a[l].astype(np.float64) @ planes_b[l].astype(np.float64).T).astype(np.int64)
    return out


# --------------------------------------------------------------------------- step 4
def round_scaled(x: int, s: int) -> float:
    """RN(x * 2^-s), correctly rounded once (Python int true division is correctly
    rounded, subnormal results included)."""
    if x == 0:
        return 0.0
    if s >= 0:
        return x / (1 << s)
    try:
        return float(x << (-s))
    except OverflowError:
        return math.copysign(math.inf, x)


def crt_integers(products: np.ndarray, r: int) -> np.ndarray:
    """CRT lift of each output's r modular products (``rns.crt_lift`` per output): object
    array of Python ints."""
    prods = np.asarray(products)
    flat = prods.reshape(r, -1)
    out = np.empty(flat.shape[1], dtype=object)
    for idx in range(flat.shape[1]):
        out[idx] = rns.crt_lift([int(v) for v in flat[:, idx]], r)
    return out.reshape(prods.shape[1:])


def reconstruct(products: np.ndarray, r: int, e: np.ndarray, f: np.ndarray) -> np.ndarray:
    """C_ij = RN(X_ij 2^-(e_i + f_j)) from the modular products; NaN where e_i or f_j
    is NONFINITE."""
    xs = crt_integers(products, r)
    rows, cols = xs.shape
    out = np.empty((rows, cols), dtype=np.float64)
    for i in range(rows):
        for j in range(cols):
            if e[i] == NONFINITE or f[j] == NONFINITE:
                out[i, j] = math.nan
            else:
                out[i, j] = round_scaled(xs[i, j], int(e[i]) + int(f[j]))
    return out


# --------------------------------------------------------------------------- pipelines
def dgemm(a: np.ndarray, b: np.ndarray, r: int, rows=None, cols=None,
          scaling: str = "max", exps=None) -> np.ndarray:
    """Emulated C = A B (A m x k, B k x n), optionally only rows x cols of C.

    Exponents always come from the full rows of A and full columns of B, so a sampled
    block equals the same block of the full product.  ``exps`` = (e, f) supplies the
    exponents of the selected rows and columns instead (they must satisfy the bound of
    the rule; ``exact_sum_bound_ok`` checks it)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    k = a.shape[1]
    rows = np.arange(a.shape[0]) if rows is None else np.asarray(rows)
    cols = np.arange(b.shape[1]) if cols is None else np.asarray(cols)
    if exps is None:
        e = exponents(a[rows], r, k, 0, "a", scaling)
        f = exponents(b[:, cols], r, k, 1, "b", scaling)
    else:
        e, f = (np.asarray(v, dtype=np.int64) for v in exps)
    pla = residue_planes(a[rows], e, r, axis=0)
    plb = residue_planes(b[:, cols], f, r, axis=1)
    prods = modular_products(pla, plb)
    return reconstruct(prods, r, e, f)


def dgemv(a: np.ndarray, x: np.ndarray, r: int, rows=None) -> np.ndarray:
    """Emulated Y = A X for X with a few columns; identical arithmetic to dgemm
    (A scaled per row with P_A, X per column with P_B)."""
    return dgemm(a, x, r, rows=rows)


def exact_scaled_product(a: np.ndarray, b: np.ndarray, r: int,
                         scaling: str = "max") -> np.ndarray:
    """The plain definition without residues, for tiny inputs: RN(2^-(e_i+f_j)
    sum_h a'_ih b'_hj) with the sum taken in Python integers."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    m, k = a.shape
    n = b.shape[1]
    e = exponents(a, r, k, 0, "a", scaling)
    f = exponents(b, r, k, 1, "b", scaling)
    ai = [[scaled_integer(float(a[i, h]), int(e[i])) for h in range(k)] for i in range(m)]
    bi = [[scaled_integer(float(b[h, j]), int(f[j])) for h in range(k)] for j in range(n)]
    out = np.empty((m, n))
    for i in range(m):
        for j in range(n):
            s = sum(x * y for x, y in zip(ai[i], bi[j]))
            out[i, j] = round_scaled(s, int(e[i]) + int(f[j]))
    return out
