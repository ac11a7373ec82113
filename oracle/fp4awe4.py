"""Exact INT4 x INT8 matrix product in 4 FP4 products (oracle side).

Test infrastructure only (see the package docstring).  [AWE], English abstract: with
free integer limb weights and stored planes that are linear combinations of limbs, an
INT4 x INT8 product needs 4 FP4 matrix products.  The page prints neither the weights nor
the planes.  Readings taken here:

* Limbs: an int4 value x (in [-8, 7]) is written x = a0 + W a1 and an int8 value y is
  written y = b0 + W b1 + W^2 b2, with one limb weight W for both: x and y are then the
  values at (W, 1) of the binary forms X(p, q) = q a0 + p a1 and Y(p, q) = q^2 b0 + p q b1
  + p^2 b2, and x y is the value at (W, 1) of the cubic form C = X Y, whose four
  coefficients c_d (of p^d q^(3-d)) follow from C at four points.
* Products: at the points (p, q) in {(0, 1), (1, 0), (1, 1), (1, 2)} the stored planes are
  U_t = X(p_t, q_t) = a0, a1, a0 + a1, 2 a0 + a1 for x and V_t = Y(p_t, q_t) = b0, b2,
  b0 + b1 + b2, 4 b0 + 2 b1 + b2 for y; every one of them must lie in S = 2 x FP4 =
  {0, +-1, +-2, +-3, +-4, +-6, +-8, +-12} (b1 itself is not stored).  Solving the 4 x 4
  system for c and evaluating at (W, 1) gives x y = sum_t coef_t U_t(x) V_t(y) with integer
  coefficients, so C = A B = sum_t coef_t U_t(A) V_t(B): four plane products.
* Weight and points: W = 5 at the points above.  ``search_encodings`` tries every weight
  2 <= W < 25 with every 4 of the 10 points (0, 1), (1, 0), (+-1, 1), (+-2, 1), (+-1, 2),
  (+-3, 1) and finds two that encode every int4 and every int8 value: W = 5 with these
  points and W = 4 with (0, 1), (1, 0), (-1, 1), (-1, 2); the first has plain sums.  Its
  coefficients are (36, 90, 45, -10); the A planes never exceed 4 and the B planes 12 in
  magnitude, so every elementary product is at most 48 and fp32 accumulation of a plane
  product is exact for K <= 349525.
* Limb choice: among the limb tuples that encode a value with every plane in S, the one
  with the smallest largest plane magnitude, then the smallest sum of squares of its
  planes, then the smallest limbs lexicographically.
* INT4 input: a byte holds one int4 value in its low four bits (two's complement); an
  int8 array of values in [-8, 7] is read as it is.
* Storage: as the other FP4 engines, a plane value d is the e2m1 code of d/2 (both MFMA
  block scales 2^1), two codes per byte with the even K index in the low nibble.  The
  fused product's planes are laid out per line in K steps of 64 codes: for line i and step
  s, 4 planes x 32 bytes = 128 consecutive bytes (plane t at byte 32 t).
"""
from __future__ import annotations

import itertools
from fractions import Fraction
from functools import lru_cache

import numpy as np

from . import fp4limb

W = 5
POINTS = ((0, 1), (1, 0), (1, 1), (1, 2))
N_PRODUCTS = 4
STEP_CODES = 64
STEP_BYTES = N_PRODUCTS * STEP_CODES // 2   # 128
CANDIDATE_POINTS = ((0, 1), (1, 0), (1, 1), (-1, 1), (2, 1), (-2, 1), (1, 2), (-1, 2),
                    (3, 1), (-3, 1))


def s_values() -> list[int]:
    """S = 2 x FP4, the 15 distinct integers."""
    return fp4limb.fp4_times_two()


def int4_value(byte: int) -> int:
    """The int4 value held in the low four bits of a byte (two's complement)."""
    return ((int(byte) & 15) ^ 8) - 8


def x_planes(a, points=POINTS) -> tuple[int, ...]:
    """U_t = q_t a0 + p_t a1 at each point."""
    return tuple(q * a[0] + p * a[1] for p, q in points)


def y_planes(b, points=POINTS) -> tuple[int, ...]:
    """V_t = q_t^2 b0 + p_t q_t b1 + p_t^2 b2 at each point."""
    return tuple(q * q * b[0] + p * q * b[1] + p * p * b[2] for p, q in points)


def coefficients(w: int = W, points=POINTS) -> tuple[int, ...]:
    """coef_t with x y = sum_t coef_t U_t V_t: the row (w^0, .., w^3) times the inverse of
    V[t][d] = p_t^d q_t^(3-d), in exact rationals; every entry must be an integer."""
    n = 4
    mat = [[Fraction(p ** d * q ** (3 - d)) for d in range(n)] for p, q in points]
    # Gauss-Jordan inverse
    aug = [row + [Fraction(int(i == j)) for j in range(n)] for i, row in enumerate(mat)]
    for col in range(n):
        piv = next(r for r in range(col, n) if aug[r][col] != 0)
        aug[col], aug[piv] = aug[piv], aug[col]
        pv = aug[col][col]
        aug[col] = [v / pv for v in aug[col]]
        for r in range(n):
            if r != col and aug[r][col] != 0:
                f = aug[r][col]
                aug[r] = [a - f * b for a, b in zip(aug[r], aug[col])]
    inv = [row[n:] for row in aug]                       # c = inv P
    coef = [sum(Fraction(w) ** d * inv[d][t] for d in range(n)) for t in range(n)]
    if any(c.denominator != 1 for c in coef):
        raise ValueError("coefficients are not integers")
    return tuple(int(c) for c in coef)


def _integer_solutions(rows, values):
    """Integer solutions of M z = v for every row v of `values` (M square, nonsingular):
    z = adj(M) v / det(M), kept where the division is exact.  Returns (z, mask)."""
    m = np.array(rows, dtype=np.int64)
    det = int(round(np.linalg.det(m)))
    if det == 0:
        return None, None
    n = m.shape[0]
    adj = np.zeros_like(m)
    for i in range(n):
        for j in range(n):
            minor = np.delete(np.delete(m, j, axis=0), i, axis=1)
            adj[i, j] = (-1) ** (i + j) * int(round(np.linalg.det(minor))) if n > 1 else 1
    num = values @ adj.T                                    # [cases][n]
    ok = np.all(num % det == 0, axis=1)
    return num // det, ok


@lru_cache(maxsize=None)
def x_limb_sets(points=POINTS):
    """Every integer limb pair (a0, a1) whose planes at all four points lie in S: the
    planes at the first two points take every pair of values of S, which fixes (a0, a1)."""
    s = s_values()
    vals = np.array(list(itertools.product(s, repeat=2)), dtype=np.int64)
    z, ok = _integer_solutions([(q, p) for p, q in points[:2]], vals)
    out = []
    if z is not None:
        for a in z[ok]:
            a = (int(a[0]), int(a[1]))
            pl = x_planes(a, points)
            if all(v in set(s) for v in pl):
                out.append((a, pl))
    return tuple(out)


@lru_cache(maxsize=None)
def y_limb_sets(points=POINTS):
    """Every integer limb triple (b0, b1, b2) whose planes at all four points lie in S: the
    planes at the first three points take every triple of values of S."""
    s = s_values()
    vals = np.array(list(itertools.product(s, repeat=3)), dtype=np.int64)
    z, ok = _integer_solutions([(q * q, p * q, p * p) for p, q in points[:3]], vals)
    out = []
    if z is not None:
        for b in z[ok]:
            b = (int(b[0]), int(b[1]), int(b[2]))
            pl = y_planes(b, points)
            if all(v in set(s) for v in pl):
                out.append((b, pl))
    return tuple(out)


def _choose(cands):
    def key(item):
        limbs, planes = item
        return (max(abs(v) for v in planes), sum(v * v for v in planes), limbs)
    return min(cands, key=key)[0] if cands else None


def x_limbs(x: int, w: int = W, points=POINTS):
    """(a0, a1) for an int4 x by the limb-choice rule, or None."""
    return _choose([c for c in x_limb_sets(points) if c[0][0] + w * c[0][1] == x])


def y_limbs(y: int, w: int = W, points=POINTS):
    """(b0, b1, b2) for an int8 y by the limb-choice rule, or None."""
    return _choose([c for c in y_limb_sets(points)
                    if c[0][0] + w * c[0][1] + w * w * c[0][2] == y])


@lru_cache(maxsize=None)
def x_table() -> dict[int, tuple[int, int]]:
    out = {}
    for x in range(-8, 8):
        a = x_limbs(x)
        if a is None:
            raise ValueError(f"int4 {x} has no encoding")
        out[x] = a
    return out


@lru_cache(maxsize=None)
def y_table() -> dict[int, tuple[int, int, int]]:
    out = {}
    for y in range(-128, 128):
        b = y_limbs(y)
        if b is None:
            raise ValueError(f"int8 {y} has no encoding")
        out[y] = b
    return out


def search_encodings(w_max: int = 25, candidates=CANDIDATE_POINTS):
    """Every (W, 4 points) with 2 <= W < w_max that encodes every int4 and int8 value with
    all planes in S."""
    hits = []
    for pts in itertools.combinations(candidates, 4):
        xa = np.array([a for a, _ in x_limb_sets(pts)], dtype=np.int64).reshape(-1, 2)
        yb = np.array([b for b, _ in y_limb_sets(pts)], dtype=np.int64).reshape(-1, 3)
        for w in range(2, w_max):
            xv = xa[:, 0] + w * xa[:, 1]
            yv = yb[:, 0] + w * yb[:, 1] + w * w * yb[:, 2]
            if np.isin(np.arange(-8, 8), xv).all() and np.isin(np.arange(-128, 128), yv).all():
                hits.append((w, pts))
    return hits


def planes_x(x: np.ndarray) -> np.ndarray:
    """The 4 plane values of an int4 matrix (int8 array, low nibble): int8 [4][rows][cols]."""
    x = np.asarray(x, dtype=np.int64)
    v = ((x & 15) ^ 8) - 8
    tab = x_table()
    lut = np.array([x_planes(tab[t]) for t in range(-8, 8)], dtype=np.int8)   # [16][4]
    return np.moveaxis(lut[v + 8], -1, 0)


def planes_y(y: np.ndarray) -> np.ndarray:
    """The 4 plane values of an int8 matrix: int8 [4][rows][cols]."""
    y = np.asarray(y, dtype=np.int64)
    tab = y_table()
    lut = np.array([y_planes(tab[t]) for t in range(-128, 128)], dtype=np.int8)  # [256][4]
    return np.moveaxis(lut[y + 128], -1, 0)


def _codes(p: np.ndarray) -> np.ndarray:
    lut = np.zeros(256, dtype=np.uint8)
    for d in s_values():
        lut[d & 0xFF] = fp4limb.encode_digit(d)
    return lut[p.astype(np.int64) & 0xFF]


def pack_lines(planes: np.ndarray, k_padded: int) -> np.ndarray:
    """Interleaved packed planes of lines (plane values [4][lines][k]; K along the last
    axis), zero-padded to k_padded codes (a multiple of 64): uint8 [lines][k_padded/64 *
    128], step s of line i at bytes 128 s .. 128 s + 127, plane t at 32 t within the step."""
    codes = _codes(planes)
    lines, k = codes.shape[1], codes.shape[2]
    if k_padded % STEP_CODES or k_padded < k:
        raise ValueError("k_padded must be a multiple of 64 and >= K")
    full = np.zeros((N_PRODUCTS, lines, k_padded), dtype=np.uint8)
    full[:, :, :k] = codes
    packed = full[..., 0::2] | (full[..., 1::2] << 4)        # [4][lines][k_padded/2]
    steps = k_padded // STEP_CODES
    packed = packed.reshape(N_PRODUCTS, lines, steps, STEP_CODES // 2)
    return np.ascontiguousarray(packed.transpose(1, 2, 0, 3)).reshape(lines, steps * STEP_BYTES)


def plane_products(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """The 4 exact plane products P_t = U_t(A) V_t(B), int64 [4][m][n]."""
    ua = planes_x(a).astype(np.int64)
    vb = planes_y(np.asarray(b).T).astype(np.int64)          # B's planes per column
    return np.stack([ua[t] @ vb[t].T for t in range(N_PRODUCTS)])


def int4_int8_gemm(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """C = sum_t coef_t P_t, the exact product of the int4 matrix A (low nibbles) and the
    int8 matrix B (int64)."""
    p = plane_products(a, b)
    c = np.zeros(p.shape[1:], dtype=np.int64)
    for t, coef in enumerate(coefficients()):
        c += coef * p[t]
    return c
