"""Exact INT8 x INT8 matrix product in 6 FP4 products (oracle side).

Test infrastructure only (see the package docstring).  [AWE], English abstract: with
free integer limb weights and stored planes that are linear combinations of limbs, an
INT8 x INT8 product needs 6 FP4 matrix products instead of the 9 of base-13 limbs.  The
page prints neither the weights nor the planes.  Readings taken here:

* Limbs and planes: an int8 value x is written x = a0 + w1 a1 + w2 a2 with every limb
  a_i in S = 2 x FP4 = {0, +-1, +-2, +-3, +-4, +-6, +-8, +-12}; the stored planes are the
  three limbs and their three pairwise sums a0 + a1, a0 + a2, a1 + a2, each of which must
  also lie in S (so that it is an FP4 value).  The same encoding serves both operands.
* Products (the three-term Karatsuba identity): with u = (a0, a1, a2, a0+a1, a0+a2,
  a1+a2) for x and v the same for y,
      x y = sum_i w_i^2 a_i b_i + sum_{i<j} w_i w_j (a_i b_j + a_j b_i)
          = sum_i c_i a_i b_i + sum_{i<j} w_i w_j (a_i + a_j)(b_i + b_j),
      c_i = w_i^2 - w_i sum_{j != i} w_j,
  so C = A B = sum_t coef_t U_t(A) V_t(B) over 6 plane products.
* Weights: (w0, w1, w2) = (1, 29, 37).  An exhaustive search over 2 <= w1 < 60,
  w1 < w2 < 400 and the sign of each pairwise combination finds 11 weight triples that
  encode every int8 value; (1, 29, 37) is the one with plain pairwise sums whose limbs and
  sums never exceed 6 in magnitude (``search_weights`` repeats the search for the sums).
  Every elementary product is then at most 36, so fp32 accumulation of a plane product
  is exact for K <= 466033 (36 K < 2^24).
* Limb choice: several limb triples may encode one x; the one taken minimises, in order,
  the largest magnitude among its six plane values, the sum of their squares, and then
  (a0, a1, a2) lexicographically.
* Storage: as the base-13 engine, a plane value d is the e2m1 code of d/2 (both MFMA
  block scales 2^1), two codes per byte with the even K index in the low nibble.  The
  fused product's planes are laid out per line in K steps of 64 codes: for line i and
  step s, 6 planes x 32 bytes = 192 consecutive bytes (plane t at byte 32 t).
"""
from __future__ import annotations

import itertools
from functools import lru_cache

import numpy as np

from . import fp4limb

WEIGHTS = (1, 29, 37)
PAIRS = ((0, 1), (0, 2), (1, 2))
N_PRODUCTS = 6
STEP_CODES = 64                  # K codes per step of the interleaved layout
STEP_BYTES = N_PRODUCTS * STEP_CODES // 2   # 192


def s_values() -> list[int]:
    """S = 2 x FP4, the 15 distinct integers."""
    return fp4limb.fp4_times_two()


def coefficients(w=WEIGHTS) -> tuple[int, ...]:
    """coef_t of the 6 plane products: c_0, c_1, c_2, then w_i w_j for the pairs."""
    c = [w[i] * w[i] - w[i] * sum(w[j] for j in range(3) if j != i) for i in range(3)]
    d = [w[i] * w[j] for i, j in PAIRS]
    return tuple(c + d)


def plane_values(a) -> tuple[int, ...]:
    """The six plane values of limbs (a0, a1, a2)."""
    return tuple(a) + tuple(a[i] + a[j] for i, j in PAIRS)


def valid_triples(x: int, w=WEIGHTS, signs=(1, 1, 1)):
    """Every limb triple in S^3 encoding x whose pairwise combinations a_i + sign a_j
    also lie in S."""
    s = s_values()
    ss = set(s)
    for a in itertools.product(s, repeat=3):
        if sum(wi * ai for wi, ai in zip(w, a)) != x:
            continue
        if all(a[i] + sg * a[j] in ss for (i, j), sg in zip(PAIRS, signs)):
            yield a


@lru_cache(maxsize=None)
def limb_table() -> dict[int, tuple[int, int, int]]:
    """x -> (a0, a1, a2) for every int8 x, by the limb-choice rule."""
    out = {}
    for x in range(-128, 128):
        cands = list(valid_triples(x))
        if not cands:
            raise ValueError(f"{x} has no encoding")

        def key(a):
            v = plane_values(a)
            return (max(abs(t) for t in v), sum(t * t for t in v), a)

        out[x] = min(cands, key=key)
    return out


def search_weights(w1_max: int = 60, w2_max: int = 400):
    """All (weights, signs) with w0 = 1, 2 <= w1 < w1_max, w1 < w2 < w2_max that encode
    every int8 value with limbs and pairwise combinations (a_i + sign a_j) in S."""
    s = np.array(s_values(), dtype=np.int64)
    ss = set(int(v) for v in s)
    trip = np.array(list(itertools.product(s, repeat=3)), dtype=np.int64)   # [3375][3]
    hits = []
    for signs in itertools.product((1, -1), repeat=3):
        ok = np.ones(len(trip), dtype=bool)
        for (i, j), sg in zip(PAIRS, signs):
            ok &= np.isin(trip[:, i] + sg * trip[:, j], list(ss))
        t = trip[ok]
        for w1 in range(2, w1_max):
            for w2 in range(w1 + 1, w2_max):
                x = t[:, 0] + w1 * t[:, 1] + w2 * t[:, 2]
                x = x[(x >= -128) & (x <= 127)]
                if np.unique(x).size == 256:
                    hits.append(((1, w1, w2), signs))
    return sorted(hits)


def planes(x: np.ndarray) -> np.ndarray:
    """The 6 plane values of an int8 matrix: int8 [6][rows][cols]."""
    x = np.asarray(x, dtype=np.int64)
    tab = limb_table()
    lut = np.array([plane_values(tab[v]) for v in range(-128, 128)], dtype=np.int8)  # [256][6]
    return np.moveaxis(lut[x + 128], -1, 0)


def plane_codes(x: np.ndarray) -> np.ndarray:
    """e2m1 codes of the plane values: uint8 [6][rows][cols], one code per byte."""
    p = planes(x).astype(np.int64)
    lut = np.zeros(256, dtype=np.uint8)
    for d in s_values():
        lut[d & 0xFF] = fp4limb.encode_digit(d)
    return lut[p & 0xFF]


def pack_lines(x: np.ndarray, k_padded: int) -> np.ndarray:
    """Interleaved packed planes of the lines of x (rows of x; K along its columns),
    zero-padded to k_padded codes (a multiple of 64): uint8 [lines][k_padded/64 * 192],
    step s of line i at bytes 192 s .. 192 s + 191, plane t at 32 t within the step."""
    codes = plane_codes(x)                                   # [6][lines][k]
    lines, k = codes.shape[1], codes.shape[2]
    if k_padded % STEP_CODES or k_padded < k:
        raise ValueError("k_padded must be a multiple of 64 and >= K")
    full = np.zeros((N_PRODUCTS, lines, k_padded), dtype=np.uint8)
    full[:, :, :k] = codes
    packed = full[..., 0::2] | (full[..., 1::2] << 4)        # [6][lines][k_padded/2]
    steps = k_padded // STEP_CODES
    packed = packed.reshape(N_PRODUCTS, lines, steps, STEP_CODES // 2)
    return np.ascontiguousarray(packed.transpose(1, 2, 0, 3)).reshape(lines, steps * STEP_BYTES)


def plane_products(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """The 6 exact plane products P_t = U_t(A) V_t(B), int64 [6][m][n]."""
    ua = planes(a).astype(np.int64)
    vb = planes(b.T).astype(np.int64)                        # B's planes per column
    return np.stack([ua[t] @ vb[t].T for t in range(N_PRODUCTS)])


def int8_gemm(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """C = sum_t coef_t P_t, the exact int8 product (int64)."""
    p = plane_products(a, b)
    c = np.zeros(p.shape[1:], dtype=np.int64)
    for t, coef in enumerate(coefficients()):
        c += coef * p[t]
    return c
