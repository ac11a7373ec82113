"""Accuracy references for the emulated fp64 product (oracle side).

Test infrastructure only (see the package docstring).

* ``dot2_matmul``: each C_ij is the Dot2 dot product of Ogita, Rump and Oishi,
  "Accurate Sum and Dot Product", SIAM J. Sci. Comput. 26(6), 2005 (section 5): the
  running sum is carried as an unevaluated pair (p, s), each product is split exactly
  by TwoProduct (Dekker's product with Veltkamp's splitting, factor 2^27 + 1) and each
  addition by Knuth's TwoSum; the result p + s is as accurate as if computed in twice
  the working precision.  Vectorised over an output block, sequential in k.
* ``exact_matmul``: the exact rational product, formed with Python integers (every
  finite double is an integer multiple of 2^-1074), rounded once to fp64.  Tiny sizes.
* ``elementwise_bound``: the a-priori error bound of the max-rule scaling.
"""
from __future__ import annotations

import numpy as np

from . import ozaki2, rns

_SPLITTER = 134217729.0  # 2^27 + 1


def _two_sum(a, b):
    x = a + b
    z = x - a
    y = (a - (x - z)) + (b - z)
    return x, y


def _split(a):
    c = _SPLITTER * a
    hi = c - (c - a)
    return hi, a - hi


def _two_product(a, b):
    x = a * b
    ah, al = _split(a)
    bh, bl = _split(b)
    y = al * bl - (((x - ah * bh) - al * bh) - ah * bl)
    return x, y


def dot2_matmul(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """C = A B with every entry computed by Dot2 (sequential over k)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    k = a.shape[1]
    p, s = _two_product(a[:, 0:1], b[0:1, :])
    for h in range(1, k):
        prod, err = _two_product(a[:, h:h + 1], b[h:h + 1, :])
        p, q = _two_sum(p, prod)
        s = s + (q + err)
    return p + s


def _as_scaled_ints(x: np.ndarray) -> np.ndarray:
    """x * 2^1074 as exact Python integers (object array)."""
    flat = np.asarray(x, dtype=np.float64).reshape(-1)
    out = np.empty(flat.size, dtype=object)
    for i, v in enumerate(flat.tolist()):
        num, den = float(v).as_integer_ratio()
        out[i] = num * ((1 << 1074) // den)
    return out.reshape(np.shape(x))


def exact_matmul_ints(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """The exact product A B times 2^2148, as Python integers (object array)."""
    return np.dot(_as_scaled_ints(a), _as_scaled_ints(b))


def exact_matmul(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """The exact product A B rounded once to fp64 (round to nearest even)."""
    s = exact_matmul_ints(a, b)
    out = np.empty(s.shape, dtype=np.float64)
    for idx in np.ndindex(s.shape):
        out[idx] = ozaki2.round_scaled(int(s[idx]), 2148)
    return out


def elementwise_bound(a: np.ndarray, b: np.ndarray, r: int) -> np.ndarray:
    """Bound on |sum_h 2^-(e_i+f_j) a'_ih b'_hj - (A B)_ij| under the max rule.

    With a = (a' + da) 2^-e, |da| <= 1/2 (RNE), and likewise for b:
    a b 2^(e+f) = a'b' + a' db + da b' + da db, so the error of the exact scaled sum
    is at most 2^-(e_i+f_j) sum_h (|a'_ih| / 2 + |b'_hj| / 2 + 1/4), and
    |a'_ih| <= |a_ih| 2^e_i + 1/2.  Returned in float64 (upper-rounded by 1%).
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    k = a.shape[1]
    pa, pb = rns.scaling_bits(r, k)
    e = ozaki2.scale_exponents(a, pa, axis=0).astype(np.float64)
    f = ozaki2.scale_exponents(b, pb, axis=1).astype(np.float64)
    abs_a = np.abs(a) * np.exp2(e)[:, None] + 0.5     # >= |a'|
    abs_b = np.abs(b) * np.exp2(f)[None, :] + 0.5     # >= |b'|
    rowsum = abs_a.sum(axis=1)[:, None]                # sum_h |a'_ih|
    colsum = abs_b.sum(axis=0)[None, :]                # sum_h |b'_hj|
    bound = (0.5 * rowsum + 0.5 * colsum + 0.25 * k) * np.exp2(-(e[:, None] + f[None, :]))
    return bound * 1.01
