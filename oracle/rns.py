"""Residue number system of Ozaki scheme II (oracle side, Python integers).

Test infrastructure only (see the package docstring).

[TME4] abstract: every fp64 operand is reduced "modulo each of the r moduli"; the pages
name neither the moduli nor the reconstruction formula.  Readings taken here:

* Moduli: pairwise-coprime integers <= 256, chosen greedily from 256 downwards (each
  candidate is kept when it is coprime to every modulus kept so far); the first r are
  used.  This gives the largest product M for every r under the <= 256 constraint.
* Symmetric residue: smod(x, m) = ((x + floor(m/2)) mod m) - floor(m/2), which lies in
  [-floor(m/2), ceil(m/2) - 1]; for odd m that is +-(m-1)/2, for m = 256 it is
  [-128, 127], so every residue fits int8.
* Reconstruction: the Chinese Remainder Theorem, X = sum_l E_l c_l mod M with
  E_l = (M/m_l) * ((M/m_l)^-1 mod m_l), lifted to the symmetric range.
* Bit budget: Q = floor(log2((M-1)/2)), beta = Q - ceil(log2 k), P_A = floor(beta/2),
  P_B = beta - P_A, each capped at WIDTH_CAP = 76.  With |a'| <= 2^P_A and |b'| <= 2^P_B
  every exact dot product of length k satisfies sum |a'||b'| <= 2^Q <= (M-1)/2, so the
  CRT lift recovers it exactly.  The cap only binds at r = 20 with k <= 2 (beta 153 or
  154); there a dot product of one or two terms still carries 76 bits per operand, far
  more than the 53 its fp64 result keeps, and every scaled integer stays at or below
  2^76, the range the norm rule already keeps to.
* Norm budget (the tighter row/column scaling): widths (alpha_A, alpha_B) for scaled
  rows and columns whose 2-norms stay below 2^alpha_A and 2^alpha_B; rounding each of
  the k entries moves a 2-norm by at most sqrt(k)/2, so by Cauchy-Schwarz
  sum |a'||b'| < (2^alpha_A + sqrt(k)/2)(2^alpha_B + sqrt(k)/2), which is kept at or
  below (M-1)/2.  alpha_A + alpha_B starts at Q - 1, each at most WIDTH_CAP = 76 (scaled
  integers then stay at or below 2^76, as under the max rule), and the larger is lowered
  until the inequality holds exactly.
"""
from __future__ import annotations

import math
from functools import lru_cache

MAX_MODULI = 20
MODULUS_BOUND = 256


def greedy_moduli(count: int, start: int = MODULUS_BOUND) -> list[int]:
    """First ``count`` pairwise-coprime integers found scanning down from ``start``."""
    chosen: list[int] = []
    cand = start
    while len(chosen) < count:
        if cand < 2:
            raise ValueError("not enough pairwise-coprime moduli below the bound")
        if all(math.gcd(cand, c) == 1 for c in chosen):
            chosen.append(cand)
        cand -= 1
    return chosen


def moduli(r: int) -> list[int]:
    if not 1 <= r <= MAX_MODULI:
        raise ValueError(f"r must be in [1, {MAX_MODULI}], got {r}")
    return greedy_moduli(r)


def product(ms) -> int:
    out = 1
    for m in ms:
        out *= m
    return out


@lru_cache(maxsize=None)
def crt_basis(r: int) -> tuple[int, tuple[int, ...]]:
    """(M, (E_1..E_r)) with E_l = 1 mod m_l and E_l = 0 mod m_j for j != l."""
    ms = moduli(r)
    big_m = product(ms)
    basis = []
    for m in ms:
        cofactor = big_m // m
        basis.append(cofactor * pow(cofactor, -1, m))
    return big_m, tuple(basis)


def budget_q(r: int) -> int:
    """Q = floor(log2((M - 1) / 2)) for the first r moduli."""
    big_m, _ = crt_basis(r)
    return ((big_m - 1) // 2).bit_length() - 1


def ceil_log2(k: int) -> int:
    if k < 1:
        raise ValueError("k must be >= 1")
    return (k - 1).bit_length()


WIDTH_CAP = 76
NORM_ALPHA_CAP = WIDTH_CAP


def scaling_bits(r: int, k: int) -> tuple[int, int]:
    """(P_A, P_B): the integer widths the scaled operands of A and B may use."""
    beta = budget_q(r) - ceil_log2(k)
    if beta < 2:
        raise ValueError(f"r={r} gives no bit budget for k={k}")
    pa = beta // 2
    return min(pa, WIDTH_CAP), min(beta - pa, WIDTH_CAP)


def norm_bound_holds(alpha_a: int, alpha_b: int, k: int, big_m: int) -> bool:
    """(2^alpha_a + sqrt(k)/2)(2^alpha_b + sqrt(k)/2) <= (M-1)/2, exactly: with
    t = isqrt(k - 1) + 1 >= sqrt(k), check (2^(alpha_a+1) + t)(2^(alpha_b+1) + t)
    <= 2 (M - 1)."""
    t = math.isqrt(k - 1) + 1
    return ((1 << (alpha_a + 1)) + t) * ((1 << (alpha_b + 1)) + t) <= 2 * (big_m - 1)


def scaling_bits_norm(r: int, k: int) -> tuple[int, int]:
    """(alpha_A, alpha_B) of the norm rule (see the module docstring)."""
    if k < 1:
        raise ValueError("k must be >= 1")
    big_m, _ = crt_basis(r)
    q = budget_q(r)
    aa = min((q - 1) // 2, NORM_ALPHA_CAP)
    ab = min(q - 1 - (q - 1) // 2, NORM_ALPHA_CAP)
    while not norm_bound_holds(aa, ab, k, big_m):
        if aa >= ab:
            aa -= 1
        else:
            ab -= 1
        if aa < 1 or ab < 1:
            raise ValueError(f"r={r} gives no norm budget for k={k}")
    return aa, ab


def smod(x: int, m: int) -> int:
    """Symmetric residue of integer x modulo m, in [-floor(m/2), ceil(m/2) - 1]."""
    h = m // 2
    return (x + h) % m - h


def crt_lift(residues, r: int) -> int:
    """The integer X in [-(M/2), M/2) congruent to residues[l] modulo m_l for every l."""
    big_m, basis = crt_basis(r)
    acc = 0
    for c, e in zip(residues, basis):
        acc += int(c) * e
    x = acc % big_m
    if x > (big_m - 1) // 2:
        x -= big_m
    return x
