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
  P_B = beta - P_A.  With |a'| <= 2^P_A and |b'| <= 2^P_B every exact dot product of
  length k satisfies sum |a'||b'| <= 2^Q <= (M-1)/2, so the CRT lift recovers it exactly.
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


def scaling_bits(r: int, k: int) -> tuple[int, int]:
    """(P_A, P_B): the integer widths the scaled operands of A and B may use."""
    beta = budget_q(r) - ceil_log2(k)
    if beta < 2:
        raise ValueError(f"r={r} gives no bit budget for k={k}")
    pa = beta // 2
    return pa, beta - pa


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
