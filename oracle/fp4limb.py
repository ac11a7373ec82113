"""Exact INT8 x INT8 matrix product through base-13 FP4 limbs (oracle side).

Test infrastructure only (see the package docstring).  Follows [AWE], English abstract:
the FP4 values scaled by 2 form S = {0, +-1, +-2, +-3, +-4, +-6, +-8, +-12}, which
holds every residue modulo 13, so with carries an integer splits into base-13 digits
that FP4 can store; each INT8 operand is split into 3 digits with weights (1, 13, 169)
and the digits are multiplied pairwise, 9 FP4 GEMMs per INT8 x INT8 product.

Readings of what the page leaves open:

* Digit choice: residues 1 and 12 have two representatives in S (1 or -12, 12 or -1);
  the one of smaller magnitude is taken, so the digit of residue rho is the element of
  S congruent to rho mod 13 with the least |d|.  Then |d0|, |d1| <= 8, d2 in {-1,0,1}.
* Storage: a digit d is stored as the e2m1 (OCP MX FP4) code of d/2; both MFMA block
  scales are 2^1, so each FP4 product equals d_a d_b.
* Packing: two codes per byte, the even K index in the low nibble.
"""
from __future__ import annotations

import numpy as np

BASE = 13
WEIGHTS = (1, 13, 169)


def e2m1_value(code: int) -> float:
    """Value of a 4-bit e2m1 code (sign, 2 exponent bits with bias 1, 1 mantissa bit)."""
    sign = (code >> 3) & 1
    exp = (code >> 1) & 3
    man = code & 1
    mag = 0.5 * man if exp == 0 else 2.0 ** (exp - 1) * (1.0 + 0.5 * man)
    return -mag if sign else mag


def fp4_times_two() -> list[int]:
    """The set 2 * FP4 as sorted integers (both zero codes give 0)."""
    return sorted({int(2 * e2m1_value(c)) for c in range(16)})


def digit_table() -> list[int]:
    """digit_table()[rho] = element of S congruent to rho (mod 13) of least magnitude."""
    s = fp4_times_two()
    table = []
    for rho in range(BASE):
        cands = [d for d in s if d % BASE == rho]
        table.append(min(cands, key=abs))
    return table


_TABLE = None


def split3(x: int) -> tuple[int, int, int]:
    """x = d0 + 13 d1 + 169 d2 with every d in S (x in [-128, 127])."""
    global _TABLE
    if _TABLE is None:
        _TABLE = digit_table()
    d0 = _TABLE[x % BASE]
    x1 = (x - d0) // BASE
    d1 = _TABLE[x1 % BASE]
    d2 = (x1 - d1) // BASE
    return d0, d1, d2


def encode_digit(d: int) -> int:
    """e2m1 code of d/2 (positive zero for 0)."""
    for code in range(16):
        if 2 * e2m1_value(code) == d:
            return code
    raise ValueError(f"digit {d} is not in S")


def limb_digits(x: np.ndarray) -> np.ndarray:
    """Digits of an int8 matrix: int8 array [3][rows][cols]."""
    x = np.asarray(x, dtype=np.int64)
    lut = np.array([split3(v) for v in range(-128, 128)], dtype=np.int8)  # [256][3]
    d = lut[x + 128]
    return np.moveaxis(d, -1, 0)


def limb_codes(x: np.ndarray) -> np.ndarray:
    """e2m1 codes of the digits: uint8 array [3][rows][cols], one code per byte."""
    codes = {d: encode_digit(d) for d in fp4_times_two()}
    d = limb_digits(x)
    lut = np.zeros(256, dtype=np.uint8)
    for dv, c in codes.items():
        lut[dv & 0xFF] = c
    return lut[d.astype(np.int64) & 0xFF]


def pack_codes(codes: np.ndarray, k_padded: int) -> np.ndarray:
    """Pack codes [..., k] two per byte along the last axis, zero-padded to k_padded
    (even); the even index goes to the low nibble."""
    k = codes.shape[-1]
    pad = np.zeros(codes.shape[:-1] + (k_padded,), dtype=np.uint8)
    pad[..., :k] = codes
    return (pad[..., 0::2] | (pad[..., 1::2] << 4)).astype(np.uint8)


def limb_products(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """The 9 exact limb products P[ia][ib] = D_ia(A) D_ib(B), int64 [3][3][m][n]."""
    da = limb_digits(a).astype(np.int64)
    db = limb_digits(b).astype(np.int64)
    out = np.empty((3, 3, da.shape[1], db.shape[2]), dtype=np.int64)
    for ia in range(3):
        for ib in range(3):
            out[ia, ib] = da[ia] @ db[ib]
    return out


def int8_gemm(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """C = sum_{ia, ib} 13^(ia+ib) P[ia][ib]: the exact int8 product, int64."""
    p = limb_products(a, b)
    c = np.zeros(p.shape[2:], dtype=np.int64)
    for ia in range(3):
        for ib in range(3):
            c += WEIGHTS[ia] * WEIGHTS[ib] * p[ia, ib]
    return c
