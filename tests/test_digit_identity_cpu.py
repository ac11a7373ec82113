"""Host check of the arithmetic identity behind the on-the-fly GEMV's digit path.

For |a'| <= 2^50 the double t = RN(a 2^e + 2^52 + 0x8808080808080) carries a' = RNE(a 2^e)
in its mantissa; the kernel feeds t's eight bytes to the int8 MFMA after XOR 0x80 on bytes
0..5, against weights 256^j mod m (zero for byte 7), and removes byte 6's bias of 56 with a
per-column constant.  This test rebuilds that byte decomposition with Python's struct and
big integers and checks, for random and boundary a', that the digits are valid int8 values
and that the weighted digit sum minus the bias equals a' modulo every modulus (and equals
a' itself with weights 256^j).  The rounding of the magic add is checked against Python's
round-half-even on ties."""
import random
import struct

import pytest

from oracle import rns

MAGIC = float.fromhex("0x1.8808080808080p+52")


def _digits(t: float):
    raw = bytearray(struct.pack("<d", t))
    for j in range(6):
        raw[j] ^= 0x80
    return [b - 256 if b >= 128 else b for b in raw]


def _values():
    rng = random.Random(7)
    edge = [0, 1, -1, 2**50, -(2**50), 2**50 - 1, -(2**50 - 1), 2**47, -(2**47), 255, -256]
    return edge + [rng.randint(-(2**50), 2**50) for _ in range(3000)]


def test_digits_reconstruct_the_integer():
    for ap in _values():
        t = MAGIC + ap
        assert t == float(2**52 + 0x8808080808080 + ap)   # exact: ulp(t) = 1
        d = _digits(t)
        assert all(-128 <= v <= 127 for v in d) and 52 <= d[6] <= 60
        assert sum(d[j] * 256**j for j in range(6)) + (d[6] - 56) * 2**48 == ap


@pytest.mark.parametrize("r", [20])
def test_weighted_digits_are_congruent(r):
    mods = rns.moduli(r)
    vals = _values()[:600]
    for m in mods:
        w = [pow(256, j, m) for j in range(7)] + [0]
        for ap in vals:
            d = _digits(MAGIC + ap)
            assert (sum(dj * wj for dj, wj in zip(d, w)) - 56 * w[6]) % m == ap % m


def test_magic_add_rounds_half_to_even():
    for x in [0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 7.5, 2.0**49 + 0.5, -(2.0**49) - 1.5,
              3.4999999999999996, 1e-300, -1e-300]:
        assert (MAGIC + x) - MAGIC == round(x)
