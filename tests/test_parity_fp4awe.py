"""GPU parity of the exact INT8 x INT8 product in 6 FP4 plane products (weights 1, 29,
37; limb and pairwise-sum planes).

Packed planes, the 6 plane products and the weighted int32 result must all be bit-exact
against the oracle (oracle/fp4awe.py) and the exact integer product."""
import numpy as np
import pytest
import torch

import fp64_gemm_emulation_ozk_amd as ozk
import ozk_inputs
from oracle import fp4awe

from gpu_common import announce, to_dev

pytestmark = pytest.mark.gpu


def _kpad(k):
    return (k + 63) // 64 * 64


@pytest.mark.parametrize("rows,cols,axis", [(37, 100, 0), (5, 64, 0), (100, 37, 1),
                                            (300, 130, 1), (1, 1, 0), (1, 1, 1),
                                            (9, 208, 0), (33, 512, 0), (70, 64, 1),
                                            (45, 260, 1)])
def test_pack_bit_exact(rows, cols, axis):
    announce(f"fp4awe pack rows={rows} cols={cols} axis={axis}")
    rng = np.random.default_rng(rows * 5 + cols)
    x = ozk_inputs.int8_matrix(rng, (rows, cols))
    x.flat[0] = -128
    x.flat[-1] = 127
    got = ozk.ozk_fp4awe_pack(to_dev(x), axis).cpu().numpy()
    src = x if axis == 0 else x.T
    want = fp4awe.pack_lines(src, _kpad(src.shape[1]))
    np.testing.assert_array_equal(got, want)


def test_pack_every_int8_value():
    announce("fp4awe pack all 256 values")
    x = np.arange(-128, 128, dtype=np.int8).reshape(2, 128)
    got = ozk.ozk_fp4awe_pack(to_dev(x), 0).cpu().numpy()
    np.testing.assert_array_equal(got, fp4awe.pack_lines(x, 128))


@pytest.mark.parametrize("m,n,k", [(33, 29, 70), (64, 96, 256), (130, 70, 1000), (1, 1, 1)])
def test_plane_products_bit_exact(m, n, k):
    announce(f"fp4awe 6 products m={m} n={n} k={k}")
    a, b = ozk_inputs.int8_operands(m, n, k, seed=m + 2 * n + k)
    pa = ozk.ozk_fp4awe_pack(to_dev(a), 0)
    pb = ozk.ozk_fp4awe_pack(to_dev(b), 1)
    got = ozk.ozk_fp4awe_products(pa, pb, k).cpu().numpy()
    np.testing.assert_array_equal(got.astype(np.int64), fp4awe.plane_products(a, b))


def _exact(a, b):
    return a.astype(np.int64) @ b.astype(np.int64)


# tiles of 128 x 128: one partial tile, several tiles with ragged edges, K not a multiple
# of 64, one K step, more steps than the 3-stage ring, odd and even step counts
@pytest.mark.parametrize("m,n,k", [(1, 1, 1), (33, 29, 70), (128, 128, 64), (300, 257, 129),
                                   (257, 520, 1000), (64, 40, 8192), (129, 130, 192),
                                   (400, 384, 3 * 64)])
def test_int8gemm_fp4awe_exact(m, n, k):
    announce(f"fp4awe int8gemm m={m} n={n} k={k}")
    a, b = ozk_inputs.int8_operands(m, n, k, seed=11 * m + n + k)
    got = ozk.ozk_int8gemm_fp4awe(to_dev(a), to_dev(b)).cpu().numpy()
    np.testing.assert_array_equal(got.astype(np.int64), _exact(a, b))


def _largest_plane_value():
    """The int8 value whose six plane values have the largest sum of magnitudes."""
    tab = fp4awe.limb_table()
    return max(range(-128, 128), key=lambda x: sum(abs(v) for v in fp4awe.plane_values(tab[x])))


@pytest.mark.parametrize("va,vb", [(-128, -128), (127, -128), ("big", "big"), ("big", -128)])
def test_int8gemm_fp4awe_accumulator_bound(va, vb):
    """Constant operands with K = 131071 (the largest K): every plane product sums K equal
    terms of up to 36 in magnitude, 4.7 M, still an integer below 2^24 in fp32."""
    big = _largest_plane_value()
    va = big if va == "big" else va
    vb = big if vb == "big" else vb
    k = 131071
    announce(f"fp4awe int8gemm bound k={k} va={va} vb={vb}")
    a = np.full((40, k), va, dtype=np.int8)
    b = np.full((k, 36), vb, dtype=np.int8)
    a[3, 5] = 0
    got = ozk.ozk_int8gemm_fp4awe(to_dev(a), to_dev(b)).cpu().numpy()
    np.testing.assert_array_equal(got.astype(np.int64), _exact(a, b))


def test_int8gemm_fp4awe_strided():
    announce("fp4awe int8gemm strided")
    a, b = ozk_inputs.int8_operands(50, 40, 77, seed=4)
    abig = np.zeros((50, 96), np.int8)
    abig[:, :77] = a
    bbig = np.zeros((77, 48), np.int8)
    bbig[:, :40] = b
    out = torch.full((50, 44), 9, dtype=torch.int32, device="cuda")
    ozk.ozk_int8gemm_fp4awe(to_dev(abig)[:, :77], to_dev(bbig)[:, :40], out=out[:, :40])
    got = out.cpu().numpy()
    assert np.all(got[:, 40:] == 9)
    np.testing.assert_array_equal(got[:, :40].astype(np.int64), _exact(a, b))


def test_int8gemm_fp4awe_equals_nine_product_engine():
    announce("fp4awe equals the 9-product engine")
    a, b = ozk_inputs.int8_operands(700, 650, 2000, seed=21)
    da, db = to_dev(a), to_dev(b)
    six = ozk.ozk_int8gemm_fp4awe(da, db)
    nine = ozk.ozk_int8gemm_fp4limb(da, db)
    torch.cuda.synchronize()
    assert torch.equal(six, nine)


def test_int8gemm_fp4awe_8192_full():
    """The 8192^3 configuration (int8 uniform in [-128, 127], seed 5): every output against
    the exact product in float64 BLAS on the host (exact: |partial sums| <= 2^27 < 2^53);
    a second call gives the same bits."""
    announce("fp4awe int8gemm 8192^3 full output")
    a, b = ozk_inputs.int8_operands(8192, 8192, 8192, seed=5)
    da, db = to_dev(a), to_dev(b)
    got = ozk.ozk_int8gemm_fp4awe(da, db)
    again = ozk.ozk_int8gemm_fp4awe(da, db)
    torch.cuda.synchronize()
    assert torch.equal(got, again)
    want = a.astype(np.float64) @ b.astype(np.float64)
    np.testing.assert_array_equal(got.cpu().numpy(), want.astype(np.int32))
