"""GPU parity of the exact INT8 x INT8 product through base-13 FP4 limbs.

Limb planes (packed e2m1 codes), the 9 digit products and the weighted int32 result
must all be bit-exact against the oracle / the exact integer product."""
import numpy as np
import pytest
import torch

import fp64_gemm_emulation_ozk_amd as ozk
import ozk_inputs
from oracle import fp4limb

from gpu_common import announce, to_dev

pytestmark = pytest.mark.gpu


def _kpad(k):
    return (k + 63) // 64 * 64


@pytest.mark.parametrize("rows,cols,axis", [(37, 100, 0), (5, 64, 0), (100, 37, 1), (300, 130, 1),
                                            (1, 1, 0), (1, 1, 1),
                                            # 16-byte rows: whole chunks by vector loads,
                                            # a ragged last chunk byte by byte
                                            (9, 208, 0), (33, 512, 0),
                                            # columns by 4-byte loads (rows a multiple of 4)
                                            (70, 64, 1), (45, 260, 1)])
def test_pack_bit_exact(rows, cols, axis):
    announce(f"fp4 pack rows={rows} cols={cols} axis={axis}")
    rng = np.random.default_rng(rows * 3 + cols)
    x = ozk_inputs.int8_matrix(rng, (rows, cols))
    x.flat[0] = -128
    x.flat[-1] = 127
    got = ozk.ozk_fp4limb_pack(to_dev(x), axis).cpu().numpy()
    src = x if axis == 0 else x.T
    kdim = src.shape[1]
    want = fp4limb.pack_codes(fp4limb.limb_codes(src), _kpad(kdim))
    np.testing.assert_array_equal(got, want)


def test_pack_all_int8_values():
    announce("fp4 pack all 256 values")
    x = np.arange(-128, 128, dtype=np.int8).reshape(2, 128)
    got = ozk.ozk_fp4limb_pack(to_dev(x), 0).cpu().numpy()
    want = fp4limb.pack_codes(fp4limb.limb_codes(x), 128)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("m,n,k", [(33, 29, 70), (64, 96, 256), (130, 70, 1000)])
def test_limb_products_bit_exact(m, n, k):
    announce(f"fp4 9 products m={m} n={n} k={k}")
    a, b = ozk_inputs.int8_operands(m, n, k, seed=m + n + k)
    pa = ozk.ozk_fp4limb_pack(to_dev(a), 0)
    pb = ozk.ozk_fp4limb_pack(to_dev(b), 1)
    got = ozk.ozk_fp4limb_products(pa, pb).cpu().numpy().reshape(3, 3, m, n)
    want = fp4limb.limb_products(a, b)
    np.testing.assert_array_equal(got.astype(np.int64), want)


def _exact(a, b):
    return a.astype(np.int64) @ b.astype(np.int64)


@pytest.mark.parametrize("m,n,k", [(1, 1, 1), (33, 29, 70), (128, 128, 64), (300, 257, 129),
                                   (257, 520, 1000), (64, 40, 8192)])
def test_int8gemm_fp4limb_exact(m, n, k):
    announce(f"fp4 int8gemm m={m} n={n} k={k}")
    a, b = ozk_inputs.int8_operands(m, n, k, seed=7 * m + n + k)
    got = ozk.ozk_int8gemm_fp4limb(to_dev(a), to_dev(b)).cpu().numpy()
    np.testing.assert_array_equal(got.astype(np.int64), _exact(a, b))


@pytest.mark.parametrize("va,vb", [(-128, -128), (127, -128), (122, 122), (-122, 121)])
def test_int8gemm_fp4limb_accumulator_bound(va, vb):
    """Constant operands with K = 131071 (the largest exact K): every digit product has
    its maximal magnitude, so the fp32 partial sums climb to just below 2^24."""
    k = 131071
    announce(f"fp4 int8gemm bound k={k} va={va} vb={vb}")
    a = np.full((40, k), va, dtype=np.int8)
    b = np.full((k, 36), vb, dtype=np.int8)
    a[3, 5] = 0
    got = ozk.ozk_int8gemm_fp4limb(to_dev(a), to_dev(b)).cpu().numpy()
    np.testing.assert_array_equal(got.astype(np.int64), _exact(a, b))


def test_int8gemm_fp4limb_strided():
    announce("fp4 int8gemm strided")
    a, b = ozk_inputs.int8_operands(50, 40, 77, seed=4)
    abig = np.zeros((50, 96), np.int8)
    abig[:, :77] = a
    bbig = np.zeros((77, 48), np.int8)
    bbig[:, :40] = b
    out = torch.full((50, 44), 9, dtype=torch.int32, device="cuda")
    ozk.ozk_int8gemm_fp4limb(to_dev(abig)[:, :77], to_dev(bbig)[:, :40], out=out[:, :40])
    got = out.cpu().numpy()
    assert np.all(got[:, 40:] == 9)
    np.testing.assert_array_equal(got[:, :40].astype(np.int64), _exact(a, b))


def test_int8gemm_fp4limb_8192_full():
    """The 8192^3 configuration (int8 uniform in [-128, 127], seed 5): every one of the
    8192^2 outputs against the exact product, computed on the host in float64 BLAS, which
    is exact here (every partial sum is an integer of magnitude <= 8192 * 2^14 = 2^27 <
    2^53, whatever order the library sums in); a second call gives the same bits."""
    announce("fp4 int8gemm 8192^3 full output")
    a, b = ozk_inputs.int8_operands(8192, 8192, 8192, seed=5)
    got = ozk.ozk_int8gemm_fp4limb(to_dev(a), to_dev(b))
    again = ozk.ozk_int8gemm_fp4limb(to_dev(a), to_dev(b))
    torch.cuda.synchronize()
    assert torch.equal(got, again)
    got = got.cpu().numpy()
    want = a.astype(np.float64) @ b.astype(np.float64)
    assert np.abs(want).max() <= 8192 * 2**14
    np.testing.assert_array_equal(got, want.astype(np.int32))
