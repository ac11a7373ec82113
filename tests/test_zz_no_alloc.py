"""GPU checks of the allocation-free GEMV entry point, ozk_dgemv_noalloc, through the C ABI.

Its scratch is the library's fixed device array instead of a workspace.  Each case calls
it twice in a row on one stream, the second time with a smaller input, so that the
second call runs over what the first left in the shared array; both results must equal
ozk_dgemv's (same kernels: bit for bit) and the oracle's (<= 2 ulp, expected bit-exact).
Covered: the base-256 digits path, the on-the-fly residue path (narrow and wide
arithmetic, two passes of moduli) and stored planes."""
import numpy as np
import pytest
import torch

import fp64_gemm_emulation_ozk_amd as ozk
import ozk_inputs
from oracle import ozaki2

from gpu_common import announce, assert_within_ulps, to_dev

pytestmark = pytest.mark.gpu


def _both(a, x, r, mode):
    da, dx = to_dev(a), to_dev(x)
    planes = exps = None
    if mode == 1:
        planes, exps = ozk.ozk_deconstruct(da, 0, r, k_budget=a.shape[1])
    out = torch.full((a.shape[0], x.shape[1]), np.nan, dtype=torch.float64, device=dx.device)
    ozk.ozk_dgemv_noalloc(da if mode == 0 else None, dx, r, mode=mode, a_planes=planes,
                          a_exps=exps, out=out)
    ref = ozk.ozk_dgemv(da if mode == 0 else None, dx, r, mode=mode, a_planes=planes,
                        a_exps=exps)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ref.cpu().numpy()


# (m, k, nrhs, r, mode) for the first call, then the smaller second call
CASES = [
    ((700, 3000, 8, 14, 0), (130, 900, 3, 14, 0)),      # digits path
    ((600, 2000, 32, 14, 0), (70, 500, 20, 12, 0)),     # residue path, narrow
    ((300, 700, 32, 20, 0), (65, 300, 17, 18, 0)),      # residue path, wide, two passes
    ((800, 4100, 32, 16, 1), (100, 1000, 5, 16, 1)),    # stored planes
]


@pytest.mark.parametrize("first,second", CASES)
def test_noalloc_equals_dgemv_twice(first, second):
    for i, (m, k, nrhs, r, mode) in enumerate((first, second)):
        announce(f"dgemv_noalloc call {i + 1}: m={m} k={k} nrhs={nrhs} r={r} mode={mode}")
        a, x = ozk_inputs.gemv_operands(m, k, nrhs, seed=m + k + nrhs + i)
        got, ref = _both(a, x, r, mode)
        np.testing.assert_array_equal(got.view(np.int64), ref.view(np.int64))
        assert assert_within_ulps(got, ozaki2.dgemv(a, x, r), 2) == 0


def test_noalloc_rejects_a_request_beyond_its_scratch():
    """32768 x 32768 with 16 columns on the fly needs about 98 MiB of scratch: the call
    returns OZK_ENOSCRATCH before touching any memory (nothing is enqueued)."""
    announce("dgemv_noalloc oversize request")
    need = ozk.ozk_dgemv_workspace_size(32768, 32768, 16, 14, 0)
    assert need > ozk.OZK_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((32768, 16), dtype=torch.float64, device="cuda")
    a = torch.zeros((32768, 32768), dtype=torch.float64, device="cuda")
    out = torch.zeros((32768, 16), dtype=torch.float64, device="cuda")
    st = ozk.library().ozk_dgemv_noalloc(32768, 32768, 16, a.data_ptr(), 32768, None, 0, 0, None,
                                         x.data_ptr(), 16, out.data_ptr(), 16, 14, 0, None)
    assert st == -6
    torch.cuda.synchronize()
    assert not torch.any(out)
