"""Helpers shared by the GPU parity tests (comparison and ulp arithmetic only)."""
import sys

import numpy as np
import torch


def device():
    return torch.device("cuda:0")


def to_dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(device())


def announce(msg: str) -> None:
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def ulp(x: np.ndarray) -> np.ndarray:
    """ulp(x) = 2^(max(ilogb|x|, -1022) - 52); 2^-1074 for zero."""
    ax = np.abs(x)
    _, ex = np.frexp(np.where(ax > 0, ax, 1.0))
    e = np.where(ax > 0, ex - 1, -1022)
    return np.ldexp(1.0, np.maximum(e, -1022) - 52)


def assert_within_ulps(got: np.ndarray, want: np.ndarray, max_ulps: int = 2) -> int:
    """|got - want| <= max_ulps * ulp(want) elementwise; NaN must match NaN.  Returns
    the number of entries that are not bitwise equal."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape
    nan_w = np.isnan(want)
    np.testing.assert_array_equal(np.isnan(got), nan_w)
    g, w = got[~nan_w], want[~nan_w]
    inf_w = np.isinf(w)
    np.testing.assert_array_equal(g[inf_w], w[inf_w])
    g, w = g[~inf_w], w[~inf_w]
    err = np.abs(g - w)
    lim = max_ulps * ulp(w)
    bad = err > lim
    assert not np.any(bad), (f"{int(bad.sum())} entries beyond {max_ulps} ulp; worst "
                             f"{float(np.max(err / lim)) * max_ulps:.3g} ulp")
    return int(np.sum(got.view(np.int64) != want.view(np.int64)))
