"""The wide-dynamic-range configuration: 8192^3 with entries (U(0,1) - 0.5) exp(4 N(0,1))
(seed 3), per-row and per-column power-of-two scaling, r = 16..20.

Sampled outputs (8 rows x 32 columns, the last row and column included) are compared
with the oracle (<= 2 ulp, expected bit-exact) for both scaling rules, and with the
exact rational product of the sampled rows and columns for accuracy: normwise 1e-15 is
reached at r = 18 by the max rule and at r = 16 by the norm rule."""
import numpy as np
import pytest
import torch

import fp64_gemm_emulation_ozk_amd as ozk
import ozk_inputs
from oracle import ozaki2, reference, rns

from gpu_common import announce, assert_within_ulps, to_dev

pytestmark = pytest.mark.gpu

N = 8192


@pytest.fixture(scope="module")
def cfg():
    announce("wide range 8192^3: generating operands")
    a, b = ozk_inputs.gemm_operands(N, N, N, seed=3, dist="phi", phi=4.0)
    rng = np.random.default_rng(2024)
    rows = np.sort(rng.choice(N, 8, replace=False))
    cols = np.sort(rng.choice(N, 32, replace=False))
    rows[-1], cols[-1] = N - 1, N - 1
    exact = reference.exact_matmul(a[rows], b[:, cols])
    da, db = to_dev(a), to_dev(b)
    ws = torch.empty(ozk.ozk_dgemm_workspace_size(N, N, N, 20), dtype=torch.uint8,
                     device=da.device)
    out = torch.empty((N, N), dtype=torch.float64, device=da.device)
    yield {"a": a, "b": b, "rows": rows, "cols": cols, "exact": exact, "da": da, "db": db,
           "ws": ws, "out": out}
    del da, db, ws, out
    torch.cuda.empty_cache()


def _sample(cfg, c: torch.Tensor) -> np.ndarray:
    r_i = torch.as_tensor(cfg["rows"], device=c.device)
    c_i = torch.as_tensor(cfg["cols"], device=c.device)
    return c[r_i][:, c_i].cpu().numpy()


def _run(cfg, r: int, rule: str) -> np.ndarray:
    ozk.ozk_dgemm_ex(cfg["da"], cfg["db"], r, rule, out=cfg["out"], workspace=cfg["ws"])
    torch.cuda.synchronize()
    return _sample(cfg, cfg["out"])


@pytest.mark.parametrize("r", [16, 17, 18, 19, 20])
def test_wide_range_max_rule_matches_oracle(cfg, r):
    announce(f"wide range 8192^3 max rule r={r}")
    got = _run(cfg, r, "max")
    want = ozaki2.dgemm(cfg["a"], cfg["b"], r, rows=cfg["rows"], cols=cfg["cols"])
    assert assert_within_ulps(got, want, 2) == 0


@pytest.mark.parametrize("r", [16, 17, 18, 19, 20])
def test_wide_range_norm_rule_matches_oracle(cfg, r):
    announce(f"wide range 8192^3 norm rule r={r}")
    got = _run(cfg, r, "norm")
    _, e_all = ozk.ozk_deconstruct_ex(cfg["da"], 0, r, "norm", k_budget=N)
    _, f_all = ozk.ozk_deconstruct_ex(cfg["db"], 1, r, "norm", k_budget=N)
    torch.cuda.synchronize()
    e = e_all.cpu().numpy().astype(np.int64)[cfg["rows"]]
    f = f_all.cpu().numpy().astype(np.int64)[cfg["cols"]]
    aa, ab = rns.scaling_bits_norm(r, N)
    np.testing.assert_array_equal(
        e, ozaki2.scale_exponents_norm(cfg["a"][cfg["rows"]], aa, 0))
    np.testing.assert_array_equal(
        f, ozaki2.scale_exponents_norm(cfg["b"][:, cfg["cols"]], ab, 1))
    want = ozaki2.dgemm(cfg["a"], cfg["b"], r, rows=cfg["rows"], cols=cfg["cols"],
                        exps=(e, f))
    assert assert_within_ulps(got, want, 2) == 0


def _normwise(got: np.ndarray, exact: np.ndarray) -> float:
    return float(np.linalg.norm(got - exact) / np.linalg.norm(exact))


def test_wide_range_accuracy_by_rule(cfg):
    """Normwise error of the sampled block against the exact product: <= 1e-15 at r = 18
    (max rule) and at r = 16 (norm rule); two fewer moduli for the same accuracy."""
    announce("wide range 8192^3 accuracy")
    ex = cfg["exact"]
    err_max_18 = _normwise(_run(cfg, 18, "max"), ex)
    err_max_16 = _normwise(_run(cfg, 16, "max"), ex)
    err_norm_16 = _normwise(_run(cfg, 16, "norm"), ex)
    assert err_max_18 <= 1e-15
    assert err_norm_16 <= 1e-15
    assert err_max_16 > 1e-15          # the max rule needs the two extra moduli here
    assert err_norm_16 < err_max_16 / 16
