"""The GPU tests' comparison gate itself (CPU only): what it must catch and what
it must let through."""
import numpy as np
import pytest

import parity
from parity import FWD_TOL, GRAD_TOL, assert_close, elem_err, rel_err


@pytest.fixture(autouse=True)
def _keep_results_clean():
    """These checks fail on purpose: keep them out of the session's headroom table."""
    n = len(parity.RESULTS)
    yield
    del parity.RESULTS[n:]


def _ref(seed=0, shape=(512, 96)):
    return np.random.default_rng(seed).standard_normal(shape)


def test_rounding_noise_passes_both_variants():
    r = _ref()
    for prec, tol in (("fp32", GRAD_TOL["fp32"]), ("bf16", GRAD_TOL["bf16"])):
        noise = {"fp32": 2.0 ** -23, "bf16": 2.0 ** -8}[prec]
        x = r * (1 + noise * np.random.default_rng(1).standard_normal(r.shape))
        assert_close(x, r, tol, prec)


@pytest.mark.parametrize("tol", [FWD_TOL["fp32"], GRAD_TOL["bf16"]])
def test_one_wrong_row_fails(tol):
    r = _ref(shape=(8192, 64))
    x = r.copy()
    x[4097] = 0.0                                   # one of 8192 rows lost: L2 error 1.1e-2
    assert rel_err(x, r) < 2e-2
    with pytest.raises(AssertionError):
        assert_close(x, r, tol)


def test_wrong_ragged_tile_fails_in_bf16():
    r = _ref(shape=(1000, 1000))
    x = r.copy()
    x[996:, 968:] = x[996:, 968:][::-1]             # the last 4 x 32 corner permuted
    assert rel_err(x, r) < 2e-2
    with pytest.raises(AssertionError):
        assert_close(x, r, GRAD_TOL["bf16"])


def test_large_rows_are_judged_at_their_own_scale():
    # a few rows 1e4 x larger than the rest (a tied embedding's gradient): errors of 4% of
    # such a row's RMS are rounding at that row's scale, which the tensor-wide RMS (0.07 of
    # the large rows') would call 7% of the gate; a tiny row off by 1% of the tensor RMS passes
    r = _ref(shape=(1000, 32)) * 1e-4
    r[:5] *= 1e4
    x = r.copy()
    rowrms = np.sqrt(np.mean(r[:5] ** 2, axis=1, keepdims=True))
    x[:5, ::8] += 0.04 * rowrms * np.sign(np.random.default_rng(2).standard_normal((5, 4)))
    x[500] += 0.01 * np.sqrt(np.mean(r ** 2))
    assert_close(x, r, GRAD_TOL["bf16"])
    # but a large row permuted is caught
    x = r.copy()
    x[3] = x[3][::-1]
    with pytest.raises(AssertionError):
        assert_close(x, r, GRAD_TOL["bf16"])


def test_zero_reference_tensor_must_be_matched_closely():
    r = np.zeros((64, 16))
    x = r.copy()
    x[10, 3] = 1e-3
    with pytest.raises(AssertionError):
        assert_close(x, r, GRAD_TOL["bf16"])
