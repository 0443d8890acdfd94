"""The comparison helpers of the parity tests (host logic)."""
import numpy as np

from helpers import GRAD_FLOOR, grad_row_err, row_rel_err


def test_grad_row_err_is_row_relative_above_the_floor():
    r = np.random.default_rng(1)
    ref = r.normal(size=(50, 8))
    got = ref * (1 + 1e-3 * r.normal(size=ref.shape))
    assert np.isclose(grad_row_err(got, ref), row_rel_err(got, ref))


def test_grad_row_err_floors_small_rows():
    r = np.random.default_rng(2)
    ref = r.normal(size=(51, 8))
    ref[7] *= 1e-4                                  # a row far below the median size
    got = ref.copy()
    got[7] += 1e-6                                  # relative 1e-2..1e-1 of the row itself
    m = np.median(np.abs(ref).max(axis=1))
    assert row_rel_err(got, ref) > 1e-3
    assert np.isclose(grad_row_err(got, ref), 1e-6 / (GRAD_FLOOR * m))
    got[3] = 0.0                                    # a real error in a typical row still counts
    assert grad_row_err(got, ref) > 0.5


def test_grad_row_err_zero_rows_must_be_zero():
    ref = np.zeros((3, 4))
    ref[0] = 1.0
    got = ref.copy()
    assert grad_row_err(got, ref) == 0.0
    got[2, 1] = 1e-30
    assert grad_row_err(got, ref) == float("inf")
