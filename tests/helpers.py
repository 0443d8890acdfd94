"""Comparison helpers shared by the GPU parity tests (no method arithmetic here)."""
import numpy as np
import torch

# Tolerances of the parity bar: max per-row relative error (see row_rel_err).
TOL_F32 = 1e-4
TOL_BF16 = 2e-2
# Gradient rows are sums of terms of the typical row size that can cancel to far below it;
# with bf16 features (relative rounding 2^-9 of q' and k', as in the forward) their absolute
# error stays at the typical scale, so rows under GRAD_FLOOR of the median row size are
# held to an absolute bound instead (see grad_row_err).
GRAD_FLOOR = 0.05


def f64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def row_rel_err(got, ref) -> float:
    """Max over rows (last axis = one output row) of ||got - ref||_inf / ||ref||_inf.

    A row whose reference is exactly zero must be exactly zero (error inf otherwise).
    """
    got, ref = f64(got), f64(ref)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    g = got.reshape(-1, got.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    num = np.abs(g - r).max(axis=1)
    den = np.abs(r).max(axis=1)
    zero = den == 0
    if (num[zero] != 0).any():
        return float("inf")
    if (~zero).sum() == 0:
        return 0.0
    return float((num[~zero] / den[~zero]).max())


def grad_row_err(got, ref, floor: float = GRAD_FLOOR) -> float:
    """Max over rows of ||got - ref||_inf / max(||ref_row||_inf, floor * m), m = the median
    of ||ref_row||_inf over the tensor's nonzero rows: the per-row relative error for every
    row at least ``floor`` of the typical row size, an absolute error in units of
    ``floor * m`` below that. A row whose reference is exactly zero must be exactly zero."""
    got, ref = f64(got), f64(ref)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    g = got.reshape(-1, got.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    num = np.abs(g - r).max(axis=1)
    den = np.abs(r).max(axis=1)
    zero = den == 0
    if (num[zero] != 0).any():
        return float("inf")
    if (~zero).sum() == 0:
        return 0.0
    scale = np.maximum(den, floor * np.median(den[~zero]))
    return float((num[~zero] / scale[~zero]).max())


def mat_rel_err(got, ref, mat_dims: int = 2) -> float:
    """Max over leading indices of max|got - ref| / max|ref| over the last ``mat_dims``
    axes (2 for states S [..., d, d], 1 for z [..., d])."""
    got, ref = f64(got), f64(ref)
    lead = got.shape[:got.ndim - mat_dims]
    return row_rel_err(got.reshape(*lead, -1), ref.reshape(*lead, -1))


def sample_rows(L: int, n_random: int, seed: int, chunk: int = 64) -> np.ndarray:
    """Rows that cover chunk boundaries, both ends and random interior positions."""
    r = np.random.default_rng(seed)
    rows = {0, 1, L - 1, L - 2}
    for c in range(chunk, L, max(chunk, (L // 16) // chunk * chunk)):
        rows.update({c - 1, c, c + 1})
    rows.update(r.integers(0, L, size=n_random).tolist())
    return np.array(sorted(x for x in rows if 0 <= x < L))


def scaled_row_err(got, ref, scale) -> float:
    """Max over rows of ||got - ref||_inf / max(||ref_row||_inf, scale_row), ``scale`` one
    value per row (the size of the terms a row is a difference of). A row whose reference and
    scale are both exactly zero must be exactly zero."""
    got, ref = f64(got), f64(ref)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    g = got.reshape(-1, got.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    s = np.asarray(scale, dtype=np.float64).reshape(-1)
    assert s.shape[0] == r.shape[0]
    num = np.abs(g - r).max(axis=1)
    den = np.maximum(np.abs(r).max(axis=1), s)
    zero = den == 0
    if (num[zero] != 0).any():
        return float("inf")
    if (~zero).sum() == 0:
        return 0.0
    return float((num[~zero] / den[~zero]).max())
