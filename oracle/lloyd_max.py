"""Lloyd-Max scalar quantiser for the standard normal distribution.

PolyKV explainer, section 2.B (value quantisation): rotated V coordinates are
mapped to precomputed Lloyd-Max centroids optimised for N(0, 1).  The page
prints no values, so the table is computed here from its definition:

* thresholds are midpoints of neighbouring centroids,
  tau_j = (c_j + c_{j+1}) / 2;
* each centroid is the conditional mean of its cell,
  c_j = (phi(tau_{j-1}) - phi(tau_j)) / (Phi(tau_j) - Phi(tau_{j-1})),
  with tau_{-1} = -inf and tau_{K-1} = +inf, K = 2^bits.

The fixed point is found by Lloyd iteration in double on the positive half
(the density is symmetric, so the table is mirrored and the middle threshold
is exactly 0).  The double values are then rounded to fp32 (nearest-even);
thresholds are computed in double from the double centroids before rounding.
Code j indexes centroids in ascending order (j = 0 is the most negative).

The MSE of a table, D = E[(X - Q(X))^2], has the closed form used in
``mse_closed_form``; tests check it against numerical integration and against
the values published by J. Max, "Quantizing for Minimum Distortion" (1960).
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import ndtr

_SQRT_2PI = math.sqrt(2.0 * math.pi)


def _phi(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    fin = np.isfinite(x)
    out[fin] = np.exp(-0.5 * x[fin] * x[fin]) / _SQRT_2PI
    return out


def _cell_mass_upper(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Phi(b) - Phi(a) for 0 <= a < b <= inf, via upper tails for accuracy."""
    return ndtr(-np.asarray(a, dtype=np.float64)) - ndtr(-np.asarray(b, dtype=np.float64))


def _positive_half(bits: int, tol: float, max_iter: int) -> tuple[np.ndarray, int, float]:
    half = (1 << bits) // 2
    # start from cell quantile midpoints of the positive half
    from scipy.special import ndtri

    c = ndtri(0.5 + (np.arange(half) + 0.5) / (2 * half))
    for it in range(1, max_iter + 1):
        lo = np.concatenate([[0.0], 0.5 * (c[:-1] + c[1:])])
        hi = np.concatenate([lo[1:], [np.inf]])
        c_new = (_phi(lo) - _phi(hi)) / _cell_mass_upper(lo, hi)
        delta = float(np.max(np.abs(c_new - c)))
        c = c_new
        if delta <= tol:
            return c, it, delta
    return c, max_iter, delta


def lloyd_max_normal(bits: int, tol: float = 1e-14, max_iter: int = 200_000):
    """Lloyd-Max centroids and thresholds for N(0, 1) in double.

    Iterates until no centroid moves by more than ``tol`` in one iteration
    (1e-14 by default: about 1e-7 of an fp32 ulp at these magnitudes).
    Returns (centroids[2^bits], thresholds[2^bits - 1]).
    """
    if bits not in (1, 2, 3, 4, 5, 6):
        raise ValueError("bits out of range")
    cpos, _, _ = _positive_half(bits, tol, max_iter)
    cent = np.concatenate([-cpos[::-1], cpos])
    tpos = 0.5 * (cpos[:-1] + cpos[1:])
    thr = np.concatenate([-tpos[::-1], [0.0], tpos])
    return cent, thr


def fixed_point_residual(cent: np.ndarray, thr: np.ndarray) -> float:
    """Max violation of the two Lloyd-Max conditions by a double table."""
    mid = 0.5 * (cent[:-1] + cent[1:])
    lo = np.concatenate([[-np.inf], thr])
    hi = np.concatenate([thr, [np.inf]])
    mass = ndtr(hi) - ndtr(lo)
    cond_mean = (_phi(lo) - _phi(hi)) / mass
    return float(max(np.max(np.abs(mid - thr)), np.max(np.abs(cond_mean - cent))))


def table_f32(bits: int) -> tuple[np.ndarray, np.ndarray]:
    """The fp32 table used by the codec: (centroids, thresholds), nearest-even rounding."""
    cent, thr = lloyd_max_normal(bits)
    return cent.astype(np.float32), thr.astype(np.float32)


def mse_closed_form(cent: np.ndarray, thr: np.ndarray) -> float:
    """E[(X - Q(X))^2] for X ~ N(0, 1) and the quantiser (cent, thr), in double.

    On a cell [a, b] with output c: integral of (x - c)^2 phi(x) dx
    = (1 + c^2)(Phi(b) - Phi(a)) - (b phi(b) - a phi(a)) + 2c (phi(b) - phi(a)).
    """
    cent = np.asarray(cent, dtype=np.float64)
    thr = np.asarray(thr, dtype=np.float64)
    lo = np.concatenate([[-np.inf], thr])
    hi = np.concatenate([thr, [np.inf]])
    mass = ndtr(hi) - ndtr(lo)

    def xphi(x):
        out = np.zeros_like(x)
        fin = np.isfinite(x)
        out[fin] = x[fin] * _phi(x[fin])
        return out

    terms = (1.0 + cent * cent) * mass - (xphi(hi) - xphi(lo)) + 2.0 * cent * (_phi(hi) - _phi(lo))
    return float(np.sum(terms))
