"""Online quantization of key and value vectors.

Test infrastructure (see ``oracle/__init__``).

Steps, in the pages' order:

1. (P3 Stage 1, PolarQuant bullet list, first and last items) normalise the
   vector and keep its norm; rotate it (``rotation``); map every rotated
   coordinate to a few bits with the Lloyd-Max quantizer for the Beta law.
2. (P3 Stage 2; P1 "One more stage so attention doesn't break") keys only:
   take the residual the MSE stage leaves and apply a 1-bit quantized
   Johnson-Lindenstrauss transform to it -- a random projection followed by
   the sign -- so that inner products with the key become unbiased.

Readings (the pages are silent on these):

* index of a coordinate = number of decision boundaries at or below it, so
  a value equal to a boundary goes to the upper cell; this is the nearest
  centroid (ties to the larger index).
* the residual and the sketch live in the rotated domain, at unit-sphere
  scale: r = y/||x|| - c[idx], z = S r (S: m x d, iid N(0,1), an input).
  The sign bit is 1 for z >= 0 and 0 otherwise (P3 Stage 2 garbles the
  two signs; they are read as +1 / -1).
* stored norms: ||x|| and ||x|| * ||r|| (the residual norm at the input's
  scale).
* a zero vector gets norm 0, the index of the cell just above 0
  (L/2), a zero residual and all sign bits 1; it contributes nothing.

``centroids`` / ``bounds`` are one codebook shared by every coordinate, or
one row per coordinate (a fractional width, ``codebook.split_codebook``).
"""

import numpy as np

from .codebook import centroid_values


def _rotate_normalise(X, Pi):
    X = np.asarray(X, dtype=np.float64)
    Pi = np.asarray(Pi, dtype=np.float64)
    norm = np.sqrt(np.sum(X * X, axis=-1))
    Y = X @ Pi.T                       # y = Pi x for every row
    safe = np.where(norm > 0.0, norm, 1.0)
    yhat = Y / safe[..., None]
    return norm, yhat


def _indices(yhat, bounds, zero_mask):
    bounds = np.asarray(bounds, dtype=np.float64)
    idx = np.zeros(yhat.shape, dtype=np.int64)
    if bounds.ndim == 1:
        for t in bounds:               # count of boundaries at or below y
            idx += (yhat >= t)
        L = bounds.size + 1
        idx[zero_mask] = L // 2
        return idx
    # one row of boundaries per coordinate (a split width; padding is +inf)
    for i in range(bounds.shape[1]):
        idx += (yhat >= bounds[:, i])
    L = np.sum(np.isfinite(bounds), axis=1) + 1      # levels of each coordinate
    idx[zero_mask] = (L // 2)[None, :].repeat(int(np.sum(zero_mask)), axis=0)
    return idx


def residual_and_sketch(yhat, idx, centroids, S, norm):
    """Residual r = yhat - c[idx], its stored norm ||x||*||r||, the sketch
    z = S r and the sign bits (z >= 0).  Zero vectors give r = 0, z = 0."""
    S = np.asarray(S, dtype=np.float64)
    zero = np.asarray(norm) == 0.0
    r = yhat - centroid_values(centroids, idx)
    r[zero] = 0.0
    rho = np.sqrt(np.sum(r * r, axis=-1))
    z = r @ S.T
    return dict(rhat=r, rnorm=np.asarray(norm) * rho, z=z, signs=(z >= 0.0))


def quantize_values(X, Pi, centroids, bounds):
    """MSE stage only: returns dict(idx, norm, yhat)."""
    norm, yhat = _rotate_normalise(X, Pi)
    idx = _indices(yhat, bounds, norm == 0.0)
    return dict(idx=idx, norm=norm, yhat=yhat)


def quantize_keys(X, Pi, S, centroids, bounds):
    """MSE stage plus the 1-bit sketch of the residual.

    Returns dict(idx, norm, yhat, rhat, rnorm, z, signs).
    """
    out = quantize_values(X, Pi, centroids, bounds)
    out.update(residual_and_sketch(out["yhat"], out["idx"], centroids, S, out["norm"]))
    return out
