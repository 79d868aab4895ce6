"""Lloyd-Max scalar codebook for one coordinate of a randomly rotated unit vector.

Test infrastructure (see ``oracle/__init__``).

What the pages fix
------------------
* P3 "How it works", Stage 1: after the random rotation every coordinate of
  the (normalised) vector follows Beta((d-1)/2, (d-1)/2) on [-1, 1], so the
  optimal centroids can be precomputed analytically.
* P1 "Rotate, then quantize": the same law is close to a normal law with
  mean 0 and variance 1/d; an MSE-optimal scalar quantizer (Lloyd-Max) is
  applied to each coordinate independently.
* P3 "How to implement", item 1: the Lloyd-Max codebook is precomputed per
  head dimension and bit width.

Reading of the law: the Beta law on [-1, 1] is t = 2u - 1 with
u ~ Beta(alpha, alpha), alpha = (d-1)/2, whose density is
f(t) = (1 - t^2)^a / Z with a = (d-3)/2 and Z = B(1/2, a+1).  Its variance
is 1/(2 alpha + 1) = 1/d, which is the P1 statement.

Lloyd-Max (the textbook two conditions): every decision boundary is the
midpoint of its two neighbouring centroids, every centroid is the mean of
the law restricted to its cell.  The law is log-concave for d >= 3, so the
fixed point is unique and the starting point does not matter.
"""

import functools

import numpy as np
from scipy import special


def _a(d):
    return (d - 3) / 2.0


@functools.lru_cache(maxsize=None)
def _norm_const(a):
    """Z = B(1/2, a+1), the integral of (1-t^2)^a over [-1, 1].

    Built by the recurrence B(1/2, x+1) = B(1/2, x) * x / (x + 1/2) from
    a0 = a - floor(a) in [0, 1); a plain product keeps full fp64 accuracy
    where gamma-function ratios of large arguments lose digits.
    """
    n = int(np.floor(a))
    a0 = a - n
    z = special.beta(0.5, a0 + 1.0)
    for k in range(1, n + 1):
        x = a0 + k
        z *= x / (x + 0.5)
    return z


def beta_density(d, t):
    """f(t) = (1-t^2)^((d-3)/2) / B(1/2, (d-1)/2) on [-1, 1] (P3 Stage 1)."""
    a = _a(d)
    t = np.asarray(t, dtype=np.float64)
    z = _norm_const(a)
    return np.where(np.abs(t) < 1.0, np.power(np.clip(1.0 - t * t, 0.0, None), a) / z, 0.0)


def bin_mass(d, t0, t1):
    """P(t0 <= T < t1) for the rotated-coordinate law, via the Beta CDF.

    T = 2U - 1 with U ~ Beta(alpha, alpha): P(T < t) = I_{(1+t)/2}(alpha, alpha).
    In the upper half the survival form is used so that small tail cells do
    not lose digits to cancellation.
    """
    al = (d - 1) / 2.0
    if t0 >= 0.0:
        return float(special.betainc(al, al, (1.0 - t0) / 2.0)
                     - special.betainc(al, al, (1.0 - t1) / 2.0))
    return float(special.betainc(al, al, (1.0 + t1) / 2.0)
                 - special.betainc(al, al, (1.0 + t0) / 2.0))


def bin_first_moment(d, t0, t1):
    """Integral of t f(t) over [t0, t1] in closed form.

    d/dt [-(1-t^2)^(a+1) / (2(a+1))] = t (1-t^2)^a.
    """
    a = _a(d)
    z = _norm_const(a)
    g0 = (1.0 - t0 * t0) ** (a + 1.0)
    g1 = (1.0 - t1 * t1) ** (a + 1.0)
    return float((g0 - g1) / (2.0 * (a + 1.0) * z))


def _edges(bounds):
    return np.concatenate([[-1.0], np.asarray(bounds, dtype=np.float64), [1.0]])


def lloyd_max(d, bits, tol=1e-15, max_iter=200000):
    """Lloyd-Max codebook for the Beta((d-1)/2,(d-1)/2) law on [-1, 1].

    Returns ``(centroids, bounds)``: ``2**bits`` ascending centroids and the
    ``2**bits - 1`` decision boundaries between them, at unit-sphere scale.
    Iterates the two Lloyd conditions (boundaries = midpoints, centroids =
    conditional means) until no centroid moves by ``tol`` or more.

    Starting point: the law's quantiles at (i + 1/2)/L (any start reaches
    the same, unique, fixed point).
    """
    if d < 3:
        raise ValueError("the law is log-concave (unique codebook) only for d >= 3")
    if bits < 1:
        raise ValueError("bits must be >= 1")
    L = 2 ** bits
    al = (d - 1) / 2.0
    c = 2.0 * special.betaincinv(al, al, (np.arange(L) + 0.5) / L) - 1.0
    for _ in range(max_iter):
        t = 0.5 * (c[:-1] + c[1:])
        e = _edges(t)
        cn = np.array([bin_first_moment(d, e[i], e[i + 1]) / bin_mass(d, e[i], e[i + 1])
                       for i in range(L)])
        moved = np.max(np.abs(cn - c))
        c = cn
        if moved < tol:
            break
    t = 0.5 * (c[:-1] + c[1:])
    return c, t


def codebook_mse(d, centroids, bounds):
    """Per-coordinate mean squared error E[(T - c(T))^2] of a codebook.

    Expanding the square cell by cell, E[T^2] + sum_i (c_i^2 P_i - 2 c_i M1_i),
    with E[T^2] = 1/d for this law (P1: variance 1/d), P_i the cell mass and
    M1_i the cell's first moment.  Valid for any centroids, not only at the
    Lloyd fixed point; summing only the centroid terms avoids the cancellation
    of forming every cell's second moment.
    """
    e = _edges(bounds)
    total = 1.0 / d
    for i, ci in enumerate(np.asarray(centroids, dtype=np.float64)):
        m0 = bin_mass(d, e[i], e[i + 1])
        m1 = bin_first_moment(d, e[i], e[i + 1])
        total += ci * (ci * m0 - 2.0 * m1)
    return total


# ------------------------------------------------------- fractional widths
# The pages report quality at 2.5 and 3.5 bits per channel (qiita page,
# "Which bit width is 'lossless'?", first table) without saying how a
# fractional width is formed.  Reading: a fixed split of the rotated
# coordinates -- the first `hi` coordinates use the (b+1)-bit Lloyd-Max
# codebook of the same Beta law, the others the b-bit one (3.5 bits: half
# the coordinates at 4 bits, half at 3).  The rotated coordinates are
# exchangeable (each follows the same law), so which ones carry the extra
# bit does not change the expected distortion, and each group's codebook
# is the MSE-optimal one for its width.

def split_codebook(d, hi, lo_codebook, hi_codebook):
    """Per-coordinate codebook of a split width: rows j < hi hold
    ``hi_codebook`` = (centroids, bounds), rows j >= hi ``lo_codebook``.

    Returns (C [d, L], B [d, L-1]) with L the larger level count; the
    shorter rows are padded (centroids with NaN, never indexed; bounds with
    +inf, never reached)."""
    (c_lo, t_lo), (c_hi, t_hi) = lo_codebook, hi_codebook
    if not 0 <= hi <= d:
        raise ValueError("need 0 <= hi <= d")
    L = max(len(c_lo), len(c_hi))
    C = np.full((d, L), np.nan)
    B = np.full((d, L - 1), np.inf)
    C[:hi, :len(c_hi)] = c_hi
    B[:hi, :len(t_hi)] = t_hi
    C[hi:, :len(c_lo)] = c_lo
    B[hi:, :len(t_lo)] = t_lo
    return C, B


def split_widths(d, bits, hi):
    """Bits of every coordinate of a split width: bits + 1 below hi, bits above."""
    return np.where(np.arange(d) < hi, bits + 1, bits)


def centroid_values(centroids, idx):
    """c[idx]: the centroid of every index.  ``centroids`` is one codebook
    (1-D, shared by every coordinate) or one row per coordinate (2-D,
    ``split_codebook``), in which case coordinate j (the last axis of idx)
    takes row j."""
    c = np.asarray(centroids, dtype=np.float64)
    idx = np.asarray(idx)
    if c.ndim == 1:
        return c[idx]
    return c[np.arange(c.shape[0]), idx]
