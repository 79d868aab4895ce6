"""Pins of the oracle's Lloyd-Max codebook against things other than itself.

* conditional means and MSE by adaptive quadrature of scipy's Beta pdf
  (independent of the oracle's incomplete-beta / closed-form moments);
* the 1-bit closed form E|T|;
* the large-d limit against the textbook Gaussian Lloyd-Max table;
* the pages' 2.7x distortion constant and 0.983 cosine at 3 bits.
"""

import json
import math
import os

import numpy as np
import pytest
from scipy import integrate, stats

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def law_pdf(d):
    """Density of t = 2u - 1, u ~ Beta((d-1)/2, (d-1)/2), from scipy.stats."""
    al = (d - 1) / 2.0
    b = stats.beta(al, al)
    return lambda t: 0.5 * b.pdf((1.0 + t) / 2.0)


def quad(f, a, b, pts=None):
    v, err = integrate.quad(f, a, b, epsabs=1e-16, epsrel=1e-14, limit=400, points=pts)
    return v


@pytest.mark.parametrize("d", [8, 128])
def test_density_normalised_and_variance(d):
    f = law_pdf(d)
    assert abs(quad(lambda t: oracle.beta_density(d, t), -1, 1, [0.0]) - 1.0) < 1e-12
    # the oracle's density equals the Beta pdf after the change of variable
    ts = np.linspace(-0.99, 0.99, 41)
    assert np.allclose(oracle.beta_density(d, ts), [f(t) for t in ts], rtol=1e-11, atol=1e-300)
    # P1: variance 1/d
    assert abs(quad(lambda t: t * t * f(t), -1, 1, [0.0]) - 1.0 / d) < 1e-13


@pytest.mark.parametrize("d,bits", [(8, 1), (8, 2), (8, 3), (128, 1), (128, 2), (128, 3), (128, 4)])
def test_lloyd_fixed_point_against_quadrature(d, bits):
    c, t = oracle.lloyd_max(d, bits)
    L = 2 ** bits
    assert c.shape == (L,) and t.shape == (L - 1,)
    assert np.all(np.diff(c) > 0)
    # boundaries are midpoints
    assert np.max(np.abs(t - 0.5 * (c[:-1] + c[1:]))) <= 1e-15
    # centroids are conditional means, checked by independent quadrature
    f = law_pdf(d)
    e = np.concatenate([[-1.0], t, [1.0]])
    for i in range(L):
        m0 = quad(f, e[i], e[i + 1])
        m1 = quad(lambda x: x * f(x), e[i], e[i + 1])
        assert abs(c[i] - m1 / m0) <= 1e-13, (i, c[i], m1 / m0)
    # symmetric law -> symmetric codebook
    assert np.max(np.abs(c + c[::-1])) <= 1e-14


@pytest.mark.parametrize("d,bits", [(8, 2), (128, 2), (128, 3), (128, 4)])
def test_mse_against_quadrature(d, bits):
    c, t = oracle.lloyd_max(d, bits)
    f = law_pdf(d)
    e = np.concatenate([[-1.0], t, [1.0]])
    ref = sum(quad(lambda x, ci=ci: (x - ci) ** 2 * f(x), e[i], e[i + 1]) for i, ci in enumerate(c))
    D = oracle.codebook_mse(d, c, t)
    assert abs(D - ref) <= 1e-12 * ref
    # at the fixed point D = 1/d - sum c_i^2 P_i
    P = np.array([quad(f, e[i], e[i + 1]) for i in range(len(c))])
    assert abs(D - (1.0 / d - np.sum(c * c * P))) <= 1e-12 * D


def _one_bit_level(d):
    # E|T| = Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2)); for d = 2k this is
    # 4^k k! (k-1)! / ((2k)! pi), evaluated exactly in rationals.
    from fractions import Fraction
    k = d // 2
    r = Fraction(4 ** k * math.factorial(k) * math.factorial(k - 1), math.factorial(2 * k))
    return float(r) / math.pi


@pytest.mark.parametrize("d", [8, 128, 1024])
def test_one_bit_closed_form(d):
    ref = _one_bit_level(d)
    c, t = oracle.lloyd_max(d, 1)
    assert abs(c[1] - ref) < 4e-16 * 1 + 1e-15 * ref and abs(c[0] + ref) < 1e-15
    assert abs(t[0]) < 1e-16
    assert abs(oracle.codebook_mse(d, c, t) - (1.0 / d - ref * ref)) < 1e-15


def test_known_values_d128_d8():
    # closed form numbers derived above, printed to 7 digits
    assert abs(oracle.lloyd_max(128, 1)[0][1] - 0.0706616) < 1e-7
    assert abs(oracle.lloyd_max(8, 1)[0][1] - 0.2910262) < 1e-7


def test_gaussian_limit_matches_textbook_table():
    g = json.load(open(os.path.join(GOLDEN, "gaussian_lloyd_max.json")))
    d = 2 ** 14
    for b in (1, 2, 3, 4):
        c, t = oracle.lloyd_max(d, b)
        pos = np.sqrt(d) * c[len(c) // 2:]
        ref = np.array(g["levels"][str(b)])
        assert np.allclose(pos, ref, rtol=2e-3, atol=6e-4), (b, pos, ref)
        dD = d * oracle.codebook_mse(d, c, t)
        assert abs(dD - g["mse"][str(b)]) <= 2e-3 * g["mse"][str(b)], (b, dD)


def test_distortion_constant_from_pages():
    # d * D * 4^b stays under sqrt(3) pi / 2 ~ 2.72 (the pages' "about 2.7x"
    # of the 4^-b lower bound) and increases with b.
    fig = json.load(open(os.path.join(GOLDEN, "page_figures.json")))
    bound = math.sqrt(3) * math.pi / 2
    assert abs(bound - fig["distortion_over_lower_bound"]["value"]) < 0.05
    for d in (8, 128):
        r = []
        for b in (1, 2, 3, 4):
            c, t = oracle.lloyd_max(d, b)
            r.append(d * oracle.codebook_mse(d, c, t) * 4 ** b)
        assert all(x < bound for x in r)
        assert all(r[i] < r[i + 1] for i in range(3))


def test_cosine_at_three_bits_matches_page():
    fig = json.load(open(os.path.join(GOLDEN, "page_figures.json")))
    c, t = oracle.lloyd_max(128, 3)
    cos = math.sqrt(1.0 - 128 * oracle.codebook_mse(128, c, t))
    assert round(cos, 3) == fig["cosine_3bit"]["value"]
