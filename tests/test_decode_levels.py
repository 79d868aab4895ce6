"""Exact float16 levels of a 2-bit codebook (decode's centroid term).

Decode takes the centroid term of 2-bit keys on exact float16 levels: under
one common factor the two magnitudes a > b of the Lloyd-Max codebook
-a, -b, b, a become l_a = Q 2^(E-11) and l_b = P 2^(e-11) l_a / Q with 11-bit
integers P, Q, chosen to make l_b / l_a closest to b / a.  The decode kernels
search Q in [1024, 2047]; this test restates that search on the oracle's
codebooks and pins the precision the kernels rely on (<= 2e-6 relative for
every head dimension, 1.3e-6 at d = 128) and that both levels are float16
numbers.  Host arithmetic only.
"""

import numpy as np
import pytest

import oracle


def best_levels(a, b):
    r = b / a
    best = None
    for Q in range(1024, 2048):
        x = r * Q
        _, e = np.frexp(x)
        P = np.rint(np.ldexp(x, 11 - int(e)))
        err = abs(np.ldexp(P, int(e) - 11) - x) / x
        if best is None or err < best[0]:
            best = (err, Q, int(P), int(e))
    err, Q, P, e = best
    _, E = np.frexp(a)
    la = np.ldexp(float(Q), int(E) - 11)
    lb = np.ldexp(float(P), int(e) + int(E) - 22)
    return err, la, lb


@pytest.mark.parametrize("d", [8, 32, 64, 128, 256, 1024])
def test_two_bit_levels_are_exact_float16_to_2e6(d):
    c, _ = oracle.lloyd_max(d, 2)
    c32 = np.asarray(c, dtype=np.float32).astype(np.float64)
    assert c32[0] == -c32[3] and c32[1] == -c32[2]          # the symmetry the kernels use
    a, b = c32[3], c32[2]
    err, la, lb = best_levels(a, b)
    assert err <= 2e-6
    # both levels are float16 numbers (no rounding when the table is built)
    assert float(np.float16(la)) == la and float(np.float16(lb)) == lb
    # the common factor a / l_a maps them back: a exactly, b within err
    f = a / la
    assert abs(la * f - a) <= 1e-7 * a
    assert abs(lb * f - b) / b <= err * 1.01 + 1e-7
    # l_a lies in a's binade, so the factor is near 1
    assert 0.5 < f < 2.0


def test_d128_error_matches_the_stated_bound():
    c, _ = oracle.lloyd_max(128, 2)
    c32 = np.asarray(c, dtype=np.float32).astype(np.float64)
    err, _, _ = best_levels(c32[3], c32[2])
    assert 1.0e-6 < err < 1.5e-6
