"""Data-independent random orthogonal rotation.

Test infrastructure (see ``oracle/__init__``).

P3 "How it works", Stage 1: every KV vector goes through a random
orthogonal transform obtained from the QR decomposition of a Gaussian
matrix; it needs no data.  P2 ("QJL" section) adds that the matrix is drawn
once before inference and cached.

Readings: the Gaussian matrix G is an input (drawn by the caller from a
seeded generator).  QR is ambiguous up to the signs of R's diagonal; the
rotation is Q after flipping columns so that diag(R) > 0, which makes it a
unique function of G (for full-rank G) and Haar-distributed.  Vectors are
rotated as y = Pi @ x with Pi = Q.

Walsh-Hadamard variant.  P1 ("What you hit when you try it") notes that
some implementations approximate the per-vector rotation with a
Walsh-Hadamard transform.  Reading: the randomized form Pi_H = H_d D / sqrt(d),
with H_d Sylvester's Hadamard matrix (d a power of two) and D a diagonal of
random signs drawn once (an input, like G); the sign flips make the rotation
random, and the 1/sqrt(d) makes it orthogonal.  Every later step uses Pi_H
exactly where it would use Pi (same codebook, same sketch).
"""

import numpy as np


def rotation_from_gaussian(G):
    """Pi = Q diag(sign(diag R)) for G = Q R (LAPACK Householder QR, fp64)."""
    G = np.asarray(G, dtype=np.float64)
    if G.ndim != 2 or G.shape[0] != G.shape[1]:
        raise ValueError("G must be square")
    Q, R = np.linalg.qr(G)
    s = np.sign(np.diag(R))
    s[s == 0] = 1.0
    return Q * s[None, :]


def hadamard_matrix(d):
    """Sylvester's construction: H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]
    (entries +-1, float64); d must be a power of two."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    H = np.ones((1, 1))
    while H.shape[0] < d:
        H = np.block([[H, H], [H, -H]])
    return H


def randomized_hadamard(signs):
    """Pi_H = H_d diag(signs) / sqrt(d) for a vector of d signs (+-1)."""
    sg = np.asarray(signs, dtype=np.float64)
    if sg.ndim != 1 or not np.all(np.abs(sg) == 1.0):
        raise ValueError("signs must be a vector of +-1")
    d = sg.shape[0]
    return hadamard_matrix(d) * sg[None, :] / np.sqrt(np.float64(d))
