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
