"""Attention logits and decode attention computed from quantized records.

Test infrastructure (see ``oracle/__init__``).

P3 "How it works", closing paragraph, and "How to implement", item 1: the
query is rotated once up front and the logits are dot products against the
stored indices, with no pass that dequantizes the whole cache.  P1 "One
more stage so attention doesn't break" and P3 Stage 2: the 1-bit sketch of
the residual corrects the inner product so that it is unbiased.

Logit estimate of <q, k> from a key record (idx, signs, n = ||k||,
rn = ||k|| * ||r||), with q' = Pi q and u = S q':

    l = n * sum_j q'_j c[idx_j] + sqrt(pi/2)/m * rn * sum_i u_i (2 s_i - 1)

The first term is <q, k_mse> (the rotation is orthogonal).  The second is
the standard unbiased 1-bit JL estimate of <q', n r>: for a row s ~ N(0, I),
E[<s, a> sign<s, r>] = sqrt(2/pi) <a, r> / ||r||, so
E[sqrt(pi/2)/m * ||r|| * sum_i <S_i, q'> sign<S_i, r>] = <q', r>.  The
constant is derived; the pages give none.

Decode (readings): one query token per (batch, query head) attends to all T
cached tokens (no mask); query head h uses KV head h // (Hq/Hkv); the
softmax is over scale * l with scale = 1/sqrt(d); values are summed in the
rotated domain, acc = sum_t a_t * ||v_t|| * c_V[idx_t], and rotated back
once, o = Pi_v^T acc, with Pi_v the rotation the values were quantized with
(the same Pi as the keys' unless the value stream has its own).
"""

import numpy as np

from .codebook import centroid_values
from .packing import unpack_key_codes, unpack_signs, unpack_value_codes


def qjl_scale(m):
    return np.sqrt(np.pi / 2.0) / m


def query_prep(q, Pi, S=None):
    """q' = Pi q and u = S q' (both fp64)."""
    q = np.asarray(q, dtype=np.float64)
    qr = q @ np.asarray(Pi, dtype=np.float64).T
    u = None if S is None else qr @ np.asarray(S, dtype=np.float64).T
    return qr, u


def key_logits(q, idx, signs, norm, rnorm, Pi, S, centroids):
    """Raw <q, k> estimates for one query q [d] against T key records.

    idx [T, d] ints, signs [T, m] bools, norm / rnorm [T] (the stored,
    possibly rounded, values)."""
    qr, u = query_prep(q, Pi, S)
    norm = np.asarray(norm, dtype=np.float64)
    mse_term = norm * (centroid_values(centroids, idx) @ qr)
    if S is None:
        return mse_term
    m = np.asarray(S).shape[0]
    pm = np.where(np.asarray(signs, dtype=bool), 1.0, -1.0)
    qjl_term = qjl_scale(m) * np.asarray(rnorm, dtype=np.float64) * (pm @ u)
    return mse_term + qjl_term


def key_logits_from_records(q, codes, sign_words, norm, rnorm, Pi, S, centroids):
    d = np.asarray(Pi).shape[0]
    idx = unpack_key_codes(codes, d)
    signs = None if S is None else unpack_signs(sign_words, np.asarray(S).shape[0])
    return key_logits(q, idx, signs, norm, rnorm, Pi, S, centroids)


def _softmax(x):
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(x - np.max(x))
    return e / np.sum(e)


def decode(q, k_idx, k_signs, k_norm, k_rnorm, v_idx, v_norm, Pi, S, ck, cv, scale=None, Pi_v=None):
    """q [B, Hq, d]; key/value records [B, Hkv, T, ...]; returns out [B, Hq, d].

    Pi rotated the keys (and so the query); Pi_v, the rotation the values
    were quantized with, rotates the value sum back (default: Pi)."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = np.asarray(k_idx).shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    Pi = np.asarray(Pi, dtype=np.float64)
    Pi_v = Pi if Pi_v is None else np.asarray(Pi_v, dtype=np.float64)
    out = np.zeros((B, Hq, d))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            l = key_logits(q[b, h], k_idx[b, g], None if S is None else k_signs[b, g],
                           k_norm[b, g], k_rnorm[b, g], Pi, S, ck)
            a = _softmax(scale * l)
            w = a * np.asarray(v_norm[b, g], dtype=np.float64)
            acc = w @ centroid_values(cv, v_idx[b, g])
            out[b, h] = Pi_v.T @ acc
    return out


def decode_from_records(q, k_codes, k_sign_words, k_norm, k_rnorm, v_codes, v_norm,
                        T, Pi, S, ck, cv, scale=None, Pi_v=None):
    """Same as ``decode`` but from the packed layout of ``packing``."""
    d = np.asarray(Pi).shape[0]
    B, Hkv = np.asarray(k_codes).shape[:2]
    k_idx = unpack_key_codes(k_codes, d)
    k_signs = None if S is None else unpack_signs(k_sign_words, np.asarray(S).shape[0])
    v_idx = unpack_value_codes(np.asarray(v_codes).reshape(B * Hkv, *np.asarray(v_codes).shape[2:]),
                               T).reshape(B, Hkv, T, d)
    return decode(q, k_idx, k_signs, k_norm, k_rnorm, v_idx, v_norm, Pi, S, ck, cv, scale, Pi_v)
