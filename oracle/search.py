"""Inner-product search over packed keys: estimated scores, then top-k.

Test infrastructure (see ``oracle/__init__``).

P3 "Benchmarks": vector search (GloVe, d = 200) is judged by the top-k recall
of the inner products the quantized codes estimate.  The scores are the
logits of ``attention.key_logits`` (the same estimator, computed straight
from the stored indices and signs).  Reading: the k best of a row are its k
largest scores, ties going to the smaller column index (a total order, so
the answer is unique); -0 and +0 are equal scores.
"""

import numpy as np

from .attention import key_logits_from_records


def topk(scores, k):
    """scores [rows, n] -> (idx [rows, k] int64, val [rows, k]) ordered by
    descending score, then ascending column."""
    S = np.asarray(scores)
    rows, n = S.shape
    if not 1 <= k <= n:
        raise ValueError("need 1 <= k <= n")
    cols = np.arange(n)
    idx = np.empty((rows, k), dtype=np.int64)
    for r in range(rows):
        order = np.lexsort((cols, -S[r]))   # primary key: -score; then column
        idx[r] = order[:k]
    val = np.take_along_axis(S, idx, axis=1)
    return idx, val


def search_from_records(queries, codes, sign_words, norm, rnorm, Pi, S, centroids, k):
    """queries [nq, d]; one packed key stream (codes [N, d/32, bits], sign
    words [N, m/32], norms [N]) -> top-k of the estimated inner products."""
    Q = np.asarray(queries, dtype=np.float64)
    scores = np.stack([key_logits_from_records(q, codes, sign_words, norm, rnorm, Pi, S, centroids)
                       for q in Q])
    return topk(scores, k) + (scores,)
