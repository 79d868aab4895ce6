"""Pins of the oracle's top-k selection (the search step)."""

import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load_scores(g):
    return np.array([float(x) for x in g["scores"]])


def test_topk_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "topk_worked_example.json")))
    s = _load_scores(g)[None, :]
    idx, val = oracle.topk(s, g["k"])
    assert idx[0].tolist() == g["idx"]
    assert np.array_equal(val[0], s[0, g["idx"]])
    idx3, _ = oracle.topk(s, 3)
    assert idx3[0].tolist() == g["k3_idx"]


def test_topk_equals_rank_count_definition():
    # position p of the answer holds the entry that exactly p entries rank
    # above (larger score, or equal score and smaller column): brute force
    rng = np.random.default_rng(5)
    for n in (1, 2, 7, 30):
        for _ in range(20):
            s = rng.integers(-3, 4, size=(3, n)).astype(np.float64)   # many ties
            s[s == 0] = rng.choice([0.0, -0.0], size=int(np.sum(s == 0)))
            k = int(rng.integers(1, n + 1))
            idx, val = oracle.topk(s, k)
            for r in range(3):
                for p, i in enumerate(idx[r]):
                    above = sum(1 for j in range(n) if s[r, j] > s[r, i] or (s[r, j] == s[r, i] and j < i))
                    assert above == p
                assert np.array_equal(val[r], s[r, idx[r]])


def test_topk_special_cases():
    rng = np.random.default_rng(6)
    s = rng.standard_normal((4, 50))
    idx, _ = oracle.topk(s, 1)
    assert np.array_equal(idx[:, 0], np.argmax(s, axis=1))        # first maximum
    idx, _ = oracle.topk(s, 50)
    assert all(sorted(r.tolist()) == list(range(50)) for r in idx)  # a permutation
    with pytest.raises(ValueError):
        oracle.topk(s, 51)
