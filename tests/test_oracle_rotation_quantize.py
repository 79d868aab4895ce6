"""Pins of the oracle's rotation, quantizer and packed layout."""

import json
import os

import numpy as np
import pytest
from scipy import stats

import oracle
from kv_cache_vector_quantize_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- rotation
@pytest.mark.parametrize("d", [8, 128])
def test_rotation_orthogonal_and_unique_qr(d):
    G, _ = inputs.table_gaussians(d, 0, seed=42)
    Pi = oracle.rotation_from_gaussian(G)
    assert np.max(np.abs(Pi.T @ Pi - np.eye(d))) < 1e-12
    # QR with a positive diagonal is unique: Pi is THE orthogonal matrix with
    # Pi^T G upper triangular and a positive diagonal.
    R = Pi.T @ G
    assert np.max(np.abs(np.tril(R, -1))) < 1e-12 * np.max(np.abs(G))
    assert np.all(np.diag(R) > 0)


def test_rotated_coordinate_follows_beta_law():
    # Haar rotation of a fixed unit vector: each coordinate ~ Beta((d-1)/2,(d-1)/2)
    d, n = 16, 3000
    x = np.zeros(d)
    x[3] = 1.0
    rng = np.random.default_rng(7)
    ys = np.array([oracle.rotation_from_gaussian(rng.standard_normal((d, d))) @ x for _ in range(n)])
    al = (d - 1) / 2
    for j in (0, 3, 11):
        p = stats.kstest((1 + ys[:, j]) / 2, stats.beta(al, al).cdf).pvalue
        assert p > 1e-3, (j, p)


# ------------------------------------------- randomized Walsh-Hadamard variant
def test_hadamard_sylvester_equals_closed_form():
    # H_d[j][k] = (-1)^popcount(j & k), and H H^T = d I in exact arithmetic
    for d in (1, 2, 4, 8, 64, 256):
        H = oracle.hadamard_matrix(d)
        j, k = np.indices((d, d))
        pc = np.vectorize(lambda v: bin(int(v)).count("1"))(j & k)
        assert np.array_equal(H, (-1.0) ** pc)
        assert np.array_equal(H @ H.T, d * np.eye(d))
    with pytest.raises(ValueError):
        oracle.hadamard_matrix(96)


def test_hadamard_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "hadamard_worked_example.json")))
    assert np.array_equal(oracle.hadamard_matrix(4), np.array(g["H4"], dtype=float))
    assert np.array_equal(oracle.hadamard_matrix(4) @ np.array(g["x"], float), np.array(g["H4_x"], float))
    P = oracle.randomized_hadamard(np.array(g["signs"], float))
    assert np.allclose(P @ np.array(g["x"], float), np.array(g["PiH_x"], float), rtol=0, atol=1e-15)


def test_randomized_hadamard_orthogonal_and_second_moment():
    P = oracle.randomized_hadamard(inputs.hadamard_signs(128))
    assert np.max(np.abs(P @ P.T - np.eye(128))) < 1e-14
    # over random signs, y_j = sum_k H_jk s_k x_k / sqrt(d) has mean 0 and
    # E[y_j^2] = ||x||^2 / d exactly (the cross terms vanish)
    d, n = 16, 40000
    rng = np.random.default_rng(3)
    x = rng.standard_normal(d)
    ys = np.stack([oracle.randomized_hadamard(rng.integers(0, 2, d) * 2.0 - 1.0) @ x for _ in range(n)])
    var = np.sum(x * x) / d
    # the sample mean of y_j^2 has standard deviation below sqrt(3) var / sqrt(n)
    assert np.all(np.abs(np.mean(ys ** 2, axis=0) - var) < 5 * np.sqrt(3.0) * var / np.sqrt(n))
    assert np.all(np.abs(np.mean(ys, axis=0)) < 5 * np.sqrt(var / n))
    with pytest.raises(ValueError):
        oracle.randomized_hadamard(np.array([1.0, 0.5]))


def test_hadamard_signs_input():
    s = inputs.hadamard_signs(128)
    assert s.shape == (128,) and set(np.unique(s)) == {-1.0, 1.0}
    assert np.array_equal(s, inputs.hadamard_signs(128))


# ---------------------------------------------------------------- quantizer
def _tables(d, m, bits, seed=42):
    G, S = inputs.table_gaussians(d, m, seed=seed)
    Pi = oracle.rotation_from_gaussian(G)
    c, t = oracle.lloyd_max(d, bits)
    return Pi, S, c, t


def test_boundary_compare_equals_brute_force_nearest_codeword_d8():
    d, bits = 8, 2
    Pi, S, c, t = _tables(d, 8, bits)
    rng = np.random.default_rng(11)
    X = rng.standard_normal((10000, d))
    q = oracle.quantize_values(X, Pi, c, t)
    # every one of the 4^8 codewords
    L = 2 ** bits
    grid = np.array(np.meshgrid(*[np.arange(L)] * d, indexing="ij")).reshape(d, -1).T
    cw = c[grid]                                     # [65536, 8]
    cw2 = np.sum(cw * cw, axis=1)
    for s in range(0, X.shape[0], 1000):
        yh = q["yhat"][s:s + 1000]
        dist = cw2[None, :] - 2.0 * yh @ cw.T
        best = grid[np.argmin(dist, axis=1)]
        assert np.array_equal(best, q["idx"][s:s + 1000])


def test_dequantize_reconstructs_input_exactly():
    d, m, bits = 128, 128, 2
    Pi, S, c, t = _tables(d, m, bits)
    X = inputs.random_vectors(64, d, seed=3).double().numpy()
    q = oracle.quantize_keys(X, Pi, S, c, t)
    # x = ||x|| Pi^T (c[idx] + r)
    rec = q["norm"][:, None] * ((c[q["idx"]] + q["rhat"]) @ Pi)
    assert np.max(np.abs(rec - X)) < 1e-12
    # residual is inside its cell: |r| <= half the cell width at the cell's side
    assert np.all(np.abs(q["rhat"]) < 1.0)
    assert np.allclose(q["rnorm"], q["norm"] * np.linalg.norm(q["rhat"], axis=1), rtol=0, atol=1e-12)
    assert np.array_equal(q["signs"], (q["rhat"] @ S.T) >= 0)


def test_mse_and_cosine_on_outlier_keys_match_codebook_and_page():
    # Rotation makes any input follow the Beta law, so the mean squared error
    # per unit vector is d * D_b even for keys with x20 outlier channels.
    d = 128
    fig = json.load(open(os.path.join(GOLDEN, "page_figures.json")))
    w = inputs.WORKLOADS[1]
    X = inputs.key_slice(w, 0, 0, T=2048).double().numpy()
    for bits in (2, 3):
        Pi, S, c, t = _tables(d, 0, bits)
        q = oracle.quantize_values(X, Pi, c, t)
        err = np.mean(np.sum((q["yhat"] - c[q["idx"]]) ** 2, axis=1))
        dD = d * oracle.codebook_mse(d, c, t)
        assert abs(err - dD) < 0.05 * dD
        if bits == 3:
            rec = c[q["idx"]]
            cos = np.mean(np.sum(q["yhat"] * rec, axis=1) / np.linalg.norm(rec, axis=1))
            assert cos >= fig["cosine_3bit"]["value"] - 1e-3


def test_zero_vector():
    d, m, bits = 128, 128, 3
    Pi, S, c, t = _tables(d, m, bits)
    X = np.zeros((2, d))
    X[1, 5] = 1.0
    q = oracle.quantize_keys(X, Pi, S, c, t)
    assert q["norm"][0] == 0 and q["rnorm"][0] == 0
    assert np.all(q["idx"][0] == 4) and np.all(q["signs"][0])
    assert q["norm"][1] == 1.0


# ---------------------------------------------------------------- packing
def test_packing_hand_worked_words():
    g = json.load(open(os.path.join(GOLDEN, "packing_layout.json")))
    idx = np.arange(32) % 4
    w = oracle.pack_key_codes(idx[None, :], 2)[0]
    assert [int(v) for v in w[0]] == [int(h, 16) for h in g["key_codes"]["words_hex"]]
    s = np.zeros(64, dtype=bool)
    s[[0, 5, 31, 32, 63]] = True
    assert [int(v) for v in oracle.pack_signs(s)] == [int(h, 16) for h in g["signs"]["words_hex"]]
    vidx = np.zeros((1, 33, 32), dtype=np.int64)
    for j in range(32):
        vidx[0, j, j] = 5
    vidx[0, 32, 7] = 7
    vidx[0, 11, 0] = 6
    vw = oracle.pack_value_codes(vidx, 3)
    assert vw.shape == (1, 2, 32, 3)
    vc = g["value_codes"]
    for blk, key in ((0, "records_hex_block0"), (1, "records_hex_block1")):
        for j, rec in vc[key].items():
            assert [int(v) for v in vw[0, blk, int(j)]] == [int(h, 16) for h in rec], (blk, j)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_packing_roundtrip(bits):
    rng = np.random.default_rng(bits)
    idx = rng.integers(0, 2 ** bits, size=(2, 45, 64))
    assert np.array_equal(oracle.unpack_key_codes(oracle.pack_key_codes(idx, bits), 64), idx)
    assert np.array_equal(oracle.unpack_value_codes(oracle.pack_value_codes(idx, bits), 45), idx)
    s = rng.integers(0, 2, size=(3, 7, 96)).astype(bool)
    assert np.array_equal(oracle.unpack_signs(oracle.pack_signs(s), 96), s)


def test_bits_per_value_matches_llama_cpp_cache_types():
    # key record at d = m = 128: b code bits + 1 sign bit per coordinate and
    # two fp16 norms per vector -> b + 1.25 bits per value: turbo3 / turbo4.
    fig = json.load(open(os.path.join(GOLDEN, "page_figures.json")))["llama_cpp_bits_per_value"]
    d = m = 128
    for bits, name in ((2, "turbo3"), (3, "turbo4")):
        idx = np.zeros((1, d), dtype=np.int64)
        nbytes = (oracle.pack_key_codes(idx, bits).nbytes + oracle.pack_signs(np.zeros((1, m), bool)).nbytes
                  + 2 * oracle.round_norms(np.zeros(1), "f16").nbytes)
        bpv = nbytes * 8 / d
        assert bpv == fig[name]
        assert round(16 / bpv, 1) == fig["compression_vs_fp16"][name]


def test_packing_pads_partial_words_with_zero_bits():
    """d = 40 coordinates take two 32-bit words per plane: coordinates 32..39
    sit at bits 0..7 of the second word and bits 8..31 stay 0 (the padded
    layout of head dimensions that are not multiples of 32, e.g. the pages'
    d = 200 search vectors).  All-ones 1-bit codes give 0xFFFFFFFF, 0x000000FF;
    41 sketch rows of sign 1 give 0xFFFFFFFF, 0x000001FF."""
    idx = np.ones((1, 40), dtype=np.int64)
    w = oracle.pack_key_codes(idx, 1)
    assert w.shape == (1, 2, 1) and w[0, :, 0].tolist() == [0xFFFFFFFF, 0x000000FF]
    assert np.array_equal(oracle.unpack_key_codes(w, 40), idx)
    sw = oracle.pack_signs(np.ones((1, 41), dtype=bool))
    assert sw[0].tolist() == [0xFFFFFFFF, 0x000001FF]
    assert np.array_equal(oracle.unpack_signs(sw, 41), np.ones((1, 41), dtype=bool))
