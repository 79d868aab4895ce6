"""GPU parity of the setup kernels (codebook, rotation) against the oracle."""

import numpy as np
import pytest
import torch

import oracle
from kv_cache_vector_quantize_amd import inputs, tq

from gpu_common import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d", [8, 64, 128, 200])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_codebook_matches_oracle(d, bits):
    say("tq_codebook", d, bits)
    c64, b64, c32, b32 = tq.tq_codebook(d, bits)
    torch.cuda.synchronize()
    c, t = oracle.lloyd_max(d, bits)
    assert np.max(np.abs(c64.cpu().numpy() - c)) <= 1e-12
    assert np.max(np.abs(b64.cpu().numpy() - t)) <= 1e-12
    # float32 tables are the library's fp64 values rounded to nearest
    assert np.array_equal(c32.cpu().numpy(), c64.cpu().numpy().astype(np.float32))
    assert np.array_equal(b32.cpu().numpy(), b64.cpu().numpy().astype(np.float32))


@pytest.mark.parametrize("d", [8, 32, 128, 129, 200, 256])
def test_rotation_matches_oracle(d):
    # up to 128 the factorization runs in LDS, past 128 in global memory
    say("tq_rotation", d)
    G, _ = inputs.table_gaussians(d, 0)
    r64, r32 = tq.tq_rotation(torch.as_tensor(G).cuda())
    torch.cuda.synchronize()
    P = r64.cpu().numpy()
    ref = oracle.rotation_from_gaussian(G)
    assert np.max(np.abs(P - ref)) <= 1e-12
    assert np.max(np.abs(P.T @ P - np.eye(d))) < 1e-12
    assert np.array_equal(r32.cpu().numpy(), P.astype(np.float32))


@pytest.mark.parametrize("d", [16, 200])
def test_rotation_rank_deficient_column(d):
    # a zero column leaves the reflector at the identity and a +1 sign
    say("tq_rotation zero column", d)
    G, _ = inputs.table_gaussians(d, 0, seed=3)
    G[:, 5] = 0.0
    r64, _ = tq.tq_rotation(torch.as_tensor(G).cuda())
    P = r64.cpu().numpy()
    assert np.max(np.abs(P.T @ P - np.eye(d))) < 1e-12
    R = P.T @ G
    assert np.max(np.abs(np.tril(R, -1))) < 1e-12 * np.max(np.abs(G))
    assert np.all(np.diag(R) >= -1e-12)
