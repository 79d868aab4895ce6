"""GPU parity of the search step: tq_topk against the oracle's top-k (bit
exact: it is index work), and inner-product search (tq_attn_logits over
one packed key database, then tq_topk) against the oracle's scores."""

import numpy as np
import pytest
import torch

import oracle
from kv_cache_vector_quantize_amd import inputs, tq

from gpu_common import gpu_tables, oracle_tables, say, to64

pytestmark = pytest.mark.gpu
D = M = 128


def _scores(rows, n, seed):
    """Scores with many exact ties, signed zeros and -inf."""
    rng = np.random.default_rng(seed)
    s = np.round(rng.standard_normal((rows, n)) * 4) / 4
    s[rng.random((rows, n)) < 0.01] = -np.inf
    z = s == 0
    s[z] = rng.choice([0.0, -0.0], size=int(np.sum(z)))
    return s.astype(np.float32)


def _check_topk(s, k):
    got_i, got_v = tq.tq_topk(torch.as_tensor(s).cuda(), k)
    torch.cuda.synchronize()
    ref_i, ref_v = oracle.topk(s.astype(np.float64), k)
    assert np.array_equal(got_i.cpu().numpy(), ref_i)
    assert np.array_equal(got_v.cpu().numpy(), ref_v.astype(np.float32))


@pytest.mark.parametrize("rows,n,k", [
    (1, 1, 1), (3, 5, 5), (2, 100, 10), (4, 16383, 16), (4, 16384, 17), (5, 16385, 32),
    (2, 100003, 10), (40, 3000, 7), (3, 4 * 16384 * 5 + 3, 32),
    (1, 300 * 16384 + 5, 7)])   # more chunk lists than the row merge has threads
def test_topk_exact(rows, n, k):
    say("topk", rows, n, k)
    _check_topk(_scores(rows, n, seed=rows * 1000 + k), k)


def test_topk_adversarial_orders():
    """All-equal rows (the answer is columns 0..k-1), ascending rows (every
    column enters a thread's list), the winners in the last chunk only."""
    say("topk adversarial")
    n = 3 * 16384 + 100
    s = np.zeros((4, n), dtype=np.float32)
    s[1] = np.arange(n, dtype=np.float32)
    s[2] = -np.arange(n, dtype=np.float32)
    s[3, :] = -1.0
    s[3, n - 40:] = np.linspace(1.0, 2.0, 40, dtype=np.float32)
    for k in (1, 13, 32):
        _check_topk(s, k)


def test_topk_many_rows_long():
    say("topk 16 x 2^20")
    _check_topk(_scores(16, 1 << 20, seed=99), 10)


def _search(w_bits, N, nq, k, seed, law="normal_outliers", d=D, m=M):
    w = inputs.Workload("search_test", 60 + seed, B=1, Hq=nq, Hkv=1, T=N, d=d, m=m, k_bits=w_bits, k_law=law)
    X = inputs.key_slice(w, 0, 0, device="cuda").unsqueeze(0).contiguous()
    tabs = gpu_tables(d, m, w_bits)
    p = tq.alloc_packed(tq.TQ_KEY, tabs, 1, N, "f16")
    tq.tq_quantize(tabs, X, p)
    q = inputs.queries(w, device="cuda")                      # [1, nq, d]
    logits = tq.tq_attn_logits(tabs, q, p, 1, nq, 1)          # [1, nq, N]
    idx, val = tq.tq_topk(logits.view(nq, N), k)
    torch.cuda.synchronize()
    return w, p, q, logits.view(nq, N).cpu().numpy(), idx.cpu().numpy(), val.cpu().numpy()


def _check_search(ref_scores_at, logits, idx, val, k, sample):
    """ref_scores_at(r, cols) -> the oracle's scores of row r at cols."""
    nq = idx.shape[0]
    for r in range(nq):
        # the returned values are the row's scores at the returned columns, in order
        assert np.array_equal(val[r], logits[r, idx[r]])
        assert np.all(np.diff(val[r]) <= 0)
        ref_sel = ref_scores_at(r, idx[r])
        tol = 1e-4 + 1e-3 * np.abs(ref_sel)
        assert np.all(np.abs(val[r] - ref_sel) <= tol), r
        # no other column beats the k-th beyond the tolerance of two estimates
        cols = np.setdiff1d(sample, idx[r])
        ref_other = ref_scores_at(r, cols)
        kth = ref_sel.min()
        assert np.all(ref_other <= kth + 2 * (1e-4 + 1e-3 * abs(kth))), r


@pytest.mark.parametrize("d", [128, 200])
def test_search_small_against_oracle_scores(d):
    """A 20000-key database, 8 queries, top 10: the oracle scores every key
    from the GPU's records; the GPU's top 10 must be a top 10 of them up to
    the logits tolerance.  d = 200 (m = 200) is the pages' search dimension."""
    say("search small", d)
    N, nq, k = 20000, 8, 10
    w, p, q, logits, idx, val = _search(3, N, nq, k, seed=1, d=d, m=d)
    Pi, S, c, _ = oracle_tables(d, d, 3)
    codes = p.codes[0].cpu().numpy().view(np.uint32)
    signs = p.signs[0].cpu().numpy().view(np.uint32)
    ridx, rval, rscores = oracle.search_from_records(to64(q)[0], codes, signs,
                                                     p.norm[0].cpu().numpy().astype(np.float64),
                                                     p.rnorm[0].cpu().numpy().astype(np.float64), Pi, S, c, k)
    _check_search(lambda r, cols: rscores[r, cols], logits, idx, val, k, np.arange(N))
    # most of the answer is the oracle's own (differences only at near-ties)
    agree = np.mean([len(set(idx[r]) & set(ridx[r])) / k for r in range(nq)])
    assert agree >= 0.9, agree


def test_search_full_size_sampled():
    """The search workload (2^20 keys, 8 queries, top 10) in the bench's
    launch configuration: the oracle scores the returned keys and a sample
    of 20000 others."""
    w6 = inputs.WORKLOADS[6]
    say("search full size", w6.name)
    X = inputs.keys(w6, device="cuda").reshape(1, w6.T, w6.d)
    tabs = gpu_tables(w6.d, w6.m, w6.k_bits)
    p = tq.alloc_packed(tq.TQ_KEY, tabs, 1, w6.T, w6.norm_dtype)
    tq.tq_quantize(tabs, X, p)
    del X
    q = inputs.queries(w6, device="cuda")
    logits = tq.tq_attn_logits(tabs, q, p, 1, w6.Hq, 1).view(w6.Hq, w6.T)
    idx, val = tq.tq_topk(logits, w6.topk)
    torch.cuda.synchronize()
    logits_h, idx, val = logits.cpu().numpy(), idx.cpu().numpy(), val.cpu().numpy()
    rng = np.random.default_rng(6)
    sample = np.unique(np.concatenate([rng.choice(w6.T, 20000, replace=False), idx.reshape(-1)]))
    Pi, S, c, _ = oracle_tables(w6.d, w6.m, w6.k_bits)
    codes = p.codes[0].cpu().numpy().view(np.uint32)[sample]
    signs = p.signs[0].cpu().numpy().view(np.uint32)[sample]
    kn = p.norm[0].cpu().numpy().astype(np.float64)[sample]
    kr = p.rnorm[0].cpu().numpy().astype(np.float64)[sample]
    q64 = to64(q)[0]
    ref = np.stack([oracle.key_logits_from_records(q64[r], codes, signs, kn, kr, Pi, S, c) for r in range(w6.Hq)])
    pos = {int(col): i for i, col in enumerate(sample)}
    _check_search(lambda r, cols: ref[r, [pos[int(x)] for x in cols]], logits_h, idx, val, w6.topk, sample)
