"""GPU parity of the randomized Walsh-Hadamard rotation variant: the table
built by tq_hadamard_rotation, then quantize (whole stream and append),
logits and decode with it, all against the oracle using its own
H_d diag(s) / sqrt(d) from the same signs."""

import functools

import numpy as np
import pytest
import torch

import oracle
from kv_cache_vector_quantize_amd import inputs, tq

from gpu_common import key_records, say, to64, value_records
from parity import check_key_stream, check_value_stream, decode_close, logits_close

pytestmark = pytest.mark.gpu
D = M = 128


@functools.lru_cache(maxsize=None)
def h_oracle_tables(m, bits):
    Pi = oracle.randomized_hadamard(inputs.hadamard_signs(D))
    _, S = inputs.table_gaussians(D, m)
    c, t = oracle.lloyd_max(D, bits)
    return Pi, S, c, t


_cache = {}


def h_gpu_tables(m, bits):
    if (m, bits) not in _cache:
        _, S = inputs.table_gaussians(D, m)
        _cache[(m, bits)] = tq.make_tables(None, S if m > 0 else None, bits,
                                           hadamard_signs=inputs.hadamard_signs(D))
    return _cache[(m, bits)]


@pytest.mark.parametrize("d", [2, 4, 128, 1024])
def test_hadamard_rotation_table_equals_oracle(d):
    say("hadamard table", d)
    s = inputs.hadamard_signs(d, seed=100 + d)
    got = tq.tq_hadamard_rotation(torch.as_tensor(s, dtype=torch.float32).cuda()).cpu().numpy()
    ref = oracle.randomized_hadamard(s).astype(np.float32)
    assert np.array_equal(got, ref)


def _keys(X, bits, nd, cap=0):
    tabs = h_gpu_tables(M, bits)
    p = tq.alloc_packed(tq.TQ_KEY, tabs, X.shape[0], X.shape[1], nd, capacity=cap)
    tq.tq_quantize(tabs, X, p)
    return tabs, p


def _values(X, bits, nd, cap=0):
    tabs = h_gpu_tables(0, bits)
    p = tq.alloc_packed(tq.TQ_VALUE, tabs, X.shape[0], X.shape[1], nd, capacity=cap)
    tq.tq_quantize(tabs, X, p)
    return tabs, p


@pytest.mark.parametrize("bits,xdt,nd", [(1, torch.bfloat16, "f16"), (2, torch.float32, "f32"),
                                         (3, torch.bfloat16, "f16"), (4, torch.float32, "f16")])
def test_hadamard_quantize_keys_and_values(bits, xdt, nd):
    """Heavy-tailed keys with outlier channels and Gaussian values, ragged
    lengths; codes, signs and norms against the oracle."""
    say("hadamard quantize", bits, xdt, nd)
    w = inputs.WORKLOADS[2]
    K = inputs.key_slice(w, 0, 1, device="cuda", T=2 * 700).reshape(2, 700, D).to(xdt).contiguous()
    _, pk = _keys(K, bits, nd)
    torch.cuda.synchronize()
    Pi, S, c, t = h_oracle_tables(M, bits)
    idx, sg, n, rn = key_records(pk)
    rep = check_key_stream(to64(K).reshape(-1, D), idx.reshape(-1, D), sg.reshape(-1, M), n.reshape(-1),
                           rn.reshape(-1), Pi, S, c, t, nd)
    assert rep["ok"], rep
    g = torch.Generator().manual_seed(bits)
    V = torch.randn((3, 333, D), generator=g).to(xdt).cuda().contiguous()
    _, pv = _values(V, bits, nd)
    torch.cuda.synchronize()
    Piv, _, cv, tv = h_oracle_tables(0, bits)
    vidx, vn = value_records(pv)
    rep = check_value_stream(to64(V).reshape(-1, D), vidx.reshape(-1, D), vn.reshape(-1), Piv, cv, tv, nd)
    assert rep["ok"], rep


def test_hadamard_append_equals_bulk():
    say("hadamard append")
    g = torch.Generator().manual_seed(12)
    X = torch.randn((2, 100, D), generator=g).to(torch.bfloat16).cuda().contiguous()
    for role, bits in ((tq.TQ_KEY, 2), (tq.TQ_VALUE, 3)):
        tabs = h_gpu_tables(M if role == tq.TQ_KEY else 0, bits)
        bulk = tq.alloc_packed(role, tabs, 2, 100, "f16", capacity=128)
        tq.tq_quantize(tabs, X, bulk)
        grown = tq.alloc_packed(role, tabs, 2, 0, "f16", capacity=128)
        for a, b in ((0, 45), (45, 46), (46, 100)):
            tq.tq_append(tabs, X[:, a:b].contiguous(), grown)
        torch.cuda.synchronize()
        for u, v in ((grown.buf_codes, bulk.buf_codes), (grown.buf_norm, bulk.buf_norm)):
            assert torch.equal(u, v)
        if role == tq.TQ_KEY:
            assert torch.equal(grown.buf_signs, bulk.buf_signs)
            assert torch.equal(grown.buf_rnorm, bulk.buf_rnorm)


def _oracle_decode(q, pk, pv, kbits, vbits, B, Hq, Hkv, rows):
    Pi, S, ck, _ = h_oracle_tables(M, kbits)
    _, _, cv, _ = h_oracle_tables(0, vbits)
    G = Hq // Hkv
    out = {}
    for (b, h) in rows:
        s = b * Hkv + h // G
        kc = pk.codes[s].cpu().numpy().view(np.uint32)
        ks = pk.signs[s].cpu().numpy().view(np.uint32)
        vc = pv.codes[s].cpu().numpy().view(np.uint32)
        out[(b, h)] = oracle.decode_from_records(
            q[b:b + 1, h:h + 1], kc[None, None], ks[None, None],
            pk.norm[s].cpu().numpy().astype(np.float64)[None, None],
            pk.rnorm[s].cpu().numpy().astype(np.float64)[None, None], vc[None, None],
            pv.norm[s].cpu().numpy().astype(np.float64)[None, None], pk.T, Pi, S, ck, cv)[0, 0]
    return out


@pytest.mark.parametrize("G,T", [(4, 1000), (8, 2500)])
def test_hadamard_logits_and_decode(G, T):
    say("hadamard decode", G, T)
    B, Hkv = 2, 2
    Hq = G * Hkv
    g = torch.Generator().manual_seed(G)
    K = (torch.randn((B * Hkv, T, D), generator=g) * 1.5).to(torch.bfloat16).cuda().contiguous()
    V = torch.randn((B * Hkv, T, D), generator=g).to(torch.bfloat16).cuda().contiguous()
    q = torch.randn((B, Hq, D), generator=g).to(torch.bfloat16).cuda()
    tk, pk = _keys(K, 2, "f16")
    tv, pv = _values(V, 3, "f16")
    got_l = tq.tq_attn_logits(tk, q, pk, B, Hq, Hkv).cpu().numpy()
    got = tq.tq_attn_decode(tk, tv, q, pk, pv, B, Hq, Hkv).cpu().numpy()
    Pi, S, ck, _ = h_oracle_tables(M, 2)
    idx, sg, n, rn = key_records(pk)
    q64 = to64(q)
    ref_l = np.zeros((B, Hq, T))
    for b in range(B):
        for h in range(Hq):
            s = b * Hkv + h // G
            ref_l[b, h] = oracle.key_logits(q64[b, h], idx[s], sg[s], n[s].astype(np.float64),
                                            rn[s].astype(np.float64), Pi, S, ck)
    ok, nbad, mx = logits_close(got_l, ref_l)
    assert ok, (nbad, mx)
    rows = [(b, h) for b in range(B) for h in range(Hq)]
    ref = _oracle_decode(q64, pk, pv, 2, 3, B, Hq, Hkv, rows)
    ok, rel = decode_close(np.stack([got[b, h] for b, h in rows]), np.stack([ref[r] for r in rows]))
    assert ok, rel


def test_hadamard_full_size_sampled():
    """The batched decode workload (16 x 8 KV heads, 131072 tokens) with the
    Walsh-Hadamard rotation, in the bench's launch configuration: sampled
    keys and value blocks against the oracle, then sampled decode rows."""
    w = inputs.WORKLOADS[3]
    say("hadamard full size", w.name)
    K = inputs.keys(w, device="cuda").reshape(w.nseq, w.T, D)
    tk, pk = _keys(K, w.k_bits, w.norm_dtype)
    rng = np.random.default_rng(77)
    rows = np.sort(rng.choice(w.nseq * w.T, size=3000, replace=False))
    Pi, S, c, t = h_oracle_tables(M, w.k_bits)
    sel = torch.as_tensor(rows, device="cuda")
    codes = pk.codes.reshape(-1, D // 32, w.k_bits)[sel].cpu().numpy().view(np.uint32)
    signs = pk.signs.reshape(-1, M // 32)[sel].cpu().numpy().view(np.uint32)
    rep = check_key_stream(to64(K.reshape(-1, D)[sel]), oracle.unpack_key_codes(codes, D),
                           oracle.unpack_signs(signs, M), pk.norm.reshape(-1)[sel].cpu().numpy(),
                           pk.rnorm.reshape(-1)[sel].cpu().numpy(), Pi, S, c, t, w.norm_dtype)
    assert rep["ok"], rep
    del K
    V = inputs.values(w, device="cuda").reshape(w.nseq, w.T, D)
    tv, pv = _values(V, w.v_bits, w.norm_dtype)
    Piv, _, cv, tvb = h_oracle_tables(0, w.v_bits)
    for s, blk in zip(rng.integers(0, w.nseq, 16), rng.integers(0, w.T // 32, 16)):
        words = pv.codes[s, blk].cpu().numpy().view(np.uint32)
        idx = oracle.unpack_value_codes(words.reshape(1, 1, D, w.v_bits), 32)[0]
        rep = check_value_stream(to64(V[s, blk * 32:(blk + 1) * 32]), idx,
                                 pv.norm[s, blk * 32:(blk + 1) * 32].cpu().numpy(), Piv, cv, tvb,
                                 w.norm_dtype)
        assert rep["ok"], (s, blk, rep)
    del V
    q = inputs.queries(w, device="cuda")
    got = tq.tq_attn_decode(tk, tv, q, pk, pv, w.B, w.Hq, w.Hkv).cpu().numpy()
    drows = [(int(rng.integers(w.B)), int(rng.integers(w.Hq))) for _ in range(2)]
    ref = _oracle_decode(to64(q), pk, pv, w.k_bits, w.v_bits, w.B, w.Hq, w.Hkv, drows)
    ok, rel = decode_close(np.stack([got[b, h] for b, h in drows]), np.stack([ref[r] for r in drows]))
    assert ok, rel
