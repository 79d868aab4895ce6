"""GPU parity of tq_attn_logits and tq_attn_decode against the oracle,
which recomputes every output from the GPU's own packed records."""

import math

import numpy as np
import pytest
import torch

import oracle
from kv_cache_vector_quantize_amd import inputs, tq

from gpu_common import gpu_tables, key_records, oracle_tables, say, to64, value_records
from parity import decode_close, logits_close

pytestmark = pytest.mark.gpu
D = M = 128


def _keys(X, bits, nd):
    tabs = gpu_tables(D, M, bits)
    p = tq.alloc_packed(tq.TQ_KEY, tabs, X.shape[0], X.shape[1], nd)
    tq.tq_quantize(tabs, X, p)
    return tabs, p


def _values(X, bits, nd):
    tabs = gpu_tables(D, 0, bits)
    p = tq.alloc_packed(tq.TQ_VALUE, tabs, X.shape[0], X.shape[1], nd)
    tq.tq_quantize(tabs, X, p)
    return tabs, p


def _oracle_logits(q, p, bits, B, Hq, Hkv):
    Pi, S, c, _ = oracle_tables(D, M, bits)
    idx, sg, n, rn = key_records(p)
    G = Hq // Hkv
    out = np.zeros((B, Hq, p.T))
    for b in range(B):
        for h in range(Hq):
            s = b * Hkv + h // G
            out[b, h] = oracle.key_logits(q[b, h], idx[s], sg[s], n[s].astype(np.float64),
                                          rn[s].astype(np.float64), Pi, S, c)
    return out


def test_tiny_logits():
    w = inputs.WORKLOADS[1]
    say("logits", w.name)
    X = inputs.key_slice(w, 0, 0, device="cuda").unsqueeze(0).contiguous()
    tk, p = _keys(X, w.k_bits, w.norm_dtype)
    q = inputs.queries(w, device="cuda")
    got = tq.tq_attn_logits(tk, q, p, 1, 1, 1)
    torch.cuda.synchronize()
    ref = _oracle_logits(to64(q), p, w.k_bits, 1, 1, 1)
    ok, nbad, mx = logits_close(got.cpu().numpy(), ref)
    assert ok, (nbad, mx)


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
def test_logits_group_sizes_ragged(G):
    say("logits group", G)
    B, Hkv, T = 2, 2, 777
    Hq = G * Hkv
    X = (torch.randn((B * Hkv, T, D), device="cuda") * 2).to(torch.bfloat16)
    tk, p = _keys(X.contiguous(), 3, "f16")
    q = torch.randn((B, Hq, D), device="cuda")
    got = tq.tq_attn_logits(tk, q, p, B, Hq, Hkv)
    torch.cuda.synchronize()
    ref = _oracle_logits(to64(q), p, 3, B, Hq, Hkv)
    ok, nbad, mx = logits_close(got.cpu().numpy(), ref)
    assert ok, (nbad, mx)


@pytest.mark.parametrize("B,Hkv,G", [(1, 3, 1), (1, 5, 2), (3, 1, 2)])
def test_odd_head_counts(B, Hkv, G):
    """3, 10 and 6 query heads (counts that are not a power of two), 3 and 5
    KV heads: logits and decode against the oracle."""
    say("odd head counts", B, Hkv, G)
    T = 300
    Hq = G * Hkv
    K = (torch.randn((B * Hkv, T, D), device="cuda") * 1.5).to(torch.bfloat16).contiguous()
    V = torch.randn((B * Hkv, T, D), device="cuda").to(torch.bfloat16).contiguous()
    tk, pk = _keys(K, 2, "f16")
    tv, pv = _values(V, 3, "f16")
    q = torch.randn((B, Hq, D), device="cuda")
    got = tq.tq_attn_logits(tk, q, pk, B, Hq, Hkv)
    torch.cuda.synchronize()
    ref = _oracle_logits(to64(q), pk, 2, B, Hq, Hkv)
    ok, nbad, mx = logits_close(got.cpu().numpy(), ref)
    assert ok, (nbad, mx)
    got = tq.tq_attn_decode(tk, tv, q, pk, pv, B, Hq, Hkv).cpu().numpy()
    rows = [(b, h) for b in range(B) for h in range(Hq)]
    ref = _oracle_decode_rows(to64(q), pk, pv, 2, 3, B, Hq, Hkv, rows)
    ok, rel = decode_close(np.stack([got[b, h] for b, h in rows]), np.stack([ref[r] for r in rows]))
    assert ok, rel


@pytest.mark.parametrize("bits,T,nd", [(1, 100, "f16"), (2, 2049, "f16"), (4, 64, "f16"), (3, 333, "f32"),
                                       (2, 4096, "f32")])
def test_logits_code_widths_and_splits(bits, T, nd):
    """Every key width and both norm storages through the matrix-core logits;
    T = 2049 leaves a one-token last split, T = 100 / 333 a partial block."""
    say("logits bits", bits, "T", T, nd)
    B, Hkv, G = 1, 4, 4
    Hq = G * Hkv
    X = (torch.randn((B * Hkv, T, D), device="cuda") * 2).to(torch.bfloat16)
    tk, p = _keys(X.contiguous(), bits, nd)
    q = torch.randn((B, Hq, D), device="cuda")
    got = tq.tq_attn_logits(tk, q, p, B, Hq, Hkv)
    torch.cuda.synchronize()
    ref = _oracle_logits(to64(q), p, bits, B, Hq, Hkv)
    ok, nbad, mx = logits_close(got.cpu().numpy(), ref)
    assert ok, (nbad, mx)


def test_llama8b_logits_full_size():
    w = inputs.WORKLOADS[2]
    say("logits full size", w.name)
    K = inputs.keys(w, device="cuda").reshape(w.nseq, w.T, D)
    tk, p = _keys(K, w.k_bits, w.norm_dtype)
    q = inputs.queries(w, device="cuda")
    got = tq.tq_attn_logits(tk, q, p, w.B, w.Hq, w.Hkv)
    torch.cuda.synchronize()
    ref = _oracle_logits(to64(q), p, w.k_bits, w.B, w.Hq, w.Hkv)
    ok, nbad, mx = logits_close(got.cpu().numpy(), ref)
    assert ok, (nbad, mx)


def _oracle_decode_rows(q, pk, pv, kbits, vbits, B, Hq, Hkv, rows):
    Pi, S, ck, _ = oracle_tables(D, M, kbits)
    _, _, cv, _ = oracle_tables(D, 0, vbits)
    G = Hq // Hkv
    out = {}
    for (b, h) in rows:
        s = b * Hkv + h // G
        kc = pk.codes[s].cpu().numpy().view(np.uint32)
        ks = pk.signs[s].cpu().numpy().view(np.uint32)
        vc = pv.codes[s].cpu().numpy().view(np.uint32)
        o = oracle.decode_from_records(
            q[b:b + 1, h:h + 1], kc[None, None], ks[None, None],
            pk.norm[s].cpu().numpy().astype(np.float64)[None, None],
            pk.rnorm[s].cpu().numpy().astype(np.float64)[None, None], vc[None, None],
            pv.norm[s].cpu().numpy().astype(np.float64)[None, None], pk.T, Pi, S, ck, cv)
        out[(b, h)] = o[0, 0]
    return out


@pytest.mark.parametrize("G,T", [(1, 1), (2, 31), (4, 1000), (8, 2500)])
def test_decode_small(G, T):
    say("decode small", G, T)
    B, Hkv = 2, 2
    Hq = G * Hkv
    K = (torch.randn((B * Hkv, T, D), device="cuda") * 1.5).to(torch.bfloat16).contiguous()
    V = torch.randn((B * Hkv, T, D), device="cuda").to(torch.bfloat16).contiguous()
    tk, pk = _keys(K, 2, "f16")
    tv, pv = _values(V, 3, "f16")
    q = torch.randn((B, Hq, D), device="cuda").to(torch.bfloat16)
    got = tq.tq_attn_decode(tk, tv, q, pk, pv, B, Hq, Hkv).cpu().numpy()
    rows = [(b, h) for b in range(B) for h in range(Hq)]
    ref = _oracle_decode_rows(to64(q), pk, pv, 2, 3, B, Hq, Hkv, rows)
    ok, rel = decode_close(np.stack([got[b, h] for b, h in rows]), np.stack([ref[r] for r in rows]))
    assert ok, rel


@pytest.mark.parametrize("T,G", [(16000, 1), (20000, 2)])
def test_decode_many_splits(T, G):
    """One KV head over a long context: 125 and 157 splits of 128 tokens,
    merged by the log-sum-exp combine (four groups of splits of uneven
    length)."""
    say("decode many splits", T, G)
    B, Hkv = 1, 1
    Hq = G * Hkv
    K = (torch.randn((B * Hkv, T, D), device="cuda") * 1.5).to(torch.bfloat16).contiguous()
    V = torch.randn((B * Hkv, T, D), device="cuda").to(torch.bfloat16).contiguous()
    tk, pk = _keys(K, 2, "f16")
    tv, pv = _values(V, 3, "f16")
    q = torch.randn((B, Hq, D), device="cuda").to(torch.bfloat16)
    got = tq.tq_attn_decode(tk, tv, q, pk, pv, B, Hq, Hkv).cpu().numpy()
    rows = [(b, h) for b in range(B) for h in range(Hq)]
    ref = _oracle_decode_rows(to64(q), pk, pv, 2, 3, B, Hq, Hkv, rows)
    ok, rel = decode_close(np.stack([got[b, h] for b, h in rows]), np.stack([ref[r] for r in rows]))
    assert ok, rel


@pytest.mark.parametrize("kbits,vbits,knd,vnd,G", [
    (1, 4, "f32", "f32", 4), (3, 1, "f16", "f32", 2), (4, 2, "f32", "f16", 8), (2, 3, "f32", "f16", 1)])
def test_decode_code_widths_and_norm_dtypes(kbits, vbits, knd, vnd, G):
    """Every key / value width and norm storage mix, several splits with a
    ragged last block."""
    say("decode widths", kbits, vbits, knd, vnd, G)
    B, Hkv, T = 2, 2, 777
    Hq = G * Hkv
    K = torch.randn((B * Hkv, T, D), device="cuda").contiguous()
    V = (torch.randn((B * Hkv, T, D), device="cuda") * 0.5).contiguous()
    tk, pk = _keys(K, kbits, knd)
    tv, pv = _values(V, vbits, vnd)
    q = torch.randn((B, Hq, D), device="cuda")
    got = tq.tq_attn_decode(tk, tv, q, pk, pv, B, Hq, Hkv).cpu().numpy()
    rows = [(b, h) for b in range(B) for h in range(Hq)]
    ref = _oracle_decode_rows(to64(q), pk, pv, kbits, vbits, B, Hq, Hkv, rows)
    ok, rel = decode_close(np.stack([got[b, h] for b, h in rows]), np.stack([ref[r] for r in rows]))
    assert ok, rel


def test_decode_value_norm_range():
    """Value norms from 0 to 1e6 rising along the context (float32 norms): the
    running largest norm and the softmax reference are raised many times
    inside a split, and the first blocks hold zero vectors only."""
    say("decode value norm range")
    B, Hkv, G, T = 1, 2, 4, 3000
    Hq = G * Hkv
    g = torch.Generator().manual_seed(5)
    K = torch.randn((B * Hkv, T, D), generator=g) * 2.0
    V = torch.randn((B * Hkv, T, D), generator=g)
    scale = torch.logspace(-6, 6, T, dtype=torch.float64).float()
    scale[:100] = 0.0
    V = V * scale[None, :, None]
    K[:, 2000:2010] *= 6.0  # a few tokens with large logits late in the context
    tk, pk = _keys(K.cuda().contiguous(), 2, "f32")
    tv, pv = _values(V.cuda().contiguous(), 3, "f32")
    q = torch.randn((B, Hq, D), generator=g).cuda()
    got = tq.tq_attn_decode(tk, tv, q, pk, pv, B, Hq, Hkv).cpu().numpy()
    rows = [(0, h) for h in range(Hq)]
    ref = _oracle_decode_rows(to64(q), pk, pv, 2, 3, B, Hq, Hkv, rows)
    ok, rel = decode_close(np.stack([got[b, h] for b, h in rows]), np.stack([ref[r] for r in rows]))
    assert ok, rel


@pytest.mark.parametrize("v_kind", ["dense_other_seed", "hadamard"])
def test_decode_separate_key_and_value_rotations(v_kind):
    """Key and value tables built separately: the values rotated by a Pi of
    their own (another Gaussian draw, or the Walsh-Hadamard rotation).  The
    output is rotated back with the value table's Pi."""
    say("decode separate rotations", v_kind)
    B, Hkv, G, T = 1, 2, 4, 700
    Hq = G * Hkv
    Gk, Sk = inputs.table_gaussians(D, M)
    Pi_k = oracle.rotation_from_gaussian(Gk)
    if v_kind == "hadamard":
        hs = inputs.hadamard_signs(D)
        tv = tq.make_tables(None, None, 3, hadamard_signs=hs)
        Pi_v = oracle.randomized_hadamard(hs)
    else:
        Gv, _ = inputs.table_gaussians(D, 0, seed=77)
        tv = tq.make_tables(Gv, None, 3)
        Pi_v = oracle.rotation_from_gaussian(Gv)
    tk = gpu_tables(D, M, 2)
    g = torch.Generator().manual_seed(21)
    K = (torch.randn((B * Hkv, T, D), generator=g) * 1.5).to(torch.bfloat16).cuda().contiguous()
    V = torch.randn((B * Hkv, T, D), generator=g).to(torch.bfloat16).cuda().contiguous()
    pk = tq.alloc_packed(tq.TQ_KEY, tk, B * Hkv, T, "f16")
    tq.tq_quantize(tk, K, pk)
    pv = tq.alloc_packed(tq.TQ_VALUE, tv, B * Hkv, T, "f16")
    tq.tq_quantize(tv, V, pv)
    q = torch.randn((B, Hq, D), generator=g).cuda()
    got = tq.tq_attn_decode(tk, tv, q, pk, pv, B, Hq, Hkv).cpu().numpy()
    # the value codes follow the value table's rotation
    _, _, cv, tbv = oracle_tables(D, 0, 3)
    vidx, vn = value_records(pv)
    vref = oracle.quantize_values(to64(V).reshape(-1, D), Pi_v, cv, tbv)
    diff = vidx.reshape(-1, D) != vref["idx"]
    near = np.min(np.abs(vref["yhat"][..., None] - tbv[None, None, :]), axis=-1) <= 1e-5
    assert not np.any(diff & ~near)
    _, S, ck, _ = oracle_tables(D, M, 2)
    qn = to64(q)
    for h in range(Hq):
        s = h // G
        kc = pk.codes[s].cpu().numpy().view(np.uint32)
        ks = pk.signs[s].cpu().numpy().view(np.uint32)
        vc = pv.codes[s].cpu().numpy().view(np.uint32)
        ref = oracle.decode_from_records(
            qn[0:1, h:h + 1], kc[None, None], ks[None, None],
            pk.norm[s].cpu().numpy().astype(np.float64)[None, None],
            pk.rnorm[s].cpu().numpy().astype(np.float64)[None, None], vc[None, None],
            pv.norm[s].cpu().numpy().astype(np.float64)[None, None], T, Pi_k, S, ck, cv,
            Pi_v=Pi_v)[0, 0]
        ok, rel = decode_close(got[0, h][None], ref[None])
        assert ok, (h, rel)
