"""GPU parity at head dimensions other than 128: the pages' search vectors
have d = 200 (a2a-mcp.org page, "Benchmarks"), quantized with m = 200 sketch
rows; other sizes check the padding of partial 32-bit words.  Quantize runs
on the vector-ALU kernels, logits on the matrix-core tiles (one or two
passes of 4 coordinate words) for up to 8 query heads per KV head and on the
vector ALU for 16.  Codes, signs and norms of every vector and every logit
are compared with the oracle; decode and appends stay at d = 128."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from kv_cache_vector_quantize_amd import inputs, tq

from gpu_common import gpu_tables, key_records, oracle_tables, say, to64, value_records
from parity import check_key_stream, check_value_stream, logits_close

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d,m,bits,dtype", [(200, 200, 2, torch.bfloat16), (200, 200, 3, torch.float32),
                                            (200, 200, 4, torch.bfloat16), (72, 40, 1, torch.float32),
                                            (256, 256, 3, torch.bfloat16), (136, 32, 2, torch.bfloat16)])
def test_generic_keys_and_values(d, m, bits, dtype):
    say("generic quantize", d, m, bits, dtype)
    w = inputs.Workload("generic", 70, B=1, Hq=1, Hkv=2, T=333, d=d, m=m, k_bits=bits)
    X = torch.stack([inputs.key_slice(w, 0, h, device="cuda") for h in range(2)]).to(dtype).contiguous()
    X[1, 7] = 0.0                                              # a zero vector
    tk = gpu_tables(d, m, bits)
    pk = tq.alloc_packed(tq.TQ_KEY, tk, 2, 333, "f16")
    tq.tq_quantize(tk, X, pk)
    Pi, S, c, t = oracle_tables(d, m, bits)
    idx, sg, n, rn = key_records(pk)
    rep = check_key_stream(to64(X).reshape(-1, d), idx.reshape(-1, d), sg.reshape(-1, m), n.reshape(-1),
                           rn.reshape(-1), Pi, S, c, t, "f16")
    assert rep["ok"], rep
    assert np.all(idx[1, 7] == 1 << (bits - 1)) and np.all(sg[1, 7]) and n[1, 7] == 0
    # padding bits of the last code word and sign word are zero
    codes = pk.buf_codes.cpu().numpy().view(np.uint32)
    if d % 32:
        assert np.all(codes[:, :, -1, :] >> (d % 32) == 0)
    if m % 32:
        assert np.all(pk.buf_signs.cpu().numpy().view(np.uint32)[:, :, -1] >> (m % 32) == 0)
    # padding tokens 333 .. 351 hold the zero-vector record
    pad = oracle.unpack_key_codes(codes[:, 333:], d)
    assert np.all(pad == 1 << (bits - 1)) and not torch.any(pk.buf_norm[:, 333:])
    tv = gpu_tables(d, 0, bits)
    pv = tq.alloc_packed(tq.TQ_VALUE, tv, 2, 333, "f32")
    tq.tq_quantize(tv, X, pv)
    Piv, _, cv, tv_ = oracle_tables(d, 0, bits)
    vidx, vn = value_records(pv)
    rep = check_value_stream(to64(X).reshape(-1, d), vidx.reshape(-1, d), vn.reshape(-1), Piv, cv, tv_, "f32")
    assert rep["ok"], rep
    full = oracle.unpack_value_codes(pv.codes.cpu().numpy().view(np.uint32), pv.Tp)
    assert np.all(full[:, 333:] == 0) and not torch.any(pv.buf_norm[:, 333:])


@pytest.mark.parametrize("d,m,G,bits,T,nd", [
    (200, 200, 1, 3, 1000, "f16"), (200, 200, 8, 3, 4097, "f16"), (200, 200, 16, 2, 300, "f16"),
    (200, 200, 4, 4, 64, "f16"), (200, 200, 2, 1, 777, "f32"), (200, 200, 8, 2, 2100, "f32"),
    (256, 256, 8, 3, 515, "f16"),      # eight full words in both passes
    (136, 32, 4, 2, 333, "f16"),       # five code words, one sign word
    (96, 64, 8, 3, 1031, "f32"),       # one pass (three code words, two sign words)
    (128, 64, 2, 4, 96, "f16")])       # d = 128 with a shorter sketch
def test_generic_logits(d, m, G, bits, T, nd):
    say("generic logits", d, m, G, bits, T, nd)
    B, Hkv = 2, 2
    Hq = G * Hkv
    X = (torch.randn((B * Hkv, T, d), device="cuda") * 2).to(torch.bfloat16).contiguous()
    tk = gpu_tables(d, m, bits)
    pk = tq.alloc_packed(tq.TQ_KEY, tk, B * Hkv, T, nd)
    tq.tq_quantize(tk, X, pk)
    q = torch.randn((B, Hq, d), device="cuda").to(torch.bfloat16)
    got = tq.tq_attn_logits(tk, q, pk, B, Hq, Hkv).cpu().numpy()
    Pi, S, c, _ = oracle_tables(d, m, bits)
    idx, sg, n, rn = key_records(pk)
    qn = to64(q)
    for b in range(B):
        for h in range(Hq):
            s = b * Hkv + h // G
            ref = oracle.key_logits(qn[b, h], idx[s], sg[s], n[s].astype(np.float64), rn[s].astype(np.float64),
                                    Pi, S, c)
            ok, nbad, mx = logits_close(got[b, h], ref)
            assert ok, (b, h, nbad, mx)


def test_generic_decode_and_append_unsupported():
    say("generic decode / append unsupported")
    d = m = 200
    tk, tv = gpu_tables(d, m, 2), gpu_tables(d, 0, 3)
    pk = tq.alloc_packed(tq.TQ_KEY, tk, 2, 64, "f16", capacity=96)
    pv = tq.alloc_packed(tq.TQ_VALUE, tv, 2, 64, "f16", capacity=96)
    q = torch.zeros((1, 4, d), device="cuda")
    with pytest.raises(tq.TQError) as e:
        tq.tq_attn_decode(tk, tv, q, pk, pv, 1, 4, 2)
    assert e.value.status == tq.TQ_EUNSUPPORTED
    with pytest.raises(tq.TQError) as e:
        tq.tq_append(tk, torch.zeros((2, 3, d), device="cuda"), pk)
    assert e.value.status == tq.TQ_EUNSUPPORTED
