"""CPU checks of the full-coverage parity harness (oracle.fanout and the
jobs in full_parity): fed the oracle's own packed records it finds no
mismatch, and it catches a wrong code, a wrong sign bit and a wrong norm
planted in those records.  Decode jobs agree with the oracle's one-call
decode."""

import numpy as np
import pytest

import oracle
from oracle import fanout

import full_parity as fp

D = M = 128
T, NSEQ = 640, 2


def _records(bits, nd="f16", seed=0):
    rng = np.random.default_rng(seed)
    X = (rng.standard_normal((NSEQ, T, D)) * (1 + 9 * (np.arange(D) % 31 == 0))).astype(np.float32)
    Pi, S, c, t = fp.tables(D, M, bits)
    r = oracle.quantize_keys(X.reshape(-1, D).astype(np.float64), Pi, S, c, t)
    rec = dict(x=X,
               codes=oracle.pack_key_codes(r["idx"], bits).reshape(NSEQ, T, D // 32, bits).view(np.int32),
               signs=oracle.pack_signs(r["signs"]).reshape(NSEQ, T, M // 32).view(np.int32),
               norm=oracle.round_norms(r["norm"], nd).reshape(NSEQ, T),
               rnorm=oracle.round_norms(r["rnorm"], nd).reshape(NSEQ, T))
    return rec, r


@pytest.fixture(scope="module")
def pool():
    with fanout.Pool(2) as p:
        yield p


def _run_keys(pool, rec, bits, nd="f16"):
    with fanout.SharedArrays() as sh:
        for k, v in rec.items():
            sh.put(k, v)
        return fp.aggregate(pool.run(fp.key_slice, fp.key_tasks(NSEQ, T, bits, nd, chunk=256), sh))


def test_own_records_pass_and_planted_errors_are_caught(pool):
    bits = 3
    rec, r = _records(bits)
    rep = _run_keys(pool, rec, bits)
    assert rep["ok"] and rep["vectors"] == NSEQ * T and rep["code_mismatch"] == 0, rep
    # a code bit flipped at a coordinate far from every boundary
    _, _, _, t = fp.tables(D, M, bits)
    dist = np.min(np.abs(r["yhat"][..., None] - t[None, None, :]), axis=-1).reshape(NSEQ, T, D)
    s, tok, j = np.unravel_index(np.argmax(dist), dist.shape)
    bad = {k: v.copy() for k, v in rec.items()}
    bad["codes"].view(np.uint32)[s, tok, j // 32, 0] ^= np.uint32(1 << (j % 32))
    rep = _run_keys(pool, bad, bits)
    assert not rep["ok"] and rep["code_bad"] >= 1, rep
    # a sign bit flipped where |z| is far from zero
    z = r["z"].reshape(NSEQ, T, M)
    s, tok, i = np.unravel_index(np.argmax(np.abs(z)), z.shape)
    bad = {k: v.copy() for k, v in rec.items()}
    bad["signs"].view(np.uint32)[s, tok, i // 32] ^= np.uint32(1 << (i % 32))
    rep = _run_keys(pool, bad, bits)
    assert not rep["ok"] and rep["sign_bad"] == 1, rep
    # a norm two float16 ulps off
    bad = {k: v.copy() for k, v in rec.items()}
    bad["norm"][1, 5] = np.nextafter(np.nextafter(bad["norm"][1, 5], np.float16(np.inf)), np.float16(np.inf))
    rep = _run_keys(pool, bad, bits)
    assert not rep["ok"] and not rep["norm_ok"], rep


def test_value_job_and_padding(pool):
    bits, Tv = 2, T - 7                      # a ragged last block
    rng = np.random.default_rng(3)
    X = rng.standard_normal((NSEQ, Tv, D)).astype(np.float32)
    Pi, _, c, t = fp.tables(D, 0, bits)
    r = oracle.quantize_values(X.reshape(-1, D).astype(np.float64), Pi, c, t)
    codes = oracle.pack_value_codes(r["idx"].reshape(NSEQ, Tv, D), bits).view(np.int32)
    rec = dict(x=X, codes=codes, norm=oracle.round_norms(r["norm"], "f32").reshape(NSEQ, Tv))
    with fanout.SharedArrays() as sh:
        for k, v in rec.items():
            sh.put(k, v)
        rep = fp.aggregate(pool.run(fp.value_slice, fp.value_tasks(NSEQ, Tv, bits, "f32", chunk_blocks=4), sh))
        assert rep["ok"] and rep["vectors"] == NSEQ * Tv, rep
        # a nonzero field in the padding of the last block is caught
        bad = codes.copy()
        bad.view(np.uint32)[1, -1, 7, bits - 1] |= np.uint32(1 << 31)
        sh.drop("codes")
        sh.put("codes", bad)
        rep = fp.aggregate(pool.run(fp.value_slice, fp.value_tasks(NSEQ, Tv, bits, "f32", chunk_blocks=4), sh))
        assert not rep["ok"], rep


def test_decode_job_matches_one_call_decode(pool):
    kb, vb, G, Tt = 2, 3, 2, 300
    rng = np.random.default_rng(4)
    K = rng.standard_normal((NSEQ, Tt, D)).astype(np.float32)
    V = rng.standard_normal((NSEQ, Tt, D)).astype(np.float32)
    q = rng.standard_normal((NSEQ, G, D)).astype(np.float32)
    Pi, S, ck, tk = fp.tables(D, M, kb)
    _, _, cv, tv = fp.tables(D, 0, vb)
    kr = oracle.quantize_keys(K.reshape(-1, D).astype(np.float64), Pi, S, ck, tk)
    vr = oracle.quantize_values(V.reshape(-1, D).astype(np.float64), Pi, cv, tv)
    rs = lambda a: a.reshape(NSEQ, Tt, *a.shape[1:])
    sh_arrays = dict(
        k=K, v=V, q=q,
        kcodes=oracle.pack_key_codes(rs(kr["idx"]), kb).view(np.int32),
        ksigns=oracle.pack_signs(rs(kr["signs"])).view(np.int32),
        knorm=oracle.round_norms(rs(kr["norm"]), "f16"), krnorm=oracle.round_norms(rs(kr["rnorm"]), "f16"),
        vcodes=oracle.pack_value_codes(rs(vr["idx"]), vb).view(np.int32),
        vnorm=oracle.round_norms(rs(vr["norm"]), "f16"))
    with fanout.SharedArrays() as sh:
        for k_, v_ in sh_arrays.items():
            sh.put(k_, v_)
        res = pool.run(fp.decode_kv_head, [(s, G, kb, vb) for s in range(NSEQ)], sh)
    f = lambda a: a.astype(np.float64).reshape(1, NSEQ, Tt)
    one = oracle.decode(q.astype(np.float64).reshape(1, NSEQ * G, D), rs(kr["idx"])[None], rs(kr["signs"])[None],
                        f(sh_arrays["knorm"]), f(sh_arrays["krnorm"]), rs(vr["idx"])[None],
                        f(sh_arrays["vnorm"]), Pi, S, ck, cv)[0].reshape(NSEQ, G, D)
    for s in range(NSEQ):
        assert np.allclose(res[s][0], one[s], rtol=1e-12, atol=1e-13)   # from the records
        assert np.allclose(res[s][1], one[s], rtol=1e-12, atol=1e-13)   # end to end (same records)
