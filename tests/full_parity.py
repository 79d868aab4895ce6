"""Worker jobs of the full-coverage parity tests (run through oracle.fanout).

Each job takes the shared host copies of a workload's inputs and of the
GPU's packed records, checks one slice of one sequence against the oracle
with the rules of ``parity``, and returns counts; the test aggregates them
over the whole workload.  Decode jobs return the oracle's output rows for
one KV head, computed from the GPU's records (the gated comparison) and from
the oracle's own quantization of the same inputs (the end-to-end figure,
reported only).
"""

import functools

import numpy as np

import oracle
from kv_cache_vector_quantize_amd import inputs

import parity


@functools.lru_cache(maxsize=None)
def tables(d, m, bits):
    G, S = inputs.table_gaussians(d, m)
    return oracle.rotation_from_gaussian(G), S, *oracle.lloyd_max(d, bits)


def as_f64(x):
    """Exact float64 values of host input vectors stored as bfloat16 bits
    (uint16) or float32."""
    if x.dtype in (np.uint16, np.int16):
        return (x.view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def key_slice(arrs, task):
    """task = (s, t0, t1, bits, norm_dtype): keys t0..t1-1 of sequence s."""
    s, t0, t1, bits, nd = task
    x = as_f64(arrs["x"][s, t0:t1])
    d = x.shape[-1]
    codes = arrs["codes"][s, t0:t1].view(np.uint32)
    signs = arrs["signs"][s, t0:t1].view(np.uint32)
    m = 32 * signs.shape[-1]
    Pi, S, c, t = tables(d, m, bits)
    idx = oracle.unpack_key_codes(codes, d)
    sg = oracle.unpack_signs(signs, m)
    rep = parity.check_key_stream(x, idx, sg, arrs["norm"][s, t0:t1], arrs["rnorm"][s, t0:t1],
                                  Pi, S, c, t, nd)
    return dict(vectors=t1 - t0, coords=idx.size + sg.size, code_mismatch=rep["code_mismatch"],
                code_bad=rep["code_mismatch_out_of_band"], sign_mismatch=rep["sign_mismatch"],
                sign_bad=rep["sign_mismatch_out_of_band"], norm_ok=rep["norm_ok"],
                rnorm_ok=rep["rnorm_ok"])


def value_slice(arrs, task):
    """task = (s, b0, b1, bits, norm_dtype): 32-token blocks b0..b1-1 of
    sequence s (the whole blocks the value records hold)."""
    s, b0, b1, bits, nd = task
    T = arrs["x"].shape[1]
    t0, t1 = 32 * b0, min(32 * b1, T)
    x = as_f64(arrs["x"][s, t0:t1])
    d = x.shape[-1]
    Pi, _, c, t = tables(d, 0, bits)
    words = arrs["codes"][s, b0:b1].view(np.uint32)[None]
    idx = oracle.unpack_value_codes(words, t1 - t0)[0]
    rep = parity.check_value_stream(x, idx, arrs["norm"][s, t0:t1], Pi, c, t, nd)
    # fields of padding tokens in the last block must be zero
    pad_ok = True
    if t1 < 32 * b1:
        full = oracle.unpack_value_codes(words, 32 * (b1 - b0))[0]
        pad_ok = bool(np.all(full[t1 - t0:] == 0))
    return dict(vectors=t1 - t0, coords=idx.size, code_mismatch=rep["code_mismatch"],
                code_bad=rep["code_mismatch_out_of_band"], sign_mismatch=0, sign_bad=0,
                norm_ok=rep["norm_ok"] and pad_ok, rnorm_ok=True)


def decode_kv_head(arrs, task):
    """task = (s, G, k_bits, v_bits): the G query heads that read KV head s.

    Returns (from_gpu_records [G, d], end_to_end [G, d]): the oracle's decode
    of those heads from the GPU's packed records, and from the oracle's own
    quantization of the same keys and values."""
    s, G, kb, vb = task
    q = as_f64(arrs["q"][s])                                   # [G, d]
    d = q.shape[-1]
    T = arrs["k"].shape[1]
    m = 32 * arrs["ksigns"].shape[-1]
    Pi, S, ck, tk = tables(d, m, kb)
    _, _, cv, tv = tables(d, 0, vb)
    f64 = lambda a: a.astype(np.float64)[None, None]
    gpu = oracle.decode_from_records(
        q[None], arrs["kcodes"][s].view(np.uint32)[None, None],
        arrs["ksigns"][s].view(np.uint32)[None, None],
        f64(arrs["knorm"][s]), f64(arrs["krnorm"][s]), arrs["vcodes"][s].view(np.uint32)[None, None],
        f64(arrs["vnorm"][s]), T, Pi, S, ck, cv)[0]
    # end to end: quantize with the oracle (in slices, to bound memory), then decode
    kidx = np.empty((T, d), dtype=np.uint8)
    ksg = np.empty((T, m), dtype=bool)
    kn, krn = np.empty(T), np.empty(T)
    vidx = np.empty((T, d), dtype=np.uint8)
    vn = np.empty(T)
    nd = "f16" if arrs["knorm"].dtype == np.float16 else "f32"
    for a in range(0, T, 32768):
        b = min(T, a + 32768)
        kr = oracle.quantize_keys(as_f64(arrs["k"][s, a:b]), Pi, S, ck, tk)
        kidx[a:b], ksg[a:b] = kr["idx"], kr["signs"]
        kn[a:b] = oracle.round_norms(kr["norm"], nd)
        krn[a:b] = oracle.round_norms(kr["rnorm"], nd)
        vr = oracle.quantize_values(as_f64(arrs["v"][s, a:b]), Pi, cv, tv)
        vidx[a:b] = vr["idx"]
        vn[a:b] = oracle.round_norms(vr["norm"], nd)
    e2e = oracle.decode(q[None], kidx[None, None], ksg[None, None], kn[None, None], krn[None, None],
                        vidx[None, None], vn[None, None], Pi, S, ck, cv)[0]
    return gpu, e2e


def logits_kv_head(arrs, task):
    """task = (s, G, k_bits): end-to-end logits of the G query heads of KV
    head s from the oracle's own quantization of the keys (reported only)."""
    s, G, kb = task
    q = as_f64(arrs["q"][s])
    d = q.shape[-1]
    m = 32 * arrs["ksigns"].shape[-1]
    Pi, S, ck, tk = tables(d, m, kb)
    kr = oracle.quantize_keys(as_f64(arrs["k"][s]), Pi, S, ck, tk)
    nd = "f16" if arrs["knorm"].dtype == np.float16 else "f32"
    kn = oracle.round_norms(kr["norm"], nd).astype(np.float64)
    krn = oracle.round_norms(kr["rnorm"], nd).astype(np.float64)
    return np.stack([oracle.key_logits(q[g], kr["idx"], kr["signs"], kn, krn, Pi, S, ck)
                     for g in range(G)])


def key_tasks(nseq, T, bits, nd, chunk=32768):
    return [(s, a, min(T, a + chunk), bits, nd) for s in range(nseq) for a in range(0, T, chunk)]


def value_tasks(nseq, T, bits, nd, chunk_blocks=1024):
    nb = (T + 31) // 32
    return [(s, a, min(nb, a + chunk_blocks), bits, nd) for s in range(nseq)
            for a in range(0, nb, chunk_blocks)]


def aggregate(results):
    tot = {k: 0 for k in ("vectors", "coords", "code_mismatch", "code_bad", "sign_mismatch", "sign_bad")}
    norm_ok = rnorm_ok = True
    for r in results:
        for k in tot:
            tot[k] += r[k]
        norm_ok &= r["norm_ok"]
        rnorm_ok &= r["rnorm_ok"]
    tot["mismatch_fraction"] = (tot["code_mismatch"] + tot["sign_mismatch"]) / max(tot["coords"], 1)
    tot["norm_ok"], tot["rnorm_ok"] = norm_ok, rnorm_ok
    tot["ok"] = (tot["code_bad"] == 0 and tot["sign_bad"] == 0 and norm_ok and rnorm_ok
                 and tot["mismatch_fraction"] <= parity.MAX_MISMATCH_FRACTION)
    return tot
