"""Full-coverage parity at the full sizes of the five hot-path workloads.

Every key and value vector of every workload is quantized on the GPU in
the launch configuration the benchmark times (one tq_quantize per stream),
and every code, sign bit and norm is checked against the oracle: the
oracle's work is fanned out over the host cores (oracle.fanout) and the
counts are aggregated, so the mismatch fraction is the fraction over the
whole workload.  Every decode row of the decode workloads is compared with
the oracle's decode of the GPU's own records (gated: 2e-3 relative per row),
and with the oracle's decode of its own quantization of the same inputs
(end to end, reported only, as is the end-to-end logits error).

Set TQ_PARITY_REPORT=<path> to append each workload's report as a JSON line.
"""

import json
import os

import numpy as np
import pytest
import torch

from oracle import fanout
from kv_cache_vector_quantize_amd import inputs, tq

import full_parity as fp
from gpu_common import gpu_tables, say
from parity import decode_close, logits_close

pytestmark = pytest.mark.gpu
D = M = 128


def report(cfg, what, rep):
    line = json.dumps({"workload": inputs.WORKLOADS[cfg].name, "check": what, **rep})
    say(line)
    path = os.environ.get("TQ_PARITY_REPORT")
    if path:
        with open(path, "a") as f:
            f.write(line + "\n")


@pytest.fixture(scope="module")
def pool():
    with fanout.Pool() as p:
        yield p


def _to_host(sh, name, t):
    """Copy a device tensor straight into a shared host array."""
    t = t.contiguous()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    dt = {torch.int16: np.int16, torch.int32: np.int32, torch.float16: np.float16,
          torch.float32: np.float32}[t.dtype]
    a = sh.empty(name, tuple(t.shape), dt)
    torch.from_numpy(a).copy_(t)
    return a


class Workload:
    """One workload's inputs and GPU records, on the device and in shared
    host memory."""

    def __init__(self, cfg):
        self.w = w = inputs.WORKLOADS[cfg]
        self.cfg = cfg
        self.keys = fanout.SharedArrays()
        self.vals = fanout.SharedArrays()
        say("full parity: generating and quantizing", w.name)
        self.tk = gpu_tables(D, M, w.k_bits)
        K = inputs.keys(w, device="cuda").reshape(w.nseq, w.T, D)
        self.pk = tq.alloc_packed(tq.TQ_KEY, self.tk, w.nseq, w.T, w.norm_dtype)
        tq.tq_quantize(self.tk, K, self.pk)
        self.q = inputs.queries(w, device="cuda").contiguous()
        torch.cuda.synchronize()
        for name, t in (("x", K), ("codes", self.pk.codes), ("signs", self.pk.signs),
                        ("norm", self.pk.norm), ("rnorm", self.pk.rnorm)):
            _to_host(self.keys, name, t)
        del K
        self.pv = None
        if w.v_bits:
            self.tv = gpu_tables(D, 0, w.v_bits)
            V = inputs.values(w, device="cuda").reshape(w.nseq, w.T, D)
            self.pv = tq.alloc_packed(tq.TQ_VALUE, self.tv, w.nseq, w.T, w.norm_dtype)
            tq.tq_quantize(self.tv, V, self.pv)
            torch.cuda.synchronize()
            for name, t in (("x", V), ("codes", self.pv.codes), ("norm", self.pv.norm)):
                _to_host(self.vals, name, t)
            del V

    def close(self):
        self.keys.close()
        self.vals.close()


@pytest.fixture(scope="module", params=[1, 2, 3, 4, 5])
def wl(request):
    W = Workload(request.param)
    yield W
    W.close()
    torch.cuda.empty_cache()


def test_every_key_vector(wl, pool):
    w = wl.w
    res = pool.run(fp.key_slice, fp.key_tasks(w.nseq, w.T, w.k_bits, w.norm_dtype), wl.keys)
    rep = fp.aggregate(res)
    report(wl.cfg, f"keys {w.k_bits}-bit + QJL, every vector", rep)
    assert rep["vectors"] == w.nseq * w.T
    assert rep["ok"], rep


def test_every_value_vector(wl, pool):
    w = wl.w
    if not w.v_bits:
        pytest.skip("workload has no value stream")
    res = pool.run(fp.value_slice, fp.value_tasks(w.nseq, w.T, w.v_bits, w.norm_dtype), wl.vals)
    rep = fp.aggregate(res)
    report(wl.cfg, f"values {w.v_bits}-bit, every vector", rep)
    assert rep["vectors"] == w.nseq * w.T
    assert rep["ok"], rep


def _attention_shared(wl):
    """Keys, values and queries of the workload, grouped per KV head, for the
    decode and logits jobs."""
    w = wl.w
    G = w.Hq // w.Hkv
    sh = fanout.SharedArrays()
    kspec, vspec = wl.keys.spec, wl.vals.spec
    # the jobs read the key / value arrays under other names: alias the blocks
    for src, dst in (("x", "k"), ("codes", "kcodes"), ("signs", "ksigns"), ("norm", "knorm"),
                     ("rnorm", "krnorm")):
        sh.spec[dst] = kspec[src]
    for src, dst in (("x", "v"), ("codes", "vcodes"), ("norm", "vnorm")):
        if src in vspec:
            sh.spec[dst] = vspec[src]
    _to_host(sh, "q", wl.q.reshape(w.B * w.Hkv, G, D))
    return sh


def test_every_decode_row(wl, pool):
    w = wl.w
    if not w.decode:
        pytest.skip("workload has no decode")
    G = w.Hq // w.Hkv
    out = tq.tq_attn_decode(wl.tk, wl.tv, wl.q, wl.pk, wl.pv, w.B, w.Hq, w.Hkv)
    got = out.reshape(w.B * w.Hkv, G, D).cpu().numpy()
    sh = _attention_shared(wl)
    try:
        res = pool.run(fp.decode_kv_head, [(s, G, w.k_bits, w.v_bits) for s in range(w.nseq)], sh)
    finally:
        sh.drop("q")
    ref = np.stack([r[0] for r in res])
    e2e = np.stack([r[1] for r in res])
    ok, worst = decode_close(got.reshape(-1, D), ref.reshape(-1, D))
    e2e_rel = np.linalg.norm(got - e2e, axis=-1) / np.linalg.norm(e2e, axis=-1)
    report(wl.cfg, "decode, every row", {
        "rows": int(got.shape[0] * got.shape[1]), "max_rel_err_vs_oracle_on_gpu_records": worst,
        "ok": ok, "end_to_end_max_rel_err": float(e2e_rel.max()),
        "end_to_end_median_rel_err": float(np.median(e2e_rel)),
        "end_to_end": "oracle codes -> oracle decode vs GPU codes -> GPU decode (reported, not gated)"})
    assert got.shape[0] * got.shape[1] == w.B * w.Hq
    assert ok, worst


def test_logits_end_to_end_report(wl, pool):
    """The gated logits parity (every logit, from the GPU's records) is in
    test_gpu_attention; this reports the end-to-end figure."""
    w = wl.w
    if not w.logits:
        pytest.skip("workload has no logits stage")
    G = w.Hq // w.Hkv
    got = tq.tq_attn_logits(wl.tk, wl.q, wl.pk, w.B, w.Hq, w.Hkv).reshape(w.nseq, G, w.T).cpu().numpy()
    sh = _attention_shared(wl)
    try:
        res = pool.run(fp.logits_kv_head, [(s, G, w.k_bits) for s in range(w.nseq)], sh)
    finally:
        sh.drop("q")
    e2e = np.stack(res)
    _, nbad, mx = logits_close(got, e2e)
    report(wl.cfg, "logits, end to end", {
        "logits": int(got.size), "outside_1e-4+1e-3|ref|": nbad,
        "fraction_outside": nbad / got.size, "max_abs_err": mx,
        "end_to_end": "oracle codes -> oracle logits vs GPU codes -> GPU logits (reported, not gated)"})
