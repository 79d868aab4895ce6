#!/usr/bin/env python
"""Benchmark of the TurboQuant hot path on one MI355X (gfx950).

One step = one pass of the whole hot path over one batch of the batched
quantize + decode workload (batch 16, 8 KV heads, 32 query heads, d = 128,
131072 cached tokens per sequence): quantize every key (2-bit Lloyd-Max +
1-bit QJL sketch) and every value (3-bit Lloyd-Max) into the packed cache,
then decode one query token per (batch, query head) through softmax to the
weighted value sum, straight from the codes.  Inputs (bf16 K, V, Q) are
resident in HBM before the timed region starts.

Prints one JSON line on stdout; progress goes to stderr.
"""

import argparse
import functools
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
FP16_MFMA_PEAK_TFLOPS = 2500.0  # dense fp16 / bf16 matrix cores, published


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def _sha(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()


def key_record_bytes(bits, d=128, m=128, norm_bytes=2, hi=0):
    """Bytes of one packed key: code planes (one more plane for the hi/32
    leading words of a split stream), sign words, two norms."""
    return (((d + 31) // 32) * bits + hi // 32) * 4 + ((m + 31) // 32) * 4 + 2 * norm_bytes


def value_record_bytes(bits, d=128, norm_bytes=2, hi=0):
    """Bytes of one packed value: d fields of bits (+1 for the hi leading
    coordinates of a split stream), one norm."""
    return (d * bits + hi) // 8 + norm_bytes


def traffic_from_profiles(kernel_src, kernel_name, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when it is missing, was taken on another workload, or the kernel
    source changed since."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        t = json.load(open(p))
        e = t.get(f"{kernel_name} @ {workload}")
        if e is None or e.get("source_sha256") != _sha(kernel_src):
            return None
        return e["hbm_bytes_per_launch"]
    except Exception:
        return None


# ------------------------------------------------------------------ oracle
# The CPU baseline: the oracle (oracle/), as it stands, on a bounded sample
# of the same workload -- once on one core, once on every core of the host
# through a process pool over independent sequences / vector chunks.  Each
# stage's sampled rate prices that stage's share of a whole step.

@functools.lru_cache(maxsize=None)
def _oracle_tables(d, m, k_bits, v_bits, hadamard, hi):
    import oracle
    from kv_cache_vector_quantize_amd import inputs
    G, S = inputs.table_gaussians(d, m)
    Pi = oracle.randomized_hadamard(inputs.hadamard_signs(d)) if hadamard else oracle.rotation_from_gaussian(G)

    def cb(bits):
        if not bits:
            return None, None
        if hi:
            return oracle.split_codebook(d, hi, oracle.lloyd_max(d, bits), oracle.lloyd_max(d, bits + 1))
        return oracle.lloyd_max(d, bits)
    return Pi, S, cb(k_bits), cb(v_bits)


def _exact64(x):
    """Exact float64 values of bfloat16 bits (int16) or float32."""
    import numpy as np
    if x.dtype == np.int16:
        return (x.view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def oracle_job(arrs, task):
    """One unit of the oracle's work for the CPU baseline; returns (units
    done, seconds).  task = (stage, cfg, a, b); cfg = (d, m, k_bits, v_bits,
    hadamard, hi, norm dtype, tokens per sequence, heads per KV head)."""
    import numpy as np
    import oracle
    stage, cfg, a, b = task
    d, m, kb, vb, had, hi, nd, T, G = cfg
    Pi, S, (ck, tk), (cv, tv) = _oracle_tables(d, m, kb, vb, had, hi)
    t0 = time.perf_counter()
    if stage == "quantize_k":                       # vectors a .. b-1 of the key sample
        r = oracle.quantize_keys(_exact64(arrs["k"][a:b]), Pi, S, ck, tk)
        if hi:
            oracle.pack_key_codes_split(r["idx"], oracle.split_widths(d, kb, hi)[::32])
        else:
            oracle.pack_key_codes(r["idx"], kb)
        oracle.pack_signs(r["signs"])
        oracle.round_norms(r["norm"], nd)
        oracle.round_norms(r["rnorm"], nd)
        n = b - a
    elif stage == "quantize_v":                     # vectors a .. b-1 of the value sample
        r = oracle.quantize_values(_exact64(arrs["v"][a:b]), Pi, cv, tv)
        if hi:
            oracle.pack_value_codes_split(r["idx"].reshape(1, b - a, d), oracle.split_widths(d, vb, hi))
        else:
            oracle.pack_value_codes(r["idx"].reshape(1, b - a, d), vb)
        oracle.round_norms(r["norm"], nd)
        n = b - a
    elif stage == "logits":                         # the G heads of sequence a over tokens 0 .. b-1
        kidx = (oracle.unpack_key_codes_split(arrs["kcodes"][a, :b].view(np.uint32), d, oracle.split_widths(d, kb, hi)[::32])
                if hi else oracle.unpack_key_codes(arrs["kcodes"][a, :b].view(np.uint32), d))
        sg = oracle.unpack_signs(arrs["ksigns"][a, :b].view(np.uint32), m)
        kn, kr = arrs["knorm"][a, :b].astype(np.float64), arrs["krnorm"][a, :b].astype(np.float64)
        q = _exact64(arrs["q"][a])
        for g in range(G):
            oracle.key_logits(q[g], kidx, sg, kn, kr, Pi, S, ck)
        n = b
    elif stage == "decode":                         # query head 0 of sequence a over all T tokens
        kw, vw = arrs["kcodes"][a].view(np.uint32), arrs["vcodes"][a].view(np.uint32)
        if hi:
            kidx = oracle.unpack_key_codes_split(kw, d, oracle.split_widths(d, kb, hi)[::32])
            vidx = oracle.unpack_value_codes_split(vw[None], T, oracle.split_widths(d, vb, hi))[0]
        else:
            kidx = oracle.unpack_key_codes(kw, d)
            vidx = oracle.unpack_value_codes(vw[None], T)[0]
        sg = oracle.unpack_signs(arrs["ksigns"][a].view(np.uint32), m)
        f = lambda x: x.astype(np.float64)[None, None]
        oracle.decode(_exact64(arrs["q"][a, :1])[None], kidx[None, None], sg[None, None], f(arrs["knorm"][a]),
                      f(arrs["krnorm"][a]), vidx[None, None], f(arrs["vnorm"][a]), Pi, S, ck, cv)
        n = 1
    else:                                           # topk of score row a, k = b
        oracle.topk(arrs["scores"][a:a + 1].astype(np.float64), b)
        n = 1
    return n, time.perf_counter() - t0


def _time_oracle(sh, names, tasks, P, share):
    """Rates (units per second) of every stage: on one core (this process,
    tasks in turn until `share` seconds) and on P cores (a pool running one
    task per worker at once, after a first round that builds the workers'
    tables)."""
    from threadpoolctl import threadpool_limits

    from oracle import fanout
    arrs = fanout._attach(sh.spec)
    one, allc = {}, {}
    with threadpool_limits(limits=1):
        for name in names:
            units, secs = 0, 0.0
            for task in tasks(name, P):
                n, t = oracle_job(arrs, task)
                units, secs = units + n, secs + t
                if secs >= share:
                    break
            one[name] = units / secs
    del arrs
    with fanout.Pool(P) as pool:
        for name in names:
            ts = tasks(name, P)
            pool.run(oracle_job, ts, sh)
            t0 = time.perf_counter()
            res = pool.run(oracle_job, ts, sh)
            allc[name] = sum(n for n, _ in res) / (time.perf_counter() - t0)
    return one, allc


def cpu_baseline(w, stages, K, V, pk, pv, q, logits, budget_s=8.0, hadamard=False, hi=0):
    """The oracle, untouched, on a bounded sample of the same workload, on 1
    core and on every core.  Per stage: chunks of 32768 vectors (quantize),
    one KV head's query group over its sequence (logits), one query head
    over a whole sequence (decode), one score row (top-k).  Each stage's
    sampled rate prices the stage's algorithmic bytes in a whole step."""
    import numpy as np
    import torch

    from oracle import fanout

    P = fanout.default_workers()
    nvec = w.nseq * w.T
    chunk = min(32768, nvec)
    nchunks = max(1, min(P, nvec // chunk))   # distinct quantize chunks in the sample (tasks cycle over them)
    G = w.Hq // w.Hkv
    cfg = (w.d, w.m, w.k_bits, w.v_bits, hadamard, hi, w.norm_dtype, w.T, G)
    names = [st["name"] for st in stages]
    sh = fanout.SharedArrays()

    def host(name, t):
        t = t.contiguous()
        if t.dtype == torch.bfloat16:
            t = t.view(torch.int16)
        a = sh.empty(name, tuple(t.shape), {torch.int16: np.int16, torch.int32: np.int32,
                                            torch.float16: np.float16, torch.float32: np.float32}[t.dtype])
        torch.from_numpy(a).copy_(t)

    nq = min(P, w.nseq)              # sequences sampled for logits / decode
    if "quantize_k" in names:
        host("k", K.reshape(-1, w.d)[:nchunks * chunk])
    if "quantize_v" in names:
        host("v", V.reshape(-1, w.d)[:nchunks * chunk])
    if "logits" in names or "decode" in names:
        host("kcodes", pk.codes[:nq])
        host("ksigns", pk.signs[:nq])
        host("knorm", pk.norm[:nq])
        host("krnorm", pk.rnorm[:nq])
        host("q", q.reshape(w.nseq, G, w.d)[:nq])
        if "decode" in names:
            host("vcodes", pv.codes[:nq])
            host("vnorm", pv.norm[:nq])
    if "topk" in names:
        host("scores", logits.reshape(-1, w.T)[:min(P, w.B * w.Hq)])

    def tasks(name, count):
        if name in ("quantize_k", "quantize_v"):
            return [(name, cfg, (i % nchunks) * chunk, (i % nchunks + 1) * chunk) for i in range(count)]
        if name == "logits":
            return [(name, cfg, i % nq, w.T) for i in range(count)]
        if name == "decode":
            return [(name, cfg, i % nq, 0) for i in range(count)]
        return [(name, cfg, i % min(P, w.B * w.Hq), w.topk) for i in range(count)]

    # units of each stage per step, and its bytes per unit (as on the GPU)
    per_step = {"quantize_k": w.nseq * w.T, "quantize_v": w.nseq * w.T, "logits": w.nseq * w.T,
                "decode": w.B * w.Hq, "topk": w.B * w.Hq}
    try:
        one, allc = _time_oracle(sh, names, tasks, P, budget_s / len(stages))
    finally:
        sh.close()
    notes = []

    # seconds the oracle would take for one whole step, stage by stage
    est1 = sum(per_step[n] / one[n] for n in names)
    estP = sum(per_step[n] / allc[n] for n in names)
    total = sum(st["bytes"] for st in stages)
    unit_txt = {"quantize_k": "key vectors", "quantize_v": "value vectors", "logits": "tokens x KV heads",
                "decode": "query heads over a whole sequence", "topk": "score rows"}
    for name in names:
        notes.append(f"{name}: {one[name]:.4g} / {allc[name]:.4g} {unit_txt[name]} per s (1 / {P} cores)")
    return {
        "value": round(total / estP / 1e9, 4), "unit": "GB/s", "cores": P, "kind": "oracle",
        "sample": ("fp64 NumPy oracle, 1 BLAS thread per process, a process pool of " + str(P)
                   + " workers over independent sequences / 32768-vector chunks: " + "; ".join(notes)
                   + "; each stage's sampled rate prices its share of one step"),
        "single_core": {"value": round(total / est1 / 1e9, 4), "unit": "GB/s", "cores": 1},
        "cpu": _cpu_model(),
    }


def serve_leg(n, w, tk, tv, K, V, q, pk, pv, ws, out):
    """The serving loop at the workload's shape: n steps of (append one new
    key and value per sequence with tq_append, decode one query token per
    (batch, query head)), the context growing from T-n+1 to T tokens.  The
    streams end as they started (the appended tokens are the workload's own
    last n tokens, re-quantized bit for bit)."""
    import torch

    from kv_cache_vector_quantize_amd import tq
    T0 = w.T - n
    # new tokens, one [nseq][1][d] slab per step
    Kn = K[:, T0:].transpose(0, 1).contiguous().unsqueeze(2)
    Vn = V[:, T0:].transpose(0, 1).contiguous().unsqueeze(2)
    pk.capacity = pv.capacity = tq.padded_tokens(w.T)  # same buffers, now growable

    def run(evs=None):
        pk.T = pv.T = T0
        for i in range(n):
            if evs is not None:
                evs[i][0].record()
            tq.tq_append(tk, Kn[i], pk)
            if evs is not None:
                evs[i][1].record()
            tq.tq_append(tv, Vn[i], pv)
            if evs is not None:
                evs[i][2].record()
            tq.tq_attn_decode(tk, tv, q, pk, pv, w.B, w.Hq, w.Hkv, ws=ws, out=out)
            if evs is not None:
                evs[i][3].record()

    run()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n)]
    run(evs)
    torch.cuda.synchronize()
    assert pk.T == pv.T == w.T
    ak = sum(e[0].elapsed_time(e[1]) for e in evs) / n
    av = sum(e[1].elapsed_time(e[2]) for e in evs) / n
    dc = sum(e[2].elapsed_time(e[3]) for e in evs) / n
    ms = evs[0][0].elapsed_time(evs[-1][3]) / n
    log(f"serving: {n} steps, {ms:.3f} ms/step (append K {ak * 1e3:.1f} us, append V {av * 1e3:.1f} us, "
        f"decode {dc * 1e3:.1f} us)")
    del Kn, Vn
    return {"steps": n, "context": [T0 + 1, w.T], "ms_per_step": round(ms, 4),
            "append_k_us": round(ak * 1e3, 2), "append_v_us": round(av * 1e3, 2),
            "decode_us": round(dc * 1e3, 2),
            "new_tokens_per_s": round(w.B / (ms * 1e-3), 1),
            "step": "tq_append(K), tq_append(V), tq_attn_decode"}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except Exception:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3,
                    help="workload number 1-5 (default 3: batched quantize + decode)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rotation", choices=["qr", "hadamard"], default="qr",
                    help="qr: Pi = Q of a seeded Gaussian (the method as described); hadamard: the "
                         "randomized Walsh-Hadamard variant H diag(s) / sqrt(d)")
    ap.add_argument("--serve-steps", type=int, default=32,
                    help="decode workloads: also time this many serving steps (append one key "
                         "and one value per sequence, then decode) ending at the full context")
    ap.add_argument("--split", action="store_true",
                    help="fractional widths: keys and values at bits + 1/2 (the leading half of the "
                         "rotated coordinates at bits + 1; e.g. 2.5-bit keys + QJL, 3.5-bit values)")
    ap.add_argument("--cold", action="store_true", default=None,
                    help="also time every stage with the Infinity Cache flushed before each rep "
                         "(default: on for the tiny and Llama-8B logits workloads)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device-to-device copy (counter scaling)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: every input lives on one MI355X and "
              "nothing is sharded (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    from kv_cache_vector_quantize_amd import inputs, tq

    if not os.path.exists(tq._LIB_PATH):
        from kv_cache_vector_quantize_amd import build
        build.build()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = inputs.WORKLOADS[args.config]
    if args.cold is None:
        args.cold = args.config in (1, 2)
    dev = "cuda"
    d, m = w.d, w.m
    xb = 2 if w.x_dtype == "bf16" else 4
    log("workload", w.name)
    G, S = inputs.table_gaussians(d, m)
    had = args.rotation == "hadamard"
    hs = inputs.hadamard_signs(d) if had else None
    hi = d // 2 if args.split else 0
    if args.split and had:
        print("--split takes the QR rotation", file=sys.stderr)
        sys.exit(2)
    tk = tq.make_tables(G, S, w.k_bits, dev, hadamard_signs=hs, hi_coords=hi)
    tv = tq.make_tables(G, None, w.v_bits, dev, hadamard_signs=hs, hi_coords=hi) if w.v_bits else None
    rtag = (", hadamard" if had else "") + (", split" if hi else "")
    t0 = time.perf_counter()
    K = inputs.keys(w, device=dev).reshape(w.nseq, w.T, d)
    V = inputs.values(w, device=dev).reshape(w.nseq, w.T, d) if w.v_bits else None
    q = inputs.queries(w, device=dev).contiguous()
    pk = tq.alloc_packed(tq.TQ_KEY, tk, w.nseq, w.T, w.norm_dtype, dev)
    pv = tq.alloc_packed(tq.TQ_VALUE, tv, w.nseq, w.T, w.norm_dtype, dev) if w.v_bits else None
    nvec = w.nseq * w.T
    nb = 2 if w.norm_dtype == "f16" else 4
    kb = key_record_bytes(w.k_bits, d, m, nb, hi)
    vb = value_record_bytes(w.v_bits, d, nb, hi) if w.v_bits else 0
    qbytes = w.B * w.Hq * d * xb

    # the stages of one step, in order, with their algorithmic bytes.  The
    # quantize kernels reach fp32-grade products on the fp16 matrix cores
    # with hi + lo splits: the rotation takes X Pi_hi + X Pi_lo (one product
    # for the +-1 Walsh-Hadamard matrix), plus x_lo Pi_hi for fp32 input, and
    # the key sketch R_hi S_hi + R_hi S_lo + R_lo S_hi (R_hi S + R_lo S for a
    # sketch exact in float16, the tables' flag); "mfma_flop_per_unit" counts
    # those executed d x d products.
    rot_products = (1 if had else 2) + (1 if w.x_dtype == "f32" else 0)
    sketch_products = 2 if tk.sketch_f16 else 3
    G_ = w.Hq // w.Hkv
    # head dimensions other than 128: vector-ALU quantize, wide matrix-core
    # logits (one or two passes of 4 coordinate words)
    generic_d = not (d == 128 and m in (0, 128))
    if generic_d:
        kq_kernel = f"quantize_generic_kernel<{w.x_dtype}>"
    else:
        kq_kernel = f"quantize_keys_pipe_kernel<{w.x_dtype}, {w.k_bits}{rtag}>"
    if generic_d and G_ <= 8:
        lg_kernel = f"logits_wide_kernel<{G_}, {w.k_bits}, {nb}, {1 if max(d, m) <= 128 else 2}>"
    elif generic_d:
        lg_kernel = f"logits_generic_kernel<{G_}, {w.k_bits}>"
    elif G_ <= 8:
        lg_kernel = f"logits_mfma_kernel<{G_}, {w.k_bits}, {nb}>"
    else:
        lg_kernel = f"logits_kernel<{G_}>"
    stages = []
    if w.quantize_timed:
        stages.append({"name": "quantize_k", "bytes": nvec * (d * xb + kb), "units": nvec,
                       "fn": lambda: tq.tq_quantize(tk, K, pk),
                       "kernel": kq_kernel,
                       "flop_per_unit": 2 * d * d + 2 * m * d,
                       "mfma_flop_per_unit": (rot_products + sketch_products) * 2 * d * d})
        if w.v_bits:
            stages.append({"name": "quantize_v", "bytes": nvec * (d * xb + vb), "units": nvec,
                           "fn": lambda: tq.tq_quantize(tv, V, pv),
                           "kernel": (f"quantize_generic_kernel<{w.x_dtype}>" if generic_d
                                      else f"quantize_mfma_kernel<{w.x_dtype}, value, {w.v_bits}{rtag}>" if hi
                                      else f"quantize_values_pipe_kernel<{w.x_dtype}, {w.v_bits}{rtag}>"),
                           "flop_per_unit": 2 * d * d,
                           "mfma_flop_per_unit": rot_products * 2 * d * d})
    else:
        tq.tq_quantize(tk, K, pk)
        if w.v_bits:
            tq.tq_quantize(tv, V, pv)
    if w.logits:
        logits = torch.empty((w.B, w.Hq, w.T), dtype=torch.float32, device=dev)
        lws = torch.empty(max(tq.logits_workspace_bytes(w.B, w.Hq, d, m), 256), dtype=torch.uint8,
                          device=dev)
        stages.append({"name": "logits", "bytes": nvec * kb + w.B * w.Hq * w.T * 4 + qbytes,
                       "units": nvec,
                       "kernel": lg_kernel,
                       "fn": lambda: tq.tq_attn_logits(tk, q, pk, w.B, w.Hq, w.Hkv, ws=lws, out=logits),
                       "flop_per_unit": 2 * (w.Hq // w.Hkv) * (d + m)})
    if w.topk:
        rows = w.B * w.Hq
        scores2d = logits.view(rows, w.T)
        tws = torch.empty(tq.topk_workspace_bytes(rows, w.T, w.topk), dtype=torch.uint8, device=dev)
        t_idx = torch.empty((rows, w.topk), dtype=torch.int32, device=dev)
        t_val = torch.empty((rows, w.topk), dtype=torch.float32, device=dev)
        stages.append({"name": "topk", "bytes": rows * w.T * 4 + rows * w.topk * 8, "units": rows * w.T,
                       "kernel": "topk_chunk_kernel<16>",
                       "fn": lambda: tq.tq_topk(scores2d, w.topk, ws=tws, idx=t_idx, val=t_val),
                       "flop_per_unit": 0})
    if w.decode:
        ws = torch.empty(tq.decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.T, d, m), dtype=torch.uint8,
                         device=dev)
        out = torch.empty((w.B, w.Hq, d), dtype=torch.float32, device=dev)
        stages.append({"name": "decode", "bytes": nvec * (kb + vb) + qbytes + w.B * w.Hq * d * 4,
                       "units": nvec,
                       "kernel": f"decode_mfma_kernel<{G_}, {w.k_bits}, {w.v_bits}>" + (" (split)" if hi else ""),
                       "fn": lambda: tq.tq_attn_decode(tk, tv, q, pk, pv, w.B, w.Hq, w.Hkv, ws=ws, out=out),
                       "flop_per_unit": 2 * G_ * (2 * d + m)})
    torch.cuda.synchronize()
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s; stages: {[st['name'] for st in stages]}")

    ns = len(stages)

    def step(ev=None):
        for i, st in enumerate(stages):
            if ev is not None:
                ev[i].record()
            st["fn"]()
        if ev is not None:
            ev[ns].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(ns + 1)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        step(evs[i])
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = start.elapsed_time(end) / args.steps
    for i, st in enumerate(stages):
        st["ms_reps"] = [e[i].elapsed_time(e[i + 1]) for e in evs]
        st["ms"] = sum(st["ms_reps"]) / args.steps              # the average launch duration
        st["ms_median"] = statistics.median(st["ms_reps"])
    log(f"step {ms_step:.3f} ms (wall {wall / args.steps * 1e3:.3f} ms): "
        + ", ".join(f"{st['name']} {st['ms']:.3f} ms (median {st['ms_median']:.3f})" for st in stages))

    # Cold-cache reps: every stage again, each rep preceded by a 512 MiB
    # write that evicts the 256 MB Infinity Cache (the small workloads'
    # packed keys would otherwise be served from it)
    if args.cold:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        for st in stages:
            reps = []
            for r in range(args.steps):
                flush.fill_(r & 0xFF)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                st["fn"]()
                e1.record()
                torch.cuda.synchronize()
                reps.append(e0.elapsed_time(e1))
            st["cold_ms_median"] = statistics.median(reps)
        del flush
        log("cold cache: " + ", ".join(f"{st['name']} {st['cold_ms_median']:.3f} ms" for st in stages))

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log("copy calibration: 3 x 1 GiB device copies done")

    serving = serve_leg(args.serve_steps, w, tk, tv, K, V, q, pk, pv, ws, out) \
        if w.decode and args.serve_steps > 0 else None

    step_bytes = sum(st["bytes"] for st in stages)
    value = step_bytes / (ms_step * 1e-3) / 1e9

    # Roofline of the dominant kernel (the stage that takes longest).  Every
    # stage is bound by HBM at its algorithmic work: a key vector moves 308 B
    # (bf16 in, packed record out) against 65536 flop, a value 306 B against
    # 32768, decode 102 B per (token, KV head) against 2G(2d+m) flop, so at
    # the fp16 matrix-core peak all of them are bandwidth-bound.
    dom = max(stages, key=lambda st: st["ms"])
    src = {"quantize_k": "generic.hip" if generic_d else "quantize.hip",
           "quantize_v": "generic.hip" if generic_d else "quantize.hip",
           "logits": ("decode_kernels.h" if w.Hq // w.Hkv <= 8 else ("generic.hip" if generic_d else "attention.hip")),
           "decode": "decode_kernels.h", "topk": "topk.hip"}[dom["name"]]
    achieved = dom["bytes"] / (dom["ms"] * 1e-3) / 1e9
    # the time divided into is the stage's event-timed call: for decode and
    # logits that call launches query preparation (and decode's combine) too
    qprep = "qprep_generic_kernel" if generic_d else "qprep_kernel"
    calls = {"decode": f"tq_attn_decode: {qprep}, {dom['kernel']}, decode_combine_kernel",
             "logits": f"tq_attn_logits: {qprep}, {dom['kernel']}"}
    roofline = {
        "kernel": dom["kernel"],
        "timed_call": calls.get(dom["name"], dom["kernel"]),
        "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
        "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": traffic_from_profiles(os.path.join(ROOT, "kv_cache_vector_quantize_amd", "csrc", src),
                                         dom["kernel"], w.name),
        "algorithmic": {"bytes_per_unit": round(dom["bytes"] / dom["units"], 2), "units_per_launch": dom["units"],
                        "unit": "vector" if dom["name"].startswith("quantize") else "token of one KV head",
                        "flop_per_unit": dom["flop_per_unit"],
                        "algorithmic_tflops": round(dom["flop_per_unit"] * dom["units"] / (dom["ms"] * 1e-3) / 1e12, 2),
                        "fp16_mfma_peak_tflops": FP16_MFMA_PEAK_TFLOPS},
    }
    if dom["name"].startswith("quantize"):
        # the kernel's own bound: its HBM bytes at 8 TB/s or its executed
        # matrix-core work (the fp16 hi/lo split products) at 2.5 PFLOP/s
        hbm_ms = dom["bytes"] / (HBM_PEAK_GBS * 1e9) * 1e3
        mfma_ms = dom["mfma_flop_per_unit"] * dom["units"] / (FP16_MFMA_PEAK_TFLOPS * 1e12) * 1e3
        roofline["split_bound"] = {"hbm_ms": round(hbm_ms, 4), "split_mfma_ms": round(mfma_ms, 4),
                                   "bound_ms": round(max(hbm_ms, mfma_ms), 4),
                                   "frac": round(max(hbm_ms, mfma_ms) / dom["ms"], 4)}
    stage_report = {st["name"]: {"ms": round(st["ms_median"], 4), "ms_mean": round(st["ms"], 4),
                                 "gbs": round(st["bytes"] / (st["ms_median"] * 1e-3) / 1e9, 2),
                                 "frac_hbm": round(st["bytes"] / (st["ms_median"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
                    for st in stages}
    for st in stages:
        if "cold_ms_median" in st:
            stage_report[st["name"]]["cold_ms"] = round(st["cold_ms_median"], 4)
            stage_report[st["name"]]["cold_gbs"] = round(st["bytes"] / (st["cold_ms_median"] * 1e-3) / 1e9, 2)
    for st in stages:
        if st["name"].startswith("quantize"):
            stage_report[st["name"]]["mvec_s"] = round(nvec / (st["ms_median"] * 1e-3) / 1e6, 2)
            mf = st["mfma_flop_per_unit"] * st["units"] / (st["ms_median"] * 1e-3) / 1e12
            stage_report[st["name"]]["mfma_executed_tflops"] = round(mf, 2)
            stage_report[st["name"]]["mfma_frac_fp16_peak"] = round(mf / FP16_MFMA_PEAK_TFLOPS, 4)
        elif st["name"] == "topk":
            stage_report[st["name"]]["scores_per_s"] = round(st["units"] / (st["ms_median"] * 1e-3), 1)
        else:
            stage_report[st["name"]]["qhead_tokens_per_s"] = round(w.B * w.Hq * w.T / (st["ms_median"] * 1e-3), 1)
    inputs_desc = ("fp32" if w.x_dtype == "f32" else "bf16") + " K" + (", V" if w.v_bits else "") + ", Q"
    res = {
        "metric": "decode attn from packed KV: GB/s & % HBM peak; quantize Mvec/s",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16 hi/lo, f32 acc", "data": "synthetic",
        "precision": ("matrix products on fp16 hi/lo operand pairs with fp32 accumulation (fp32-grade "
                      "rotation, sketch and logits" +
                      ("; the sketch matrix is exact in fp16, so the sketch takes R_hi S + R_lo S"
                       if tk.sketch_f16 else "") +
                      "); decode's value contraction takes fp16 weights "
                      "and fp16 centroids; norms and softmax in fp32"),
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "T": w.T, "d": d,
                   "k_bits": w.k_bits + (0.5 if hi else 0), "qjl_m": m,
                   "v_bits": (w.v_bits + (0.5 if hi else 0)) if w.v_bits else 0, "norms": w.norm_dtype,
                   "inputs": inputs_desc, "rotation": args.rotation,
                   "step": [st["name"] for st in stages],
                   "parallelism": "1 GPU"},
        "frac_hbm_step": round(value / HBM_PEAK_GBS, 4),
        "stages": stage_report,
        "roofline": roofline,
        "serving": serving,
        "cpu_baseline": None,
    }
    if w.topk:
        call_ms = sum(st["ms"] for st in stages if st["name"] in ("logits", "topk"))
        res["search"] = {"database_keys": w.T, "queries_per_call": w.B * w.Hq, "k": w.topk,
                         "ms_per_call": round(call_ms, 4),
                         "queries_per_s": round(w.B * w.Hq / (call_ms * 1e-3), 1),
                         "step": "tq_attn_logits (scores of every key), tq_topk"}
    if not args.no_cpu_baseline:
        log("timing the oracle on a bounded CPU sample")
        res["cpu_baseline"] = cpu_baseline(w, stages, K, V, pk, pv, q, logits if w.logits else None,
                                           hadamard=had, hi=hi)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
