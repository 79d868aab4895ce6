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
import hashlib
import json
import math
import os
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


def key_record_bytes(bits, d=128, m=128, norm_bytes=2):
    return (d // 32) * bits * 4 + (m // 32) * 4 + 2 * norm_bytes


def value_record_bytes(bits, d=128, norm_bytes=2):
    return (d // 32) * bits * 4 + norm_bytes


def traffic_from_profiles(kernel_src, kernel_name):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when it is missing or the kernel source changed since."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        t = json.load(open(p))
        e = t.get(kernel_name)
        if e is None or e.get("source_sha256") != _sha(kernel_src):
            return None
        return e["hbm_bytes_per_launch"]
    except Exception:
        return None


def cpu_baseline(w, K, V, pk, pv, q, budget_s=12.0):
    """The oracle, untouched, on a bounded sample of the same workload:
    quantize chunks of keys and values (and pack them) until about
    `budget_s` seconds have passed, plus one decode row over a full
    sequence from the GPU's packed records.  BLAS pinned to one thread."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    from kv_cache_vector_quantize_amd import inputs

    d, m = w.d, w.m
    G, S = inputs.table_gaussians(d, m)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        Pi = oracle.rotation_from_gaussian(G)
        ck, tk = oracle.lloyd_max(d, w.k_bits)
        cv, tv = oracle.lloyd_max(d, w.v_bits)
        setup_s = time.perf_counter() - t0
        # decode of one (batch 0, head 0) row over all T tokens
        kc = pk.codes[0].cpu().numpy().view(np.uint32)[None, None]
        ks = pk.signs[0].cpu().numpy().view(np.uint32)[None, None]
        kn = pk.norm[0].cpu().numpy().astype(np.float64)[None, None]
        kr = pk.rnorm[0].cpu().numpy().astype(np.float64)[None, None]
        vc = pv.codes[0].cpu().numpy().view(np.uint32)[None, None]
        vn = pv.norm[0].cpu().numpy().astype(np.float64)[None, None]
        qq = q[0:1, 0:1].float().double().cpu().numpy()
        t0 = time.perf_counter()
        oracle.decode_from_records(qq, kc, ks, kn, kr, vc, vn, w.T, Pi, S, ck, cv)
        dec_s = time.perf_counter() - t0
        dec_bytes = w.T * (key_record_bytes(w.k_bits) + value_record_bytes(w.v_bits))
        # quantize + pack chunks of 32768 keys and 32768 values
        chunk, nvec, q_s = 32768, 0, 0.0
        flat_k = K.reshape(-1, d)
        flat_v = V.reshape(-1, d)
        while q_s < budget_s and (nvec + chunk) <= flat_k.shape[0]:
            xk = flat_k[nvec:nvec + chunk].float().double().cpu().numpy()
            xv = flat_v[nvec:nvec + chunk].float().double().cpu().numpy()
            t0 = time.perf_counter()
            rk = oracle.quantize_keys(xk, Pi, S, ck, tk)
            oracle.pack_key_codes(rk["idx"], w.k_bits)
            oracle.pack_signs(rk["signs"])
            oracle.round_norms(rk["norm"], w.norm_dtype)
            oracle.round_norms(rk["rnorm"], w.norm_dtype)
            rv = oracle.quantize_values(xv, Pi, cv, tv)
            oracle.pack_value_codes(rv["idx"].reshape(1, chunk, d), w.v_bits)
            oracle.round_norms(rv["norm"], w.norm_dtype)
            q_s += time.perf_counter() - t0
            nvec += chunk
    q_bytes = nvec * (2 * w.d * 2 + key_record_bytes(w.k_bits) + value_record_bytes(w.v_bits))
    total_s = q_s + dec_s
    gbs = (q_bytes + dec_bytes) / total_s / 1e9
    return {
        "value": round(gbs, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
        "sample": (f"fp64 NumPy oracle, 1 BLAS thread: quantize+pack {nvec} keys and {nvec} values "
                   f"({q_s:.1f} s) and one decode row over all {w.T} tokens of a sequence "
                   f"({dec_s:.1f} s); {nvec * 2 / q_s / 1e6:.3f} Mvec/s quantize, "
                   f"{dec_bytes / dec_s / 1e9:.3f} GB/s decode; table setup {setup_s:.1f} s excluded"),
        "cpu": _cpu_model(),
    }


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
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3, help="workload number (3 = batched quantize+decode)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device-to-device copy (counter scaling)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build measures one GPU only; every input lives on one MI355X and "
              "nothing is sharded (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    from kv_cache_vector_quantize_amd import inputs, tq

    if not os.path.exists(tq._LIB_PATH):
        from kv_cache_vector_quantize_amd import build
        build.build()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = inputs.WORKLOADS[args.config]
    if not (w.decode and w.v_bits):
        raise SystemExit("bench.py runs the quantize + decode workloads (3)")
    dev = "cuda"
    d, m = w.d, w.m
    log("workload", w.name)
    G, S = inputs.table_gaussians(d, m)
    tk = tq.make_tables(G, S, w.k_bits, dev)
    tv = tq.make_tables(G, None, w.v_bits, dev)
    t0 = time.perf_counter()
    K = inputs.keys(w, device=dev).reshape(w.nseq, w.T, d)
    V = inputs.values(w, device=dev).reshape(w.nseq, w.T, d)
    q = inputs.queries(w, device=dev).contiguous()
    pk = tq.alloc_packed(tq.TQ_KEY, tk, w.nseq, w.T, w.norm_dtype, dev)
    pv = tq.alloc_packed(tq.TQ_VALUE, tv, w.nseq, w.T, w.norm_dtype, dev)
    ws = torch.empty(tq.decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.T, d, m), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((w.B, w.Hq, d), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s")

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        tq.tq_quantize(tk, K, pk)
        if ev is not None:
            ev[1].record()
        tq.tq_quantize(tv, V, pv)
        if ev is not None:
            ev[2].record()
        tq.tq_attn_decode(tk, tv, q, pk, pv, w.B, w.Hq, w.Hkv, ws=ws, out=out)
        if ev is not None:
            ev[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
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
    qk_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    qv_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    dec_ms = sum(e[2].elapsed_time(e[3]) for e in evs) / args.steps
    log(f"step {ms_step:.3f} ms (wall {wall / args.steps * 1e3:.3f} ms): quantize K {qk_ms:.3f}, "
        f"quantize V {qv_ms:.3f}, decode {dec_ms:.3f} ms")

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log("copy calibration: 3 x 1 GiB device copies done")

    nvec = w.nseq * w.T
    kb, vb = key_record_bytes(w.k_bits), value_record_bytes(w.v_bits)
    qk_bytes = nvec * (d * 2 + kb)
    qv_bytes = nvec * (d * 2 + vb)
    dec_bytes = nvec * (kb + vb) + w.B * w.Hq * d * (2 + 4)
    step_bytes = qk_bytes + qv_bytes + dec_bytes
    qk_flops = nvec * (2 * d * d + 2 * m * d)
    value = step_bytes / (ms_step * 1e-3) / 1e9

    # Roofline of the dominant kernel (key quantization).  Per key vector the
    # method reads d bf16 elements and writes one packed record, and does
    # 2 d^2 (rotation) + 2 m d (sketch) flops: 308 B against 65536 flop, so
    # at the fp16 matrix-core peak it is bound by HBM.
    qsrc = os.path.join(ROOT, "kv_cache_vector_quantize_amd", "csrc", "quantize.hip")
    kname = f"quantize_mfma_kernel<bf16, key, {w.k_bits}>"
    achieved = qk_bytes / (qk_ms * 1e-3) / 1e9
    traffic = traffic_from_profiles(qsrc, kname)
    roofline = {
        "kernel": kname,
        "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
        "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": traffic,
        "algorithmic": {"bytes_per_vector": d * 2 + kb, "vectors_per_launch": nvec,
                        "flop_per_vector": 2 * d * d + 2 * m * d,
                        "algorithmic_tflops": round(qk_flops / (qk_ms * 1e-3) / 1e12, 2),
                        "fp16_mfma_peak_tflops": FP16_MFMA_PEAK_TFLOPS},
    }
    dec_gbs = dec_bytes / (dec_ms * 1e-3) / 1e9
    res = {
        "metric": "decode attn from packed KV: GB/s & % HBM peak; quantize Mvec/s",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "T": w.T, "d": d,
                   "k_bits": w.k_bits, "qjl_m": m, "v_bits": w.v_bits, "norms": w.norm_dtype,
                   "inputs": "bf16 K, V, Q", "parallelism": "1 GPU"},
        "frac_hbm_step": round(value / HBM_PEAK_GBS, 4),
        "quantize_mvec_s": round(2 * nvec / ((qk_ms + qv_ms) * 1e-3) / 1e6, 2),
        "quantize_k_ms": round(qk_ms, 4), "quantize_v_ms": round(qv_ms, 4),
        "decode_ms": round(dec_ms, 4), "decode_gbs": round(dec_gbs, 2),
        "decode_frac_hbm": round(dec_gbs / HBM_PEAK_GBS, 4),
        "decode_qhead_tokens_per_s": round(w.B * w.Hq * w.T / (dec_ms * 1e-3), 1),
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("timing the oracle on a bounded CPU sample")
        res["cpu_baseline"] = cpu_baseline(w, K, V, pk, pv, q)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
