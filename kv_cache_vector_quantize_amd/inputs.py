"""Seeded synthetic inputs shared by the HIP path and the oracle.

This module draws random numbers and knows the workload shapes; it holds
none of the quantizer's arithmetic.  The Gaussian matrices that the method
itself needs (the one the rotation is built from and the sketch matrix) are
drawn here and handed to both sides as inputs.

Workloads stand in for the models and long-context suites the pages
evaluate on (P1 "Rotate, then quantize": Gemma, Mistral, Llama-3.1-8B on
LongBench / RULER / ZeroSCROLLS; P3 "Benchmarks"): only their shapes are
used -- 32 query / 8 KV heads for an 8B Llama layer, 64 / 8 for a 70B-class
layer, head dimension 128 -- with heavy-tailed keys and a few outlier
channels, the situation P1 gives as the reason for rotating first.
"""

from dataclasses import dataclass, field

import numpy as np
import torch

KIND_K, KIND_V, KIND_Q, KIND_OUTLIER = 0, 1, 2, 3
TABLE_SEED = 42


def table_gaussians(d=128, m=128, seed=TABLE_SEED):
    """G (d x d) for the rotation, then S (m x d) for the sketch, drawn in
    that order from one numpy PCG64 stream; float64.  The sketch matrix is
    stored at float16 precision: its draw is rounded once to float16 (a
    relative change of at most 2^-11 per entry), so that both sides use a
    matrix that is exact in float16."""
    rng = np.random.default_rng(seed)
    G = rng.standard_normal((d, d))
    S = rng.standard_normal((m, d)).astype(np.float16).astype(np.float64) if m > 0 else None
    return G, S


HADAMARD_SEED = 43


def hadamard_signs(d=128, seed=HADAMARD_SEED):
    """The d random signs (+-1, float64) of a randomized Walsh-Hadamard
    rotation, from a numpy PCG64 stream of their own."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, 2, size=d).astype(np.float64) * 2.0 - 1.0


@dataclass(frozen=True)
class Workload:
    name: str
    cfg: int
    B: int
    Hq: int
    Hkv: int
    T: int
    d: int = 128
    m: int = 128
    k_bits: int = 2
    v_bits: int = 0            # 0: no value stream
    x_dtype: str = "bf16"      # input dtype of K / V / Q
    norm_dtype: str = "f16"
    k_law: str = "normal_outliers"   # or "student_t_outliers"
    v_sigma: float = 1.0
    decode: bool = False       # whole decode (softmax + values) is part of it
    logits: bool = False       # logits only
    quantize_timed: bool = True
    topk: int = 0              # search: the k best keys per query after the logits

    @property
    def nseq(self):
        return self.B * self.Hkv


WORKLOADS = {
    1: Workload("tiny_logits_d128_n4096", 1, B=1, Hq=1, Hkv=1, T=4096, k_bits=2,
                x_dtype="f32", norm_dtype="f32", logits=True),
    2: Workload("llama8b_logits_32q8kv_T32768", 2, B=1, Hq=32, Hkv=8, T=32768, k_bits=3,
                k_law="student_t_outliers", logits=True, quantize_timed=False),
    3: Workload("batched_quant_decode_B16_8kv_T131072", 3, B=16, Hq=32, Hkv=8, T=131072,
                k_bits=2, v_bits=3, v_sigma=0.5, decode=True),
    4: Workload("prefill_quantize_1M_tokens_8kv", 4, B=1, Hq=8, Hkv=8, T=1048576,
                k_bits=3, v_bits=4, v_sigma=1.0),
    5: Workload("70b_long_decode_64q8kv_T524288", 5, B=1, Hq=64, Hkv=8, T=524288,
                k_bits=2, v_bits=3, k_law="student_t_outliers", v_sigma=1.0, decode=True,
                quantize_timed=False),
    # Inner-product search (the pages' second workload: GloVe vectors, d = 200,
    # judged by top-k recall), as a synthetic stand-in at the pages' dimension:
    # one database of 2^20 keys (3-bit codes + QJL with m = d = 200 sketch
    # rows), 8 queries per call, top 10.
    6: Workload("search_d200_N1M_q8_top10", 6, B=1, Hq=8, Hkv=1, T=1048576, d=200, m=200, k_bits=3,
                logits=True, quantize_timed=False, topk=10),
}

# Channels scaled x20 in the "normal with outliers" key law (tiny workload).
FIXED_OUTLIER_CHANNELS = (3, 17, 64, 101)


def _seed(cfg, kind, b, h):
    return ((((1000 + cfg) * 8 + kind) * 4096 + b) * 4096 + h) & 0x7FFFFFFFFFFFFFFF


def _gen(device, cfg, kind, b, h):
    g = torch.Generator(device=device)
    g.manual_seed(_seed(cfg, kind, b, h))
    return g


def _cast(x, dtype):
    return x.to(torch.bfloat16) if dtype == "bf16" else x.to(torch.float32)


def key_slice(w, b, h, device="cpu", T=None):
    """Keys of one (batch, kv-head) sequence: [T, d] in the workload dtype."""
    T = w.T if T is None else T
    g = _gen(device, w.cfg, KIND_K, b, h)
    if w.k_law == "normal_outliers":
        x = torch.randn((T, w.d), generator=g, device=device, dtype=torch.float32)
        scale = torch.ones(w.d, device=device)
        scale[list(c for c in FIXED_OUTLIER_CHANNELS if c < w.d)] = 20.0
        x = x * scale
    elif w.k_law == "student_t_outliers":
        z = torch.randn((T, w.d), generator=g, device=device, dtype=torch.float32)
        u1 = 1.0 - torch.rand((T, w.d), generator=g, device=device, dtype=torch.float32)
        u2 = 1.0 - torch.rand((T, w.d), generator=g, device=device, dtype=torch.float32)
        chi2_4 = -2.0 * torch.log(u1 * u2)          # chi-square with 4 dof
        x = z / torch.sqrt(chi2_4 / 4.0)            # Student-t, nu = 4 (variance 2)
        go = _gen(device, w.cfg, KIND_OUTLIER, b, h)
        n_out = int(round(0.02 * w.d))
        ch = torch.randperm(w.d, generator=go, device=device)[:n_out]
        scale = torch.ones(w.d, device=device)
        scale[ch] = 10.0
        x = x * scale
    else:
        raise ValueError(w.k_law)
    return _cast(x, w.x_dtype)


def value_slice(w, b, h, device="cpu", T=None):
    T = w.T if T is None else T
    g = _gen(device, w.cfg, KIND_V, b, h)
    x = torch.randn((T, w.d), generator=g, device=device, dtype=torch.float32) * w.v_sigma
    return _cast(x, w.x_dtype)


def queries(w, device="cpu"):
    """[B, Hq, d] queries, N(0, 1), in the workload dtype."""
    out = []
    for b in range(w.B):
        g = _gen(device, w.cfg, KIND_Q, b, 0)
        out.append(torch.randn((w.Hq, w.d), generator=g, device=device, dtype=torch.float32))
    return _cast(torch.stack(out), w.x_dtype)


def keys(w, device="cpu", T=None):
    """[B, Hkv, T, d]."""
    T = w.T if T is None else T
    t = torch.empty((w.B, w.Hkv, T, w.d), device=device,
                    dtype=torch.bfloat16 if w.x_dtype == "bf16" else torch.float32)
    for b in range(w.B):
        for h in range(w.Hkv):
            t[b, h] = key_slice(w, b, h, device, T)
    return t


def values(w, device="cpu", T=None):
    T = w.T if T is None else T
    t = torch.empty((w.B, w.Hkv, T, w.d), device=device,
                    dtype=torch.bfloat16 if w.x_dtype == "bf16" else torch.float32)
    for b in range(w.B):
        for h in range(w.Hkv):
            t[b, h] = value_slice(w, b, h, device, T)
    return t


def random_vectors(n, d, seed, device="cpu", dtype="f32", scale=1.0):
    """Plain N(0, scale^2) vectors for unit tests."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn((n, d), generator=g, device=device, dtype=torch.float32) * scale
    return _cast(x, dtype)
