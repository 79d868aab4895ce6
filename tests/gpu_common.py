"""Shared set-up for the GPU parity tests: tables built on the device by
libtq and, independently, by the oracle from the same Gaussian draws."""

import functools
import sys

import numpy as np
import torch

import oracle
from kv_cache_vector_quantize_amd import inputs, tq


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


@functools.lru_cache(maxsize=None)
def oracle_tables(d, m, bits):
    G, S = inputs.table_gaussians(d, m)
    Pi = oracle.rotation_from_gaussian(G)
    c, t = oracle.lloyd_max(d, bits)
    return Pi, S, c, t


_gpu_cache = {}


def gpu_tables(d, m, bits):
    key = (d, m, bits)
    if key not in _gpu_cache:
        G, S = inputs.table_gaussians(d, m)
        _gpu_cache[key] = tq.make_tables(G, S if m > 0 else None, bits)
    return _gpu_cache[key]


def host(t):
    return t.detach().cpu()


def key_records(p):
    """Unpack a GPU key stream to (idx [nseq,T,d], signs [nseq,T,m], norm, rnorm)."""
    codes = host(p.codes).numpy().view(np.uint32)
    signs = host(p.signs).numpy().view(np.uint32)
    idx = oracle.unpack_key_codes(codes, p.d)
    sg = oracle.unpack_signs(signs, p.m)
    return idx, sg, host(p.norm).numpy(), host(p.rnorm).numpy()


def value_records(p):
    codes = host(p.codes).numpy().view(np.uint32)
    idx = oracle.unpack_value_codes(codes, p.T)
    return idx, host(p.norm).numpy()


def to64(x):
    """Exact fp64 values of a float32 / bfloat16 tensor."""
    return host(x).float().double().numpy()
