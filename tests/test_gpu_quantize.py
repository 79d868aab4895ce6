"""GPU parity of tq_quantize against the oracle (codes, signs, norms)."""

import numpy as np
import pytest
import torch

import oracle
from kv_cache_vector_quantize_amd import inputs, tq

from gpu_common import gpu_tables, key_records, oracle_tables, say, to64, value_records
from parity import check_key_stream, check_value_stream

pytestmark = pytest.mark.gpu
D = M = 128


def _quantize_keys(X, bits, norm_dtype):
    nseq, T, _ = X.shape
    tabs = gpu_tables(D, M, bits)
    p = tq.alloc_packed(tq.TQ_KEY, tabs, nseq, T, norm_dtype)
    tq.tq_quantize(tabs, X, p)
    torch.cuda.synchronize()
    return p


def _quantize_values(X, bits, norm_dtype):
    nseq, T, _ = X.shape
    tabs = gpu_tables(D, 0, bits)
    p = tq.alloc_packed(tq.TQ_VALUE, tabs, nseq, T, norm_dtype)
    tq.tq_quantize(tabs, X, p)
    torch.cuda.synchronize()
    return p


def _check_keys(X, p, bits, norm_dtype, rows=None):
    Pi, S, c, t = oracle_tables(D, M, bits)
    idx, sg, n, rn = key_records(p)
    x = to64(X).reshape(-1, D)
    idx, sg, n, rn = idx.reshape(-1, D), sg.reshape(-1, M), n.reshape(-1), rn.reshape(-1)
    if rows is not None:
        x, idx, sg, n, rn = x[rows], idx[rows], sg[rows], n[rows], rn[rows]
    rep = check_key_stream(x, idx, sg, n, rn, Pi, S, c, t, norm_dtype)
    assert rep["ok"], rep
    return rep


def _check_values(X, p, bits, norm_dtype):
    Pi, _, c, t = oracle_tables(D, 0, bits)
    idx, n = value_records(p)
    rep = check_value_stream(to64(X).reshape(-1, D), idx.reshape(-1, D), n.reshape(-1), Pi, c, t,
                             norm_dtype)
    assert rep["ok"], rep
    return rep


def test_tiny_keys_fp32_input_fp32_norms():
    w = inputs.WORKLOADS[1]
    say("quantize tiny keys", w.name)
    X = inputs.key_slice(w, 0, 0, device="cuda").unsqueeze(0).contiguous()
    p = _quantize_keys(X, w.k_bits, "f32")
    _check_keys(X, p, w.k_bits, "f32")


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_bf16_keys_student_t_ragged(bits):
    w = inputs.WORKLOADS[2]
    say("quantize bf16 keys", bits)
    X = inputs.key_slice(w, 0, 3, device="cuda", T=1000).reshape(2, 500, D).contiguous()
    p = _quantize_keys(X, bits, "f16")
    _check_keys(X, p, bits, "f16")
    # the padding tokens 500 .. 511 of each sequence hold a zero vector's record
    assert p.Tp == 512
    codes = p.buf_codes[:, 500:].cpu().numpy().view(np.uint32)
    idx = oracle.unpack_key_codes(codes, D)
    assert np.all(idx == 1 << (bits - 1))
    assert np.all(p.buf_signs[:, 500:].cpu().numpy().view(np.uint32) == 0xFFFFFFFF)
    assert not torch.any(p.buf_norm[:, 500:]) and not torch.any(p.buf_rnorm[:, 500:])


@pytest.mark.parametrize("bits", [2, 3])
def test_keys_general_sketch(bits):
    """A sketch that is not exact in float16 takes the three-product sketch
    (R_hi S_hi + R_hi S_lo + R_lo S_hi): parity with the oracle on that S."""
    say("quantize keys, sketch not exact in float16", bits)
    G, _ = inputs.table_gaussians(D, M)
    S = np.random.default_rng(7).standard_normal((M, D))
    tabs = tq.make_tables(G, S, bits)
    assert tabs.sketch_f16 == 0
    # 2 x 16000 tokens: 1000 units, so that workgroups of the pipelined kernel
    # take several units (its loop body, not only its prologue and epilogue)
    w = inputs.WORKLOADS[2]
    X = inputs.key_slice(w, 0, 1, device="cuda", T=32000).reshape(2, 16000, D).contiguous()
    p = tq.alloc_packed(tq.TQ_KEY, tabs, 2, 16000, "f16")
    tq.tq_quantize(tabs, X, p)
    torch.cuda.synchronize()
    Pi = oracle.rotation_from_gaussian(G)
    c, t = oracle.lloyd_max(D, bits)
    idx, sg, n, rn = key_records(p)
    rep = check_key_stream(to64(X).reshape(-1, D), idx.reshape(-1, D), sg.reshape(-1, M), n.reshape(-1),
                           rn.reshape(-1), Pi, S, c, t, "f16")
    assert rep["ok"], rep


@pytest.mark.parametrize("x_dtype,rotation,hi", [
    (torch.bfloat16, "dense", 0), (torch.float32, "dense", 0), (torch.bfloat16, "hadamard", 0),
    (torch.float32, "hadamard", 0), (torch.bfloat16, "dense", D // 2), (torch.float32, "dense", D // 2)])
def test_float16_sketch_flag_gives_the_same_records(x_dtype, rotation, hi):
    """With a sketch exact in float16, the two-product path (tables flag set)
    writes the records of the three-product one bit for bit -- the dropped
    product only adds zeros -- for every instance of the whole-stream key
    kernel: both input types, both rotations, uniform and split widths."""
    say("quantize keys, float16 sketch flag on / off", x_dtype, rotation, hi)
    G, S = inputs.table_gaussians(D, M)
    hs = inputs.hadamard_signs(D) if rotation == "hadamard" else None
    t16 = tq.make_tables(G, S, 2, hadamard_signs=hs, hi_coords=hi)
    t32 = tq.make_tables(G, S, 2, hadamard_signs=hs, hi_coords=hi, sketch_f16=False)
    assert t16.sketch_f16 == 1 and t32.sketch_f16 == 0
    w = inputs.WORKLOADS[3]
    # 4 x 10000 tokens: 1252 units, several per workgroup
    X = inputs.key_slice(w, 1, 2, device="cuda", T=40000).to(x_dtype).reshape(4, 10000, D).contiguous()
    out = []
    for tabs in (t16, t32):
        p = tq.alloc_packed(tq.TQ_KEY, tabs, 4, 10000, "f16")
        tq.tq_quantize(tabs, X, p)
        out.append(p)
    torch.cuda.synchronize()
    a, b = out
    for f in ("buf_codes", "buf_signs", "buf_norm", "buf_rnorm"):
        assert torch.equal(getattr(a, f).view(torch.uint8), getattr(b, f).view(torch.uint8)), f


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_bf16_values_ragged_blocks(bits):
    w = inputs.WORKLOADS[4]
    say("quantize bf16 values", bits)
    X = inputs.value_slice(w, 0, 1, device="cuda", T=3 * 333).reshape(3, 333, D).contiguous()
    p = _quantize_values(X, bits, "f16")
    _check_values(X, p, bits, "f16")
    # fields of the padded tokens of the last block are zero
    codes = p.codes.cpu().numpy().view(np.uint32)
    tail = 333 - 32 * 10
    for s_ in range(3):
        for j in range(D):
            rec = sum(int(codes[s_, 10, j, q]) << (32 * q) for q in range(bits))
            assert rec >> (bits * tail) == 0
    assert not torch.any(p.buf_norm[:, 333:])


def test_fp32_values_ragged():
    w = inputs.WORKLOADS[1]
    say("quantize fp32 values", w.name)
    X = inputs.value_slice(w, 0, 0, device="cuda", T=2 * 77).reshape(2, 77, D).contiguous()
    assert X.dtype == torch.float32
    for bits in (2, 4):
        p = _quantize_values(X, bits, "f32")
        _check_values(X, p, bits, "f32")


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_bf16_streams_several_units_per_workgroup(bits):
    """Keys and values of every width through the pipelined kernels' loop
    body: 32000 + 9 tokens, about 1000 units, more than the workgroups."""
    w = inputs.WORKLOADS[4]
    say("quantize bf16 streams of many units", bits)
    T = 32009
    K = inputs.key_slice(w, 0, 2, device="cuda", T=T).reshape(1, T, D).contiguous()
    _check_keys(K, _quantize_keys(K, bits, "f16"), bits, "f16")
    V = inputs.value_slice(w, 0, 2, device="cuda", T=T).reshape(1, T, D).contiguous()
    _check_values(V, _quantize_values(V, bits, "f16"), bits, "f16")


@pytest.mark.parametrize("role", ["key", "value"])
def test_fp32_streams_several_units_per_workgroup(role):
    """fp32 input keeps one unit of input in flight in the pipelined kernels
    (one register buffer for every unit): streams of more units than
    workgroups run their loop body, with a ragged last block."""
    w = inputs.WORKLOADS[1]
    say("quantize fp32 stream of many units", role)
    T = 3 * 10000 + 17
    if role == "key":
        X = inputs.key_slice(w, 0, 0, device="cuda", T=T).reshape(1, T, D).contiguous()
        p = _quantize_keys(X, 2, "f32")
        _check_keys(X, p, 2, "f32")
    else:
        X = inputs.value_slice(w, 0, 0, device="cuda", T=T).reshape(1, T, D).contiguous()
        p = _quantize_values(X, 3, "f32")
        _check_values(X, p, 3, "f32")
    assert X.dtype == torch.float32


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_extreme_magnitudes(dtype):
    """Per-vector power-of-two range scaling: vectors from 1e-30 to 1e30 (the
    squares of the large ones overflow float32, the small ones' underflow)
    quantize exactly as at unit scale."""
    say("quantize extreme magnitudes", dtype)
    g = torch.Generator().manual_seed(11)
    scales = torch.tensor([1e-30, 1e-12, 1e-3, 1.0, 1e3, 1e12, 1e30], dtype=torch.float64)
    X = torch.randn((len(scales), 40, D), generator=g, dtype=torch.float64) * scales[:, None, None]
    X = X.to(dtype).to("cuda").contiguous()
    p = _quantize_keys(X, 3, "f32")
    _check_keys(X, p, 3, "f32")
    pv = _quantize_values(X, 2, "f32")
    _check_values(X, pv, 2, "f32")


def test_zero_vectors_and_single_token():
    say("quantize zero vectors")
    X = torch.randn((3, 1, D), device="cuda")
    X[1] = 0.0
    p = _quantize_keys(X.contiguous(), 2, "f32")
    idx, sg, n, rn = key_records(p)
    assert n[1, 0] == 0 and rn[1, 0] == 0
    assert np.all(idx[1, 0] == 2) and np.all(sg[1, 0])
    _check_keys(X, p, 2, "f32")
    pv = _quantize_values(X.contiguous(), 3, "f32")
    vidx, vn = value_records(pv)
    assert vn[1, 0] == 0 and np.all(vidx[1, 0] == 4)


def test_empty_inputs_are_noops():
    say("quantize empty")
    tabs = gpu_tables(D, M, 2)
    for nseq, T in ((0, 5), (2, 0)):
        p = tq.alloc_packed(tq.TQ_KEY, tabs, nseq, T, "f16")
        tq.tq_quantize(tabs, torch.empty((nseq, T, D), device="cuda"), p)
    torch.cuda.synchronize()


def test_deterministic_across_runs():
    w = inputs.WORKLOADS[2]
    say("quantize determinism")
    X = inputs.key_slice(w, 0, 0, device="cuda", T=4096).unsqueeze(0).contiguous()
    a = _quantize_keys(X, 3, "f16")
    b = _quantize_keys(X, 3, "f16")
    for u, v in ((a.codes, b.codes), (a.signs, b.signs), (a.norm, b.norm), (a.rnorm, b.rnorm)):
        assert torch.equal(u, v)
