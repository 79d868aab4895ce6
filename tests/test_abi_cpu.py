"""C ABI checks that need no GPU: the library loads, exports every function
include/tq.h declares, and rejects bad arguments on the host before any
launch."""

import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tq.h")


@pytest.fixture(scope="module")
def L():
    from kv_cache_vector_quantize_amd import tq
    if not os.path.exists(tq._LIB_PATH):
        from kv_cache_vector_quantize_amd import build
        build.build()
    return tq.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert len(names) == 15, names
    for n in names:
        assert hasattr(L, n), n
    assert L.tq_abi_version() == 6


def test_status_strings(L):
    for code in (0, -1, -2, -3, -4, 7):
        s = L.tq_status_str(code)
        assert isinstance(s, bytes) and len(s) > 0


def test_workspace_sizes(L):
    assert L.tq_logits_workspace(1, 32, 128, 128) == 32 * 128 * 4 * 2
    assert L.tq_logits_workspace(1, 1, 128, 0) == 512
    # rotated queries (q', u: 2 x 64 heads x 128 floats) and one (d + 2)-float
    # partial per query head per split; T = 524288 over 8 KV heads is cut into
    # 96 splits of 5472 tokens (768 workgroups: one round of the chip at 3 per
    # CU), 131072 tokens over 128 sequences into 16 splits of 8192 (the
    # longest decode split).
    ws = L.tq_decode_workspace(1, 64, 8, 524288, 128, 128)
    assert ws == 2 * 64 * 128 * 4 + 64 * 96 * 130 * 4
    ws = L.tq_decode_workspace(16, 32, 8, 131072, 128, 128)
    assert ws == 2 * 512 * 128 * 4 + 512 * 16 * 130 * 4
    assert L.tq_decode_workspace(-1, 1, 1, 1, 128, 128) == 0


# Fake, aligned device addresses: every call below must be rejected by the
# host-side validation, so nothing is ever launched with them.  On a machine
# with a GPU the cases are skipped (the GPU tests cover the same paths with
# real buffers).
FAKE = 0x10000
needs_no_gpu = pytest.mark.skipif(torch.cuda.is_available(),
                                  reason="fake device pointers are only used without a GPU")


def _tables(tq, d=128, m=128, bits=2, rot_kind=0, sketch=True, hi=0, sketch_f16=0):
    return tq.Tables(d, m, bits, rot_kind, FAKE, FAKE if sketch else None, FAKE, FAKE, hi,
                     FAKE if hi else None, FAKE if hi else None, sketch_f16)


def _packed(tq, role=0, bits=2, d=128, m=128, nseq=1, T=4, nd=2, cap=0, hi=0):
    key = role == 0
    return tq.Packed(role, bits, d, m, nseq, T, FAKE, FAKE if key else None, FAKE,
                     FAKE if key else None, nd, cap, hi)


@needs_no_gpu
def test_codebook_and_rotation_validation(L):
    vp = ctypes.c_void_p
    assert L.tq_codebook(2, 2, None, None, vp(FAKE), vp(FAKE), None) == -1      # d < 3
    assert L.tq_codebook(128, 5, None, None, vp(FAKE), vp(FAKE), None) == -1    # bits > 4
    assert L.tq_codebook(128, 0, None, None, vp(FAKE), vp(FAKE), None) == -1
    assert L.tq_codebook(128, 2, None, None, None, vp(FAKE), None) == -1        # null out
    assert L.tq_codebook(128, 2, None, None, vp(FAKE + 4), vp(FAKE), None) == -1  # misaligned
    assert L.tq_rotation(1025, vp(FAKE), vp(FAKE), None, None) == -1      # past the global-memory kernel
    assert L.tq_rotation(1, vp(FAKE), vp(FAKE), None, None) == -1
    assert L.tq_rotation(128, None, vp(FAKE), None, None) == -1
    assert L.tq_hadamard_rotation(96, vp(FAKE), vp(FAKE), None) == -1     # not a power of two
    assert L.tq_hadamard_rotation(8192, vp(FAKE), vp(FAKE), None) == -1
    assert L.tq_hadamard_rotation(128, None, vp(FAKE), None) == -1
    assert L.tq_hadamard_rotation(128, vp(FAKE), vp(FAKE + 4), None) == -1  # misaligned


@needs_no_gpu
def test_quantize_validation(L):
    from kv_cache_vector_quantize_amd import tq
    by = ctypes.byref
    x = ctypes.c_void_p(FAKE)
    cases = [
        (_tables(tq, rot_kind=2), _packed(tq), -1),            # unknown rotation kind
        (_tables(tq, bits=5), _packed(tq, bits=5), -1),
        (_tables(tq, d=300), _packed(tq, d=300), -2),          # valid, past the generic kernels' 256
        (_tables(tq, d=4), _packed(tq, d=4), -2),              # below the generic kernels' 8
        (_tables(tq, m=512), _packed(tq, m=512), -2),          # sketch past the generic kernels' 256
        (_tables(tq, d=200, hi=64), _packed(tq, d=200, hi=64), -2),  # split widths only at d = 128
        (_tables(tq), _packed(tq, bits=3), -1),                # bits mismatch
        (_tables(tq, m=0, sketch=False), _packed(tq, role=0, m=0), -1),  # key without sketch
        (_tables(tq, m=0, sketch=False), _packed(tq, role=1, m=0, nd=7), -1),  # bad norm dtype
        (_tables(tq), _packed(tq, role=3), -1),
        (_tables(tq), _packed(tq, T=-1), -1),
        (_tables(tq), _packed(tq, T=4, cap=48), -1),           # capacity not a multiple of 32
        (_tables(tq), _packed(tq, T=70, cap=64), -1),          # capacity below T
        (_tables(tq), _packed(tq, T=4, cap=-32), -1),
        (_tables(tq, sketch_f16=2), _packed(tq), -1),          # the float16-sketch flag is 0 or 1
        (_tables(tq, m=0, sketch=False, sketch_f16=1), _packed(tq, role=1, m=0), -1),  # values have no sketch
    ]
    for t, p, want in cases:
        assert L.tq_quantize(by(t), x, 1, by(p), None) == want, (want,)
    # bad input dtype
    assert L.tq_quantize(by(_tables(tq)), x, 2, by(_packed(tq)), None) == -1
    # null input with work to do
    assert L.tq_quantize(by(_tables(tq)), None, 1, by(_packed(tq)), None) == -1
    # empty stream: nothing to do, OK without touching any pointer
    assert L.tq_quantize(by(_tables(tq)), None, 1, by(_packed(tq, nseq=0)), None) == 0


def test_topk_workspace_sizes(L):
    # one sorted list of 16 (k <= 16) or 32 keys of 8 bytes per 16384-column chunk and row
    assert L.tq_topk_workspace(8, 1 << 20, 10) == 8 * 64 * 16 * 8
    assert L.tq_topk_workspace(3, 16385, 17) == 3 * 2 * 32 * 8
    assert L.tq_topk_workspace(1, 5, 6) == 0          # k > n
    assert L.tq_topk_workspace(1, 100, 33) == 0       # k > 32
    assert L.tq_topk_workspace(70000, 100, 3) == 0


@needs_no_gpu
def test_topk_validation(L):
    vp = ctypes.c_void_p
    f = vp(FAKE)
    ws = L.tq_topk_workspace(4, 1000, 10)
    assert L.tq_topk(f, 4, 1000, 0, f, f, f, ws, None) == -1          # k < 1
    assert L.tq_topk(f, 4, 1000, 33, f, f, f, ws, None) == -1         # k > 32
    assert L.tq_topk(f, 4, 5, 6, f, f, f, ws, None) == -1             # k > n
    assert L.tq_topk(f, 4, 1 << 31, 6, f, f, f, ws, None) == -1       # n too large
    assert L.tq_topk(None, 4, 1000, 10, f, f, f, ws, None) == -1
    assert L.tq_topk(f, 4, 1000, 10, vp(FAKE + 4), f, f, ws, None) == -1
    assert L.tq_topk(f, 4, 1000, 10, f, f, f, ws - 1, None) == -3
    assert L.tq_topk(f, 70000, 1000, 10, f, f, f, 1 << 40, None) == -2
    assert L.tq_topk(None, 0, 1000, 10, None, None, None, 0, None) == 0   # no rows


@needs_no_gpu
def test_append_validation(L):
    from kv_cache_vector_quantize_amd import tq
    by = ctypes.byref
    x = ctypes.c_void_p(FAKE)
    t = _tables(tq)
    # no capacity (a stream sized for its T only) cannot grow
    assert L.tq_append(by(t), x, 1, 1, by(_packed(tq, T=4)), None) == -1
    # past the capacity, or a negative count
    assert L.tq_append(by(t), x, 1, 61, by(_packed(tq, T=4, cap=64)), None) == -1
    assert L.tq_append(by(t), x, 1, -1, by(_packed(tq, T=4, cap=64)), None) == -1
    assert L.tq_append(by(t), x, 1, (1 << 62), by(_packed(tq, T=4, cap=64)), None) == -1
    # bad dtype, null input, role mismatch with the tables
    assert L.tq_append(by(t), x, 2, 1, by(_packed(tq, T=4, cap=64)), None) == -1
    assert L.tq_append(by(t), None, 1, 1, by(_packed(tq, T=4, cap=64)), None) == -1
    assert L.tq_append(by(t), x, 1, 1, by(_packed(tq, T=4, cap=64, bits=3)), None) == -1
    # nothing to do: OK without touching any pointer
    assert L.tq_append(by(t), None, 1, 0, by(_packed(tq, T=4, cap=64)), None) == 0
    assert L.tq_append(by(t), None, 1, 5, by(_packed(tq, nseq=0, T=4, cap=64)), None) == 0


@needs_no_gpu
def test_attention_validation(L):
    from kv_cache_vector_quantize_amd import tq
    by = ctypes.byref
    vp = ctypes.c_void_p
    tk, tv = _tables(tq), _tables(tq, m=0, sketch=False, bits=3)
    pk = _packed(tq, nseq=16, T=64)
    pv = _packed(tq, role=1, m=0, bits=3, nseq=16, T=64)
    ws = L.tq_decode_workspace(2, 32, 8, 64, 128, 128)
    q = vp(FAKE)
    # Hq not a multiple of Hkv
    assert L.tq_attn_logits(by(tk), q, 1, 2, 30, 8, by(pk), vp(FAKE), vp(FAKE), ws, None) == -1
    # nseq != B * Hkv
    assert L.tq_attn_logits(by(tk), q, 1, 3, 32, 8, by(pk), vp(FAKE), vp(FAKE), ws, None) == -1
    # group of 32 query heads per kv head: unsupported
    assert L.tq_attn_logits(by(tk), q, 1, 16, 32, 1, by(pk), vp(FAKE), vp(FAKE), ws, None) == -2
    # workspace too small
    assert L.tq_attn_logits(by(tk), q, 1, 2, 32, 8, by(pk), vp(FAKE), vp(FAKE), 16, None) == -3
    # value stream passed as keys
    assert L.tq_attn_logits(by(tv), q, 1, 2, 32, 8, by(pv), vp(FAKE), vp(FAKE), ws, None) == -1
    args = lambda scale, k, v, w: (by(tk), by(tv), q, 1, 2, 32, 8, by(k), by(v), scale, vp(FAKE),
                                   vp(FAKE), w, None)
    assert L.tq_attn_decode(*args(0.0, pk, pv, ws)) == -1                   # bad scale
    assert L.tq_attn_decode(*args(float("nan"), pk, pv, ws)) == -1
    assert L.tq_attn_decode(*args(0.1, pk, _packed(tq, role=1, m=0, bits=3, nseq=16, T=65), ws)) == -1
    assert L.tq_attn_decode(*args(0.1, pk, pv, ws - 1)) == -3
    # key and value tables of different head dimensions (their rotations
    # may differ, even in kind: the GPU tests cover that case)
    tv96 = _tables(tq, d=96, m=0, sketch=False, bits=3)
    assert L.tq_attn_decode(by(tk), by(tv96), q, 1, 2, 32, 8, by(pk), by(pv), 0.1, vp(FAKE), vp(FAKE),
                            ws, None) == -1
    assert L.tq_attn_decode(*args(0.1, _packed(tq, nseq=16, T=0),
                                  _packed(tq, role=1, m=0, bits=3, nseq=16, T=0), ws)) == -1
    # 16 query heads per kv head: fine for logits, unsupported for decode
    pk2 = _packed(tq, nseq=2, T=64)
    pv2 = _packed(tq, role=1, m=0, bits=3, nseq=2, T=64)
    assert L.tq_attn_decode(by(tk), by(tv), q, 1, 1, 32, 2, by(pk2), by(pv2), 0.1, vp(FAKE),
                            vp(FAKE), 1 << 30, None) == -2


@needs_no_gpu
def test_static_decode_rejects_shapes_beyond_its_array(L):
    """tq_attn_decode_static checks the workspace its shape needs against the
    array's capacity before anything else: 64 sequences x 64 query heads
    over 524288 tokens need far more than 16 MiB of split partials."""
    from kv_cache_vector_quantize_amd import tq
    by, vp = ctypes.byref, ctypes.c_void_p
    assert L.tq_attn_decode_static_capacity() == 16 << 20
    B, Hq, Hkv, T = 64, 64, 8, 524288
    assert L.tq_decode_workspace(B, Hq, Hkv, T, 128, 128) > 16 << 20
    tk, tv = _tables(tq), _tables(tq, m=0, sketch=False, bits=3)
    pk = _packed(tq, nseq=B * Hkv, T=T)
    pv = _packed(tq, role=1, m=0, bits=3, nseq=B * Hkv, T=T)
    assert L.tq_attn_decode_static(by(tk), by(tv), vp(FAKE), 1, B, Hq, Hkv, by(pk), by(pv), 0.088,
                                   vp(FAKE), None) == -3
    # a bad argument is still rejected as such
    assert L.tq_attn_decode_static(by(tk), by(tv), vp(FAKE), 1, 1, 30, 8, by(_packed(tq, nseq=8, T=64)),
                                   by(_packed(tq, role=1, m=0, bits=3, nseq=8, T=64)), 0.088,
                                   vp(FAKE), None) == -1


@needs_no_gpu
def test_split_width_validation(L):
    """Fractional widths: hi_coords 0 or d/2 (others unsupported or invalid),
    the second codebook present exactly for split tables, packed and tables
    agreeing, bits + 1 <= 4, dense rotation for quantize; logits take split
    keys of 2 or 3 bits, decode needs both streams split with float16 norms."""
    from kv_cache_vector_quantize_amd import tq
    by, vp = ctypes.byref, ctypes.c_void_p
    x = vp(FAKE)
    q = lambda t, p: L.tq_quantize(by(t), x, 1, by(p), None)
    # hi_coords not a multiple of 32, or past d: invalid; 32 / 96: unsupported
    for hi, want in ((16, -1), (160, -1), (32, -2), (96, -2)):
        assert q(_tables(tq, hi=hi), _packed(tq, hi=hi)) == want, hi
    # split tables need the second codebook; uniform ones must not carry it
    t = tq.Tables(128, 128, 2, 0, FAKE, FAKE, FAKE, FAKE, 64, None, None)
    assert q(t, _packed(tq, hi=64)) == -1
    t = tq.Tables(128, 128, 2, 0, FAKE, FAKE, FAKE, FAKE, 0, FAKE, None)
    assert q(t, _packed(tq)) == -1
    # bits + 1 must stay <= 4
    assert q(_tables(tq, bits=4, hi=64), _packed(tq, bits=4, hi=64)) == -1
    # packed and tables disagree
    assert q(_tables(tq, hi=64), _packed(tq, hi=0)) == -1
    # Walsh-Hadamard rotation with a split: unsupported
    assert q(_tables(tq, hi=64, rot_kind=1), _packed(tq, hi=64)) == -2
    # logits: split 1-bit keys unsupported
    tk1 = _tables(tq, bits=1, hi=64)
    assert L.tq_attn_logits(by(tk1), x, 1, 1, 4, 1, by(_packed(tq, bits=1, hi=64)), vp(FAKE), vp(FAKE),
                            1 << 20, None) == -2
    # decode: one stream split, the other not -> unsupported; f32 norms -> unsupported
    tk, tv = _tables(tq, hi=64), _tables(tq, m=0, sketch=False, bits=3)
    pk, pv = _packed(tq, nseq=8, T=64, hi=64), _packed(tq, role=1, m=0, bits=3, nseq=8, T=64)
    args = lambda tv_, pk_, pv_: (by(tk), by(tv_), x, 1, 1, 32, 8, by(pk_), by(pv_), 0.1, vp(FAKE),
                                  vp(FAKE), 1 << 30, None)
    assert L.tq_attn_decode(*args(tv, pk, pv)) == -2
    tvs = _tables(tq, m=0, sketch=False, bits=3, hi=64)
    pvs32 = _packed(tq, role=1, m=0, bits=3, nseq=8, T=64, nd=0, hi=64)
    assert L.tq_attn_decode(*args(tvs, pk, pvs32)) == -2
