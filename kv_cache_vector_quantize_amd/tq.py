"""Thin ctypes binding of libtq.so over torch tensors.

torch supplies device memory and the current stream; every step of the
computation runs in the library's HIP kernels.  The names follow the C ABI
in ``include/tq.h``.  Any non-OK status raises ``TQError``; a missing
library raises ``ImportError`` (there is no other code path).
"""

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtq.so")

TQ_OK, TQ_EINVAL, TQ_EUNSUPPORTED, TQ_EWORKSPACE, TQ_EHIP = 0, -1, -2, -3, -4
TQ_F32, TQ_BF16, TQ_F16 = 0, 1, 2
TQ_KEY, TQ_VALUE = 0, 1
TQ_ROT_DENSE, TQ_ROT_HADAMARD = 0, 1


class TQError(RuntimeError):
    def __init__(self, status, what):
        super().__init__(f"{what}: {lib().tq_status_str(status).decode()} ({status})")
        self.status = status


class Tables(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("m", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("rot_kind", ctypes.c_int32), ("rot", ctypes.c_void_p),
                ("sketch", ctypes.c_void_p), ("centroids", ctypes.c_void_p),
                ("bounds", ctypes.c_void_p), ("hi_coords", ctypes.c_int32),
                ("centroids_hi", ctypes.c_void_p), ("bounds_hi", ctypes.c_void_p),
                ("sketch_f16", ctypes.c_int32)]


class Packed(ctypes.Structure):
    _fields_ = [("role", ctypes.c_int32), ("bits", ctypes.c_int32), ("d", ctypes.c_int32),
                ("m", ctypes.c_int32), ("nseq", ctypes.c_int64), ("T", ctypes.c_int64),
                ("codes", ctypes.c_void_p), ("signs", ctypes.c_void_p),
                ("norm", ctypes.c_void_p), ("rnorm", ctypes.c_void_p),
                ("norm_dtype", ctypes.c_int32), ("capacity", ctypes.c_int32),
                ("hi_coords", ctypes.c_int32)]


_lib = None


def lib():
    """Load libtq.so once (raises ImportError if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} not found: build it with "
                          "`python -m kv_cache_vector_quantize_amd.build`")
    L = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    L.tq_abi_version.restype = i32
    L.tq_status_str.restype = ctypes.c_char_p
    L.tq_status_str.argtypes = [i32]
    L.tq_codebook.restype = i32
    L.tq_codebook.argtypes = [i32, i32, vp, vp, vp, vp, vp]
    L.tq_rotation.restype = i32
    L.tq_rotation.argtypes = [i32, vp, vp, vp, vp]
    L.tq_hadamard_rotation.restype = i32
    L.tq_hadamard_rotation.argtypes = [i32, vp, vp, vp]
    L.tq_quantize.restype = i32
    L.tq_quantize.argtypes = [ctypes.POINTER(Tables), vp, i32, ctypes.POINTER(Packed), vp]
    L.tq_topk_workspace.restype = sz
    L.tq_topk_workspace.argtypes = [i64, i64, i32]
    L.tq_topk.restype = i32
    L.tq_topk.argtypes = [vp, i64, i64, i32, vp, vp, vp, sz, vp]
    L.tq_append.restype = i32
    L.tq_append.argtypes = [ctypes.POINTER(Tables), vp, i32, i64, ctypes.POINTER(Packed), vp]
    L.tq_logits_workspace.restype = sz
    L.tq_logits_workspace.argtypes = [i32, i32, i32, i32]
    L.tq_attn_logits.restype = i32
    L.tq_attn_logits.argtypes = [ctypes.POINTER(Tables), vp, i32, i32, i32, i32,
                                 ctypes.POINTER(Packed), vp, vp, sz, vp]
    L.tq_decode_workspace.restype = sz
    L.tq_decode_workspace.argtypes = [i32, i32, i32, i64, i32, i32]
    L.tq_attn_decode.restype = i32
    L.tq_attn_decode.argtypes = [ctypes.POINTER(Tables), ctypes.POINTER(Tables), vp, i32, i32,
                                 i32, i32, ctypes.POINTER(Packed), ctypes.POINTER(Packed),
                                 ctypes.c_float, vp, vp, sz, vp]
    L.tq_attn_decode_static_capacity.restype = sz
    L.tq_attn_decode_static_capacity.argtypes = []
    L.tq_attn_decode_static.restype = i32
    L.tq_attn_decode_static.argtypes = [ctypes.POINTER(Tables), ctypes.POINTER(Tables), vp, i32, i32,
                                        i32, i32, ctypes.POINTER(Packed), ctypes.POINTER(Packed),
                                        ctypes.c_float, vp, vp]
    _lib = L
    return L


def loaded_path():
    return _LIB_PATH if _lib is not None else None


def _stream(device=None):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(status, what):
    if status != TQ_OK:
        raise TQError(status, what)


def _dtype_code(t):
    if t.dtype == torch.float32:
        return TQ_F32
    if t.dtype == torch.bfloat16:
        return TQ_BF16
    if t.dtype == torch.float16:
        return TQ_F16
    raise TypeError(f"unsupported dtype {t.dtype}")


# --------------------------------------------------------------- setup calls
def tq_codebook(d, bits, device="cuda"):
    """Returns (centroids64, bounds64, centroids32, bounds32) device tensors."""
    L = 2 ** bits
    c64 = torch.empty(L, dtype=torch.float64, device=device)
    b64 = torch.empty(max(L - 1, 1), dtype=torch.float64, device=device)
    c32 = torch.empty(L, dtype=torch.float32, device=device)
    b32 = torch.empty(max(L - 1, 1), dtype=torch.float32, device=device)
    _check(lib().tq_codebook(d, bits, _ptr(c64), _ptr(b64), _ptr(c32), _ptr(b32), _stream()),
           "tq_codebook")
    return c64, b64[:L - 1], c32, b32[:L - 1]


def tq_rotation(G):
    """G: device float64 [d, d].  Returns (rot64, rot32)."""
    d = G.shape[0]
    G = G.contiguous()
    r64 = torch.empty((d, d), dtype=torch.float64, device=G.device)
    r32 = torch.empty((d, d), dtype=torch.float32, device=G.device)
    _check(lib().tq_rotation(d, _ptr(G), _ptr(r64), _ptr(r32), _stream()), "tq_rotation")
    return r64, r32


def tq_hadamard_rotation(signs):
    """signs: device float32 [d] (+-1).  Returns rot32 = H_d diag(signs) / sqrt(d)."""
    signs = signs.contiguous()
    d = signs.shape[0]
    r32 = torch.empty((d, d), dtype=torch.float32, device=signs.device)
    _check(lib().tq_hadamard_rotation(d, _ptr(signs), _ptr(r32), _stream()), "tq_hadamard_rotation")
    return r32


@dataclass
class StreamTables:
    """Device tables of one stream (tensors kept alive here)."""
    d: int
    m: int
    bits: int
    rot: torch.Tensor
    sketch: Optional[torch.Tensor]
    centroids: torch.Tensor
    bounds: torch.Tensor
    rot_kind: int = TQ_ROT_DENSE
    hi_coords: int = 0
    centroids_hi: Optional[torch.Tensor] = None
    bounds_hi: Optional[torch.Tensor] = None
    sketch_f16: int = 0

    def c_struct(self):
        return Tables(self.d, self.m, self.bits, self.rot_kind, self.rot.data_ptr(),
                      None if self.sketch is None else self.sketch.data_ptr(),
                      self.centroids.data_ptr(), self.bounds.data_ptr(), self.hi_coords,
                      _dp(self.centroids_hi), _dp(self.bounds_hi), self.sketch_f16)

    def coord_bits(self):
        """Bits of every coordinate (bits + 1 for the leading hi_coords)."""
        return [self.bits + 1 if j < self.hi_coords else self.bits for j in range(self.d)]


def make_tables(G, S, bits, device="cuda", hadamard_signs=None, hi_coords=0, sketch_f16=None):
    """Rotation from the Gaussian G (numpy/torch float64 [d, d]) -- or, given
    hadamard_signs (d values +-1), the randomized Walsh-Hadamard rotation
    from them (G is then unused) -- sketch S (float64 [m, d] or None) and the
    Lloyd-Max codebook, all built on the device by the library.  hi_coords
    > 0 makes a split (fractional-width) stream: the leading hi_coords
    rotated coordinates take the (bits+1)-bit codebook, built here too.
    sketch_f16 (the tables' flag) is, by default, whether every entry of S
    is exact in float16; False forces the general sketch products."""
    if hadamard_signs is not None:
        sg = torch.as_tensor(hadamard_signs, dtype=torch.float32).to(device)
        rot32, kind = tq_hadamard_rotation(sg), TQ_ROT_HADAMARD
    else:
        _, rot32 = tq_rotation(torch.as_tensor(G, dtype=torch.float64).to(device))
        kind = TQ_ROT_DENSE
    d = rot32.shape[0]
    s64 = None if S is None else torch.as_tensor(S, dtype=torch.float64)
    exact = s64 is not None and bool(torch.equal(s64, s64.to(torch.float16).to(torch.float64)))
    f16 = exact if sketch_f16 is None else (bool(sketch_f16) and exact)
    sk = None if s64 is None else s64.to(device).float().contiguous()
    _, _, c32, b32 = tq_codebook(d, bits, device)
    b32 = b32.clone() if b32.numel() else torch.zeros(1, dtype=torch.float32, device=device)
    ch, bh = None, None
    if hi_coords:
        _, _, ch, bh = tq_codebook(d, bits + 1, device)
        bh = bh.clone()
    return StreamTables(d, 0 if sk is None else sk.shape[0], bits, rot32, sk, c32, b32, kind,
                        hi_coords, ch, bh, int(f16))


@dataclass
class PackedStream:
    """A packed key or value stream.  The device buffers (``buf_*``) hold Tp
    tokens per sequence: the capacity, or with capacity 0, 32 * ceil(T / 32).
    ``codes``/``signs``/``norm``/``rnorm`` are views of the first T tokens
    (value codes are block records already)."""
    role: int
    bits: int
    d: int
    m: int
    nseq: int
    T: int
    buf_codes: torch.Tensor
    buf_signs: Optional[torch.Tensor]
    buf_norm: torch.Tensor
    buf_rnorm: Optional[torch.Tensor]
    norm_dtype: int
    capacity: int = 0
    hi_coords: int = 0

    @property
    def Tp(self):
        return self.capacity if self.capacity else padded_tokens(self.T)

    @property
    def codes(self):
        return self.buf_codes[:, : self.T] if self.role == TQ_KEY else self.buf_codes

    @property
    def signs(self):
        return None if self.buf_signs is None else self.buf_signs[:, : self.T]

    @property
    def norm(self):
        return self.buf_norm[:, : self.T]

    @property
    def rnorm(self):
        return None if self.buf_rnorm is None else self.buf_rnorm[:, : self.T]

    def c_struct(self):
        return Packed(self.role, self.bits, self.d, self.m, self.nseq, self.T,
                      self.buf_codes.data_ptr(), _dp(self.buf_signs), self.buf_norm.data_ptr(),
                      _dp(self.buf_rnorm), self.norm_dtype, self.capacity, self.hi_coords)


def padded_tokens(T):
    """Tokens per sequence stored in a packed stream: T rounded up to a 32-token block."""
    return (T + 31) // 32 * 32


def _dp(t):
    return None if t is None else t.data_ptr()


def alloc_packed(role, tables, nseq, T, norm_dtype="f16", device="cuda", capacity=0):
    """Allocate a packed stream in the canonical layout (see include/tq.h) of
    T tokens; a nonzero capacity (a multiple of 32, >= T) sizes it for
    tokens appended later by tq_append."""
    nd = TQ_F16 if norm_dtype == "f16" else TQ_F32
    tdt = torch.float16 if norm_dtype == "f16" else torch.float32
    d, m, bits = tables.d, tables.m, tables.bits
    if capacity and (capacity % 32 or capacity < T):
        raise ValueError(f"capacity {capacity} must be a multiple of 32 and >= T = {T}")
    Tp = capacity if capacity else padded_tokens(T)
    hi = tables.hi_coords
    if role == TQ_KEY:
        if hi:   # split stream: one record of (d/32) bits + hi/32 words per token
            codes = torch.zeros((nseq, Tp, (d // 32) * bits + hi // 32), dtype=torch.int32, device=device)
        else:   # coordinates padded to whole 32-bit words (bits of padding are 0)
            codes = torch.zeros((nseq, Tp, (d + 31) // 32, bits), dtype=torch.int32, device=device)
        signs = torch.zeros((nseq, Tp, (m + 31) // 32), dtype=torch.int32, device=device)
        rnorm = torch.zeros((nseq, Tp), dtype=tdt, device=device)
    else:
        if hi:   # split stream: one record of d bits + hi words per block
            codes = torch.zeros((nseq, Tp // 32, d * bits + hi), dtype=torch.int32, device=device)
        else:
            codes = torch.zeros((nseq, Tp // 32, d, bits), dtype=torch.int32, device=device)
        signs, rnorm = None, None
    norm = torch.zeros((nseq, Tp), dtype=tdt, device=device)
    return PackedStream(role, bits, d, m if role == TQ_KEY else 0, nseq, T, codes, signs, norm,
                        rnorm, nd, capacity, hi)


# ------------------------------------------------------------ hot-path calls
def tq_quantize(tables, x, out):
    """x: [nseq, T, d] float32 / bfloat16 on the device; out: PackedStream."""
    assert x.is_contiguous()
    t, p = tables.c_struct(), out.c_struct()
    _check(lib().tq_quantize(ctypes.byref(t), _ptr(x), _dtype_code(x), ctypes.byref(p),
                             _stream(x.device)), "tq_quantize")
    return out


def tq_append(tables, x, out):
    """Quantize x: [nseq, n, d] (float32 / bfloat16, on the device) onto the
    end of ``out`` (which needs a capacity of at least T + n), then advance
    ``out.T`` by n."""
    assert x.is_contiguous() and x.dim() == 3 and x.shape[0] == out.nseq
    t, p = tables.c_struct(), out.c_struct()
    _check(lib().tq_append(ctypes.byref(t), _ptr(x), _dtype_code(x), x.shape[1], ctypes.byref(p),
                           _stream(x.device)), "tq_append")
    out.T += x.shape[1]
    return out


def logits_workspace_bytes(B, Hq, d, m):
    return lib().tq_logits_workspace(B, Hq, d, m)


def tq_attn_logits(tk, q, k, B, Hq, Hkv, ws=None, out=None):
    """q: [B, Hq, d]; k: packed keys with nseq = B*Hkv.  Returns [B, Hq, T] float32."""
    assert q.is_contiguous()
    L = lib()
    need = L.tq_logits_workspace(B, Hq, tk.d, tk.m)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, k.T), dtype=torch.float32, device=q.device)
    assert out.is_contiguous() and out.numel() == B * Hq * k.T and out.dtype == torch.float32
    t, p = tk.c_struct(), k.c_struct()
    _check(L.tq_attn_logits(ctypes.byref(t), _ptr(q), _dtype_code(q), B, Hq, Hkv, ctypes.byref(p),
                            _ptr(out), _ptr(ws), ws.numel(), _stream(q.device)), "tq_attn_logits")
    return out


def decode_workspace_bytes(B, Hq, Hkv, T, d, m):
    return lib().tq_decode_workspace(B, Hq, Hkv, T, d, m)


def tq_attn_decode(tk, tv, q, k, v, B, Hq, Hkv, scale=None, ws=None, out=None):
    """Returns out [B, Hq, d] float32."""
    assert q.is_contiguous()
    L = lib()
    if scale is None:
        scale = 1.0 / math.sqrt(tk.d)
    need = L.tq_decode_workspace(B, Hq, Hkv, k.T, tk.d, tk.m)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, tk.d), dtype=torch.float32, device=q.device)
    t1, t2, p1, p2 = tk.c_struct(), tv.c_struct(), k.c_struct(), v.c_struct()
    _check(L.tq_attn_decode(ctypes.byref(t1), ctypes.byref(t2), _ptr(q), _dtype_code(q), B, Hq,
                            Hkv, ctypes.byref(p1), ctypes.byref(p2), float(scale), _ptr(out),
                            _ptr(ws), ws.numel(), _stream(q.device)), "tq_attn_decode")
    return out


def tq_attn_decode_static(tk, tv, q, k, v, B, Hq, Hkv, scale=None, out=None):
    """tq_attn_decode with the library's own per-GPU workspace (no allocation
    by the library; ``out`` is allocated here only when not given)."""
    assert q.is_contiguous()
    if scale is None:
        scale = 1.0 / math.sqrt(tk.d)
    if out is None:
        out = torch.empty((B, Hq, tk.d), dtype=torch.float32, device=q.device)
    t1, t2, p1, p2 = tk.c_struct(), tv.c_struct(), k.c_struct(), v.c_struct()
    _check(lib().tq_attn_decode_static(ctypes.byref(t1), ctypes.byref(t2), _ptr(q), _dtype_code(q), B,
                                       Hq, Hkv, ctypes.byref(p1), ctypes.byref(p2), float(scale),
                                       _ptr(out), _stream(q.device)), "tq_attn_decode_static")
    return out


def topk_workspace_bytes(rows, n, k):
    return lib().tq_topk_workspace(rows, n, k)


def tq_topk(scores, k, ws=None, idx=None, val=None):
    """scores: [rows, n] float32 on the device.  Returns (idx int32 [rows, k],
    val float32 [rows, k]): each row's k largest scores, larger first, ties
    to the smaller column."""
    assert scores.dtype == torch.float32 and scores.is_contiguous() and scores.dim() == 2
    rows, n = scores.shape
    need = lib().tq_topk_workspace(rows, n, k)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=scores.device)
    if idx is None:
        idx = torch.empty((rows, k), dtype=torch.int32, device=scores.device)
    if val is None:
        val = torch.empty((rows, k), dtype=torch.float32, device=scores.device)
    _check(lib().tq_topk(_ptr(scores), rows, n, k, _ptr(idx), _ptr(val), _ptr(ws), ws.numel(),
                         _stream(scores.device)), "tq_topk")
    return idx, val

