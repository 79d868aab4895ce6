"""In-bounds checks of the matrix-core fragment layouts (16x16x32 and
32x32x16 fp16) and the DPP row shift that the kernels are written against."""

import ctypes
import os

import numpy as np
import pytest
import torch

from kv_cache_vector_quantize_amd import tq

pytestmark = pytest.mark.gpu

PROBE_LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "probes", "libtq_probe.so")


def _probe_lib():
    if not os.path.exists(PROBE_LIB):   # normally built ahead by __graft_entry__.build()
        from probes import build as probe_build
        probe_build.build()
    return ctypes.CDLL(PROBE_LIB)


def test_mfma_16x16x32_f16_layout_and_dpp_row_shift():
    tq.lib()
    L = _probe_lib()
    L.tq_probe_mfma_layout.restype = ctypes.c_int
    L.tq_probe_mfma_layout.argtypes = [ctypes.c_void_p] * 5
    rng = np.random.default_rng(0)
    A = rng.integers(-3, 4, size=(16, 32)).astype(np.float16)
    B = rng.integers(-3, 4, size=(32, 16)).astype(np.float16)
    a, b = torch.tensor(A).cuda(), torch.tensor(B).cuda()
    d = torch.zeros((16, 16), dtype=torch.float32, device="cuda")
    dpp = torch.zeros(64, dtype=torch.float32, device="cuda")
    assert L.tq_probe_mfma_layout(ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(b.data_ptr()),
                                  ctypes.c_void_p(d.data_ptr()), ctypes.c_void_p(dpp.data_ptr()),
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) == 0
    torch.cuda.synchronize()
    assert np.array_equal(d.cpu().numpy(), A.astype(np.float32) @ B.astype(np.float32))
    got = dpp.cpu().numpy().astype(int)
    # row_shl:4 within rows of 16 lanes: lane i receives lane i + 4 (rows end -> old value -1)
    want = np.array([(l + 4) if (l % 16) + 4 < 16 else -1 for l in range(64)])
    assert np.array_equal(got, want), got


def test_mfma_32x32x16_f16_layout():
    tq.lib()
    L = _probe_lib()
    L.tq_probe_mfma_32x32x16.restype = ctypes.c_int
    L.tq_probe_mfma_32x32x16.argtypes = [ctypes.c_void_p] * 4
    rng = np.random.default_rng(1)
    A = rng.integers(-3, 4, size=(32, 16)).astype(np.float16)
    B = rng.integers(-3, 4, size=(16, 32)).astype(np.float16)
    a, b = torch.tensor(A).cuda(), torch.tensor(B).cuda()
    d = torch.zeros((32, 32), dtype=torch.float32, device="cuda")
    assert L.tq_probe_mfma_32x32x16(ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(b.data_ptr()),
                                    ctypes.c_void_p(d.data_ptr()),
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) == 0
    torch.cuda.synchronize()
    assert np.array_equal(d.cpu().numpy(), A.astype(np.float32) @ B.astype(np.float32))
