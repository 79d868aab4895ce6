"""tq_attn_decode_static (the decode entry point that allocates nothing: its
workspace is the library's per-GPU array) against tq_attn_decode with a
caller workspace, through the C ABI: two calls in a row, the second with a
smaller input, each output equal to the workspace entry point's."""

import pytest
import torch

from kv_cache_vector_quantize_amd import tq

from gpu_common import gpu_tables, say

pytestmark = pytest.mark.gpu
D = M = 128


def _streams(B, Hkv, T, kb, vb, seed):
    g = torch.Generator().manual_seed(seed)
    K = (torch.randn((B * Hkv, T, D), generator=g) * 1.5).to(torch.bfloat16).cuda().contiguous()
    V = torch.randn((B * Hkv, T, D), generator=g).to(torch.bfloat16).cuda().contiguous()
    tk, tv = gpu_tables(D, M, kb), gpu_tables(D, 0, vb)
    pk = tq.alloc_packed(tq.TQ_KEY, tk, B * Hkv, T, "f16")
    pv = tq.alloc_packed(tq.TQ_VALUE, tv, B * Hkv, T, "f16")
    tq.tq_quantize(tk, K, pk)
    tq.tq_quantize(tv, V, pv)
    return tk, tv, pk, pv


def test_static_workspace_decode_matches_workspace_decode_twice():
    assert tq.lib().tq_attn_decode_static_capacity() == 16 << 20
    # first call: 4 KV heads x 2 sequences, several splits per sequence;
    # second call smaller, so it reads only part of what the first wrote
    for (B, Hq, Hkv, T, kb, vb, seed) in ((2, 16, 4, 20000, 2, 3, 1), (1, 8, 2, 777, 3, 2, 2)):
        say("static decode", B, Hq, Hkv, T, kb, vb)
        need = tq.decode_workspace_bytes(B, Hq, Hkv, T, D, M)
        assert need <= tq.lib().tq_attn_decode_static_capacity()
        tk, tv, pk, pv = _streams(B, Hkv, T, kb, vb, seed)
        q = torch.randn((B, Hq, D), generator=torch.Generator().manual_seed(seed + 10)).cuda()
        ref = tq.tq_attn_decode(tk, tv, q, pk, pv, B, Hq, Hkv)
        out = torch.full((B, Hq, D), float("nan"), device="cuda")
        got = tq.tq_attn_decode_static(tk, tv, q, pk, pv, B, Hq, Hkv, out=out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.isfinite(got).all()
        assert torch.equal(got, ref), float((got - ref).abs().max())
