"""The hot path under HIP graph capture: quantize + decode recorded once and
replayed, as a serving loop would.  The entry points allocate nothing and
issue no memset, so they can be captured; each replay, with eager work in
between, must equal the eager result exactly."""

import pytest
import torch

from kv_cache_vector_quantize_amd import tq

from gpu_common import gpu_tables, say

pytestmark = pytest.mark.gpu
D = M = 128


def test_quantize_and_decode_replayed_from_a_graph():
    say("graph capture: quantize + decode")
    B, Hkv, G, T = 2, 2, 4, 1000
    Hq = G * Hkv
    g = torch.Generator().manual_seed(21)
    K = torch.randn((B * Hkv, T, D), generator=g).to(torch.bfloat16).cuda().contiguous()
    V = torch.randn((B * Hkv, T, D), generator=g).to(torch.bfloat16).cuda().contiguous()
    q = torch.randn((B, Hq, D), generator=g).to(torch.bfloat16).cuda().contiguous()
    tk, tv = gpu_tables(D, M, 2), gpu_tables(D, 0, 3)
    pk = tq.alloc_packed(tq.TQ_KEY, tk, B * Hkv, T, "f16")
    pv = tq.alloc_packed(tq.TQ_VALUE, tv, B * Hkv, T, "f16")
    ws = torch.empty(tq.decode_workspace_bytes(B, Hq, Hkv, T, D, M), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, Hq, D), device="cuda")

    def step():
        tq.tq_quantize(tk, K, pk)
        tq.tq_quantize(tv, V, pv)
        tq.tq_attn_decode(tk, tv, q, pk, pv, B, Hq, Hkv, ws=ws, out=out)

    step()
    torch.cuda.synchronize()
    ref = out.clone()
    codes = pk.buf_codes.clone()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for i in range(3):
        out.zero_()
        pk.buf_codes.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), i
        assert torch.equal(pk.buf_codes, codes), i
        # eager work between the replays
        tq.tq_attn_decode(tk, tv, q, pk, pv, B, Hq, Hkv)
        torch.cuda.synchronize()
