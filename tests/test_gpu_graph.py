"""The library's calls captured in a HIP graph: quantize, both dequants,
the fused attention and the speculative verification recorded once on a
capture stream, then replayed three times with the program's own eager
work and synchronizations between the replays; every replay must give the
eager results bit for bit (no call records a memset, an allocation or a
host synchronization)."""
import math

import pytest
import torch

from progressive_kv_transfer_amd import kvgen, lynx

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_graph_replays_match_eager():
    print("[gpu-graph] capture codec + attention + verify, 3 replays", flush=True)
    # two tensors of 512 tokens x 2 KV heads (K and V of one layer): 8 blocks
    kv = torch.stack([kvgen.kv_tensor(900 + i, 512, 256, [3], True, DEV) for i in range(2)])
    other = torch.stack([kvgen.kv_tensor(910 + i, 512, 256, [], True, DEV) for i in range(2)])
    q = kvgen.queries(901, 1, 4, device=DEV)
    scale = 1.0 / math.sqrt(128)
    d, t, s, u, us = kvgen.verify_inputs(902, 4, 1000, 0.3)
    d, t, s, u = d.to(DEV), t.to(DEV), s.to(DEV), u.to(DEV)

    def run(codes, oa, of, att, ws, ver, vws, stream):
        lynx.quantize_pages(kv, out=codes, stream=stream)
        lynx.dequant_anchor(codes, oa, stream=stream)
        lynx.dequant_full(codes, of, stream=stream)
        lynx.decode_attn_dequant(q, lynx.CodeView(codes, 0, 4), lynx.CodeView(codes, 4, 8),
                                 512, 2, scale, out=att, workspace=ws, stream=stream)
        lynx.spec_verify(d, t, s, u, us, out=ver, workspace=vws, stream=stream)

    def buffers():
        return (lynx.alloc_codes(8, DEV), torch.empty_like(kv), torch.empty_like(kv),
                torch.empty(q.shape, dtype=torch.bfloat16, device=DEV),
                torch.empty(max(lynx.attn_workspace_bytes(1, 4, 2, 512), 16),
                            dtype=torch.uint8, device=DEV),
                torch.empty(2, dtype=torch.int32, device=DEV),
                torch.empty(max(lynx.spec_verify_workspace_bytes(4, 1000), 16),
                            dtype=torch.uint8, device=DEV))

    eager = buffers()
    run(*eager, torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = [x.clone() for x in eager[0].tensors()] + [y.clone() for y in eager[1:4]] + \
        [eager[5].clone()]

    g_bufs = buffers()
    run(*g_bufs, torch.cuda.current_stream())  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=cap):
        run(*g_bufs, cap)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()

    scratch = lynx.alloc_codes(8, DEV)
    for r in range(3):
        # the program's own eager work between replays: poison every graph
        # output, quantize other data through the library
        for x in list(g_bufs[0].tensors()) + list(g_bufs[1:4]) + [g_bufs[5]]:
            x.view(torch.uint8).fill_(0xA5)
        lynx.quantize_pages(other, out=scratch)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = list(g_bufs[0].tensors()) + list(g_bufs[1:4]) + [g_bufs[5]]
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (r, i)
    del graph
