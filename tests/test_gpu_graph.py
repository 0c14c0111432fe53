"""GPU: the fused calls captured in a HIP graph (torch.cuda.graph on the
stream the binding passes to the library) and replayed several times, with
new inputs written into the captured buffers and eager work and
synchronizations between the replays: every replay must give the bits the
same calls give eagerly on those inputs.  Covers the W4A4 linear with its
epilogue amax (the amax word is cleared by a kernel inside the graph, not a
memset), the no-allocation linear (static scratch), the one-pass KV
quantizer fed by that amax, and the per-chunk KV quantizer."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_helpers import dev_from_host, packed_to_device

pytestmark = pytest.mark.gpu

nv = pytest.importorskip("nvfp4_w4a4_quantized_04_amd")


def _inputs(seed, m, k, heads, tokens, d):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = (torch.randn((m, k), generator=g, device="cuda") * (1 + seed)).to(torch.bfloat16)
    kv = (torch.randn((2, heads, tokens, d), generator=g, device="cuda") * (0.5 + seed)).to(torch.bfloat16)
    return x, kv


def _eager(x, w, kv, tpc):
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    y = nv.linear(x, w, torch.bfloat16, amax_out=amax)
    y2 = torch.empty_like(y)
    nv.linear_no_alloc(x, w, y2)
    p = nv.kv_quantize(y.view(-1, 64), "4over6", amax=amax)
    ch = nv.kv_quantize_chunked(kv, tpc)
    torch.cuda.synchronize()
    return y, y2, amax, p, ch


def test_graph_replays_match_eager():
    m, k, n, heads, tokens, d, tpc = 300, 512, 384, 3, 50, 64, 16
    print("[case] graph replays: linear, linear_no_alloc, kv_quantize(amax), kv_quantize_chunked", flush=True)
    rng = np.random.default_rng(90)
    w = packed_to_device(oracle.quantize(workloads.f32_to_bf16_bits(
        (rng.standard_normal((n, k)) * 0.02).astype(np.float32)), oracle.TILE16, 1))
    # captured buffers
    x, kv = _inputs(0, m, k, heads, tokens, d)
    y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty_like(y)
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    ws = nv.linear_workspace(m, k)
    p = nv.empty_packed(m * n // 64, 64, nv.ROW16)
    ch = nv.kv_quantize_chunked(kv, tpc)
    cws = torch.empty(nv.lib.nvfp4_kv_chunked_workspace_size(2, heads, tokens, d, tpc), dtype=torch.uint8,
                      device="cuda")
    kws = torch.empty(nv.lib.nvfp4_quantize_workspace_size(m * n // 64, 64), dtype=torch.uint8, device="cuda")

    def calls():
        nv.linear(x, w, torch.bfloat16, out=y, workspace=ws, amax_out=amax)
        nv.linear_no_alloc(x, w, y2)
        nv.kv_quantize(y.view(-1, 64), "4over6", out=p, workspace=kws, amax=amax)
        nv.kv_quantize_chunked(kv, tpc, out=ch, workspace=cws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()                                   # warm-up on a side stream, as capture wants
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()
    for rep in range(4):
        xn, kvn = _inputs(rep + 1, m, k, heads, tokens, d)
        x.copy_(xn)
        kv.copy_(kvn)
        y.fill_(0)
        amax.fill_(-1.0)                          # the graph's own clearing must reset it
        graph.replay()
        torch.cuda.synchronize()
        ey, ey2, eamax, ep, ech = _eager(xn, w, kvn, tpc)
        assert torch.equal(y, ey), rep
        assert torch.equal(y2, ey2), rep
        assert torch.equal(amax, eamax), rep
        assert torch.equal(p.codes, ep.codes) and torch.equal(p.scales, ep.scales), rep
        assert torch.equal(p.alpha, ep.alpha), rep
        assert torch.equal(ch.codes, ech.codes) and torch.equal(ch.scales, ech.scales), rep
        assert torch.equal(ch.alphas, ech.alphas), rep
        # eager work on the same buffers between replays
        nv.linear(xn, w, torch.bfloat16, out=y, workspace=ws)
        torch.cuda.synchronize()
