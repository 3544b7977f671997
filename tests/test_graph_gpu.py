"""The library under HIP graph capture: the binding's calls record only the
library's kernels (no allocation by the library, no memset), so a captured
prefill + split-KV decode step replays with the eager results, bit for bit."""

import pytest
import torch

import streaming_attention_amd as sa

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_prefill_and_decode_step_replays_in_a_graph():
    g = torch.Generator(device=DEV).manual_seed(2024)

    def rnd(*shape):
        return torch.randn(shape, generator=g, device=DEV).to(torch.bfloat16)

    q, k, v = rnd(1, 8, 300, 128), rnd(1, 2, 300, 128), rnd(1, 2, 300, 128)
    qd, kc, vc = rnd(3, 16, 1, 64), rnd(3, 2, 900, 64), rnd(3, 2, 900, 64)
    lens = torch.tensor([900, 17, 512], dtype=torch.int32, device=DEV)
    o, lse = torch.empty_like(q), torch.empty((1, 8, 300), dtype=torch.float32, device=DEV)
    o2, lse2 = torch.empty_like(q), torch.empty_like(lse)
    po = torch.empty((3, 16, 8, 64), dtype=torch.float32, device=DEV)
    pl = torch.empty((3, 16, 8), dtype=torch.float32, device=DEV)
    od, lsed = torch.empty_like(qd), torch.empty((3, 16), dtype=torch.float32, device=DEV)

    def step():
        sa.prefill(q, k, v, causal=True, out=o, lse=lse, num_splits=1)
        sa.prefill(q, k, v, causal=True, out=o2, lse=lse2, num_splits=3)       # split-KV + merge
        sa.decode(qd, kc, vc, lens, None, 8, part_o=po, part_lse=pl, out=od, lse=lsed)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o, lse, o2, lse2, od, lsed)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                   # warm-up on the capture stream's side, as torch asks
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()

    for _ in range(3):
        for t in (o, lse, o2, lse2, od, lsed):   # eager work between replays
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip((o, lse, o2, lse2, od, lsed), ref):
            assert torch.equal(got, want)
