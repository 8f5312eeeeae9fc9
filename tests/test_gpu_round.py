"""Streaming round driver: rounds replayed from captured HIP graphs equal the eager rounds bitwise.

Two identical stacks of layers (paged rings of 6 x 256 tokens, 512-token
chunks over a 1280-key window, so the round repeats every 3 rounds) run side by side: one eagerly, one from
the captured graphs.  Between rounds, eager torch work writes new q / k / v
into both, and every replay is compared with the eager round: outputs, cache
bytes and metadata, bitwise.  Both schedules are covered (the workspace
drives the split schedule for this small workload).
"""
import numpy as np
import pytest
import torch

import chunk_causal_dit_wf_amd as wf
from chunk_causal_dit_wf_amd.round import Layer, StreamingRound

pytestmark = pytest.mark.gpu


def make_stack(seed, layers, H, D, P, T, n):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    out = []
    for l in range(layers):
        table = list(np.random.default_rng(seed + l).permutation(T + 1)[:T])
        cache = wf.KVCache(T + 1, P, H, D, "bf16", table, device="cuda")
        bufs = [torch.empty((n, H, D), dtype=torch.bfloat16, device="cuda") for _ in range(4)]
        out.append(Layer(cache, bufs[0], bufs[1], bufs[2], bufs[3]))
    return out, g


def refill(layers, g):
    for L in layers:
        for t in (L.q, L.k_new, L.v_new):
            t.copy_(torch.randn(t.shape, generator=g, device="cuda").to(torch.bfloat16))


@pytest.mark.parametrize("workspace", ["auto", None])
def test_graph_rounds_equal_eager_rounds(workspace):
    print("case: graph rounds, workspace=%s" % workspace, flush=True)
    H, D, P, T, n, W = 2, 128, 256, 6, 512, 1280
    A, ga = make_stack(7, 2, H, D, P, T, n)
    B, gb = make_stack(7, 2, H, D, P, T, n)
    ra = StreamingRound(A, n, W, workspace=workspace)
    rb = StreamingRound(B, n, W, workspace=workspace)
    assert ra.period == 3
    while not ra.steady():
        refill(A, ga)
        refill(B, gb)
        ra.step()
        rb.step()
    rb.capture()
    assert len(rb.graphs) == 3
    for r in range(8):
        refill(A, ga)
        refill(B, gb)
        ra.step()
        rb.replay()
        torch.cuda.synchronize()
        for La, Lb in zip(A, B):
            assert torch.equal(La.o.view(torch.int16), Lb.o.view(torch.int16)), "round %d output" % r
            assert torch.equal(La.cache.k.view(torch.int16), Lb.cache.k.view(torch.int16)), "round %d K" % r
            assert torch.equal(La.cache.v.view(torch.int16), Lb.cache.v.view(torch.int16)), "round %d V" % r
            assert (La.cache.start, La.cache.end) == (Lb.cache.start, Lb.cache.end)
        # eager work on the same stream between replays
        _ = (A[0].o.float() * 2).sum().item()
