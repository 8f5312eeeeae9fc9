"""Streaming round driver (needs an MI355X): rounds replayed from captured HIP graphs against the
oracle, and against eager rounds.

Oracle test.  A stack of two layers (paged rings of 256-token pages, 512-token chunks, a
1280-key window) runs the driver for 4 + 12 rounds: eager rounds until the pipeline and the rings
are full, then graph replays covering every ring phase and wrapping.  Before every round the
producer writes new seeded Q / K / V for the in-flight chunks; the host mirror of the cache
(oracle.KVCacheModel) receives the same evictions and appends, derived from the definition of the
round (the oldest tokens leave once the ring is full; the in-flight chunks' K/V are written at
their positions, rewriting the older ones -- the mixed-noise frontier and the timestep-0 refresh;
chunk c attends to the last W keys up to its own end that the cache still holds).  After every
round: cache bytes and window metadata equal the mirror bitwise, and every output row is within
the bf16 bars of oracle.chunk_attention over the mirror's keys.

Stages 1 (one chunk per round) and 3 (a 1F1C wave: three chunks in flight, the oldest being
refreshed; ring = W + 2 chunks so every chunk sees its whole window) are covered, each with and
without a workspace (split schedule where it applies).
"""
import numpy as np
import pytest
import torch

import chunk_causal_dit_wf_amd as wf
import oracle
from chunk_causal_dit_wf_amd.round import Layer, StreamingRound, WaveRound
from gpu_util import dev, errors, host_codes, host_values

pytestmark = pytest.mark.gpu

H, D, P, N, W = 2, 128, 256, 512, 1280
BF16_MAX, BF16_MEAN, BF16_REL = 1e-2, 1e-3, 1e-2


def say(*a):
    print(*a, flush=True)


def make_stack(seed, layers, S):
    ring = W + (S - 1) * N
    T = ring // P
    out, mirrors = [], []
    for l in range(layers):
        table = list(np.random.default_rng(seed + l).permutation(T + 1)[:T])
        cache = wf.KVCache(T + 1, P, H, D, "bf16", table, device="cuda")
        bufs = [torch.zeros((S * N, H, D), dtype=torch.bfloat16, device="cuda") for _ in range(4)]
        out.append(Layer(cache, bufs[0], bufs[1], bufs[2], bufs[3]))
        mirrors.append(oracle.KVCacheModel(T + 1, P, H, D, "bf16", table))
    return out, mirrors


def bf16_codes(rng, shape):
    x = torch.from_numpy(rng.standard_normal(shape, dtype=np.float32))
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def produce(rng, layers, S):
    """New Q / K / V codes for the in-flight chunks of every layer, written to the device buffers."""
    data = []
    for L in layers:
        q, k, v = (bf16_codes(rng, (S * N, H, D)) for _ in range(3))
        for t, c in ((L.q, q), (L.k_new, k), (L.v_new, v)):
            t.copy_(dev(c, "bf16"))
        data.append((q, k, v))
    return data


def mirror_round(model, r, S, q, k, v):
    """The round on the host mirror, from its definition; returns the expected outputs of the
    in-flight rows and the row block they start at."""
    chunks = list(range(max(0, r - S + 1), r + 1))
    new_end = (r + 1) * N
    if new_end - model.start > model.capacity:
        model.evict(new_end - model.capacity - model.start)
    j0 = chunks[0] - (r - S + 1)
    model.append(chunks[0] * N, k[j0 * N:], v[j0 * N:])
    kb = [max(model.start, (c + 1) * N - W) for c in chunks]
    ke = [(c + 1) * N for c in chunks]
    K, V = model.gather(min(kb), max(ke))
    q_off = [i * N for i in range(len(chunks) + 1)]
    o, _ = oracle.chunk_attention(oracle.decode_bf16(q[j0 * N:]), K, V, q_off, kb, ke, kv_origin=min(kb))
    return o, j0


def cache_equal(L, model):
    return (np.array_equal(host_codes(L.cache.k), model.k) and np.array_equal(host_codes(L.cache.v), model.v)
            and (L.cache.start, L.cache.end) == (model.start, model.end))


@pytest.mark.parametrize("S", [1, 3])
@pytest.mark.parametrize("workspace", ["auto", None])
def test_graph_rounds_match_the_oracle(S, workspace):
    say("case: round driver vs oracle, stages=%d workspace=%s" % (S, workspace))
    rng = np.random.default_rng(500 + S)
    layers, mirrors = make_stack(61, 2, S)
    drv = WaveRound(layers, N, W, stages=S, workspace=workspace)
    r = 0
    replays = 0
    while r < 16:
        data = produce(rng, layers, S)
        if drv.graphs is None and drv.steady():
            drv.capture()
            say("captured %d phases at round %d" % (len(drv.graphs), r))
        if drv.graphs is None:
            drv.step()
        else:
            drv.replay()
            replays += 1
        torch.cuda.synchronize()
        for L, M, (q, k, v) in zip(layers, mirrors, data):
            want, j0 = mirror_round(M, r, S, q, k, v)
            assert cache_equal(L, M), "round %d: cache differs from the mirror" % r
            got = host_values(L.o)[j0 * N:]
            mx, mean, rel = errors(got, want)
            assert mx <= BF16_MAX and mean <= BF16_MEAN and rel <= BF16_REL, (r, mx, mean, rel)
        say("round %d (%s): max-abs %.2e rel-L2 %.2e" % (r, "graph" if drv.graphs else "eager", mx, rel))
        r += 1
    assert replays >= 8 and drv.period == (W + (S - 1) * N) // 256


@pytest.mark.parametrize("S", [1, 3])
@pytest.mark.parametrize("workspace", ["auto", None])
def test_graph_rounds_equal_eager_rounds(S, workspace):
    """Two identical stacks, one eager and one replayed from graphs, with eager torch work between
    replays: outputs, cache bytes and metadata are bitwise equal every round."""
    say("case: graph vs eager rounds, stages=%d workspace=%s" % (S, workspace))
    A, _ = make_stack(7, 2, S)
    B, _ = make_stack(7, 2, S)
    ra = WaveRound(A, N, W, stages=S, workspace=workspace)
    rb = WaveRound(B, N, W, stages=S, workspace=workspace)
    rng_a, rng_b = np.random.default_rng(8), np.random.default_rng(8)
    while not ra.steady():
        produce(rng_a, A, S)
        produce(rng_b, B, S)
        ra.step()
        rb.step()
    rb.capture()
    assert len(rb.graphs) == rb.period
    for r in range(rb.period + 2):
        produce(rng_a, A, S)
        produce(rng_b, B, S)
        ra.step()
        rb.replay()
        torch.cuda.synchronize()
        for La, Lb in zip(A, B):
            assert torch.equal(La.o.view(torch.int16), Lb.o.view(torch.int16)), "round %d output" % r
            assert torch.equal(La.cache.k.view(torch.int16), Lb.cache.k.view(torch.int16)), "round %d K" % r
            assert torch.equal(La.cache.v.view(torch.int16), Lb.cache.v.view(torch.int16)), "round %d V" % r
            assert (La.cache.start, La.cache.end) == (Lb.cache.start, Lb.cache.end)
        _ = (A[0].o.float() * 2).sum().item()


def test_streaming_round_is_one_stage():
    layers, _ = make_stack(3, 1, 1)
    assert StreamingRound(layers, N, W).stages == 1
