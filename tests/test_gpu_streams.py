"""Attention calls on two HIP streams at once (needs an MI355X).

The library keeps no device state between calls apart from the allocation-free entry point's
array: calls on different streams with their own caches, outputs and workspaces are independent.
Each stream here attends a chunk table over its own cache -- a bf16 ring under the split schedule
(a workspace of its own) and an E4M3FN ring per tile -- several times in a row, interleaved with
the other stream's calls; every result must equal, bit for bit, the same call made alone on the
default stream (each kernel's arithmetic is fixed by its inputs).
"""
import numpy as np
import pytest
import torch

import chunk_causal_dit_wf_amd as wf
import synth
from gpu_util import Pair, dev

pytestmark = pytest.mark.gpu

H, D, P, T = 4, 128, 256, 12


def cache(dtype, seed):
    rng = np.random.default_rng(seed)
    pair = Pair(T, P, H, D, dtype, list(rng.permutation(T)), fill_seed=seed + 1)
    n = T * P
    k = rng.standard_normal((n, H, D)).astype(np.float32)
    v = rng.standard_normal((n, H, D)).astype(np.float32)
    if dtype == "fp8":
        kc, ks = synth.quantize_e4m3_pages(k, P)
        vc, vs = synth.quantize_e4m3_pages(v, P)
        pair.append(0, kc, vc, ks, vs)
    else:
        pair.append(0, synth.encode(k * 0.5, dtype), synth.encode(v * 0.5, dtype))
    q = dev(synth.encode(rng.standard_normal((700, H, D)).astype(np.float32) * 0.5, "bf16"), "bf16")
    return pair.gpu, q


def test_two_streams_match_the_default_stream():
    print("case: two streams, bf16 split + fp8 per tile", flush=True)
    cb, qb = cache("bf16", 11)
    c8, q8 = cache("fp8", 12)
    q_off, kb, ke = [0, 300, 700], [5, 8], [3000, 3008]
    wsb = torch.empty(wf.wf_chunk_attn_workspace_bytes(cb), dtype=torch.uint8, device="cuda")
    assert wf.wf_chunk_attn_plan(cb, q_off, kb, ke, "bf16", wsb.numel())["schedule"] == "split"
    assert wf.wf_chunk_attn_plan(c8, q_off, kb, ke, "bf16", 0)["kernel"] == "dma_fp8"
    ref_b, ref_lb = wf.wf_chunk_attn_fwd(cb, qb, q_off, kb, ke, return_lse=True, workspace=wsb)
    ref_8, ref_l8 = wf.wf_chunk_attn_fwd(c8, q8, q_off, kb, ke, return_lse=True, workspace=None)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(4):
        ob, lb = torch.empty_like(qb), torch.empty((H, qb.shape[0]), dtype=torch.float32, device="cuda")
        o8, l8 = torch.empty_like(q8), torch.empty((H, q8.shape[0]), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            wf.wf_chunk_attn_fwd(cb, qb, q_off, kb, ke, o=ob, lse=lb, workspace=wsb)
        with torch.cuda.stream(s2):
            wf.wf_chunk_attn_fwd(c8, q8, q_off, kb, ke, o=o8, lse=l8, workspace=None)
        outs.append((ob, lb, o8, l8))
    torch.cuda.synchronize()
    for ob, lb, o8, l8 in outs:
        assert torch.equal(ob.view(torch.int16), ref_b.view(torch.int16))
        assert torch.equal(lb, ref_lb)
        assert torch.equal(o8.view(torch.int16), ref_8.view(torch.int16))
        assert torch.equal(l8, ref_l8)
