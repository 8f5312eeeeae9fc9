"""Host planning of an attention call (wf_chunk_attn_plan without a workspace), over random
cache shapes, windows and chunk tables, against the rules include/wf_chunk_attn.h states:
which kernel serves which cache, how many (query tile, head) items a call makes, and which
chunk tables are rejected, with which status.  No GPU: without a workspace the plan is pure
host logic."""
import hypothesis.strategies as st
import pytest
import torch
from hypothesis import HealthCheck, assume, given, settings

import chunk_causal_dit_wf_amd as wf

ROWS = {"f32": 128, "staged_bf16": 128, "staged_fp8": 128, "dma_bf16": 256, "dma_fp8": 256}
FP8_MAX_KEYS = 8 * 4096  # lead + keys of a chunk that the fp8 LDS-DMA kernel's scale table holds


@st.composite
def calls(draw):
    dtype = draw(st.sampled_from(["f32", "bf16", "fp8"]))
    P = draw(st.sampled_from([8, 16, 40, 56, 64, 72, 128, 1560]))
    H = draw(st.sampled_from([1, 2, 3, 12]))
    D = draw(st.sampled_from([64, 128]))
    T = draw(st.integers(1, 24 if P == 1560 else 8))
    extra = draw(st.integers(0, 2))
    pages = draw(st.permutations(list(range(T + extra))))[:T]
    cap = T * P
    end = draw(st.integers(1, 3 * cap))
    start = draw(st.integers(max(0, end - cap), end - 1))
    nc = draw(st.integers(1, 6))
    q_len = [draw(st.integers(0, 700)) for _ in range(nc)]
    kb, ke = [], []
    for _ in range(nc):
        a = draw(st.integers(start, end - 1))
        kb.append(a)
        ke.append(draw(st.integers(a + 1, end)))
    return dict(dtype=dtype, P=P, H=H, D=D, pages=pages, num_pages=T + extra, start=start, end=end,
                q_len=q_len, kb=kb, ke=ke)


def make(c):
    """The cache descriptor over host buffers that are allocated but never touched (planning
    reads only the descriptor and the page table)."""
    st_dtype = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}[c["dtype"]]
    shape_k = (c["num_pages"], c["H"], c["P"], c["D"])
    shape_v = (c["num_pages"], c["H"], c["D"], c["P"])
    cache = wf.KVCache(c["num_pages"], c["P"], c["H"], c["D"], c["dtype"], c["pages"], device="cpu",
                       k=torch.empty(shape_k, dtype=st_dtype), v=torch.empty(shape_v, dtype=st_dtype))
    cache.c.start, cache.c.end = c["start"], c["end"]
    q_off = [0]
    for n in c["q_len"]:
        q_off.append(q_off[-1] + n)
    return cache, q_off


def expected_kernel(c):
    if c["dtype"] == "f32":
        return "f32"
    if c["P"] < 64:
        return "staged_" + c["dtype"]
    if c["dtype"] == "bf16":
        return "dma_bf16"
    fits = all(a % 8 + (b - a) <= FP8_MAX_KEYS for a, b in zip(c["kb"], c["ke"]))
    return "dma_fp8" if fits else "staged_fp8"


@settings(max_examples=300, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(calls())
def test_plan_kernel_items_and_grid(c):
    cache, q_off = make(c)
    q_dtype = "f32" if c["dtype"] == "f32" else "bf16"
    plan = wf.wf_chunk_attn_plan(cache, q_off, c["kb"], c["ke"], q_dtype=q_dtype)
    kernel = expected_kernel(c)
    rows = ROWS[kernel]
    items = c["H"] * sum(-(-n // rows) for n in c["q_len"])
    assert plan["kernel"] == kernel
    assert plan["schedule"] == "per_tile" and plan["parts"] == 1 and plan["tail_tiles"] == 0
    assert plan["rows_per_item"] == rows
    assert plan["items"] == items and plan["grid"] == items


@settings(max_examples=200, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(calls(), st.integers(0, 5), st.data())
def test_plan_rejects_tables_outside_the_window(c, which, data):
    """Each kind of bad table is rejected with its own status, and a rejected plan leaves the
    cache's window as it was."""
    cache, q_off = make(c)
    q_dtype = "f32" if c["dtype"] == "f32" else "bf16"
    kb, ke = list(c["kb"]), list(c["ke"])
    i = data.draw(st.integers(0, len(kb) - 1))
    if which == 0:    # a range that begins before the window
        assume(c["start"] > 0)
        kb[i] = data.draw(st.integers(0, c["start"] - 1))
        want = wf.WF_ERR_RANGE
    elif which == 1:  # a range that ends after the window
        ke[i] = data.draw(st.integers(c["end"] + 1, c["end"] + 100))
        want = wf.WF_ERR_RANGE
    elif which == 2:  # an empty or reversed range
        ke[i] = data.draw(st.integers(c["start"], kb[i]))
        want = wf.WF_ERR_RANGE
    elif which == 3:  # q_off not starting at zero
        q_off = [1] + q_off[1:]
        assume(q_off[1] >= 1)
        want = wf.WF_ERR_INVALID_ARG
    elif which == 4:  # q_off decreasing
        assume(len(q_off) > 2 and q_off[1] > 0)
        q_off = list(q_off)
        q_off[2] = q_off[1] - 1
        want = wf.WF_ERR_INVALID_ARG
    else:             # the window itself is longer than the ring
        cache.c.end = cache.c.start + c["P"] * len(c["pages"]) + 8
        want = wf.WF_ERR_INVALID_ARG
    before = (cache.start, cache.end)
    try:
        wf.wf_chunk_attn_plan(cache, q_off, kb, ke, q_dtype=q_dtype)
        got = wf.WF_OK
    except wf.WfError as e:
        got = e.status
    assert got == want
    assert (cache.start, cache.end) == before


def split_rule(items, S, resident):
    """The split schedule as include/wf_chunk_attn.h states it: (parts, tail tiles, tails per
    block, grid), or None for the per-tile schedule."""
    if items >= resident:
        return None
    m = max(1, min(resident // items, S // 32, 8))
    na = items * m
    spare = resident - na
    b, q = 0, 1
    if spare > 0:
        q = -(-na // spare)
        b = (S // m) // (q + 1)
        if b < 8 or q > 5:
            b = 0
    if m == 1 and b == 0:
        return None
    return m, b, (q if b > 0 else 0), na + (-(-na // q) if b > 0 else 0)


@st.composite
def split_calls(draw):
    dtype = draw(st.sampled_from(["bf16", "fp8"]))
    H = draw(st.sampled_from([1, 2, 4, 12, 40]))
    P = 1560
    T = 21
    end = T * P
    S_keys = draw(st.integers(64, 30000))
    nc = draw(st.integers(1, 4))
    q_len = [draw(st.integers(0, 1200)) for _ in range(nc)]
    lead = draw(st.integers(0, 7))
    same = draw(st.booleans())
    kb, ke = [], []
    for _ in range(nc):
        n = S_keys if same else draw(st.integers(64, 30000))
        a = draw(st.integers(0, (end - n - 8) // 8)) * 8 + lead
        kb.append(a)
        ke.append(a + n)
    return dict(dtype=dtype, P=P, H=H, D=128, pages=list(range(T)), num_pages=T, start=0, end=end,
                q_len=q_len, kb=kb, ke=ke)


@pytest.mark.gpu
@settings(max_examples=200, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(split_calls())
def test_split_plan_follows_the_stated_rule(c):
    """With a workspace, the schedule wf_chunk_attn_plan reports is the one the header states
    (the resident-workgroup count comes from the workspace size the library asks for)."""
    cache, q_off = make(c)
    ws = wf.wf_chunk_attn_workspace_bytes(cache)
    resident = ws // (2 * 4 * (256 * c["D"] + 2 * 256))
    assert resident > 0
    plan = wf.wf_chunk_attn_plan(cache, q_off, c["kb"], c["ke"], q_dtype="bf16", workspace_bytes=ws)
    items = c["H"] * sum(-(-n // 256) for n in c["q_len"])
    steps = {(a % 8 + (b - a) + 63) // 64 for a, b, n in zip(c["kb"], c["ke"], c["q_len"]) if n > 0}
    want = split_rule(items, steps.pop(), resident) if items > 0 and len(steps) == 1 else None
    assert plan["items"] == items
    if want is None:
        assert plan["schedule"] == "per_tile" and plan["grid"] == items
    else:
        m, b, q, grid = want
        assert plan["schedule"] == "split"
        assert (plan["parts"], plan["tail_tiles"], plan["tails_per_block"], plan["grid"]) == (m, b, q, grid)
