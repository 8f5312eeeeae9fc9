"""GPU parity at the documented limits (needs an MI355X).

- A bf16 or E4M3FN cache of more than 4 GiB per tensor: the plan takes the
  register-staged kernel (64-bit page addressing), with the window's pages
  on both sides of the 4 GiB line.
- WF_MAX_CHUNKS = 64 chunks in one call, empty and ragged ones included.
- A ring of WF_MAX_TABLE_LEN = 256 slots whose live window wraps from the last
  slot to the first.
Every case is compared with the float64 oracle at the bf16 bars.
"""
import numpy as np
import pytest
import torch

import chunk_causal_dit_wf_amd as wf
from chunk_causal_dit_wf_amd import _lib
import oracle
import synth
from gpu_util import Pair, dev, errors, host_values, values_of

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN, BF16_REL = 1e-2, 1e-3, 1e-2


def say(*a):
    print(*a, flush=True)


def within_bars(got, ro, what):
    mx, mean, rel = errors(got, ro)
    say("%s: max-abs %.3e mean-abs %.3e rel-L2 %.3e" % (what, mx, mean, rel))
    assert mx <= BF16_MAX and mean <= BF16_MEAN and rel <= BF16_REL, (what, mx, mean, rel)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_cache_over_4gib_takes_the_staged_kernel(dtype):
    """H1 D128 P64 with more than 4 GiB per tensor (262208 bf16 or 524352 E4M3FN pages); the 16 ring
    slots map to pages on both sides of the 4 GiB line.  1024 tokens appended, 300 query rows over
    keys [5, 1000).  The oracle reads the same rows through a 16-page cache model."""
    H, D, P = 1, 128, 64
    esize = 2 if dtype == "bf16" else 1
    per_page = H * P * D * esize
    line = (1 << 32) // per_page
    num_pages = line + 64
    assert num_pages * per_page > (1 << 32)
    rng = np.random.default_rng([42, 901, esize])
    table = [num_pages - 1, line + 3, 100, line + 6, 7, num_pages - 5, line, 33,
             line + 56, 1, line + 16, 5000, line + 26, line + 1, line // 2, line + 46]
    say("case: %s cache over 4 GiB, %d pages, table %s" % (dtype, num_pages, table))
    cache = wf.KVCache(num_pages, P, H, D, dtype, table, device="cuda")
    ref = oracle.KVCacheModel(len(table), P, H, D, dtype, list(range(len(table))))
    n = len(table) * P
    kf = rng.standard_normal((n, H, D)).astype(np.float32)
    vf = rng.standard_normal((n, H, D)).astype(np.float32)
    if dtype == "bf16":
        k, v = synth.bf16_codes(kf), synth.bf16_codes(vf)
        wf.wf_kv_append(cache, 0, dev(k, "bf16"), dev(v, "bf16"))
        ref.append(0, k, v)
    else:
        (k, ks), (v, vs) = synth.quantize_e4m3_pages(kf, P), synth.quantize_e4m3_pages(vf, P)
        wf.wf_kv_append(cache, 0, dev(k, "fp8"), dev(v, "fp8"), dev(ks, "scale"), dev(vs, "scale"))
        ref.append(0, k, v, ks, vs)
    q = synth.bf16_codes(rng.standard_normal((300, H, D)).astype(np.float32))
    q_off, kb, ke = [0, 300], [5], [1000]
    pl = wf.wf_chunk_attn_plan(cache, q_off, kb, ke, "bf16", 0)
    say("plan:", pl)
    assert pl["kernel"] == "staged_" + dtype, pl
    o, lse = wf.wf_chunk_attn_fwd(cache, dev(q, "bf16"), q_off, kb, ke, return_lse=True, workspace=None)
    torch.cuda.synchronize()
    K, V = ref.gather(0, n)
    ro, rl = oracle.chunk_attention(values_of(q, "bf16"), K, V, q_off, kb, ke, kv_origin=0)
    within_bars(host_values(o), ro, "%s over 4 GiB" % dtype)
    assert np.abs(lse.cpu().numpy() - rl).max() < 2e-3
    del cache, o, lse
    torch.cuda.empty_cache()


def test_max_chunks_in_one_call():
    """WF_MAX_CHUNKS = 64 chunks (0 to 300 rows, 11 of them empty) over their own windows of a
    paged bf16 cache (P256, LDS-DMA kernel), in one call."""
    assert _lib.WF_MAX_CHUNKS == 64
    say("case: 64 chunks")
    rng = np.random.default_rng([42, 902])
    H, D, P, T = 2, 128, 256, 40
    pair = Pair(T, P, H, D, "bf16", list(rng.permutation(T)), fill_seed=903)
    n = T * P
    k = synth.bf16_codes(rng.standard_normal((n, H, D)).astype(np.float32))
    v = synth.bf16_codes(rng.standard_normal((n, H, D)).astype(np.float32))
    pair.append(0, k, v)
    lens = rng.integers(1, 300, size=64)
    lens[rng.choice(64, size=11, replace=False)] = 0
    q_off = [0] + np.cumsum(lens).tolist()
    kb, ke = [], []
    for _ in range(64):
        a = int(rng.integers(0, n - 64))
        b = int(rng.integers(a + 1, min(n, a + 6000) + 1))
        kb.append(a)
        ke.append(b)
    q = synth.bf16_codes(rng.standard_normal((q_off[-1], H, D)).astype(np.float32))
    pl = wf.wf_chunk_attn_plan(pair.gpu, q_off, kb, ke, "bf16", 0)
    say("plan:", pl, "rows", q_off[-1])
    assert pl["kernel"] == "dma_bf16"
    o, lse = pair.attend(dev(q, "bf16"), q_off, kb, ke, workspace=None)
    ro, rl = pair.reference(values_of(q, "bf16"), q_off, kb, ke)
    within_bars(host_values(o), ro, "64 chunks")
    assert np.abs(lse.cpu().numpy() - rl).max() < 2e-3


@pytest.mark.parametrize("P", [64, 40])
def test_ring_of_max_slots_wraps(P):
    """WF_MAX_TABLE_LEN = 256 ring slots (P64: LDS-DMA kernel; P40: register-staged): the ring is
    filled, 8000 tokens are evicted and 8000 more appended, so the live window runs from slot 125
    (P64) across the last slot to the first; 200 query rows over most of it."""
    assert _lib.WF_MAX_TABLE_LEN == 256
    say("case: 256-slot ring, P%d" % P)
    rng = np.random.default_rng([42, 904, P])
    H, D, T = 2, 128, 256
    pair = Pair(T + 8, P, H, D, "bf16", list(rng.permutation(T + 8)[:T]), fill_seed=905)
    cap = T * P
    k = synth.bf16_codes(rng.standard_normal((cap + 8000, H, D)).astype(np.float32))
    v = synth.bf16_codes(rng.standard_normal((cap + 8000, H, D)).astype(np.float32))
    pair.append(0, k[:cap], v[:cap])
    pair.evict(8000)
    pair.append(cap, k[cap:], v[cap:])
    assert (pair.gpu.start, pair.gpu.end) == (8000, cap + 8000)
    q = synth.bf16_codes(rng.standard_normal((200, H, D)).astype(np.float32))
    q_off, kb, ke = [0, 120, 200], [8003, 9000], [cap + 8000, cap + 7001]
    o, lse = pair.attend(dev(q, "bf16"), q_off, kb, ke, workspace=None)
    ro, rl = pair.reference(values_of(q, "bf16"), q_off, kb, ke)
    within_bars(host_values(o), ro, "256-slot ring P%d" % P)
    assert np.abs(lse.cpu().numpy() - rl).max() < 2e-3


@pytest.mark.parametrize("P", [256, 40])
@pytest.mark.parametrize("s0", [(1 << 31) - 3000, (1 << 32) - 3000, (1 << 40) + 17])
def test_long_running_stream_positions(s0, P):
    """A stream whose logical positions have passed 2^31, 2^32 or 2^40 tokens (about a day of
    Wan-rate generation passes 2^31): the cache starts at position s0, is filled, 2000 tokens are
    evicted and 2000 appended, so the window crosses the boundary; cache bytes bit-exact and two
    chunks' attention against the oracle (P256: LDS-DMA kernel; P40: register-staged)."""
    say("case: stream positions from %d, P%d" % (s0, P))
    rng = np.random.default_rng([42, 906, P, s0 % 1000])
    H, D, T = 2, 128, (24 if P == 256 else 128)  # rings of 6144 and 5120 tokens
    pair = Pair(T + 4, P, H, D, "bf16", list(rng.permutation(T + 4)[:T]), fill_seed=907)
    pair.gpu.c.start = pair.gpu.c.end = s0
    pair.ref.start = pair.ref.end = s0
    cap = T * P
    k = synth.bf16_codes(rng.standard_normal((cap + 2000, H, D)).astype(np.float32))
    v = synth.bf16_codes(rng.standard_normal((cap + 2000, H, D)).astype(np.float32))
    pair.append(s0, k[:cap], v[:cap])
    pair.evict(2000)
    pair.append(s0 + cap, k[cap:], v[cap:])
    assert (pair.gpu.start, pair.gpu.end) == (s0 + 2000, s0 + cap + 2000)
    assert pair.pages_equal()
    q = synth.bf16_codes(rng.standard_normal((300, H, D)).astype(np.float32))
    q_off = [0, 180, 300]
    kb, ke = [s0 + 2005, s0 + 3000], [s0 + cap + 2000, s0 + cap + 1000]
    o, lse = pair.attend(dev(q, "bf16"), q_off, kb, ke, workspace=None)
    ro, rl = pair.reference(values_of(q, "bf16"), q_off, kb, ke)
    within_bars(host_values(o), ro, "positions from %d, P%d" % (s0, P))
    assert np.abs(lse.cpu().numpy() - rl).max() < 2e-3


@pytest.mark.parametrize("s0", [(1 << 31) - 3 * 256, (1 << 32) - 12 * 256, 1 << 40])
def test_long_running_stream_positions_fp8(s0):
    """The same on an E4M3FN cache (P256, fp8-MFMA kernel): whole-page appends of pre-quantised
    pages, then 8 pages evicted and 8 appended through the quantising append; cache bytes and
    scales bit-exact, attention against the oracle at the fp8 bars."""
    say("case: fp8 stream positions from %d" % s0)
    P, H, D, T = 256, 2, 128, 24
    rng = np.random.default_rng([42, 908, s0 % 1000])
    pair = Pair(T + 4, P, H, D, "fp8", list(rng.permutation(T + 4)[:T]), fill_seed=909)
    pair.gpu.c.start = pair.gpu.c.end = s0
    pair.ref.start = pair.ref.end = s0
    cap = T * P
    kc, ks = synth.quantize_e4m3_pages(rng.standard_normal((cap, H, D)).astype(np.float32), P)
    vc, vs = synth.quantize_e4m3_pages(rng.standard_normal((cap, H, D)).astype(np.float32), P)
    pair.append(s0, kc, vc, ks, vs)
    pair.evict(8 * P)
    kn = synth.bf16_codes(rng.standard_normal((8 * P, H, D)).astype(np.float32))
    vn = synth.bf16_codes(rng.standard_normal((8 * P, H, D)).astype(np.float32))
    pair.append_quantize(s0 + cap, kn, vn)
    assert (pair.gpu.start, pair.gpu.end) == (s0 + 8 * P, s0 + cap + 8 * P)
    assert pair.pages_equal()
    q = synth.bf16_codes(rng.standard_normal((300, H, D)).astype(np.float32))
    q_off = [0, 180, 300]
    kb, ke = [s0 + 8 * P + 5, s0 + 3000], [s0 + cap + 8 * P, s0 + cap + 1000]
    pl = wf.wf_chunk_attn_plan(pair.gpu, q_off, kb, ke, "bf16", 0)
    assert pl["kernel"] == "dma_fp8", pl
    o, lse = pair.attend(dev(q, "bf16"), q_off, kb, ke, workspace=None)
    ro, rl = pair.reference(values_of(q, "bf16"), q_off, kb, ke)
    got = host_values(o)
    mx, mean, rel = errors(got, ro)
    say("fp8 positions from %d: max-abs %.3e mean-abs %.3e rel-L2 %.3e" % (s0, mx, mean, rel))
    assert mx <= 5e-2 and rel <= 6e-2, (mx, rel)
    assert np.abs(lse.cpu().numpy() - rl).max() < 3e-2
