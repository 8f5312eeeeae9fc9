"""GPU parity of wf_chunk_attn_fwd against the float64 oracle (needs an MI355X).

Bars: bf16 max-abs 1e-2 and mean-abs 1e-3 (plus rel-L2 1e-2, since the
outputs of flat softmax are small); E4M3FN K/V max-abs 5e-2 (plus rel-L2
6e-2); the fp32 path 1e-5 max-abs.  Inputs are seeded (synth) and identical on
both sides; the oracle reads the cache through its own byte mirror.
"""
import numpy as np
import pytest
import torch

import chunk_causal_dit_wf_amd as wf
import synth
from gpu_util import Pair, dev, errors, host_codes, host_values, values_of

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN, BF16_REL = 1e-2, 1e-3, 1e-2
FP8_MAX, FP8_REL = 5e-2, 6e-2
F32_MAX = 1e-5


def say(*a):
    print(*a, flush=True)


def check_bf16(got, ref, what):
    mx, mean, rel = errors(got, ref)
    say("%s: max-abs %.3e mean-abs %.3e rel-L2 %.3e" % (what, mx, mean, rel))
    assert mx <= BF16_MAX and mean <= BF16_MEAN and rel <= BF16_REL, (what, mx, mean, rel)


# ----------------------------------------------------------------------------- tiny fp32 workload

def tiny_pair(dtype):
    cfg = synth.TINY
    H, D, L = cfg["H"], cfg["D"], cfg["chunk"]
    pair = Pair(1, cfg["page_size"], H, D, dtype, [0], fill_seed=11)
    for c in range(cfg["num_chunks"]):
        k, v = synth.chunk_kv(cfg, 0, c)
        pair.append(c * L, synth.encode(k, dtype), synth.encode(v, dtype))
    return pair


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tiny_last_chunk(dtype):
    cfg = synth.TINY
    say("case: tiny last chunk", dtype)
    pair = tiny_pair(dtype)
    q = synth.encode(synth.queries(cfg, 0, 64), dtype)
    o, lse = pair.attend(dev(q, dtype), [0, 64], [0], [192])
    ro, rl = pair.reference(values_of(q, dtype), [0, 64], [0], [192])
    got = host_values(o)
    if dtype == "f32":
        mx = np.abs(got - ro).max()
        say("f32 max-abs %.3e" % mx)
        assert mx <= F32_MAX
    else:
        check_bf16(got, ro, "tiny bf16")
    assert np.abs(lse.cpu().numpy() - rl).max() < (1e-5 if dtype == "f32" else 2e-3)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tiny_varlen_prefixes(dtype):
    cfg = synth.TINY
    say("case: tiny varlen", dtype)
    pair = tiny_pair(dtype)
    q = synth.encode(synth.queries(cfg, 0, 192, stream=1), dtype)
    q_off, kb, ke = [0, 64, 128, 192], [0, 0, 0], [64, 128, 192]
    o, lse = pair.attend(dev(q, dtype), q_off, kb, ke)
    ro, rl = pair.reference(values_of(q, dtype), q_off, kb, ke)
    got = host_values(o)
    if dtype == "f32":
        assert np.abs(got - ro).max() <= F32_MAX
    else:
        check_bf16(got, ro, "tiny varlen bf16")
    assert np.abs(lse.cpu().numpy() - rl).max() < (1e-5 if dtype == "f32" else 2e-3)


# ----------------------------------------------------------------------------- Wan-1.3B shapes

def wan_pair(cfg, kv_stds):
    H, D, L = cfg["H"], cfg["D"], cfg["chunk"]
    pair = Pair(cfg["num_pages"], cfg["page_size"], H, D, "bf16", synth.identity_table(cfg["table_len"]))
    for c in range(4):
        k, v = synth.chunk_kv(cfg, 0, c, std=kv_stds[c])
        pair.append(c * L, synth.bf16_codes(k), synth.bf16_codes(v))
    return pair


@pytest.mark.parametrize("sharp", [False, True])
def test_wan_single_call(sharp):
    """4680 query rows of chunk 3 over 18720 keys, 12 heads x 128 (sharp: Q scaled x4)."""
    cfg = synth.WAN_CALL
    say("case: wan single call sharp=%s" % sharp)
    pair = wan_pair(cfg, [cfg["std"]] * 4)
    qf = synth.queries(cfg, 0, cfg["chunk"]) * (4.0 if sharp else 1.0)
    q = synth.bf16_codes(qf)
    o, lse = pair.attend(dev(q, "bf16"), [0, 4680], [0], [18720])
    ro, rl = pair.reference(values_of(q, "bf16"), [0, 4680], [0], [18720])
    check_bf16(host_values(o), ro, "wan call")
    assert np.abs(lse.cpu().numpy() - rl).max() < 2e-3


def test_wave_four_chunks_one_launch():
    """Staggered wave: 4 query chunks with prefixes 4680..18720, per-chunk K/V noise levels."""
    cfg = synth.WAVE
    say("case: wave 4 chunks")
    pair = wan_pair(cfg, list(cfg["kv_std"]))
    q = synth.bf16_codes(synth.queries(cfg, 0, 4 * 4680))
    q_off = [0, 4680, 9360, 14040, 18720]
    kb, ke = [0] * 4, [4680, 9360, 14040, 18720]
    o, lse = pair.attend(dev(q, "bf16"), q_off, kb, ke)
    ro, rl = pair.reference(values_of(q, "bf16"), q_off, kb, ke)
    check_bf16(host_values(o), ro, "wave")
    assert np.abs(lse.cpu().numpy() - rl).max() < 2e-3


def sample_rows(n, count, seed):
    return np.sort(np.random.default_rng(seed).choice(n, size=count, replace=False))


@pytest.mark.parametrize("layer", [0, 29])
def test_round_paged_ring_full_size(layer):
    """The forward-round shape: paged ring (P 1560, T 21, permuted), prefill 18 frames, then
    evict -> append -> attend for 8 rounds (the ring wraps).  Sampled rows vs the oracle."""
    cfg = synth.WAN_ROUND
    H, D, L = cfg["H"], cfg["D"], cfg["chunk"]
    say("case: round layer", layer)
    table = synth.permuted_table(cfg["workload"], layer, cfg["table_len"])
    pair = Pair(cfg["num_pages"], cfg["page_size"], H, D, "bf16", table)
    for c in range(cfg["prefill_chunks"]):
        k, v = synth.chunk_kv(cfg, layer, c)
        pair.append(c * L, synth.bf16_codes(k), synth.bf16_codes(v))
    for r in range(8):
        if pair.gpu.end - pair.gpu.start + L > pair.gpu.capacity:
            pair.evict(L)
        k, v = synth.chunk_kv(cfg, layer, cfg["prefill_chunks"] + r)
        pos = pair.gpu.end
        pair.append(pos, synth.bf16_codes(k), synth.bf16_codes(v))
        if r not in (0, 3, 7):
            continue
        assert pair.pages_equal()
        q = synth.bf16_codes(synth.queries(cfg, layer, L, stream=r))
        kb, ke = max(pair.gpu.start, pair.gpu.end - synth.WINDOW_TOKENS), pair.gpu.end
        assert ke - kb == 32760
        o, lse = pair.attend(dev(q, "bf16"), [0, L], [kb], [ke])
        rows = sample_rows(L, 384, 100 + r)
        ro, rl = pair.reference(values_of(q, "bf16")[rows], [0, len(rows)], [kb], [ke])
        check_bf16(host_values(o)[rows], ro, "round %d" % r)
        assert np.abs(lse.cpu().numpy()[:, rows] - rl).max() < 2e-3


def test_fp8_kv_14b_shape_sampled():
    """40 heads, bf16 Q over E4M3FN K/V with per-(page, head, 128-token) scales, 32760 keys."""
    cfg = synth.FP8_14B
    H, D, L, P = cfg["H"], cfg["D"], cfg["chunk"], cfg["page_size"]
    say("case: fp8 14b")
    table = synth.permuted_table(cfg["workload"], 0, cfg["table_len"])
    pair = Pair(cfg["num_pages"], P, H, D, "fp8", table)
    for c in range(cfg["prefill_chunks"] + 2):
        if pair.gpu.end - pair.gpu.start + L > pair.gpu.capacity:
            pair.evict(L)
        k, v = synth.chunk_kv(cfg, 0, c)
        kc, ks = synth.quantize_e4m3_pages(k, P)
        vc, vs = synth.quantize_e4m3_pages(v, P)
        pair.append(pair.gpu.end, kc, vc, ks, vs)
    assert pair.pages_equal()
    q = synth.bf16_codes(synth.queries(cfg, 0, L))
    kb, ke = pair.gpu.start, pair.gpu.end
    assert ke - kb == 32760
    o, lse = pair.attend(dev(q, "bf16"), [0, L], [kb], [ke])
    rows = sample_rows(L, 128, 7)
    heads = [0, 7, 13, 22, 31, 39]
    qv = values_of(q, "bf16")[rows][:, heads]
    ro, rl = pair.reference(qv, [0, len(rows)], [kb], [ke], heads=heads)
    got = host_values(o)[rows][:, heads]
    mx, mean, rel = errors(got, ro)
    say("fp8: max-abs %.3e mean-abs %.3e rel-L2 %.3e" % (mx, mean, rel))
    assert mx <= FP8_MAX and rel <= FP8_REL
    assert np.abs(lse.cpu().numpy()[heads][:, rows] - rl).max() < 2e-2


# ----------------------------------------------------------------------------- ragged / edge shapes

@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
def test_ragged_chunks_small_pages(dtype, D):
    """Pages smaller than a key tile, unaligned window starts, chunks of 1..300 rows, empty chunks."""
    rng = np.random.default_rng(1000 + D)
    H, P, T, pool = 3, 24, 9, 13
    table = rng.permutation(pool)[:T]
    pair = Pair(pool, P, H, D, dtype, table, fill_seed=5)
    # fill 200 tokens in uneven appends, evict 13, rewrite a suffix
    pos = 0
    for n in [7, 64, 1, 50, 78]:
        k = synth.encode(rng.standard_normal((n, H, D)).astype(np.float32), dtype)
        v = synth.encode(rng.standard_normal((n, H, D)).astype(np.float32), dtype)
        pair.append(pos, k, v)
        pos += n
    pair.evict(13)
    k = synth.encode(rng.standard_normal((30, H, D)).astype(np.float32), dtype)
    pair.append(pair.gpu.end - 30, k, k)
    assert pair.pages_equal()
    lens = [1, 129, 0, 37, 128, 300, 5]
    q_off = np.concatenate([[0], np.cumsum(lens)]).tolist()
    kb, ke = [], []
    for i in range(len(lens)):
        a = int(rng.integers(pair.gpu.start, pair.gpu.end - 1))
        b = int(rng.integers(a + 1, pair.gpu.end + 1))
        kb.append(a)
        ke.append(b)
    kb[0], ke[0] = 13, 14            # a single visible key
    kb[1], ke[1] = 13, 200           # the whole window
    q = synth.encode(rng.standard_normal((q_off[-1], H, D)).astype(np.float32), dtype)
    o, lse = pair.attend(dev(q, dtype), q_off, kb, ke)
    ro, rl = pair.reference(values_of(q, dtype), q_off, kb, ke)
    got = host_values(o)
    if dtype == "f32":
        mx = np.abs(got - ro).max()
        say("ragged f32 D%d max-abs %.3e" % (D, mx))
        assert mx <= F32_MAX
    else:
        check_bf16(got, ro, "ragged bf16 D%d" % D)
    assert np.abs(lse.cpu().numpy() - rl).max() < (1e-5 if dtype == "f32" else 2e-3)


# ----------------------------------------------------------------------------- invariants

def small_bf16_pair(seed, n=300, H=2, D=128, P=40, table=(3, 1, 4, 0, 2, 6, 5, 7)):
    rng = np.random.default_rng(seed)
    pair = Pair(8, P, H, D, "bf16", list(table), fill_seed=seed + 1)
    k = synth.bf16_codes(rng.standard_normal((n, H, D)).astype(np.float32))
    v = synth.bf16_codes(rng.standard_normal((n, H, D)).astype(np.float32))
    pair.append(0, k, v)
    return pair, rng


def test_single_key_returns_value_bitwise():
    pair, rng = small_bf16_pair(1)
    q = synth.bf16_codes(rng.standard_normal((70, 2, 128)).astype(np.float32))
    o, _ = pair.attend(dev(q, "bf16"), [0, 70], [123], [124])
    _, vc = pair.ref.gather_codes(123, 124)
    assert np.array_equal(host_codes(o), np.broadcast_to(vc[0], (70, 2, 128)))


def test_constant_values_give_ones():
    rng = np.random.default_rng(2)
    pair = Pair(8, 40, 2, 128, "bf16", list(range(8)))
    k = synth.bf16_codes(rng.standard_normal((300, 2, 128)).astype(np.float32))
    ones = np.full((300, 2, 128), 0x3F80, np.uint16)
    pair.append(0, k, ones)
    q = synth.bf16_codes(rng.standard_normal((130, 2, 128)).astype(np.float32) * 3)
    o, _ = pair.attend(dev(q, "bf16"), [0, 130], [3], [297])
    assert np.abs(host_values(o) - 1.0).max() <= 2.0 ** -8


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_coverage_counts_exact_visible_set(dtype):
    """Q = 0 and V[j,h,d] = bit d of j: O[:,h,d] = (# visible keys with bit d set) / n."""
    H, D, n = 2, 64, 2000
    pair = Pair(5, 400, H, D, dtype, [4, 2, 0, 1, 3])
    bits = ((np.arange(n)[:, None] >> np.arange(D)[None, :]) & 1).astype(np.float32)
    bits[:, 17:] = 0
    v = np.repeat(bits[:, None, :], H, axis=1)
    k = np.random.default_rng(3).standard_normal((n, H, D)).astype(np.float32)
    pair.append(0, synth.encode(k, dtype), synth.encode(v, dtype))
    q = synth.encode(np.zeros((3, H, D), np.float32), dtype)
    kb, ke = [5, 777, 1999], [1601, 2000, 2000]
    o, _ = pair.attend(dev(q, dtype), [0, 1, 2, 3], kb, ke)
    got = host_values(o)
    for c in range(3):
        js = np.arange(kb[c], ke[c])
        want = ((js[:, None] >> np.arange(D)[None, :]) & 1).sum(0) / len(js)
        want[17:] = 0
        tol = 1e-6 if dtype == "f32" else 2.0 ** -8
        assert np.all(np.abs(got[c, 0] - want) <= tol * np.maximum(want, 1e-3)), (c, got[c, 0][:17], want[:17])


def test_keys_outside_the_window_are_never_read():
    pair, rng = small_bf16_pair(4)
    q = synth.bf16_codes(rng.standard_normal((90, 2, 128)).astype(np.float32))
    qd = dev(q, "bf16")
    o1, l1 = pair.attend(qd, [0, 40, 90], [41, 60], [203, 250])
    # NaN-poison keys of later chunks (rewrite [250, 300)) and the evicted prefix [0, 41)
    nan = np.full((50, 2, 128), 0x7FC0, np.uint16)
    pair.append(250, nan, nan)
    pair.evict(41, poison=True)
    o2, l2 = pair.attend(qd, [0, 40, 90], [41, 60], [203, 250])
    assert np.array_equal(host_codes(o1), host_codes(o2))
    assert np.array_equal(l1.cpu().numpy(), l2.cpu().numpy())


def test_paged_equals_contiguous_bitwise():
    rng = np.random.default_rng(5)
    H, D, P = 3, 128, 64
    a = Pair(6, P, H, D, "bf16", list(range(6)))
    b = Pair(10, P, H, D, "bf16", [9, 2, 7, 0, 5, 3])
    for r in range(5):
        if a.gpu.end - a.gpu.start + 100 > a.gpu.capacity:
            a.evict(100)
            b.evict(100)
        k = synth.bf16_codes(rng.standard_normal((100, H, D)).astype(np.float32))
        v = synth.bf16_codes(rng.standard_normal((100, H, D)).astype(np.float32))
        a.append(a.gpu.end, k, v)
        b.append(b.gpu.end, k, v)
    q = dev(synth.bf16_codes(rng.standard_normal((200, H, D)).astype(np.float32)), "bf16")
    args = ([0, 77, 200], [a.gpu.start + 3, a.gpu.start], [a.gpu.end - 10, a.gpu.end])
    oa, la = a.attend(q, *args)
    ob, lb = b.attend(q, *args)
    assert np.array_equal(host_codes(oa), host_codes(ob))
    assert np.array_equal(la.cpu().numpy(), lb.cpu().numpy())


def test_run_to_run_deterministic():
    pair, rng = small_bf16_pair(6)
    q = dev(synth.bf16_codes(rng.standard_normal((257, 2, 128)).astype(np.float32)), "bf16")
    outs = [pair.attend(q, [0, 100, 257], [0, 50], [300, 280]) for _ in range(3)]
    for o, l in outs[1:]:
        assert np.array_equal(host_codes(o), host_codes(outs[0][0]))
        assert np.array_equal(l.cpu().numpy(), outs[0][1].cpu().numpy())
