"""Pins for the host KV-cache mirror and the storage decoders (CPU only).

The cache model is checked against an independently written logical model (a
dict from logical position to row), so the run splitting, ring wrap and page
table indirection are pinned by something that knows nothing about pages.
The decoders are pinned against torch's own dtype casts and against code
points printed in the OCP 8-bit float specification.
"""
import os

import numpy as np
import pytest
import torch

from oracle import KVCacheModel, decode_bf16, decode_e4m3fn

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_decode_matches_torch():
    bits = np.random.default_rng(0).integers(0, 1 << 16, size=20000, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = decode_bf16(bits)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])


def test_e4m3fn_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = decode_e4m3fn(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.isnan(got).sum() == 2  # 0x7F and 0xFF only


def test_e4m3fn_decode_golden_code_points():
    for line in open(os.path.join(GOLDEN, "e4m3fn_code_points.txt")):
        if not line.strip() or line.startswith("#"):
            continue
        code, val = line.split()
        got = decode_e4m3fn(np.array([int(code, 16)], np.uint8))[0]
        if val == "nan":
            assert np.isnan(got)
        else:
            assert got == float(val), (code, got, val)


class LogicalModel:
    """Position -> row dictionary; no pages, no ring."""

    def __init__(self):
        self.rows = {}
        self.start = self.end = 0

    def append(self, pos, k, v):
        for i in range(k.shape[0]):
            self.rows[pos + i] = (k[i].copy(), v[i].copy())
        self.end = max(self.end, pos + k.shape[0])

    def evict(self, n):
        for t in range(self.start, self.start + n):
            self.rows.pop(t, None)
        self.start += n


def _codes(rng, n, h, d, dtype):
    if dtype == "bf16":
        return rng.integers(0, 1 << 15, size=(n, h, d), dtype=np.uint16)
    if dtype == "fp8":
        return rng.integers(0, 0x7F, size=(n, h, d), dtype=np.uint8)  # finite codes
    return rng.standard_normal((n, h, d)).astype(np.float32)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("layout", ["identity", "permuted", "ring", "pool"])
def test_cache_matches_logical_model_over_many_rounds(dtype, layout):
    rng = np.random.default_rng(1)
    h, d = 3, 4
    if layout == "identity":
        P, table, pages = 8, np.arange(5), 5
    elif layout == "permuted":
        P, table, pages = 8, rng.permutation(5), 5
    elif layout == "ring":
        P, table, pages = 40, np.array([0]), 1
    else:  # a ring of 5 slots drawn from a larger pool of pages
        P, table, pages = 8, rng.permutation(9)[:5], 9
    cache = KVCacheModel(pages, P, h, d, dtype, table)
    ref = LogicalModel()
    for step in range(60):
        n = int(rng.integers(1, 13))
        live = cache.end - cache.start
        if live + n > cache.capacity:
            ev = live + n - cache.capacity + int(rng.integers(0, 3))
            ev = min(ev, live)
            cache.evict(ev)
            ref.evict(ev)
        # sometimes rewrite a suffix of the live window (timestep-0 refresh)
        pos = cache.end if rng.random() < 0.7 else int(rng.integers(cache.start, cache.end + 1))
        n = min(n, cache.start + cache.capacity - pos)
        k, v = _codes(rng, n, h, d, dtype), _codes(rng, n, h, d, dtype)
        cache.append(pos, k, v)
        ref.append(pos, k, v)
        assert (cache.start, cache.end) == (ref.start, ref.end)
        kc, vc = cache.gather_codes(cache.start, cache.end)
        for i, t in enumerate(range(cache.start, cache.end)):
            assert np.array_equal(kc[i], ref.rows[t][0]) and np.array_equal(vc[i], ref.rows[t][1])


def test_page_byte_layout():
    # K page [H][P][D]: token-major rows per head; V page [H][D][P]: transposed rows per head.
    rng = np.random.default_rng(2)
    P, h, d = 6, 2, 3
    table = np.array([2, 0, 1])
    cache = KVCacheModel(3, P, h, d, "bf16", table)
    k, v = _codes(rng, 14, h, d, "bf16"), _codes(rng, 14, h, d, "bf16")
    cache.append(0, k, v)
    for t in range(14):
        page, off = int(table[(t // P) % 3]), t % P
        for hh in range(h):
            for dd in range(d):
                assert cache.k[page, hh, off, dd] == k[t, hh, dd]
                assert cache.v[page, hh, dd, off] == v[t, hh, dd]


def test_paged_equals_contiguous_values():
    rng = np.random.default_rng(3)
    h, d, P = 2, 5, 10
    a = KVCacheModel(7, P, h, d, "f32", np.arange(7))
    b = KVCacheModel(9, P, h, d, "f32", rng.permutation(9)[:7])
    for r in range(12):
        if a.end + 9 > a.start + a.capacity:
            a.evict(9)
            b.evict(9)
        k, v = _codes(rng, 9, h, d, "f32"), _codes(rng, 9, h, d, "f32")
        a.append(a.end, k, v)
        b.append(b.end, k, v)
        ka, va = a.gather(a.start, a.end)
        kb, vb = b.gather(b.start, b.end)
        assert np.array_equal(ka, kb) and np.array_equal(va, vb)


def test_fp8_values_use_per_page_block_scales():
    rng = np.random.default_rng(4)
    P, h, d = 300, 2, 4          # 3 scale blocks per page: 128, 128, 44 tokens
    cache = KVCacheModel(2, P, h, d, "fp8", [1, 0])
    k, v = _codes(rng, 600, h, d, "fp8"), _codes(rng, 600, h, d, "fp8")
    ks = rng.uniform(0.5, 2.0, size=(2, h, 3)).astype(np.float32)
    vs = rng.uniform(0.5, 2.0, size=(2, h, 3)).astype(np.float32)
    cache.append(0, k, v, ks, vs)
    kv, vv = cache.gather(0, 600)
    for t in [0, 127, 128, 255, 256, 299, 300, 427, 428, 599]:
        p, off = t // P, t % P
        blk = off // 128
        for hh in range(h):
            assert np.array_equal(kv[t, hh], decode_e4m3fn(k[t, hh]) * np.float64(ks[p, hh, blk]))
            assert np.array_equal(vv[t, hh], decode_e4m3fn(v[t, hh]) * np.float64(vs[p, hh, blk]))
    # the scales landed on the physical pages named by the table
    assert np.array_equal(cache.k_scale[1], ks[0]) and np.array_equal(cache.k_scale[0], ks[1])


def test_poison_marks_evicted_rows():
    rng = np.random.default_rng(5)
    cache = KVCacheModel(2, 4, 1, 2, "bf16", [0, 1])
    cache.append(0, _codes(rng, 8, 1, 2, "bf16"), _codes(rng, 8, 1, 2, "bf16"))
    cache.evict(3, poison=True)
    assert np.all(cache.k[0, 0, :3, :] == 0x7FC0) and np.all(cache.v[0, 0, :, :3] == 0x7FC0)
    assert not np.any(cache.k[0, 0, 3:, :] == 0x7FC0)


def test_cache_rejects_bad_operations():
    rng = np.random.default_rng(6)
    c = KVCacheModel(2, 4, 1, 2, "bf16", [0, 1])
    k = _codes(rng, 5, 1, 2, "bf16")
    c.append(0, k, k)
    with pytest.raises(ValueError):
        c.append(6, k[:1], k[:1])          # gap after end
    with pytest.raises(ValueError):
        c.append(5, k[:4], k[:4])          # overruns live tokens (capacity 8)
    with pytest.raises(ValueError):
        c.evict(6)                         # more than the window
    with pytest.raises(ValueError):
        c.gather_codes(0, 6)
    with pytest.raises(ValueError):
        KVCacheModel(2, 4, 1, 2, "bf16", [0, 0])   # duplicate pages
    f = KVCacheModel(2, 4, 1, 2, "fp8", [0, 1])
    k8 = _codes(rng, 2, 1, 2, "fp8")
    with pytest.raises(ValueError):
        f.append(0, k8, k8, np.ones((0, 1, 1)), np.ones((0, 1, 1)))   # not page aligned


def test_gather_head_subset_matches_full_gather():
    rng = np.random.default_rng(7)
    P, h, d = 128, 5, 3
    c = KVCacheModel(3, P, h, d, "fp8", [2, 0, 1])
    k, v = _codes(rng, 256, h, d, "fp8"), _codes(rng, 256, h, d, "fp8")
    s = rng.uniform(0.5, 2, size=(2, h, 1)).astype(np.float32)
    c.append(0, k, v, s, s * 2)
    kf, vf = c.gather(10, 250)
    ks, vs = c.gather(10, 250, heads=[4, 1])
    assert np.array_equal(ks, kf[:, [4, 1]]) and np.array_equal(vs, vf[:, [4, 1]])
