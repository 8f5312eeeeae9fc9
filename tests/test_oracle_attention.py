"""Pins for the float64 chunk-attention oracle (CPU only).

Each test ties the oracle to something other than itself: an independently
written brute force, a library routine, a closed form, or an invariant that
the definition of softmax attention forces.  Definition followed: chunk-wise
causal attention (Wave Forcing abstract) -- chunk c sees logical keys
[kv_begin[c], kv_end[c]).
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import brute_force_attention, chunk_attention, merge_partials

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


def test_brute_force_toy_varlen():
    # 3 chunks x 4 tokens, queries of every chunk, block-causal prefixes 4/8/12.
    q, k, v = _rand((12, 2, 5), 1), _rand((12, 2, 5), 2), _rand((12, 2, 5), 3)
    q_off, kb, ke = [0, 4, 8, 12], [0, 0, 0], [4, 8, 12]
    o, lse = chunk_attention(q, k, v, q_off, kb, ke)
    ob, lseb = brute_force_attention(q, k, v, q_off, kb, ke)
    assert np.max(np.abs(o - np.array(ob))) < 1e-12
    assert np.max(np.abs(lse - np.array(lseb))) < 1e-12


def test_brute_force_rolling_window_and_origin():
    # keys given for logical positions [100, 130); chunk windows start after evictions.
    q, k, v = _rand((9, 3, 4), 4), _rand((30, 3, 4), 5), _rand((30, 3, 4), 6)
    q_off, kb, ke = [0, 2, 9], [103, 110], [118, 130]
    o, lse = chunk_attention(q, k, v, q_off, kb, ke, scale=0.37, kv_origin=100)
    kk = np.concatenate([np.zeros((100, 3, 4)), k])
    vv = np.concatenate([np.zeros((100, 3, 4)), v])
    ob, lseb = brute_force_attention(q, kk, vv, q_off, kb, ke, scale=0.37)
    assert np.max(np.abs(o - np.array(ob))) < 1e-12
    assert np.max(np.abs(lse - np.array(lseb))) < 1e-12


def test_brute_force_tiny_workload_shape():
    # The tiny fp32 workload: 2 heads x 64 dims, last chunk (64 rows) over 3 chunks (192 keys).
    q, k, v = _rand((64, 2, 64), 7), _rand((192, 2, 64), 8), _rand((192, 2, 64), 9)
    o, lse = chunk_attention(q, k, v, [0, 64], [0], [192])
    ob, lseb = brute_force_attention(q, k, v, [0, 64], [0], [192])
    assert np.max(np.abs(o - np.array(ob))) < 1e-12
    assert np.max(np.abs(lse - np.array(lseb))) < 1e-12


def test_library_sdpa_float64_block_causal_mask():
    # torch's scaled_dot_product_attention (default scale 1/sqrt(D)) with an explicit boolean mask.
    nq, nk, h, d = 24, 40, 3, 16
    q, k, v = _rand((nq, h, d), 10), _rand((nk, h, d), 11), _rand((nk, h, d), 12)
    q_off, kb, ke = [0, 5, 13, 24], [0, 8, 19], [10, 30, 40]
    o, _ = chunk_attention(q, k, v, q_off, kb, ke)
    mask = torch.zeros(nq, nk, dtype=torch.bool)
    for c in range(3):
        mask[q_off[c]:q_off[c + 1], kb[c]:ke[c]] = True
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(k).permute(1, 0, 2)[None]
    tv = torch.from_numpy(v).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)
    ref = ref[0].permute(1, 0, 2).numpy()
    assert np.max(np.abs(o - ref)) < 1e-12


def test_rows_sum_to_one():
    q, k = _rand((16, 2, 8), 13), _rand((20, 2, 8), 14)
    v = np.ones((20, 2, 8))
    o, _ = chunk_attention(q, k, v, [0, 7, 16], [0, 3], [12, 20])
    assert np.max(np.abs(o - 1.0)) < 1e-14


def test_single_visible_key_returns_its_value():
    q, k, v = _rand((6, 2, 8), 15), _rand((10, 2, 8), 16), _rand((10, 2, 8), 17)
    o, lse = chunk_attention(q, k, v, [0, 3, 6], [4, 9], [5, 10])
    assert np.array_equal(o[:3], np.broadcast_to(v[4], (3, 2, 8)))
    assert np.array_equal(o[3:], np.broadcast_to(v[9], (3, 2, 8)))
    s = (q[:3] * k[4]).sum(-1) / math.sqrt(8)
    assert np.max(np.abs(lse[:, :3] - s.T)) < 1e-14


def test_zero_queries_give_mean_and_log_n():
    k, v = _rand((30, 2, 8), 18), _rand((30, 2, 8), 19)
    q = np.zeros((5, 2, 8))
    o, lse = chunk_attention(q, k, v, [0, 2, 5], [3, 10], [13, 30])
    assert np.max(np.abs(o[:2] - v[3:13].mean(0))) < 1e-14
    assert np.max(np.abs(o[2:] - v[10:30].mean(0))) < 1e-14
    assert np.max(np.abs(lse[:, :2] - math.log(10))) < 1e-14
    assert np.max(np.abs(lse[:, 2:] - math.log(20))) < 1e-14


def test_two_keys_sigmoid_closed_form():
    q, k, v = _rand((4, 1, 6), 20), _rand((2, 1, 6), 21), _rand((2, 1, 6), 22)
    o, lse = chunk_attention(q, k, v, [0, 4], [0], [2], scale=0.5)
    s = 0.5 * (q[:, 0, :] @ k[:, 0, :].T)
    a = 1.0 / (1.0 + np.exp(-(s[:, 0] - s[:, 1])))
    ref = a[:, None] * v[0, 0] + (1 - a)[:, None] * v[1, 0]
    assert np.max(np.abs(o[:, 0, :] - ref)) < 1e-14
    assert np.max(np.abs(lse[0] - np.log(np.exp(s[:, 0]) + np.exp(s[:, 1])))) < 1e-13


def test_golden_two_key_values():
    """Hand-derived fixture: see tests/golden/two_key_closed_form.txt."""
    rows = [l.split() for l in open(os.path.join(GOLDEN, "two_key_closed_form.txt"))
            if l.strip() and not l.startswith("#")]
    for r in rows:
        s1, s2, v1, v2, expect_o, expect_lse = map(float, r)
        q = np.array([[[1.0]]])
        k = np.array([[[s1]], [[s2]]])
        v = np.array([[[v1]], [[v2]]])
        o, lse = chunk_attention(q, k, v, [0, 1], [0], [2], scale=1.0)
        assert abs(o[0, 0, 0] - expect_o) < 1e-15 * max(1, abs(expect_o)) * 4
        assert abs(lse[0, 0] - expect_lse) < 1e-14


def test_coverage_pins_exact_visible_set():
    # Q = 0 and V[j,h,d] = bit d of j  =>  O[:,h,d] = (# visible keys with bit d set) / n.
    nk, d = 3000, 12
    v = ((np.arange(nk)[:, None] >> np.arange(d)[None, :]) & 1).astype(np.float64)
    v = np.repeat(v[:, None, :], 2, axis=1)
    k = _rand((nk, 2, d), 23)
    q = np.zeros((3, 2, d))
    kb, ke = [17, 1000, 2047], [1234, 2999, 2049]
    o, _ = chunk_attention(q, k, v, [0, 1, 2, 3], kb, ke)
    for c in range(3):
        js = np.arange(kb[c], ke[c])
        want = ((js[:, None] >> np.arange(d)[None, :]) & 1).sum(0) / len(js)
        assert np.max(np.abs(o[c, 0] - want)) < 1e-14


def test_keys_outside_window_do_not_matter():
    q, k, v = _rand((8, 2, 8), 24), _rand((40, 2, 8), 25), _rand((40, 2, 8), 26)
    o, lse = chunk_attention(q, k, v, [0, 8], [10], [25])
    k2, v2 = k.copy(), v.copy()
    k2[:10] = np.nan
    v2[25:] = np.inf
    o2, lse2 = chunk_attention(q, k2, v2, [0, 8], [10], [25])
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_lse_merge_of_disjoint_key_sets():
    q, k, v = _rand((10, 2, 8), 27), _rand((50, 2, 8), 28), _rand((50, 2, 8), 29)
    o, lse = chunk_attention(q, k, v, [0, 10], [0], [50])
    oa, la = chunk_attention(q, k, v, [0, 10], [0], [17])
    ob, lb = chunk_attention(q, k, v, [0, 10], [17], [50])
    om, lm = merge_partials(oa, la, ob, lb)
    assert np.max(np.abs(o - om)) < 1e-13 and np.max(np.abs(lse - lm)) < 1e-13


def test_key_order_does_not_matter():
    q, k, v = _rand((10, 2, 8), 30), _rand((33, 2, 8), 31), _rand((33, 2, 8), 32)
    perm = np.random.default_rng(33).permutation(33)
    o, lse = chunk_attention(q, k, v, [0, 10], [0], [33])
    o2, lse2 = chunk_attention(q, k[perm], v[perm], [0, 10], [0], [33])
    assert np.max(np.abs(o - o2)) < 1e-13 and np.max(np.abs(lse - lse2)) < 1e-13


def test_default_scale_is_inverse_sqrt_head_dim():
    q, k, v = _rand((4, 1, 9), 34), _rand((7, 1, 9), 35), _rand((7, 1, 9), 36)
    o1, _ = chunk_attention(q, k, v, [0, 4], [0], [7])
    o2, _ = chunk_attention(q, k, v, [0, 4], [0], [7], scale=1 / 3.0)
    assert np.array_equal(o1, o2)


@pytest.mark.parametrize("bad", [
    dict(q_off=[0, 4], kb=[3], ke=[3]),          # empty window
    dict(q_off=[0, 4], kb=[0], ke=[11]),         # beyond the given keys
    dict(q_off=[0, 3], kb=[0], ke=[5]),          # offsets do not cover the rows
    dict(q_off=[0, 3, 2, 4], kb=[0, 0, 0], ke=[1, 1, 1]),  # decreasing offsets
])
def test_rejects_bad_chunk_tables(bad):
    q, k, v = _rand((4, 1, 2), 37), _rand((10, 1, 2), 38), _rand((10, 1, 2), 39)
    with pytest.raises(ValueError):
        chunk_attention(q, k, v, bad["q_off"], bad["kb"], bad["ke"])
