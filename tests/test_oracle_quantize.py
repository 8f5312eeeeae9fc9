"""Pins of the oracle's E4M3FN encoder and of its page quantiser (used by the quantising append).

The encoder is checked against torch's float8_e4m3fn cast (a library routine)
on every code value, every midpoint between neighbouring codes (ties round to
even), random magnitudes across the whole range and both signs; saturation and
NaN follow the OCP definition (satfinite).  The quantiser is checked against
properties its definition fixes: the block's largest magnitude encodes to
+-448, every element is within half an e4m3 step (times the scale) of its
input, all-zero blocks get scale 1, and scale = amax / 448 in float32.
"""
import numpy as np
import torch

import oracle
import synth


def torch_e4m3(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def finite_codes():
    c = np.arange(256, dtype=np.uint8)
    return c[(c & 0x7F) != 0x7F]


def test_encode_matches_torch_on_codes_midpoints_and_random():
    vals = oracle.decode_e4m3fn(finite_codes()).astype(np.float32)
    pos = np.sort(oracle.decode_e4m3fn(np.arange(0x7F, dtype=np.uint8)))
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)  # exact in float32: ties
    rng = np.random.default_rng(1)
    rnd = (np.exp(rng.uniform(np.log(1e-4), np.log(447.0), 20000)) * rng.choice([-1, 1], 20000)).astype(np.float32)
    for x in (vals, mids, -mids, rnd):
        got, want = oracle.encode_e4m3fn(x), torch_e4m3(x)
        zero = (oracle.decode_e4m3fn(got) == 0) & (oracle.decode_e4m3fn(want) == 0)
        assert np.array_equal(got[~zero], want[~zero])
        assert np.array_equal(np.signbit(oracle.decode_e4m3fn(got)), np.signbit(x))


def test_encode_roundtrip_saturation_nan():
    c = finite_codes()
    assert np.array_equal(oracle.encode_e4m3fn(oracle.decode_e4m3fn(c).astype(np.float32)), c)
    x = np.array([448.0, 449.0, 463.9, 464.0, 1e6, -1e6, np.inf, -np.inf, np.nan], np.float32)
    assert oracle.encode_e4m3fn(x).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x7E, 0xFE, 0x7F]
    # below half the smallest subnormal: signed zero
    t = np.array([2.0 ** -11, -(2.0 ** -11), 2.0 ** -10, 1.5 * 2.0 ** -10], np.float32)
    assert oracle.encode_e4m3fn(t).tolist() == [0x00, 0x80, 0x00, 0x01]


def test_quantize_pages_properties():
    P, H, D = 200, 3, 64          # 2 blocks per page: 128 + 72 tokens
    m = oracle.KVCacheModel(4, P, H, D, "fp8", [0, 1, 2, 3])
    rng = np.random.default_rng(2)
    x = rng.standard_normal((2 * P, H, D)).astype(np.float32)
    x[P + 128:2 * P, 1] = 0.0                       # an all-zero block (page 1, block 1, head 1)
    x[0:128, 2] *= 1e-3                             # a block of small values
    xc = synth.bf16_codes(x)
    codes, scales = m.quantize_pages(xc)
    xv = oracle.decode_bf16(xc)
    for j in range(2):
        for b in range(2):
            r0, r1 = j * P + 128 * b, min(j * P + 128 * (b + 1), (j + 1) * P)
            for h in range(H):
                blk = xv[r0:r1, h].astype(np.float32)
                amax = np.abs(blk).max()
                s = scales[j, h, b]
                if amax == 0:
                    assert s == 1.0 and not codes[r0:r1, h].any()
                    continue
                assert s == np.float32(amax) / np.float32(448.0)
                deq = oracle.decode_e4m3fn(codes[r0:r1, h]) * np.float64(s)
                q = np.abs(blk.astype(np.float64)) / s
                tol = np.maximum(q * 2.0 ** -4, 2.0 ** -10) * s * (1 + 1e-6)
                assert (np.abs(deq - blk) <= tol).all()
                top = np.argmax(np.abs(blk).ravel())
                assert (codes[r0:r1, h].ravel()[top] & 0x7F) == 0x7E


def test_append_quantized_equals_append_of_quantized():
    P, H, D = 64, 2, 32
    a = oracle.KVCacheModel(6, P, H, D, "fp8", [3, 1, 0, 5, 2, 4])
    b = oracle.KVCacheModel(6, P, H, D, "fp8", [3, 1, 0, 5, 2, 4])
    rng = np.random.default_rng(3)
    k = synth.bf16_codes(rng.standard_normal((3 * P, H, D)).astype(np.float32))
    v = synth.bf16_codes(rng.standard_normal((3 * P, H, D)).astype(np.float32))
    a.append_quantized(0, k, v)
    kc, ks = b.quantize_pages(k)
    vc, vs = b.quantize_pages(v)
    b.append(0, kc, vc, ks, vs)
    assert np.array_equal(a.k, b.k) and np.array_equal(a.v, b.v)
    assert np.array_equal(a.k_scale, b.k_scale) and np.array_equal(a.v_scale, b.v_scale)
