"""Checks of the seeded input generators (CPU only)."""
import numpy as np

import synth
from oracle import decode_bf16, decode_e4m3fn


def test_streams_are_reproducible_and_distinct():
    a = synth.normal_f32((4, 3), 1.0, 1, 2, 3)
    b = synth.normal_f32((4, 3), 1.0, 1, 2, 3)
    c = synth.normal_f32((4, 3), 1.0, 1, 2, 4)
    assert np.array_equal(a, b) and not np.array_equal(a, c)


def test_bf16_codes_round_to_nearest():
    x = synth.normal_f32((1000,), 3.0, 9)
    got = decode_bf16(synth.bf16_codes(x))
    # |x - bf16(x)| <= half an ulp of bf16 (8 significand bits)
    ulp = np.exp2(np.floor(np.log2(np.abs(x.astype(np.float64)))) - 7)
    assert np.all(np.abs(got - x) <= ulp / 2)


def test_e4m3_page_quantiser_scales_and_error():
    P = 300
    x = synth.normal_f32((600, 2, 8), 1.0, 10)
    codes, scales = synth.quantize_e4m3_pages(x, P)
    assert scales.shape == (2, 2, 3)
    deq = np.empty(x.shape)
    for t in range(600):
        deq[t] = decode_e4m3fn(codes[t]) * scales[t // P, :, (t % P) // 128][:, None]
    # the block maximum maps to +-448 exactly; relative error of e4m3 is <= 2^-4
    rel = np.abs(deq - x) / np.maximum(np.abs(x), 1e-30)
    big = np.abs(x) > 0.05
    assert np.all(rel[big] <= 2.0 ** -4 + 1e-6)
    assert np.max(decode_e4m3fn(codes)) == 448.0 or np.min(decode_e4m3fn(codes)) == -448.0
