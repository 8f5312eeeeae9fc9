"""CPU checks of the peaked-score input generator and of the host-side
rescale-event detector the GPU tests use to prove their inputs reach the
kernels' rescale branches."""
import numpy as np

import synth
from gpu_util import rescale_events


def test_staircase_rises_by_the_stated_log2_units():
    q = synth.normal_f32((50, 2, 128), 0.5, 99, 1)
    k = synth.normal_f32((1024, 2, 128), 0.5, 99, 2)
    pos = np.arange(1024)
    qs, ks = synth.staircase(q, k, pos, origin=0, step_keys=256, rise_log2=16.0, seed_words=(99, 3))
    assert np.array_equal(ks[:, :, 1:], k[:, :, 1:])
    a = qs[:, 0, 0].astype(np.float64)
    assert set(np.unique(a)) <= {0.0, 8.0, 4.0, 2.0, 1.0, 0.5, 0.25}
    assert np.mean(a == 8.0) > 0.25
    for i in range(50):  # a row of level L is the input row times 2^-L; flat rows are unchanged
        f = a[i] / 8.0 if a[i] > 0 else 1.0
        assert np.array_equal(qs[i, :, 1:], (q[i, :, 1:] * np.float32(f)).astype(np.float32))
        assert a[i] == 0 or a[i] >= np.abs(qs[i, :, 1:]).max()   # dimension 0 is the row's largest
    # score offset of dimension 0 under scale 1/sqrt(D), in log2 units: rise * a / 8 per step
    off = np.outer(a, ks[:, 0, 0]) / np.sqrt(128) / np.log(2.0)
    steps = pos // 256
    assert np.allclose(off, np.outer(a * 2.0, steps), rtol=1e-5, atol=1e-4)


def test_rescale_event_detector():
    q = synth.normal_f32((64, 1, 128), 0.5, 98, 1)
    k = synth.normal_f32((2048, 1, 128), 0.5, 98, 2)
    # flat scores: no tile can exceed the running maximum by 8 or 11 log2 units
    assert rescale_events(q[:, 0], k[:, 0], 0, 2048, "max11") == []
    assert rescale_events(q[:, 0], k[:, 0], 0, 2048, "max") == []
    qs, ks = synth.staircase(q, k, np.arange(2048), 0, 256, 16.0, seed_words=(98, 3))
    ev = rescale_events(qs[:, 0], ks[:, 0], 0, 2048, "max11")
    assert ev == [4, 8, 12, 16, 20, 24, 28]          # every step tile of the steepest rows
    assert rescale_events(qs[:, 0], ks[:, 0], 0, 2048, "max") == ev
    # a window starting at 5 keeps the tile grid (base 0); a window ending mid-tile drops no step
    assert rescale_events(qs[:, 0, :], ks[5:2000, 0], 5, 2000, "max11") == ev
