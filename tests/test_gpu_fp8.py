"""GPU parity of attention over E4M3FN caches (needs an MI355X).

Pages of >= 64 keys go to the fp8-MFMA kernel: Q quantised per row in the
kernel, P quantised after folding in the V scale, K/V scales per (page, head,
128-token block).  Smaller pages go to the kernel that dequantises to bf16.
Bars: max-abs 5e-2 and rel-L2 6e-2 against the float64 oracle on the exact
dequantised K/V.  Cases cover pages of 72 keys (a page break inside most
tiles, and V chunks that straddle one), head_dim 64 and 128, window starts off
the 8-key grid, ragged chunk ends, block scales 100x apart,
both schedules, NaN outside the windows and paged == contiguous.
"""
import numpy as np
import pytest

import synth
from gpu_util import Pair, dev, errors, host_codes, host_values, values_of

pytestmark = pytest.mark.gpu

FP8_MAX, FP8_REL = 5e-2, 6e-2


def say(*a):
    print(*a, flush=True)


def fp8_pair(seed, H, D, P, T, pages, num_pages=None, page_mult=None):
    """A paged fp8 cache holding `pages` whole pages of N(0,1) K/V (times page_mult[page])."""
    rng = np.random.default_rng(seed)
    num_pages = num_pages or T
    table = list(rng.permutation(num_pages)[:T])
    pair = Pair(num_pages, P, H, D, "fp8", table, fill_seed=seed + 1)
    n = pages * P
    k = rng.standard_normal((n, H, D)).astype(np.float32)
    v = rng.standard_normal((n, H, D)).astype(np.float32)
    if page_mult is not None:
        mult = np.repeat(np.asarray(page_mult, np.float32), P)[:, None, None]
        k *= mult
        v *= mult[::-1]
    kc, ks = synth.quantize_e4m3_pages(k, P)
    vc, vs = synth.quantize_e4m3_pages(v, P)
    pair.append(0, kc, vc, ks, vs)
    return pair, rng


def check(pair, q, q_off, kb, ke, what, workspace="auto"):
    o, lse = pair.attend(dev(q, "bf16"), q_off, kb, ke, workspace=workspace)
    ro, rl = pair.reference(values_of(q, "bf16"), q_off, kb, ke)
    got = host_values(o)
    assert np.isfinite(got).all()
    mx, mean, rel = errors(got, ro)
    say("%s: max-abs %.3e mean-abs %.3e rel-L2 %.3e" % (what, mx, mean, rel))
    assert mx <= FP8_MAX and rel <= FP8_REL, (what, mx, rel)
    assert np.abs(lse.cpu().numpy() - rl).max() < 3e-2
    return o, lse


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("workspace", ["auto", None])
def test_fp8_pages_of_72_ragged(D, workspace):
    """Pages of 72 keys: most 64-key tiles cross a page, half of the breaks inside a 16-key chunk."""
    say("case: fp8 P72 D%d workspace=%s" % (D, workspace))
    pair, rng = fp8_pair(31, H=3, D=D, P=72, T=14, pages=12)
    q = synth.bf16_codes(rng.standard_normal((300, 3, D)).astype(np.float32))
    check(pair, q, [0, 50, 300], [5, 77], [860, 651], "P72 D%d" % D, workspace)


def test_fp8_block_scales_far_apart():
    """Pages whose K (and, reversed, V) magnitudes span 100x: the V scales folded into P differ per tile."""
    say("case: fp8 scale spread")
    mult = [10.0, 1.0, 0.1, 3.0, 0.3, 5.0, 1.0, 0.5]
    pair, rng = fp8_pair(32, H=2, D=128, P=128, T=8, pages=8, page_mult=mult)
    q = synth.bf16_codes(rng.standard_normal((260, 2, 128)).astype(np.float32) * 0.1)
    check(pair, q, [0, 260], [0], [1024], "scale spread")


def test_fp8_split_schedule_parts_and_tails():
    """1 tile x 2 heads x 100 key tiles: 3 key parts per item plus B tails, merged."""
    say("case: fp8 split schedule")
    pair, rng = fp8_pair(33, H=2, D=128, P=256, T=26, pages=25)
    q = synth.bf16_codes(rng.standard_normal((100, 2, 128)).astype(np.float32))
    o, l = check(pair, q, [0, 100], [0], [6400], "fp8 split")
    o1, l1 = check(pair, q, [0, 100], [0], [6400], "fp8 per-tile", workspace=None)
    assert np.abs(host_values(o) - host_values(o1)).max() < 1e-2


def test_fp8_nan_outside_windows_never_read():
    """NaN codes on the masked keys of both edge tiles (before kv_begin inside the first tile, after
    kv_end inside the last) and in later pages leave the result bitwise unchanged."""
    say("case: fp8 NaN outside")
    pair, rng = fp8_pair(34, H=2, D=128, P=64, T=24, pages=20)
    q = dev(synth.bf16_codes(rng.standard_normal((300, 2, 128)).astype(np.float32)), "bf16")
    args = ([0, 120, 300], [70, 136], [1270, 1216])
    o1, l1 = pair.attend(q, *args)
    # rewrite page [1216, 1280) with NaN codes on keys 1270.. (past chunk 0's window, same tile)
    kc, vc = pair.ref.gather_codes(1216, 1280)
    kc, vc = kc.copy(), vc.copy()
    kc[54:] = 0x7F
    vc[54:] = 0x7F
    page = pair.ref.table[(1216 // 64) % pair.ref.T]
    pair.append(1216, kc, vc, pair.ref.k_scale[page][None].copy(), pair.ref.v_scale[page][None].copy())
    nan = np.full((64, 2, 128), 0x7F, np.uint8)
    ones = np.ones((1, 2, 1), np.float32)
    pair.append(1280, nan, nan, ones, ones)
    pair.evict(68, poison=True)  # keys 64..67 share chunk 0's first tile
    o2, l2 = pair.attend(q, *args)
    assert np.array_equal(host_codes(o1), host_codes(o2))
    assert np.array_equal(l1.cpu().numpy(), l2.cpu().numpy())


def test_fp8_paged_equals_contiguous_and_deterministic():
    say("case: fp8 paged == contiguous")
    rng = np.random.default_rng(35)
    H, D, P = 2, 128, 64
    k = rng.standard_normal((1152, H, D)).astype(np.float32)
    v = rng.standard_normal((1152, H, D)).astype(np.float32)
    kc, ks = synth.quantize_e4m3_pages(k, P)
    vc, vs = synth.quantize_e4m3_pages(v, P)
    a = Pair(18, P, H, D, "fp8", list(range(18)))
    b = Pair(22, P, H, D, "fp8", list(rng.permutation(22)[:18]))
    a.append(0, kc, vc, ks, vs)
    b.append(0, kc, vc, ks, vs)
    q = dev(synth.bf16_codes(rng.standard_normal((400, H, D)).astype(np.float32)), "bf16")
    args = ([0, 150, 400], [3, 40], [1150, 1000])
    outs = [a.attend(q, *args) for _ in range(2)] + [b.attend(q, *args)]
    for o, l in outs[1:]:
        assert np.array_equal(host_codes(o), host_codes(outs[0][0]))
        assert np.array_equal(l.cpu().numpy(), outs[0][1].cpu().numpy())


def test_fp8_small_pages_dequantising_kernel():
    """Pages of 40 keys (under one tile) take the kernel that dequantises K/V to bf16."""
    say("case: fp8 P40")
    pair, rng = fp8_pair(36, H=2, D=128, P=40, T=16, pages=15)
    q = synth.bf16_codes(rng.standard_normal((200, 2, 128)).astype(np.float32))
    check(pair, q, [0, 90, 200], [3, 0], [600, 433], "P40")
