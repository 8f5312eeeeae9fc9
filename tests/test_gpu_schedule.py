"""GPU parity of the split attention schedule (needs an MI355X).

With a workspace, bf16 caches with pages of >= 64 tokens whose chunks all span
the same number S of 64-key tiles, and that have fewer query tiles ("items")
than resident workgroups, are processed by the split schedule.  Each item's
key tiles are cut into m parts (>= 32 key tiles each), and the workgroups
still idle take the last b key tiles of q parts each.  Partial results are
merged by log-sum-exp in a second kernel (slots in the workspace).  The shapes
below hit m > 1 with and without B parts, B workgroups with several parts,
parts whose first key tile is masked by the window start (lead) and whose last
is partial, several chunks in one call, and NaN outside the windows.  Every
case is checked against the float64 oracle at the bf16 bars and against the
one-workgroup-per-tile schedule.
"""
import numpy as np
import pytest

import synth
from gpu_util import Pair, dev, errors, host_codes, host_values, values_of

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN, BF16_REL = 1e-2, 1e-3, 1e-2


def say(*a):
    print(*a, flush=True)


def check(pair, q, q_off, kb, ke, what):
    o, lse = pair.attend(dev(q, "bf16"), q_off, kb, ke)                   # split (default)
    o1, lse1 = pair.attend(dev(q, "bf16"), q_off, kb, ke, workspace=None)  # one block per tile
    ro, rl = pair.reference(values_of(q, "bf16"), q_off, kb, ke)
    for name, got, gl in (("split", o, lse), ("per-tile", o1, lse1)):
        mx, mean, rel = errors(host_values(got), ro)
        say("%s %s: max-abs %.3e mean-abs %.3e rel-L2 %.3e" % (what, name, mx, mean, rel))
        assert mx <= BF16_MAX and mean <= BF16_MEAN and rel <= BF16_REL, (what, name, mx, mean, rel)
        assert np.abs(gl.cpu().numpy() - rl).max() < 2e-3
    # the two schedules differ only in fp32 rounding before the final bf16 cast
    d = np.abs(host_values(o) - host_values(o1)).max()
    scale = np.abs(ro).max()
    say("%s split vs per-tile max diff %.3e (|O| max %.3e)" % (what, d, scale))
    assert d <= 2 ** -7 * scale + 1e-6
    return o, lse


def filled_pair(seed, H, P, T, n, num_pages=None, table=None):
    rng = np.random.default_rng(seed)
    num_pages = num_pages or T
    table = list(table) if table is not None else list(rng.permutation(num_pages)[:T])
    pair = Pair(num_pages, P, H, 128, "bf16", table, fill_seed=seed + 1)
    k = synth.bf16_codes(rng.standard_normal((n, H, 128)).astype(np.float32))
    v = synth.bf16_codes(rng.standard_normal((n, H, 128)).astype(np.float32))
    pair.append(0, k, v)
    return pair, rng


def test_three_parts_with_b_tails():
    """1 tile x 2 heads x 100 key tiles: m = 3 parts per item, each part's last 16 tiles on B blocks."""
    say("case: 3 parts + B tails")
    pair, rng = filled_pair(21, H=2, P=256, T=26, n=6400)
    q = synth.bf16_codes(rng.standard_normal((100, 2, 128)).astype(np.float32) * 2)
    check(pair, q, [0, 100], [0], [6400], "3 parts")


def test_b_blocks_with_two_parts_lead_and_ragged_end():
    """3 tiles x 8 heads x 200 key tiles (lead 5, last tile partial): m = 6, B blocks take 2 parts."""
    say("case: q = 2 B blocks, lead and ragged end")
    pair, rng = filled_pair(22, H=8, P=512, T=26, n=12800)
    q = synth.bf16_codes(rng.standard_normal((768, 8, 128)).astype(np.float32))
    check(pair, q, [0, 768], [5], [12795], "q=2 B blocks")


def test_multi_chunk_equal_key_tiles():
    """Four chunks (37, 263, 1, 399 rows) whose key ranges all span 47 key tiles, in one call."""
    say("case: multi-chunk, equal key tiles")
    pair, rng = filled_pair(23, H=3, P=128, T=26, n=3200)
    q = synth.bf16_codes(rng.standard_normal((700, 3, 128)).astype(np.float32))
    q_off = [0, 37, 300, 301, 700]
    kb = [3, 0, 64, 130]
    ke = [3003, 3000, 3054, 3129]
    check(pair, q, q_off, kb, ke, "multi-chunk")


def test_split_nan_outside_windows_never_read():
    """NaN-poisoned keys before kv_begin and after kv_end leave the split result bitwise unchanged."""
    say("case: split schedule, NaN outside windows")
    pair, rng = filled_pair(24, H=2, P=64, T=24, n=1400)
    q = dev(synth.bf16_codes(rng.standard_normal((300, 2, 128)).astype(np.float32)), "bf16")
    args = ([0, 120, 300], [70, 136], [1270, 1336])
    o1, l1 = pair.attend(q, *args)
    nan = np.full((60, 2, 128), 0x7FC0, np.uint16)
    pair.append(1400, nan, nan)
    pair.evict(70, poison=True)
    o2, l2 = pair.attend(q, *args)
    assert np.array_equal(host_codes(o1), host_codes(o2))
    assert np.array_equal(l1.cpu().numpy(), l2.cpu().numpy())
    assert not np.isnan(host_values(o2)).any()


def test_split_run_to_run_and_paged_bitwise():
    """Split-schedule results are bitwise reproducible and identical for paged and contiguous caches."""
    say("case: split determinism + paging")
    rng = np.random.default_rng(25)
    H, P = 2, 64
    a = Pair(20, P, H, 128, "bf16", list(range(20)))
    b = Pair(24, P, H, 128, "bf16", list(rng.permutation(24)[:20]))
    k = synth.bf16_codes(rng.standard_normal((1200, H, 128)).astype(np.float32))
    v = synth.bf16_codes(rng.standard_normal((1200, H, 128)).astype(np.float32))
    a.append(0, k, v)
    b.append(0, k, v)
    q = dev(synth.bf16_codes(rng.standard_normal((520, H, 128)).astype(np.float32)), "bf16")
    args = ([0, 260, 520], [0, 16], [1200, 1200])
    outs = [a.attend(q, *args) for _ in range(3)] + [b.attend(q, *args)]
    for o, l in outs[1:]:
        assert np.array_equal(host_codes(o), host_codes(outs[0][0]))
        assert np.array_equal(l.cpu().numpy(), outs[0][1].cpu().numpy())


def test_frame_wise_chunk_over_full_window_sampled():
    """Frame-wise generation: one 1560-row frame over the 32760-key window of a paged ring
    (7 tiles x 12 heads = 84 items: 3 parts per item).  Sampled rows vs the oracle."""
    cfg = synth.WAN_ROUND
    H, D, P = cfg["H"], cfg["D"], cfg["page_size"]
    say("case: frame-wise 1560 rows over 32760 keys")
    table = synth.permuted_table(cfg["workload"], 3, cfg["table_len"])
    pair = Pair(cfg["num_pages"], P, H, D, "bf16", table)
    for c in range(7):
        k, v = synth.chunk_kv(cfg, 3, c)
        pair.append(c * cfg["chunk"], synth.bf16_codes(k), synth.bf16_codes(v))
    pair.evict(pair.gpu.end - 32760)
    kb, ke = pair.gpu.start, pair.gpu.end
    q = synth.bf16_codes(synth.queries(cfg, 3, P) * 2.0)
    o, lse = pair.attend(dev(q, "bf16"), [0, P], [kb], [ke])
    o1, lse1 = pair.attend(dev(q, "bf16"), [0, P], [kb], [ke], workspace=None)
    rows = np.sort(np.random.default_rng(7).choice(P, size=256, replace=False))
    ro, rl = pair.reference(values_of(q, "bf16")[rows], [0, len(rows)], [kb], [ke])
    for name, got, gl in (("split", o, lse), ("per-tile", o1, lse1)):
        mx, mean, rel = errors(host_values(got)[rows], ro)
        say("frame-wise %s: max-abs %.3e mean-abs %.3e rel-L2 %.3e" % (name, mx, mean, rel))
        assert mx <= BF16_MAX and mean <= BF16_MEAN and rel <= BF16_REL
        assert np.abs(gl.cpu().numpy()[:, rows] - rl).max() < 2e-3
