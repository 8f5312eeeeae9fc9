"""The forward-round workloads at full size against the float64 oracle (needs an MI355X).

Wan-1.3B round (30 layers, H12 D128 bf16, paged ring P1560 T21, 32760-key window):
  - layers 0 and 29 in full: every query row of every head, after the ring has
    wrapped (8 rounds of evict -> append -> attend);
  - every layer: 512 seeded query rows per head, after the prefill and one round.
14B-shaped fp8 round (H40, E4M3FN K/V with per-(page, head, 128-token block) scales):
  - layer 0 in full (every row of every head);
  - layers 13, 26 and 39: 128 seeded rows of every head.
Bars as in test_gpu_attention.py: bf16 O max-abs 1e-2, mean-abs 1e-3, rel-L2
1e-2 and LSE 4e-3; E4M3FN O max-abs 5e-2 and rel-L2 6e-2, LSE 2e-2.  Inputs are
seeded (synth) and identical on both sides; the oracle reads the cache through
its own byte mirror.
"""
import numpy as np
import pytest

import synth
from gpu_util import Pair, dev, errors, host_values, values_of

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN, BF16_REL, BF16_LSE = 1e-2, 1e-3, 1e-2, 4e-3
FP8_MAX, FP8_REL, FP8_LSE = 5e-2, 6e-2, 2e-2


def say(*a):
    print(*a, flush=True)


def wan_layer(layer, rounds):
    """A Wan-round layer's paged ring after the 18-frame prefill and `rounds` rounds of
    evict -> append; returns the pair and the last round's index."""
    cfg = synth.WAN_ROUND
    L = cfg["chunk"]
    table = synth.permuted_table(cfg["workload"], layer, cfg["table_len"])
    pair = Pair(cfg["num_pages"], cfg["page_size"], cfg["H"], cfg["D"], "bf16", table)
    for c in range(cfg["prefill_chunks"]):
        k, v = synth.chunk_kv(cfg, layer, c)
        pair.append(c * L, synth.bf16_codes(k), synth.bf16_codes(v))
    for r in range(rounds):
        if pair.gpu.end - pair.gpu.start + L > pair.gpu.capacity:
            pair.evict(L)
        k, v = synth.chunk_kv(cfg, layer, cfg["prefill_chunks"] + r)
        pair.append(pair.gpu.end, synth.bf16_codes(k), synth.bf16_codes(v))
    assert pair.pages_equal()
    return pair


def attend_window(pair, q_codes):
    L = q_codes.shape[0]
    kb, ke = max(pair.gpu.start, pair.gpu.end - synth.WINDOW_TOKENS), pair.gpu.end
    assert ke - kb == synth.WINDOW_TOKENS
    o, lse = pair.attend(dev(q_codes, "bf16"), [0, L], [kb], [ke])
    return o, lse.cpu().numpy(), kb, ke


def check(got, ref, lse_got, lse_ref, bars, what):
    mx, mean, rel = errors(got, ref)
    dl = float(np.abs(lse_got - lse_ref).max())
    say("%s: max-abs %.3e mean-abs %.3e rel-L2 %.3e lse %.2e" % (what, mx, mean, rel, dl))
    if bars == "bf16":
        assert mx <= BF16_MAX and mean <= BF16_MEAN and rel <= BF16_REL and dl <= BF16_LSE, what
    else:
        assert mx <= FP8_MAX and rel <= FP8_REL and dl <= FP8_LSE, what


@pytest.mark.parametrize("layer", [0, 29])
def test_wan_round_layer_in_full(layer):
    say("case: Wan round, layer %d in full" % layer)
    cfg = synth.WAN_ROUND
    pair = wan_layer(layer, 8)
    q = synth.bf16_codes(synth.queries(cfg, layer, cfg["chunk"], stream=100))
    o, lse, kb, ke = attend_window(pair, q)
    ro, rl = pair.reference(values_of(q, "bf16"), [0, cfg["chunk"]], [kb], [ke])
    check(host_values(o), ro, lse, rl, "bf16", "layer %d, all %d rows x %d heads" % (layer, cfg["chunk"], cfg["H"]))


@pytest.mark.parametrize("group", [0, 1, 2])
def test_wan_round_every_layer_sampled(group):
    cfg = synth.WAN_ROUND
    for layer in range(10 * group, 10 * group + 10):
        say("case: Wan round, layer %d, 512 rows per head" % layer)
        pair = wan_layer(layer, 1)
        q = synth.bf16_codes(synth.queries(cfg, layer, cfg["chunk"], stream=200))
        o, lse, kb, ke = attend_window(pair, q)
        rows = np.sort(np.random.default_rng([300, layer]).choice(cfg["chunk"], size=512, replace=False))
        ro, rl = pair.reference(values_of(q, "bf16")[rows], [0, len(rows)], [kb], [ke])
        check(host_values(o)[rows], ro, lse[:, rows], rl, "bf16", "layer %d" % layer)
        del pair


def fp8_layer(layer):
    cfg = synth.FP8_14B
    L, P = cfg["chunk"], cfg["page_size"]
    table = synth.permuted_table(cfg["workload"], layer, cfg["table_len"])
    pair = Pair(cfg["num_pages"], P, cfg["H"], cfg["D"], "fp8", table)
    for c in range(cfg["prefill_chunks"] + 1):
        k, v = synth.chunk_kv(cfg, layer, c)
        kc, ks = synth.quantize_e4m3_pages(k, P)
        vc, vs = synth.quantize_e4m3_pages(v, P)
        pair.append(c * L, kc, vc, ks, vs)
    assert pair.pages_equal()
    return pair


def test_fp8_14b_layer0_in_full():
    say("case: 14B fp8 round, layer 0 in full")
    cfg = synth.FP8_14B
    pair = fp8_layer(0)
    q = synth.bf16_codes(synth.queries(cfg, 0, cfg["chunk"], stream=100))
    o, lse, kb, ke = attend_window(pair, q)
    ro, rl = pair.reference(values_of(q, "bf16"), [0, cfg["chunk"]], [kb], [ke])
    check(host_values(o), ro, lse, rl, "fp8", "14B layer 0, all %d rows x %d heads" % (cfg["chunk"], cfg["H"]))


@pytest.mark.parametrize("layer", [13, 26, 39])
def test_fp8_14b_layers_sampled(layer):
    say("case: 14B fp8 round, layer %d, 128 rows per head" % layer)
    cfg = synth.FP8_14B
    pair = fp8_layer(layer)
    q = synth.bf16_codes(synth.queries(cfg, layer, cfg["chunk"], stream=200))
    o, lse, kb, ke = attend_window(pair, q)
    rows = np.sort(np.random.default_rng([301, layer]).choice(cfg["chunk"], size=128, replace=False))
    ro, rl = pair.reference(values_of(q, "bf16")[rows], [0, len(rows)], [kb], [ke])
    check(host_values(o)[rows], ro, lse[:, rows], rl, "fp8", "14B layer %d" % layer)
