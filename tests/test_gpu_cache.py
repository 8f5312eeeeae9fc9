"""GPU append / evict against the oracle's byte mirror of the cache: bit-exact
(needs an MI355X)."""
import numpy as np
import pytest

import synth
from gpu_util import Pair, random_pages

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("P,T,pool", [(24, 7, 11), (40, 1, 1), (1560, 3, 5)])
def test_append_evict_rewrite_bitexact(dtype, D, P, T, pool):
    say("case: append", dtype, D, P, T, pool)
    rng = np.random.default_rng(P * 7 + D + T)
    table = rng.permutation(pool)[:T]
    H = 3
    pair = Pair(pool, P, H, D, dtype, table, fill_seed=P + D)
    cap = P * T
    for step in range(12):
        n = int(rng.integers(1, max(2, cap // 3)))
        live = pair.gpu.end - pair.gpu.start
        if live + n > cap:
            pair.evict(min(live, live + n - cap + int(rng.integers(0, 5))))
        if rng.random() < 0.3 and pair.gpu.end > pair.gpu.start:   # rewrite inside the window
            pos = int(rng.integers(pair.gpu.start, pair.gpu.end + 1))
        else:
            pos = pair.gpu.end
        n = min(n, pair.gpu.start + cap - pos)
        if n <= 0:
            continue
        k = random_pages(rng, (n, H, D), dtype)
        v = random_pages(rng, (n, H, D), dtype)
        pair.append(pos, k, v)
        assert pair.pages_equal(), step


def test_append_full_chunk_paged_ring():
    cfg = synth.WAN_ROUND
    say("case: append full chunk")
    table = synth.permuted_table(cfg["workload"], 3, cfg["table_len"])
    pair = Pair(cfg["num_pages"], cfg["page_size"], cfg["H"], cfg["D"], "bf16", table, fill_seed=1)
    for c in range(9):
        if pair.gpu.end - pair.gpu.start + cfg["chunk"] > pair.gpu.capacity:
            pair.evict(cfg["chunk"])
        k, v = synth.chunk_kv(cfg, 3, c)
        pair.append(pair.gpu.end, synth.bf16_codes(k), synth.bf16_codes(v))
    assert pair.pages_equal()
    # timestep-0 refresh: rewrite the newest chunk in place
    k, v = synth.chunk_kv(cfg, 3, 99)
    pair.append(pair.gpu.end - cfg["chunk"], synth.bf16_codes(k), synth.bf16_codes(v))
    assert pair.pages_equal()


@pytest.mark.parametrize("P", [128, 200, 1560])
def test_fp8_append_with_scales_bitexact(P):
    say("case: fp8 append", P)
    rng = np.random.default_rng(P)
    H, D, T = 5, 128, 4
    pair = Pair(6, P, H, D, "fp8", [5, 0, 3, 1], fill_seed=2)
    nblk = -(-P // 128)
    for step in range(7):
        npg = int(rng.integers(1, 3))
        if pair.gpu.end - pair.gpu.start + npg * P > pair.gpu.capacity:
            pair.evict(npg * P)
        k = random_pages(rng, (npg * P, H, D), "fp8")
        v = random_pages(rng, (npg * P, H, D), "fp8")
        ks = rng.uniform(0.01, 3, size=(npg, H, nblk)).astype(np.float32)
        vs = rng.uniform(0.01, 3, size=(npg, H, nblk)).astype(np.float32)
        pair.append(pair.gpu.end, k, v, ks, vs)
        assert pair.pages_equal(), step


@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
def test_evict_poison_bitexact(dtype):
    rng = np.random.default_rng(9)
    P = 128 if dtype == "fp8" else 24
    pair = Pair(4, P, 2, 64, dtype, [2, 3, 0, 1], fill_seed=3)
    n = 3 * P
    k = random_pages(rng, (n, 2, 64), dtype)
    ks = np.ones((3, 2, 1), np.float32) if dtype == "fp8" else None
    pair.append(0, k, k, ks, ks)
    pair.evict(P + 5, poison=True)
    assert pair.pages_equal()


@pytest.mark.parametrize("P,D", [(64, 128), (200, 64), (1560, 128)])
def test_quantizing_append_bitexact(P, D):
    """bf16 rows -> E4M3FN codes + per-(page, head, block) scales, byte-exact with the oracle's
    quantiser over several rounds (overwrite, evict, ring wrap), including all-zero and tiny blocks."""
    print("case: quantizing append P%d D%d" % (P, D), flush=True)
    H, T = 3, 5
    rng = np.random.default_rng(P + D)
    pair = Pair(T + 2, P, H, D, "fp8", list(rng.permutation(T + 2)[:T]), fill_seed=9)
    pos = 0
    for r in range(7):
        n = P * (1 + r % 2)
        if pair.gpu.end - pair.gpu.start + n > pair.gpu.capacity:
            pair.evict(pair.gpu.end - pair.gpu.start + n - pair.gpu.capacity)
        x = rng.standard_normal((2, n, H, D)).astype(np.float32) * rng.choice([1.0, 30.0, 1e-3])
        x[:, : min(n, 128), r % H] = 0.0                      # an all-zero block
        x[1, -8:, (r + 1) % H] *= 1e-6                        # tiny values (code rounding to zero)
        k, v = synth.bf16_codes(x[0]), synth.bf16_codes(x[1])
        if r == 4:
            pos = pair.gpu.end - n                            # rewrite the newest pages
        else:
            pos = pair.gpu.end
        pair.append_quantize(pos, k, v)
        assert pair.pages_equal(), "round %d" % r


def test_attention_over_quantized_cache():
    """The fp8 attention kernel over pages written by the quantising append, vs the oracle."""
    from gpu_util import dev, errors, host_values, values_of
    print("case: attention over quantized cache", flush=True)
    H, D, P = 4, 128, 256
    rng = np.random.default_rng(12)
    pair = Pair(12, P, H, D, "fp8", list(rng.permutation(12)))
    x = rng.standard_normal((2, 10 * P, H, D)).astype(np.float32)
    pair.append_quantize(0, synth.bf16_codes(x[0]), synth.bf16_codes(x[1]))
    q = synth.bf16_codes(rng.standard_normal((300, H, D)).astype(np.float32))
    o, lse = pair.attend(dev(q, "bf16"), [0, 100, 300], [5, 0], [2560, 1999])
    ro, rl = pair.reference(values_of(q, "bf16"), [0, 100, 300], [5, 0], [2560, 1999])
    mx, mean, rel = errors(host_values(o), ro)
    print("max-abs %.3e rel-L2 %.3e" % (mx, rel), flush=True)
    assert mx <= 5e-2 and rel <= 6e-2
