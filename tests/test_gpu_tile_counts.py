"""The two LDS-DMA kernels over every count of 64-key tiles from 1 to 10, against the float64
oracle (needs an MI355X).

The kernels run a chunk's key tiles as a prologue, a loop unrolled by three (the ring slot of
every step is a compile-time constant), an edge step for the last masked tile and a final P V
product whose slot depends on the tile count modulo 3.  The bf16 kernel runs one copy of the loop
per residue of the tile count, the fp8 kernel one loop and a switch over the remainder; each tile
count 1..10 reaches a different combination.  Every count runs with the chunk's first key on the
8-key grid and off it (a lead of 5 keys: the first tile masked as well), with three chunks whose
query rows straddle a query tile.  Bars as in test_gpu_paths.py: bf16 O max-abs 1e-2, mean-abs
1e-3, rel-L2 1e-2, LSE 4e-3; E4M3FN O rel-L2 6e-2, max-abs max(5e-2, (2^-4 + 2 Delta) max|V|),
LSE 3e-2.
"""
import numpy as np
import pytest

import chunk_causal_dit_wf_amd as wf
import synth
from gpu_util import Pair, dev, errors, host_values, score_error_bounds, values_of

pytestmark = pytest.mark.gpu

H, D, P = 2, 128, 256
N_KEYS = 10 * 64 + 8


def build(dtype, seed):
    rng = np.random.default_rng(seed)
    T = -(-N_KEYS // P)
    pair = Pair(T + 1, P, H, D, dtype, list(rng.permutation(T + 1)[:T]), fill_seed=seed + 1)
    if dtype == "fp8":
        k = rng.standard_normal((T * P, H, D)).astype(np.float32)
        v = rng.standard_normal((T * P, H, D)).astype(np.float32)
        kc, ks = synth.quantize_e4m3_pages(k, P)
        vc, vs = synth.quantize_e4m3_pages(v, P)
        pair.append(0, kc, vc, ks, vs)
    else:
        k = rng.standard_normal((N_KEYS, H, D)).astype(np.float32) * 0.5
        v = rng.standard_normal((N_KEYS, H, D)).astype(np.float32) * 0.5
        pair.append(0, synth.encode(k, dtype), synth.encode(v, dtype))
    return pair, rng


@pytest.mark.parametrize("dtype,kernel", [("bf16", "dma_bf16"), ("fp8", "dma_fp8")])
@pytest.mark.parametrize("lead", [0, 5])
@pytest.mark.parametrize("ntiles", list(range(1, 11)))
def test_every_tile_count(dtype, kernel, lead, ntiles):
    print("case: tile count", dtype, "tiles", ntiles, "lead", lead, flush=True)
    pair, rng = build(dtype, 100 * ntiles + lead + (7 if dtype == "fp8" else 0))
    # keys [kb, ke) with kb % 8 == lead span exactly ntiles tiles of the kernel's 64-key grid
    # (which starts at kb - lead): the last tile ends 1..13 keys short of its edge.
    kb0 = 8 * int(rng.integers(0, 2)) + lead
    n = 64 * ntiles - lead - int(rng.integers(1, 14)) if ntiles > 1 else int(rng.integers(1, 64 - lead))
    kb, ke = [kb0, kb0, kb0], [kb0 + n, kb0 + n, kb0 + n]
    q_off = [0, 200, 300, 563]
    qs = 1.0 if dtype == "fp8" else 0.5
    q = synth.encode(rng.standard_normal((q_off[-1], H, D)).astype(np.float32) * qs, "bf16")
    plan = wf.wf_chunk_attn_plan(pair.gpu, q_off, kb, ke, q_dtype="bf16")
    assert plan["kernel"] == kernel and plan["schedule"] == "per_tile"
    o, lse = pair.attend(dev(q, "bf16"), q_off, kb, ke, workspace=None)
    ro, rl = pair.reference(values_of(q, "bf16"), q_off, kb, ke)
    got = host_values(o)
    assert np.isfinite(got).all()
    mx, mean, rel = errors(got, ro)
    dl = float(np.abs(lse.cpu().numpy() - rl).max())
    if dtype == "bf16":
        bars = (1e-2, 1e-3, 1e-2, 4e-3)
    else:
        K, V = pair.ref.gather(kb0, kb0 + n)
        delta = score_error_bounds(values_of(q, "bf16"), K, q_off, kb, ke, kb0).max()
        bars = (max(5e-2, (2.0 ** -4 + 2.0 * delta) * float(np.abs(V).max()) * 1.01), 1.0, 6e-2, 3e-2)
    print("  keys", n, "max-abs %.3e mean-abs %.3e rel-L2 %.3e lse %.2e" % (mx, mean, rel, dl), flush=True)
    assert mx <= bars[0] and mean <= bars[1] and rel <= bars[2] and dl <= bars[3], (mx, mean, rel, dl)
