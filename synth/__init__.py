"""Seeded synthetic inputs for chunk-wise causal attention workloads.

Shared by the tests, the oracle-timing leg of the benchmark and the GPU
parity checks.  Holds no attention or cache arithmetic: it only draws random
numbers, casts them to the storage formats, and describes the workload shapes.

Base seed 42 is the streaming plugin's default ``base_seed`` (scope-causal-
forcing README, "Configuration").  Each tensor has its own numpy stream
``default_rng([42, workload, layer, tensor, ...])``.

Workload shapes.  The pages give 480x832 output and the Wan2.1-T2V-1.3B model;
one latent frame is 1560 tokens and a chunk is 3 latent frames (4680 tokens);
the rolling window is 21 latent frames (32760 keys).  The Wan-1.3B shape has
12 heads of 128 dims, the 14B shape 40 heads.
"""
import numpy as np
import torch

SEED = 42
FRAME_TOKENS = 1560
CHUNK_TOKENS = 3 * FRAME_TOKENS
WINDOW_TOKENS = 21 * FRAME_TOKENS
E4M3_MAX = 448.0
SCALE_BLOCK = 128

# Workload ids used as the second seed word.
W_TINY, W_WAN_CALL, W_WAVE, W_WAN_ROUND, W_14B_FP8 = 1, 2, 3, 4, 5
T_Q, T_K, T_V, T_TABLE, T_INIT = 0, 1, 2, 3, 4


def rng(*words):
    return np.random.default_rng([SEED] + [int(w) for w in words])


def normal_f32(shape, std, *words):
    """i.i.d. N(0, std^2) samples as float32."""
    return (rng(*words).standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def bf16_codes(x):
    """float32 -> bfloat16 codes (uint16), round-to-nearest-even (torch CPU cast)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def quantize_e4m3_pages(x, page_size):
    """Quantise token-major K or V rows x [n, H, D] (n a multiple of page_size) to E4M3FN.

    One float32 scale per (page, head, 128-token block counted inside the page):
    scale = amax(|block|) / 448 (1 for an all-zero block); codes are
    RNE(x / scale) saturated to +-448 (torch's float8_e4m3fn cast).
    Returns codes uint8 [n, H, D] and scales float32 [n/page_size, H, ceil(page_size/128)].
    """
    x = np.asarray(x, dtype=np.float32)
    n, h, d = x.shape
    if n % page_size:
        raise ValueError("quantised appends are whole pages")
    nblk = -(-page_size // SCALE_BLOCK)
    scales = np.ones((n // page_size, h, nblk), np.float32)
    scaled = np.empty_like(x)
    for p in range(n // page_size):
        for b in range(nblk):
            r0 = p * page_size + b * SCALE_BLOCK
            r1 = min(r0 + SCALE_BLOCK, (p + 1) * page_size)
            blk = x[r0:r1]                                   # [rows, H, D]
            amax = np.abs(blk).max(axis=(0, 2)).astype(np.float32)
            s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
            scales[p, :, b] = s
            scaled[r0:r1] = blk / s[None, :, None]
    scaled = np.clip(scaled, -E4M3_MAX, E4M3_MAX)
    codes = torch.from_numpy(scaled).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return codes, scales


def identity_table(n):
    return np.arange(n, dtype=np.int32)


def permuted_table(workload, layer, num_slots, num_pages=None):
    """Random page table: num_slots distinct physical pages out of num_pages (default num_slots)."""
    num_pages = num_slots if num_pages is None else num_pages
    perm = rng(workload, layer, T_TABLE).permutation(num_pages)
    return perm[:num_slots].astype(np.int32)


# ----------------------------------------------------------------------------
# Workload descriptions (shapes only; the arrays come from the helpers above).
# ----------------------------------------------------------------------------

TINY = dict(  # fp32, 2 heads x 64 dims, 3 chunks of 64 tokens, last chunk over 192 keys
    name="tiny-fp32 H2 D64, 3 chunks x 64 tokens, contiguous cache",
    workload=W_TINY, H=2, D=64, dtype="f32", chunk=64, num_chunks=3, std=1.0,
    page_size=192, table_len=1, num_pages=1)

WAN_CALL = dict(  # one Wan-1.3B attention call: chunk 3 of 4 over 18720 keys
    name="wan1.3b-call H12 D128 bf16, 4680 q x 18720 k",
    workload=W_WAN_CALL, H=12, D=128, dtype="bf16", chunk=CHUNK_TOKENS, num_chunks=4, std=0.5,
    page_size=FRAME_TOKENS, table_len=12, num_pages=12)

WAVE = dict(  # staggered mixed-noise wave: 4 query chunks with prefixes 4680..18720
    name="wave-4chunk H12 D128 bf16, prefixes 4680/9360/14040/18720",
    workload=W_WAVE, H=12, D=128, dtype="bf16", chunk=CHUNK_TOKENS, num_chunks=4, q_std=0.5,
    kv_std=(1.0, 0.75, 0.5, 0.25), page_size=FRAME_TOKENS, table_len=12, num_pages=12)

WAN_ROUND = dict(  # full forward round: 30 layers over a 21-frame paged ring
    name="wan1.3b-round 30 layers, H12 D128 bf16, 4680 q x 32760 k, paged ring P1560 T21",
    workload=W_WAN_ROUND, layers=30, H=12, D=128, dtype="bf16", chunk=CHUNK_TOKENS, std=0.5,
    page_size=FRAME_TOKENS, table_len=21, num_pages=21, prefill_chunks=6)

FP8_14B = dict(  # 14B shape, fp8 K/V
    name="14b-round 40 layers, H40 D128, bf16 Q + e4m3 K/V, 4680 q x 32760 k, paged ring P1560 T21",
    workload=W_14B_FP8, layers=40, H=40, D=128, dtype="fp8", chunk=CHUNK_TOKENS, std=1.0,
    page_size=FRAME_TOKENS, table_len=21, num_pages=21, prefill_chunks=6)


def chunk_kv(cfg, layer, chunk_index, std=None):
    """New K/V rows [chunk, H, D] (float32 values) for one chunk of one layer."""
    std = cfg.get("std", 1.0) if std is None else std
    shape = (cfg["chunk"], cfg["H"], cfg["D"])
    k = normal_f32(shape, std, cfg["workload"], layer, T_K, chunk_index)
    v = normal_f32(shape, std, cfg["workload"], layer, T_V, chunk_index)
    return k, v


def queries(cfg, layer, rows, std=None, stream=0):
    std = cfg.get("q_std", cfg.get("std", 1.0)) if std is None else std
    return normal_f32((rows, cfg["H"], cfg["D"]), std, cfg["workload"], layer, T_Q, stream)


def staircase(q, k, key_pos, origin, step_keys, rise_log2=16.0, seed_words=(0,)):
    """Peaked-score variant of float32 inputs q [Nq, H, D] and k [L, H, D] (copies are returned).

    Dimension 0 of key j is set to b_j = c * floor((key_pos[j] - origin) / step_keys), with c
    chosen so that a query whose dimension 0 is 8 gains rise_log2 log2 units of score (under the
    default softmax scale 1/sqrt(D)) per step of step_keys keys.  Every query row gets a level
    L: 40 % of the rows L = 0, the rest spread evenly over L = 1..5 and "flat".  A row of level L
    is scaled by 2^-L and its dimension 0 set to 8 * 2^-L, so it climbs rise_log2 * 2^-L per step;
    a flat row keeps its values and gets dimension 0 = 0.  One call thus mixes flat rows, rows
    whose last few steps all contribute, and rows dominated by their last step.  Dimension 0 is
    a power of two and the largest element of its row, so it is exact in bf16 and in a per-row
    E4M3FN quantisation.
    """
    q = np.array(q, dtype=np.float32, copy=True)
    k = np.array(k, dtype=np.float32, copy=True)
    d = q.shape[-1]
    g = rng(*seed_words)
    lv = g.choice(7, size=q.shape[0], p=[0.4, 0.1, 0.1, 0.1, 0.1, 0.1, 0.1])
    for L in range(6):
        rows = lv == L
        q[rows] *= np.float32(2.0 ** -L)
        q[rows, :, 0] = np.float32(8.0 * 2.0 ** -L)
    q[lv == 6, :, 0] = 0.0
    steps = np.floor((np.asarray(key_pos, np.float64) - origin) / step_keys)
    b = steps * rise_log2 * np.log(2.0) * np.sqrt(d) / 8.0
    k[:, :, 0] = b[:, None]
    return q, k


def encode(x, dtype):
    """float32 values -> storage codes of a cache dtype ('f32', 'bf16'); fp8 goes through quantize_e4m3_pages."""
    if dtype == "f32":
        return np.ascontiguousarray(x, np.float32)
    if dtype == "bf16":
        return bf16_codes(x)
    raise ValueError(dtype)
