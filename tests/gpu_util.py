"""Helpers for the GPU parity tests: drive the HIP library and the oracle's
cache model with the same seeded inputs, and measure the difference."""
import numpy as np
import torch

import chunk_causal_dit_wf_amd as wf
import oracle


def dev(codes, dtype):
    """Host storage codes -> device tensor in the library's storage dtype."""
    if codes is None:
        return None
    a = np.ascontiguousarray(codes)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    if dtype == "scale":
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    return torch.from_numpy(a).cuda()


def host_codes(t):
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def host_values(t):
    c = host_codes(t)
    if c.dtype == np.uint16:
        return oracle.decode_bf16(c)
    return c.astype(np.float64)


def values_of(codes, dtype):
    if dtype == "bf16":
        return oracle.decode_bf16(codes)
    return np.asarray(codes, np.float64)


def random_pages(rng, shape, dtype):
    """Finite random storage codes used to pre-fill pages (so unwritten rows are not zero)."""
    if dtype == "f32":
        return rng.standard_normal(shape, dtype=np.float32)
    if dtype == "bf16":
        return rng.integers(0, 1 << 15, size=shape, dtype=np.uint16) & np.uint16(0xBF7F)
    return rng.integers(0, 0x7F, size=shape, dtype=np.uint8)


class Pair:
    """A device cache and the oracle's cache model, driven with identical operations."""

    def __init__(self, num_pages, page_size, heads, dim, dtype, table, fill_seed=None):
        self.dtype = dtype
        kp = vp = None
        if fill_seed is not None:
            rng = np.random.default_rng(fill_seed)
            kp = random_pages(rng, (num_pages, heads, page_size, dim), dtype)
            vp = random_pages(rng, (num_pages, heads, dim, page_size), dtype)
        self.ref = oracle.KVCacheModel(num_pages, page_size, heads, dim, dtype, table, k_pages=kp, v_pages=vp)
        kt = dev(self.ref.k.copy(), dtype) if dtype != "fp8" else torch.from_numpy(self.ref.k.copy()).cuda()
        vt = dev(self.ref.v.copy(), dtype) if dtype != "fp8" else torch.from_numpy(self.ref.v.copy()).cuda()
        self.gpu = wf.KVCache(num_pages, page_size, heads, dim, dtype, list(table), k=kt, v=vt)

    def append(self, pos, k, v, ks=None, vs=None):
        d = "fp8" if self.dtype == "fp8" else self.dtype
        wf.wf_kv_append(self.gpu, pos, dev(k, d), dev(v, d), dev(ks, "scale"), dev(vs, "scale"))
        self.ref.append(pos, k, v, ks, vs)

    def append_quantize(self, pos, k_bf16, v_bf16):
        wf.wf_kv_append_quantize(self.gpu, pos, dev(k_bf16, "bf16"), dev(v_bf16, "bf16"))
        self.ref.append_quantized(pos, k_bf16, v_bf16)

    def evict(self, n, poison=False):
        wf.wf_kv_evict(self.gpu, n, poison=poison)
        self.ref.evict(n, poison=poison)

    def pages_equal(self):
        torch.cuda.synchronize()
        ok = np.array_equal(host_codes(self.gpu.k).view(np.uint8), self.ref.k.view(np.uint8)) and \
            np.array_equal(host_codes(self.gpu.v).view(np.uint8), self.ref.v.view(np.uint8))
        if self.dtype == "fp8":
            ok = ok and np.array_equal(self.gpu.k_scale.cpu().numpy(), self.ref.k_scale) and \
                np.array_equal(self.gpu.v_scale.cpu().numpy(), self.ref.v_scale)
        return ok and (self.gpu.start, self.gpu.end) == (self.ref.start, self.ref.end)

    def attend(self, q_dev, q_off, kb, ke, scale=0.0, workspace="auto"):
        o, lse = wf.wf_chunk_attn_fwd(self.gpu, q_dev, q_off, kb, ke, scale, return_lse=True, workspace=workspace)
        torch.cuda.synchronize()
        return o, lse

    def reference(self, q_vals, q_off, kb, ke, scale=None, heads=None):
        """Oracle output for q_vals [Nq, H', D] (H' = len(heads) when a head subset is given)."""
        a, b = int(min(kb)), int(max(ke))
        K, V = self.ref.gather(a, b, heads=heads)
        return oracle.chunk_attention(q_vals, K, V, q_off, kb, ke, scale=scale, kv_origin=a)


def errors(got, ref):
    d = np.abs(got - ref)
    rel = np.sqrt((d ** 2).sum() / max((ref ** 2).sum(), 1e-300))
    return float(d.max()), float(d.mean()), float(rel)


LOG2E = 1.4426950408889634


def rescale_events(q_vals, k_vals, kb, ke, kind, scale=None):
    """Key tiles at which the online softmax of the attention kernels must move its
    reference point, derived from the inputs alone (one head).

    q_vals [R, D] query rows, k_vals [ke - kb, D] the keys kb .. ke - 1.  Tiles are
    the kernels' 64-key tiles, counted from base = kb - kb % 8.  Whatever the
    rescale history, the kernels' reference point m never exceeds M(t), the largest
    score (log2 units) of the keys before tile t, so tile t forces a rescale when
      kind "max11" (bf16 LDS-DMA kernel: some x = score - m above 11):
          the tile's maximum is above M(t) + 11.01;
      kind "max" (E4M3FN kernels: a lane's sum of P' = 2^(x + c), c <= log2(1.75),
          above 448; register-staged kernel: tile maximum > m + 8):
          the tile's maximum is above M(t) + 8.01.
    Tile 0 only sets m.  Returns the sorted tile indices t >= 1 at which some row
    forces a rescale; the events hold for any cut of the key range into
    segments, except at a segment's first tile.
    """
    thr = {"max11": 11.01, "max": 8.01}[kind]
    q = np.asarray(q_vals, np.float64)
    k = np.asarray(k_vals, np.float64)
    d = q.shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    s = (q @ k.T) * (scale * LOG2E)
    base = kb - kb % 8
    tile = (np.arange(kb, ke) - base) // 64
    nt = int(tile[-1]) + 1
    events = []
    run_max = np.full(q.shape[0], -np.inf)
    for t in range(nt):
        cols = np.nonzero(tile == t)[0]
        st = s[:, cols]
        if t > 0 and bool(np.any(st.max(axis=1) > run_max + thr)):
            events.append(t)
        run_max = np.maximum(run_max, st.max(axis=1))
    return events


def score_error_bounds(q_vals, K, q_off, kb, ke, kb0):
    """Delta_row per (head, row): 2^-8 * scale * max over the row's visible keys of sum_d |q_d k_jd|."""
    qa = np.abs(np.asarray(q_vals, np.float64))
    ka = np.abs(np.asarray(K, np.float64))
    nq, h, d = qa.shape
    out = np.zeros((h, nq))
    for c in range(len(q_off) - 1):
        a, b = kb[c] - kb0, ke[c] - kb0
        for hh in range(h):
            m = qa[q_off[c]:q_off[c + 1], hh] @ ka[a:b, hh].T
            out[hh, q_off[c]:q_off[c + 1]] = m.max(axis=1) if m.size else 0.0
    return out * 2.0 ** -8 / np.sqrt(d)
