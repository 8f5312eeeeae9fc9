"""Host mirror of the paged ring KV cache, byte for byte (oracle; test infrastructure only).

What the cache holds.  In KV-cached streaming generation every new chunk's
K/V is written into a per-layer cache that later chunks read, and a re-run at
timestep 0 rewrites a chunk's entries with clean K/V (scope-causal-forcing
README, "How It Works", steps 1-2; Wave Forcing abstract, cache-refresh
stages).  The cache keeps a bounded rolling window: the oldest tokens leave as
new ones arrive.

Logical positions.  Tokens are numbered by a monotone logical position t.  The
live window is [start, end).  Storage is a ring of T page slots, each slot
naming a physical page of P tokens through a page table:

    slot(t) = (t div P) mod T,   page(t) = table[slot(t)],   offset(t) = t mod P.

Capacity is T*P tokens.  One rule covers a contiguous cache (identity table),
a plain ring (T = 1, P = capacity) and a paged ring (random permutation).

Byte layout of one physical page (per layer):
    K codes [H][P][D]   (per head, token-major rows of D elements)
    V codes [H][D][P]   (per head, value rows stored transposed: D rows of P)
    K/V scales (E4M3FN storage only) [H][ceil(P/128)] float32; scale block b
    of a page covers offsets [128 b, min(128(b+1), P)) of that page.
A stored E4M3FN code x with block scale s represents the value decode(x) * s.

Operations (the plainest reading of the pages' loop: write the new chunk,
drop the oldest):
    append(pos, k_new, v_new[, scales])  needs start <= pos <= end and
        pos + n <= start + capacity; writes tokens [pos, pos+n) (rewriting
        any already there) and sets end = max(end, pos + n).  E4M3FN appends
        must be page aligned (pos and n multiples of P) so scale blocks stay
        whole.
    evict(n)  needs n <= end - start; start += n.  With poison=True the
        evicted rows are overwritten with NaN codes (a test aid).
    append_quantized(pos, k_bf16, v_bf16)  (E4M3FN storage) quantises bf16
        rows page by page and appends codes and scales.  For each page, head
        and 128-token block: amax = max |x| over the block's tokens and dims
        (float32), scale = amax / 448 and r = 448 / amax (float32 divisions
        rounded to nearest; 1 and 1 for an all-zero block), code =
        E4M3FN(x * r) with the product a float32 multiply rounded to nearest and
        the conversion rounding to nearest-even with saturation at 448.
"""
import numpy as np

from .numerics import decode_bf16, decode_e4m3fn, decode_f32, encode_e4m3fn

_STORAGE = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}
_NAN_CODE = {"f32": np.float32(np.nan), "bf16": np.uint16(0x7FC0), "fp8": np.uint8(0x7F)}
SCALE_BLOCK = 128


class KVCacheModel:
    def __init__(self, num_pages, page_size, num_heads, head_dim, dtype, page_table,
                 k_pages=None, v_pages=None, k_scale=None, v_scale=None):
        if dtype not in _STORAGE:
            raise ValueError("dtype must be one of %s" % sorted(_STORAGE))
        table = np.asarray(page_table, dtype=np.int64).reshape(-1)
        if table.size < 1:
            raise ValueError("page table must not be empty")
        if table.min() < 0 or table.max() >= num_pages or len(set(table.tolist())) != table.size:
            raise ValueError("page table entries must be distinct physical pages in [0, num_pages)")
        self.num_pages, self.P, self.H, self.D = int(num_pages), int(page_size), int(num_heads), int(head_dim)
        self.dtype = dtype
        self.table = table
        self.T = int(table.size)
        self.nblk = -(-self.P // SCALE_BLOCK)
        st = _STORAGE[dtype]
        shape_k = (self.num_pages, self.H, self.P, self.D)
        shape_v = (self.num_pages, self.H, self.D, self.P)
        self.k = np.zeros(shape_k, st) if k_pages is None else np.array(k_pages, dtype=st).reshape(shape_k)
        self.v = np.zeros(shape_v, st) if v_pages is None else np.array(v_pages, dtype=st).reshape(shape_v)
        if dtype == "fp8":
            sshape = (self.num_pages, self.H, self.nblk)
            self.k_scale = np.ones(sshape, np.float32) if k_scale is None else np.array(k_scale, np.float32).reshape(sshape)
            self.v_scale = np.ones(sshape, np.float32) if v_scale is None else np.array(v_scale, np.float32).reshape(sshape)
        else:
            self.k_scale = self.v_scale = None
        self.start = 0
        self.end = 0

    @property
    def capacity(self):
        return self.T * self.P

    def locate(self, t):
        """Logical position -> (physical page, offset in page)."""
        t = int(t)
        return int(self.table[(t // self.P) % self.T]), t % self.P

    def _runs(self, a, b):
        """Split logical [a, b) into (logical_start, page, offset, length) runs inside one page."""
        t = a
        while t < b:
            page, off = self.locate(t)
            n = min(b - t, self.P - off)
            yield t, page, off, n
            t += n

    def append(self, pos, k_new, v_new, k_scale_new=None, v_scale_new=None):
        st = _STORAGE[self.dtype]
        k_new = np.asarray(k_new)
        v_new = np.asarray(v_new)
        if k_new.dtype != st or v_new.dtype != st:
            raise TypeError("new K/V must be %s codes" % np.dtype(st))
        n = k_new.shape[0]
        if k_new.shape != (n, self.H, self.D) or v_new.shape != k_new.shape:
            raise ValueError("new K/V must be [n, H, D]")
        pos = int(pos)
        if not (self.start <= pos <= self.end):
            raise ValueError("append position %d outside [start=%d, end=%d]" % (pos, self.start, self.end))
        if pos + n > self.start + self.capacity:
            raise ValueError("append would overrun live tokens (capacity %d)" % self.capacity)
        if self.dtype == "fp8":
            if pos % self.P or n % self.P:
                raise ValueError("E4M3FN appends must be page aligned")
            sshape = (n // self.P, self.H, self.nblk)
            k_scale_new = np.asarray(k_scale_new, np.float32)
            v_scale_new = np.asarray(v_scale_new, np.float32)
            if k_scale_new.shape != sshape or v_scale_new.shape != sshape:
                raise ValueError("new scales must be [n/P, H, ceil(P/128)]")
        for t, page, off, cnt in self._runs(pos, pos + n):
            i = t - pos
            # K page [H][P][D] <- rows [i, i+cnt) of [n][H][D]
            self.k[page, :, off:off + cnt, :] = k_new[i:i + cnt].transpose(1, 0, 2)
            # V page [H][D][P] <- the same rows, transposed
            self.v[page, :, :, off:off + cnt] = v_new[i:i + cnt].transpose(1, 2, 0)
            if self.dtype == "fp8":
                j = i // self.P
                self.k_scale[page] = k_scale_new[j]
                self.v_scale[page] = v_scale_new[j]
        self.end = max(self.end, pos + n)

    def quantize_pages(self, x_bf16):
        """bf16 codes [n, H, D] (n a multiple of P) -> E4M3FN codes [n, H, D], scales [n/P, H, nblk]."""
        x_bf16 = np.asarray(x_bf16)
        n = x_bf16.shape[0]
        if n % self.P:
            raise ValueError("quantised appends must be whole pages")
        x = decode_bf16(x_bf16).astype(np.float32)  # exact: bf16 values are float32 values
        codes = np.empty(x.shape, np.uint8)
        scales = np.empty((n // self.P, self.H, self.nblk), np.float32)
        f448 = np.float32(448.0)
        for j in range(n // self.P):
            for b in range(self.nblk):
                r0 = j * self.P + b * SCALE_BLOCK
                r1 = min(r0 + SCALE_BLOCK, (j + 1) * self.P)
                blk = x[r0:r1]                                       # [rows, H, D] float32
                amax = np.abs(blk).max(axis=(0, 2))                  # [H] float32
                pos = amax > 0
                with np.errstate(divide="ignore", invalid="ignore"):
                    scale = np.where(pos, amax / f448, np.float32(1.0)).astype(np.float32)
                    r = np.where(pos, f448 / amax, np.float32(1.0)).astype(np.float32)
                scales[j, :, b] = scale
                codes[r0:r1] = encode_e4m3fn(blk * r[None, :, None])  # float32 products
        return codes, scales

    def append_quantized(self, pos, k_bf16, v_bf16):
        if self.dtype != "fp8":
            raise TypeError("append_quantized needs an E4M3FN cache")
        kc, ks = self.quantize_pages(k_bf16)
        vc, vs = self.quantize_pages(v_bf16)
        self.append(pos, kc, vc, ks, vs)

    def evict(self, n, poison=False):
        n = int(n)
        if n < 0 or n > self.end - self.start:
            raise ValueError("cannot evict %d tokens from a window of %d" % (n, self.end - self.start))
        if poison:
            nan = _NAN_CODE[self.dtype]
            for _, page, off, cnt in self._runs(self.start, self.start + n):
                self.k[page, :, off:off + cnt, :] = nan
                self.v[page, :, :, off:off + cnt] = nan
        self.start += n

    def gather_codes(self, a, b):
        """Stored codes of logical tokens [a, b) as K [b-a, H, D], V [b-a, H, D]."""
        if not (self.start <= a <= b <= self.end):
            raise ValueError("gather [%d,%d) outside the live window [%d,%d)" % (a, b, self.start, self.end))
        ks, vs = [], []
        for _, page, off, cnt in self._runs(a, b):
            ks.append(self.k[page, :, off:off + cnt, :].transpose(1, 0, 2))
            vs.append(self.v[page, :, :, off:off + cnt].transpose(2, 0, 1))
        st = _STORAGE[self.dtype]
        if not ks:
            z = np.zeros((0, self.H, self.D), st)
            return z, z.copy()
        return np.concatenate(ks), np.concatenate(vs)

    def gather(self, a, b, heads=None):
        """Values (float64) of logical tokens [a, b): K [b-a, H', D], V [b-a, H', D].

        heads optionally selects a subset of heads (H' = len(heads)); default all.
        """
        kc, vc = self.gather_codes(a, b)
        hs = np.arange(self.H) if heads is None else np.asarray(heads, dtype=np.int64)
        kc, vc = kc[:, hs], vc[:, hs]
        if self.dtype == "f32":
            return decode_f32(kc), decode_f32(vc)
        if self.dtype == "bf16":
            return decode_bf16(kc), decode_bf16(vc)
        kd, vd = decode_e4m3fn(kc), decode_e4m3fn(vc)
        ksc = np.empty((b - a, len(hs)), np.float64)
        vsc = np.empty((b - a, len(hs)), np.float64)
        for t, page, off, cnt in self._runs(a, b):
            blk = (np.arange(off, off + cnt) // SCALE_BLOCK)
            ksc[t - a:t - a + cnt] = self.k_scale[page][hs][:, blk].T
            vsc[t - a:t - a + cnt] = self.v_scale[page][hs][:, blk].T
        return kd * ksc[:, :, None], vd * vsc[:, :, None]
