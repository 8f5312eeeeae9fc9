"""Streaming round driver: one forward round over a stack of layers, eager or as captured HIP graphs.

A round is, per layer, the cache step of chunk-wise streaming generation
(scope-causal-forcing README, "How It Works"; Wave Forcing abstract): drop the
oldest chunk once the window is full, append the new chunk's K/V, then let the
chunk's queries attend to the window [max(start, end - W), end).

Every launch argument depends only on ring-relative positions (page slot and
offset, the position within 8 keys, key counts), so once the window is full a
round repeats with period T*P / gcd(T*P, n) rounds (7 for 4680-token chunks on
a 21 x 1560-token ring).  `capture()` records one graph per phase; `replay()`
runs the graph of the current phase and then applies the round's metadata
change (start += n, end += n) on the host, exactly what the eager calls would
have done.  The graphs read the layers' q / k_new / v_new buffers at replay
time, so a producer refills those buffers between rounds.

This module only orders library calls and metadata; all computation is in the
HIP library.
"""
import math

import torch

from . import _lib


class Layer:
    """One layer's cache and the fixed device buffers of its chunk (q, k_new, v_new, o)."""

    def __init__(self, cache, q, k_new, v_new, o, k_scale_new=None, v_scale_new=None):
        self.cache, self.q, self.k_new, self.v_new, self.o = cache, q, k_new, v_new, o
        self.k_scale_new, self.v_scale_new = k_scale_new, v_scale_new


class StreamingRound:
    def __init__(self, layers, chunk, window, workspace="auto"):
        self.layers = list(layers)
        self.n = int(chunk)
        self.window = int(window)
        c0 = self.layers[0].cache
        self.ring = c0.capacity
        for L in self.layers:
            if L.cache.capacity != self.ring:
                raise ValueError("all layers must share one ring geometry")
        if self.window > self.ring:
            raise ValueError("window exceeds the ring capacity")
        self.period = self.ring // math.gcd(self.ring, self.n)
        self.workspace = workspace
        self.graphs = None

    def _layer_step(self, L):
        c = L.cache
        if c.end - c.start + self.n > c.capacity:
            _lib.wf_kv_evict(c, c.end - c.start + self.n - c.capacity)
        _lib.wf_kv_append(c, c.end, L.k_new, L.v_new, L.k_scale_new, L.v_scale_new)
        kb = max(c.start, c.end - self.window)
        _lib.wf_chunk_attn_fwd(c, L.q, [0, int(L.q.shape[0])], [kb], [c.end], o=L.o, workspace=self.workspace)

    def step(self):
        """One eager round on the current stream."""
        for L in self.layers:
            self._layer_step(L)

    def steady(self):
        """True when every layer's window is full (the state from which rounds repeat)."""
        return all(L.cache.end - L.cache.start + self.n > L.cache.capacity for L in self.layers)

    def phase(self):
        """Ring position of the next append: it fixes every launch argument of the round."""
        return self.layers[0].cache.end % self.ring

    def capture(self):
        """Record one graph per phase of the ring, starting from the current (steady) state."""
        if not self.steady():
            raise RuntimeError("capture needs full windows: run eager rounds first")
        if isinstance(self.workspace, str):
            q = self.layers[0].q
            self.workspace = _lib.workspace_for(self.layers[0].cache, q.device)
        saved = [(L.cache.c.start, L.cache.c.end) for L in self.layers]
        torch.cuda.synchronize()
        graphs = {}
        for _ in range(self.period):
            ph = self.phase()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self.step()
            graphs[ph] = g
        for L, (s, e) in zip(self.layers, saved):
            L.cache.c.start, L.cache.c.end = s, e
        self.graphs = graphs
        return self

    def replay(self):
        """Run the captured round of the current phase, then advance the host metadata by one round."""
        if self.graphs is None:
            raise RuntimeError("capture() first")
        self.graphs[self.phase()].replay()
        for L in self.layers:
            c = L.cache.c
            c.end += self.n
            c.start = max(c.start, c.end - c.table_len * c.page_size)
