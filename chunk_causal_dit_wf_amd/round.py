"""Streaming round driver: forward rounds over a stack of layers, eager or as captured HIP graphs.

A round is, per layer, the cache step of chunk-wise streaming generation
(scope-causal-forcing README, "How It Works"; Wave Forcing abstract):

* ``stages == 1`` -- one chunk per round: drop the oldest chunk once the ring
  is full, append the new chunk's K/V, let its queries attend to the window
  [max(start, end - W), end).
* ``stages == S > 1`` -- the staggered wave (Wave Forcing abstract: staggered
  denoising and cache-refresh stages, one output chunk per concurrent forward
  round after pipeline fill, "1F1C").  S consecutive chunks are in flight,
  chunk f - S + 1 (oldest) .. f (newest), each at a different stage; the
  oldest one's stage is the timestep-0 cache refresh (README "How It Works",
  step 2).  Per layer and round:
    - evict what the ring can no longer hold once chunk f is in
      (start = max(start, (f + 1) n - capacity));
    - append the in-flight chunks' K/V at [(f - S + 1) n, (f + 1) n) in one
      call: the S - 1 older chunks are rewritten in place (their K/V changed
      with their noise level; the oldest one's rewrite is the clean refresh),
      the newest is appended at the end;
    - one attention launch for all S chunks: the queries of chunk c see
      [max(start, e_c - W), e_c) with e_c = (c + 1) n -- their own chunk,
      bidirectionally, and every earlier chunk in the window, including the
      in-flight ones whose denoising is not finished (the mixed-noise
      frontier).  Later chunks are not visible to earlier ones.
  During pipeline fill (rounds 0 .. S - 2) only chunks 0 .. f are in flight.
  A ring of W + (S - 1) n tokens lets every in-flight chunk see its full
  window; a smaller ring shortens the oldest chunks' windows (the range
  starts at `start`).

Per-layer buffers hold the in-flight chunks in chunk order: rows
[j n, (j + 1) n) of q / k_new / v_new / o belong to chunk f - S + 1 + j.  A
producer writes the round's q / k_new / v_new before the round and reads o
after it.

Every launch argument depends only on ring-relative positions (page slot and
offset, the position within 8 keys, key counts), so once the pipeline is full
a round repeats with period capacity / gcd(capacity, n) rounds.  `capture()`
records one graph per phase; `replay()` runs the graph of the current phase
and then applies the round's metadata change on the host, exactly what the
eager calls would have done.  The graphs read the layers' buffers at replay
time.

This module only orders library calls and metadata; all computation is in the
HIP library.
"""
import math

import torch

from . import _lib


class Layer:
    """One layer's cache and the fixed device buffers of its in-flight chunks (q, k_new, v_new, o)."""

    def __init__(self, cache, q, k_new, v_new, o, k_scale_new=None, v_scale_new=None):
        self.cache, self.q, self.k_new, self.v_new, self.o = cache, q, k_new, v_new, o
        self.k_scale_new, self.v_scale_new = k_scale_new, v_scale_new


class WaveRound:
    def __init__(self, layers, chunk, window, stages=1, workspace="auto"):
        self.layers = list(layers)
        self.n = int(chunk)
        self.window = int(window)
        self.stages = int(stages)
        if self.stages < 1:
            raise ValueError("stages must be >= 1")
        c0 = self.layers[0].cache
        self.ring = c0.capacity
        for L in self.layers:
            if L.cache.capacity != self.ring:
                raise ValueError("all layers must share one ring geometry")
            if L.q.shape[0] != self.stages * self.n:
                raise ValueError("per-layer buffers hold stages * chunk rows")
        if self.window > self.ring or self.stages * self.n > self.ring:
            raise ValueError("window and in-flight chunks must fit the ring")
        self.period = self.ring // math.gcd(self.ring, self.n)
        self.workspace = workspace
        self.graphs = None
        # Index of the next round = its newest chunk: positions [r n, (r + 1) n).  A stack whose
        # caches already hold whole chunks continues after them.
        ends = {L.cache.end for L in self.layers}
        if len(ends) != 1 or next(iter(ends)) % self.n:
            raise ValueError("all caches must end at the same whole-chunk position")
        self.round = ends.pop() // self.n

    def in_flight(self, r=None):
        """Chunks in flight in round r (default: the next round), oldest first."""
        r = self.round if r is None else r
        return list(range(max(0, r - self.stages + 1), r + 1))

    def _layer_step(self, L, r):
        c = L.cache
        n, S = self.n, self.stages
        chunks = self.in_flight(r)
        first = chunks[0]
        new_end = (r + 1) * n
        drop = max(0, new_end - (c.start + c.capacity))
        if drop:
            _lib.wf_kv_evict(c, drop)
        j0 = first - (r - S + 1)  # buffer block of the oldest in-flight chunk
        rows = slice(j0 * n, S * n)
        ks = None if L.k_scale_new is None else L.k_scale_new[j0 * n // c.c.page_size:]
        vs = None if L.v_scale_new is None else L.v_scale_new[j0 * n // c.c.page_size:]
        _lib.wf_kv_append(c, first * n, L.k_new[rows], L.v_new[rows], ks, vs)
        kb = [max(c.start, (ch + 1) * n - self.window) for ch in chunks]
        ke = [(ch + 1) * n for ch in chunks]
        q_off = [i * n for i in range(len(chunks) + 1)]
        _lib.wf_chunk_attn_fwd(c, L.q[rows], q_off, kb, ke, o=L.o[rows], workspace=self.workspace)

    def step(self):
        """One eager round on the current stream."""
        for L in self.layers:
            self._layer_step(L, self.round)
        self.round += 1

    def steady(self):
        """True once the pipeline is full and every ring is full (the state from which rounds repeat)."""
        r = self.round
        return r >= self.stages - 1 and (r + 1) * self.n > self.ring

    def phase(self):
        """Ring position of the next round's newest chunk: it fixes every launch argument of the round."""
        return (self.round * self.n) % self.ring

    def capture(self):
        """Record one graph per phase of the ring, starting from the current (steady) state."""
        if not self.steady():
            raise RuntimeError("capture needs a full pipeline and full rings: run eager rounds first")
        if isinstance(self.workspace, str):
            q = self.layers[0].q
            self.workspace = _lib.workspace_for(self.layers[0].cache, q.device)
        saved = [(L.cache.c.start, L.cache.c.end) for L in self.layers]
        saved_round = self.round
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
        self.round = saved_round
        self.graphs = graphs
        return self

    def replay(self):
        """Run the captured round of the current phase, then advance the host metadata by one round."""
        if self.graphs is None:
            raise RuntimeError("capture() first")
        self.graphs[self.phase()].replay()
        new_end = (self.round + 1) * self.n
        for L in self.layers:
            c = L.cache.c
            c.end = max(c.end, new_end)
            c.start = max(c.start, new_end - c.table_len * c.page_size)
        self.round += 1


class StreamingRound(WaveRound):
    """One chunk per round (stages == 1)."""

    def __init__(self, layers, chunk, window, workspace="auto"):
        super().__init__(layers, chunk, window, stages=1, workspace=workspace)
