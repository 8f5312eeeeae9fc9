"""Oracle for chunk-wise causal attention over a rolling, paged KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call, link
or run anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library (``chunk_causal_dit_wf_amd``) and never imports it.

What it computes (plain definitions, float64 throughout):

* ``attention.chunk_attention`` -- for every chunk c, head h and query row i
  of the chunk, softmax-weighted sum of the value rows of the keys that chunk
  is allowed to see, i.e. the logical key positions [kv_begin[c], kv_end[c]).
  Source: "Wave Forcing: Towards Speed-of-Light Streaming Video Generation",
  abstract (chunk-wise causal attention over earlier, possibly still-noisy
  chunks); the hellomarvisaitoday Wave Forcing article, first paragraph
  (mixed-noise frontier; K/V state of earlier chunks).
* ``brute.brute_force_attention`` -- the same quantity with an explicit
  dense visibility mask and pure-Python exact sums, for tiny inputs.
* ``cache.KVCacheModel`` -- a byte-for-byte host mirror of the paged ring KV
  cache (append, eviction, logical->physical addressing, gather).  Source: the
  scope-causal-forcing README, "How It Works" (each new frame's K/V is written
  into a cache that later frames read; a timestep-0 re-run rewrites it) and the
  Wave Forcing abstract (cache refresh stages).
* ``numerics`` -- exact decoding of bfloat16 and OCP E4M3FN codes to float64.

Pins that tie these functions to something other than themselves live in
``tests/test_oracle_*.py``.  No function here is "parity unpinned".
"""
from .numerics import decode_bf16, decode_e4m3fn, decode_f32, encode_e4m3fn
from .attention import chunk_attention, merge_partials
from .brute import brute_force_attention
from .cache import KVCacheModel

__all__ = [
    "decode_bf16", "decode_e4m3fn", "decode_f32", "encode_e4m3fn",
    "chunk_attention", "merge_partials", "brute_force_attention", "KVCacheModel",
]
