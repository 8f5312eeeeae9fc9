// Device helpers shared by the attention kernels (bf16 and E4M3FN tiles):
// vector types, lane-half reductions, work-item decoding, the lazy exact
// rescale of the online softmax, LDS-DMA primitives, page cursors over the
// paged ring and the split schedule's block -> segment walk.
#pragma once
#include <type_traits>

#include "wf_internal.h"

namespace wf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kTileKeys = 64;  // keys per LDS tile; ChunkDesc::nsteps counts these

// Value of the other 32-lane half (lane l <-> l ^ 32) combined with op.
__device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Work item -> (chunk, query tile, head).  All query tiles of one (chunk,
// head) read the same keys, and each of the 8 XCDs has its own L2, so inside
// a chunk the items are dealt (deal_position) so that the workgroups that run
// together on one XCD share as few heads' keys as possible.
struct Item {
  int c, qt, head;
};
__device__ __forceinline__ int chunk_of_item(const AttnParams& p, int item) {
  int c = 0;
  while (c + 1 < p.num_chunks && item >= p.chunk[c + 1].item0) ++c;
  return c;
}
__device__ __forceinline__ Item decode_item(const AttnParams& p, int item) {
  Item it;
  it.c = chunk_of_item(p, item);
  const int T = p.chunk[it.c].ntiles;
  const int pos = deal_position(T * p.H, item - p.chunk[it.c].item0);
  it.head = pos / T;
  it.qt = pos - it.head * T;
  return it;
}
// Inverse of decode_item inside chunk c: (query tile, head) -> item.
__device__ __forceinline__ int encode_item(const AttnParams& p, int c, int qt, int head) {
  const int T = p.chunk[c].ntiles;
  return p.chunk[c].item0 + deal_index(T * p.H, head * T + qt);
}

constexpr float kRescaleThreshold = 8.0f;  // log2 units: p <= 2^8 between rescales

// Exact lazy rescaling: the reference point m moves only when a row maximum
// exceeds it by more than the threshold; O and l are always relative to m.
template <int D>
__device__ __forceinline__ void maybe_rescale(float mx, float& m, float& l, f32x16 (&o)[D / 32]) {
  if (__builtin_amdgcn_ballot_w64(mx > m + kRescaleThreshold) != 0) {
    const float m_new = fmaxf(m, mx);
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
  }
}

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0] | vmcnt[5:4] << 14,
// expcnt[6:4] = 7, lgkmcnt[11:8] = 15).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// LDS-DMA: each lane loads 16 (or 4) bytes from src; lane L's bytes land at
// lds + 16 L (or lds + 4 L); lds is wave-uniform.
__device__ __forceinline__ void dma16(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)lds, 4, 0, 0);
}

// Scalar cursor over the chunk's keys for one DMA stream (K or V^T runs):
// ring slot and in-page offset of the next run, plus the byte bases of the
// (page, head) blocks of that slot (b0) and of the next slot (b1) in both the
// K and the V cache.  A run spans at most two pages (pages hold >= 64 keys).
// With RB bytes per K row (head_dim x element size) and EB bytes per element,
// for key k of the run (0-based) the K row is at byte
// (k < split ? kb0 : kb1) + k * RB and the V^T column at
// (k < split ? vb0 : vb1) + d * P * EB + k * EB, relative to the cache bases;
// kb1 / vb1 are biased by -P so one formula serves both pages.  The bases are
// refreshed only when the cursor crosses into the next page.
struct Cursor {
  int32_t slot, off;
  uint32_t k0, k1, v0, v1;
};
struct RunGeom {
  uint32_t kb0, kb1, vb0, vb1;
  int32_t split;
};

template <int RB>
__device__ __forceinline__ void slot_bases(const AttnParams& p, int head, int slot, uint32_t& kb, uint32_t& vb) {
  const uint32_t r = (uint32_t)(p.table[slot] * p.H + head);
  kb = r * (uint32_t)p.P * RB;
  vb = r * (uint32_t)p.P * RB;  // V^T block of (page, head): D rows of P keys, same size as K's
}

__device__ __forceinline__ int next_slot(const AttnParams& p, int s) { return s + 1 == p.T ? 0 : s + 1; }

template <int RB>
__device__ __forceinline__ Cursor cursor_at(const AttnParams& p, const ChunkDesc& cd, int head, int rel0) {
  const uint32_t x = (uint32_t)cd.map.base_off + (uint32_t)rel0;
  const uint32_t pg = fastdiv(x, p.divP);
  Cursor c;
  c.off = (int32_t)(x - pg * p.divP.d);
  const uint32_t slot = (uint32_t)cd.map.base_slot + pg;
  c.slot = (int32_t)(slot - fastdiv(slot, p.divT) * p.divT.d);
  slot_bases<RB>(p, head, c.slot, c.k0, c.v0);
  slot_bases<RB>(p, head, next_slot(p, c.slot), c.k1, c.v1);
  return c;
}

template <int RB, int EB>
__device__ __forceinline__ RunGeom run_geom(const AttnParams& p, const Cursor& c) {
  RunGeom g;
  g.split = p.P - c.off;
  g.kb0 = c.k0 + (uint32_t)c.off * RB;
  g.kb1 = c.k1 + (uint32_t)(c.off - p.P) * RB;
  g.vb0 = c.v0 + (uint32_t)c.off * EB;
  g.vb1 = c.v1 + (uint32_t)(c.off - p.P) * EB;
  return g;
}

template <int RB>
__device__ __forceinline__ void advance(const AttnParams& p, int head, Cursor& c, int n) {
  c.off += n;
  if (c.off >= p.P) {
    c.off -= p.P;
    c.slot = next_slot(p, c.slot);
    c.k0 = c.k1;
    c.v0 = c.v1;
    slot_bases<RB>(p, head, next_slot(p, c.slot), c.k1, c.v1);
  }
}

// Split schedule helpers.  Part p of an item covers key tiles [p S / m, (p + 1) S / m).
__device__ __forceinline__ int part_begin(const SplitSched& sp, int p) { return (int)(((int64_t)p * sp.S) / sp.m); }

// Tile index t (over all chunks, in launch order) and head -> chunk, item.
__device__ __forceinline__ void tile_item(const AttnParams& p, int t, int head, int& c, int& item) {
  c = 0;
  while (c + 1 < p.num_chunks && t * p.H >= p.chunk[c + 1].item0) ++c;
  item = encode_item(p, c, t - p.chunk[c].item0 / p.H, head);
}

// Head-major index of the B part of (item, part p): u = (head * m + p) * tiles + tile.
__device__ __forceinline__ int b_index(const AttnParams& p, int item, int part) {
  const Item it = decode_item(p, item);
  const int t = p.chunk[it.c].item0 / p.H + it.qt;
  return (it.head * p.sp.m + part) * p.sp.tiles + t;
}

// The work of block g as (item, key tiles [j0, j1), slot) segments, handed to
// body in order (one call site, so the body is inlined once):
//   no workspace: item = block, whole key range, slot -1 (final output);
//   split schedule, A block: one part of one item minus the part's tail;
//   split schedule, B block: the tails of B parts [u0, u1).
template <typename Body>
__device__ __forceinline__ void walk_segments(const AttnParams& p, int g, Body&& body) {
  const SplitSched& sp = p.sp;
  const int na = p.ws != nullptr ? sp.n * sp.m : 0;
  int u = 0, u1 = 1;
  if (p.ws != nullptr && g >= na) {
    u = (g - na) * sp.q;
    u1 = min(u + sp.q, na);
  }
  for (; u < u1; ++u) {
    int item, j0, j1, slot;
    if (p.ws == nullptr) {
      item = g;
      j0 = 0;
      j1 = p.chunk[chunk_of_item(p, g)].nsteps;
      slot = -1;
    } else if (g < na) {
      const int part = g / sp.n;
      item = g - part * sp.n;
      j0 = part_begin(sp, part);
      j1 = part_begin(sp, part + 1) - sp.b;
      slot = g;
    } else {
      const int mt = sp.m * sp.tiles;
      const int head = u / mt;
      const int rem = u - head * mt;
      const int part = rem / sp.tiles;
      int c;
      tile_item(p, rem - part * sp.tiles, head, c, item);
      j1 = part_begin(sp, part + 1);
      j0 = j1 - sp.b;
      slot = na + u;
    }
    body(item, j0, j1, slot);
  }
}

}  // namespace
}  // namespace wf
