// Internal kernel parameter blocks and launchers shared by the host layer
// (api.cpp) and the HIP kernels.  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/wf_chunk_attn.h"

namespace wf {

// Unsigned 32-bit division by a runtime-invariant divisor via multiply-high
// (round-up method, Granlund & Montgomery 1994 / Hacker's Delight 10-8).
// Exact for every n < 2^32 and 1 <= d < 2^31.
struct FastDiv {
  uint32_t d;      // divisor
  uint32_t mult;   // magic multiplier
  uint32_t shift;  // ceil(log2 d)
};

inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  f.shift = l;
  f.mult = (uint32_t)((((1ull << l) - d) << 32) / d + 1);
  return f;
}

__host__ __device__ inline uint32_t fastdiv(uint32_t n, const FastDiv& f) {
#if defined(__HIP_DEVICE_COMPILE__)
  uint32_t t = __umulhi(n, f.mult);
#else
  uint32_t t = (uint32_t)(((uint64_t)n * f.mult) >> 32);
#endif
  if (f.shift == 0) return n;  // d == 1
  return (t + ((n - t) >> 1)) >> (f.shift - 1);
}

// XCD deal of a chunk's N work items (head-major positions 0 .. N-1).  The
// dispatcher sends workgroup L to XCD L % 8, so XCD x runs Q + 1 workgroups
// for x < R and Q for the rest (N = 8 Q + R).  The head-major order is cut
// into 8 runs with evenly spread ends, run r = [start(r), start(r + 1)),
// start(r) = floor((N r + 4) / 8), so that run ends fall on head ends where
// they can (each head's keys then sit in as few L2s as possible); run r is
// long (Q + 1 items) iff (R r + 4) mod 8 >= 8 - R.  XCD x < R takes the x-th
// long run, XCD x >= R the (x - R)-th short one, and its k-th workgroup
// (k = L / 8) the k-th position of that run.
__host__ __device__ inline int deal_run_start(int N, int r) { return (int)(((int64_t)N * r + 4) >> 3); }
__host__ __device__ inline bool deal_run_long(int R, int r) { return ((R * r + 4) & 7) >= 8 - R; }

// Workgroup index L (0 <= L < N) -> head-major position.
__host__ __device__ inline int deal_position(int N, int L) {
  const int R = N & 7, x = L & 7, k = L >> 3;
  const bool lng = x < R;
  int idx = lng ? x : x - R, r = 0;
  for (; r < 8; ++r)
    if (deal_run_long(R, r) == lng && idx-- == 0) break;
  return deal_run_start(N, r) + k;
}

// Inverse: head-major position (0 <= pos < N) -> workgroup index L.
__host__ __device__ inline int deal_index(int N, int pos) {
  const int R = N & 7;
  int r = 0;
  while (r < 7 && deal_run_start(N, r + 1) <= pos) ++r;
  const bool lng = deal_run_long(R, r);
  int rank = 0;
  for (int q = 0; q < r; ++q) rank += deal_run_long(R, q) == lng;
  return 8 * (pos - deal_run_start(N, r)) + (lng ? rank : R + rank);
}

// Page addressing of a window that starts at a known logical position.  For a
// logical token t >= base, with rel = t - base (32-bit):
//   slot   = (base_slot + (base_off + rel) / P) mod T
//   offset = (base_off + rel) mod P
struct PageMap {
  int32_t base_slot;  // (base / P) mod T
  int32_t base_off;   // base mod P
};

// ---------------------------------------------------------------- append
struct AppendParams {
  const void* k_new;      // [n][H][D]
  const void* v_new;      // [n][H][D]
  const float* ks_new;    // [n/P][H][nblk] or null
  const float* vs_new;
  void* k;                // [pages][H][P][D]
  void* v;                // [pages][H][D][P]
  float* ks;              // [pages][H][nblk]
  float* vs;
  int32_t n;              // tokens
  int32_t H, D, P, T, nblk;
  int32_t esize;          // bytes per element (4, 2, 1)
  int32_t lead;           // pos mod P: page offset of the first appended token
  PageMap map;            // for logical base = pos - lead (the start of pos's page)
  FastDiv div_tpp;        // tiles per page, ceil(P / 64)
  FastDiv divH;           // heads
  FastDiv divT;
  int32_t table[WF_MAX_TABLE_LEN];
};

struct PoisonParams {
  void* k;
  void* v;
  int32_t n, H, D, P, T;
  int32_t esize;
  PageMap map;  // base = first evicted token
  FastDiv divP, divT;
  int32_t table[WF_MAX_TABLE_LEN];
};

hipError_t launch_append(const AppendParams& p, int ntiles, hipStream_t s);

// Quantising append: bf16 rows -> E4M3FN codes + per-(page, head, block) scales.
struct QuantAppendParams {
  const void* k_new;      // bf16 [n][H][D]
  const void* v_new;
  void* k;                // E4M3FN pages [pages][H][P][D]
  void* v;                // [pages][H][D][P]
  float* ks;              // [pages][H][nblk]
  float* vs;
  int32_t npages;         // new pages (n / P)
  int32_t H, D, P, T, nblk;
  int32_t base_slot;      // ring slot of the first new page
  int32_t table[WF_MAX_TABLE_LEN];
};
hipError_t launch_quant_append(const QuantAppendParams& p, hipStream_t s);
hipError_t launch_poison(const PoisonParams& p, hipStream_t s);

// ---------------------------------------------------------------- attention
struct ChunkDesc {
  int32_t q_begin;   // first query row
  int32_t q_len;     // rows
  int32_t ntiles;    // query tiles of this chunk
  int32_t item0;     // first work item of this chunk
  int32_t lead;      // kv_begin - tile origin (0..7): keys skipped in the first tile
  int32_t nkeys;     // kv_end - kv_begin
  PageMap map;       // for logical base = kv_begin - lead
  int32_t nsteps;    // 64-key tiles per query tile, ceil((lead + nkeys) / 64)
};

// Split schedule of the DMA kernel (all chunks with the same nsteps S, fewer
// items n than resident blocks).  Item i's key tiles are cut into m parts,
// part p = [p S / m, (p + 1) S / m).  Block g < n m ("A" block) runs part
// g / n of item g % n minus the part's last b key tiles; those tails ("B"
// parts, numbered head-major: u = (head * m + p) * tiles + tile) are run q at a
// time by blocks n m + u / q.  A parts start at the same key for all items of
// one part index, so blocks of one head stream its K/V in step.  Partial
// results: A part in slot g, B part u in slot n m + u; a merge kernel combines
// the 2m (or m) partials of each item.
struct SplitSched {
  int32_t m;       // key parts per item (>= 1)
  int32_t b;       // key tiles moved from the end of every part to B blocks (0: none)
  int32_t q;       // B parts per B block
  int32_t n;       // items
  int32_t tiles;   // query tiles over all chunks (n / H)
  int32_t S;       // key tiles per item
};

struct AttnParams {
  const void* q;     // [Nq][H][D]
  void* o;           // [Nq][H][D]
  float* lse;        // [H][Nq] or null
  const void* k;     // cache pages
  const void* v;
  const float* ks;   // E4M3FN scales or null
  const float* vs;
  int32_t nq;        // total query rows
  int32_t H, P, T, nblk;
  float scale_log2;  // softmax scale * log2(e)
  int32_t num_chunks;
  int32_t num_items;
  float* ws;             // split schedule: partial results, or null (one block per item)
  SplitSched sp;
  FastDiv divP, divT;
  ChunkDesc chunk[WF_MAX_CHUNKS];
  int32_t table[WF_MAX_TABLE_LEN];
};

// Query rows per workgroup of each attention kernel (the host needs them for the grid).
constexpr int kBlockMF32 = 128;     // fp32 kernel
constexpr int kBlockMStaged = 128;  // bf16 Q, register-staged tile loads (E4M3FN or small pages)
constexpr int kBlockMDma = 256;     // bf16 Q and cache, LDS-DMA tile loads

// Split schedule: each partial-result slot holds, for the BMD rows of one
// query tile, the unnormalised O (fp32 [BMD][D]), the reference maximum m
// (log2 domain) and the row sum l.  At most 2 slots per resident block.
constexpr int64_t ws_slot_floats(int head_dim) { return (int64_t)kBlockMDma * head_dim + 2 * kBlockMDma; }
constexpr int kMergeRows = 32;  // query rows per merge block

hipError_t launch_attn_bf16_dma(const AttnParams& p, int head_dim, int grid, hipStream_t s);
// E4M3FN cache, fp8 MFMA: pages of >= 64 keys, cache < 4 GiB, and per chunk
// lead + nkeys <= 8 * kFp8MaxGroups (the per-8-key scale table in LDS).
constexpr int kFp8MaxGroups = 4096;
hipError_t launch_attn_fp8_dma(const AttnParams& p, int head_dim, int grid, hipStream_t s);
hipError_t attn_fp8_resident_blocks(int head_dim, int* blocks);
hipError_t launch_attn_merge(const AttnParams& p, int head_dim, hipStream_t s);
// Blocks of the DMA kernel that can be resident at once on the current device.
hipError_t attn_dma_resident_blocks(int head_dim, int* blocks);
hipError_t launch_attn_bf16_staged(const AttnParams& p, int head_dim, hipStream_t s);
hipError_t launch_attn_f32(const AttnParams& p, int head_dim, hipStream_t s);
hipError_t launch_attn_fp8kv(const AttnParams& p, int head_dim, hipStream_t s);

// Host layer shared by the entry points (api.cpp): the attention call with a
// caller workspace (scratch_mode false) or with the library's scratch array
// (scratch_mode true), and the thread-local error text of wf_last_error().
wf_status attn_fwd_impl(const wf_kv_cache* c, const void* q, int32_t q_dtype, void* o, float* lse,
                        int32_t num_chunks, const int32_t* q_off, const int64_t* kv_begin, const int64_t* kv_end,
                        float softmax_scale, void* workspace, uint64_t workspace_bytes, bool scratch_mode,
                        void* stream);
wf_status set_error(wf_status s, const char* msg);

}  // namespace wf
