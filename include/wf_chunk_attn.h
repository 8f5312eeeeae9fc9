/*
 * wf_chunk_attn.h -- C ABI of the chunk-causal attention library for AMD
 * Instinct MI355X (gfx950).
 *
 * The operation comes from streaming video diffusion transformers that
 * generate a video chunk by chunk ("Wave Forcing: Towards Speed-of-Light
 * Streaming Video Generation", abstract; scope-causal-forcing README, "How It
 * Works"):
 *   - every chunk's queries attend, bidirectionally, to their own chunk's
 *     tokens and to the K/V of earlier chunks held in a KV cache, including
 *     chunks whose denoising is not finished yet (the mixed-noise frontier,
 *     hellomarvisaitoday Wave Forcing article, first paragraph);
 *   - each new chunk's K/V is written into the cache, and a re-run at
 *     timestep 0 rewrites it with clean K/V (README "How It Works", steps 1-2);
 *   - the cache keeps a rolling window: the oldest chunk leaves as a new one
 *     arrives.
 *
 * Conventions for every entry point
 *   - Device pointers point to GPU memory the caller owns (e.g. torch
 *     tensors).  The library never allocates, frees or synchronises; all work
 *     is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 *     Calls on one stream execute in order, so append -> attend needs no sync.
 *   - Host pointers (page table, chunk tables) are read during the call only.
 *   - Every argument is validated on the host before anything is enqueued.  A
 *     status other than WF_OK means nothing was enqueued and no cache
 *     metadata changed; wf_last_error() returns the reason (thread-local).
 *   - WF_ERR_HIP means a HIP call or launch failed; metadata is unchanged.
 *   - Calls that use the same cache must not run concurrently from two host
 *     threads.  Nothing throws across the ABI.
 */
#ifndef WF_CHUNK_ATTN_H
#define WF_CHUNK_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum wf_status {
  WF_OK = 0,
  WF_ERR_INVALID_ARG = 1, /* null/aliased pointer, bad range or table       */
  WF_ERR_UNSUPPORTED = 2, /* dtype / head_dim / size outside what is built   */
  WF_ERR_CAPACITY = 3,    /* append would overwrite live tokens              */
  WF_ERR_RANGE = 4,       /* position outside the live window                */
  WF_ERR_HIP = 5          /* HIP runtime or launch failure                   */
} wf_status;

typedef enum wf_dtype {
  WF_F32 = 0,      /* IEEE binary32                                         */
  WF_BF16 = 1,     /* bfloat16                                              */
  WF_FP8_E4M3 = 2  /* OCP E4M3FN (bias 7, max 448, NaN = S.1111.111)        */
} wf_dtype;

#define WF_MAX_TABLE_LEN 256 /* ring slots per cache                       */
#define WF_MAX_CHUNKS 64     /* query chunks per attention call            */
#define WF_SCALE_BLOCK 128   /* tokens per E4M3FN scale block (in a page)  */
#define WF_EVICT_POISON 1u   /* evict flag: overwrite evicted rows with NaN */

/*
 * One layer's KV cache: a ring of `table_len` slots; slot s holds physical
 * page page_table[s] of `page_size` tokens.  Logical token t (positions grow
 * without bound as the video streams) lives at
 *     page = page_table[(t / page_size) % table_len],  offset = t % page_size.
 * Identity table = contiguous cache; table_len 1 = plain ring buffer; a
 * random permutation = paged ring.  The live window is [start, end);
 * capacity = table_len * page_size tokens.
 *
 * Device buffers (caller-owned, 16-byte aligned; element type = kv_dtype):
 *   k       [num_pages][num_heads][page_size][head_dim]
 *           (per page and head: token-major rows of head_dim elements)
 *   v       [num_pages][num_heads][head_dim][page_size]
 *           (per page and head: value rows stored transposed, so the key
 *            index is contiguous -- the layout the P*V product consumes)
 *   The pages fix no cache layout.  Heads are outermost inside a page (a
 *   (page, head) block is one contiguous run), and V is transposed once per
 *   token when it is appended, so that every attention call reads V^T rows
 *   of consecutive keys instead of gathering them.
 *   k_scale, v_scale   E4M3FN only, float32 [num_pages][num_heads][nblk],
 *           nblk = ceil(page_size / 128); block b of a page covers offsets
 *           [128 b, min(128 (b+1), page_size)).  Value = decode(code) * scale.
 *           NULL for other dtypes.
 * Host: page_table [table_len] distinct physical pages in [0, num_pages).
 * Constraints: head_dim in {64, 128}; page_size a positive multiple of 8;
 * table_len <= WF_MAX_TABLE_LEN.  The struct itself is host memory owned by
 * the caller; the library updates start/end in place.
 */
typedef struct wf_kv_cache {
  void *k;
  void *v;
  float *k_scale;
  float *v_scale;
  const int32_t *page_table;
  int32_t table_len;
  int32_t num_pages;
  int32_t page_size;
  int32_t num_heads;
  int32_t head_dim;
  int32_t kv_dtype; /* wf_dtype */
  int64_t start;
  int64_t end;
} wf_kv_cache;

/*
 * Validate a cache description (pointers non-null, sizes supported, page
 * table entries distinct and in range, 0 <= start <= end <= start+capacity).
 * Host only; enqueues nothing.
 */
wf_status wf_kv_cache_check(const wf_kv_cache *cache);

/*
 * Bytes the caller must allocate for c->k (== c->v) and for each scale array
 * (0 unless E4M3FN).  Host only.  Returns WF_OK or WF_ERR_INVALID_ARG /
 * WF_ERR_UNSUPPORTED for an invalid description (start/end ignored).
 */
wf_status wf_kv_cache_bytes(const wf_kv_cache *cache, uint64_t *kv_bytes, uint64_t *scale_bytes);

/*
 * Append (or rewrite) n tokens at logical positions [pos, pos + n).
 * Source: each new chunk's K/V enters the per-layer cache; the timestep-0
 * re-run rewrites a chunk already there (scope-causal-forcing README, "How
 * It Works", steps 1-2; Wave Forcing abstract, cache-refresh stages).
 *   k_new, v_new   device [n][num_heads][head_dim] token-major, kv_dtype.
 *   k_scale_new, v_scale_new   E4M3FN only: device float32
 *                  [n / page_size][num_heads][nblk], copied to the pages the
 *                  tokens land on; NULL otherwise.
 * Requires start <= pos <= end (no gaps) and pos + n <= start + capacity
 * (live tokens are never overwritten by wrap-around: WF_ERR_CAPACITY).  For
 * E4M3FN, pos and n must be multiples of page_size.  On success
 * end = max(end, pos + n).  n == 0 is a no-op.  The copy is bit-exact.
 */
wf_status wf_kv_append(wf_kv_cache *cache, int64_t pos, int32_t n, const void *k_new,
                       const void *v_new, const float *k_scale_new, const float *v_scale_new,
                       void *stream);

/*
 * Quantise bf16 rows to E4M3FN and append them to an E4M3FN cache: the
 * producer side of a cache held in fp8 (the pages' quantised attention
 * backends; scope-causal-forcing README, "How It Works", step 2 writes the
 * cache).  For each new page, head and 128-token scale block:
 *     amax  = max |x| over the block's tokens and dims (float32),
 *     scale = amax / 448,  r = 448 / amax  (float32 divisions rounded to
 *             nearest; 1 and 1 for an all-zero block),
 *     code  = E4M3FN(x * r)  (float32 product rounded to nearest, converted
 *             with round-to-nearest-even, saturating at +-448).
 *   k_new, v_new   device bf16 [n][num_heads][head_dim] token-major, finite.
 * Requires kv_dtype == WF_FP8_E4M3, pos and n multiples of page_size, and the
 * position rules of wf_kv_append.  On success end = max(end, pos + n).  Codes
 * and scales are bit-exact with the definition above.
 */
wf_status wf_kv_append_quantize(wf_kv_cache *cache, int64_t pos, int32_t n, const void *k_new,
                                const void *v_new, void *stream);

/*
 * Drop the n oldest live tokens: start += n (rolling window).  Source: the
 * KV-cached loop advances one chunk at a time (scope-causal-forcing README,
 * "How It Works", step 4) over a bounded, rolling history (the Rolling
 * Forcing baseline named in the Wave Forcing abstract).  Requires
 * 0 <= n <= end - start.  No kernel is launched unless flags has
 * WF_EVICT_POISON, which overwrites the evicted rows with NaN codes so that a
 * later read of them shows up (a test aid).
 */
wf_status wf_kv_evict(wf_kv_cache *cache, int32_t n, uint32_t flags, void *stream);

/*
 * Chunk-wise causal attention (Wave Forcing abstract: queries reach earlier,
 * possibly still-noisy chunks; hellomarvisaitoday article, first paragraph).
 * For chunk c, query rows [q_off[c], q_off[c+1]) attend to logical keys
 * [kv_begin[c], kv_end[c]) of the cache:
 *     O[i,h,:] = sum_j softmax_j(scale * Q[i,h,:].K[j,h,:]) V[j,h,:]
 *     lse[h,i] = ln sum_j exp(scale * Q[i,h,:].K[j,h,:])
 *   q          device [Nq][num_heads][head_dim], Nq = q_off[num_chunks]
 *   q_dtype    WF_F32 with an F32 cache; WF_BF16 with a BF16 or E4M3FN cache
 *   o          device, same shape and dtype as q; must not overlap q or cache
 *   lse        device float32 [num_heads][Nq], natural log, or NULL
 *   q_off      host int32 [num_chunks + 1], q_off[0] = 0, non-decreasing
 *   kv_begin, kv_end   host int64 [num_chunks];
 *              start <= kv_begin[c] < kv_end[c] <= end
 *   softmax_scale      <= 0 selects 1/sqrt(head_dim)
 *   workspace, workspace_bytes
 *              optional device scratch (caller-owned, 256-byte aligned, at
 *              least wf_chunk_attn_workspace_bytes() bytes, not overlapping
 *              any other argument).  NULL (with workspace_bytes 0) selects
 *              one workgroup per query tile of 256 rows ("per-tile"
 *              schedule).  With a workspace, calls on the LDS-DMA kernels
 *              (bf16 or E4M3FN caches with pages of >= 64 tokens) may take
 *              the split schedule instead: it is used when every chunk spans
 *              the same number S of 64-key tiles and there are fewer work
 *              items (query tiles x heads) than resident workgroups.  Each
 *              item's key tiles are then cut into m = min(resident / items,
 *              S / 32, 8) parts; workgroups still idle take the last b key
 *              tiles of q parts each (used only when q <= 5 and b >= 8);
 *              each part leaves fp32 partial results in the workspace and a
 *              second kernel merges them by their log-sum-exp (an exact
 *              re-association of the softmax).  When m = 1 and no tails are
 *              taken the call runs per-tile even with a workspace.
 *              wf_chunk_attn_plan() reports the choice.  Calls that share a
 *              workspace must be ordered (same stream).
 * 1 <= num_chunks <= WF_MAX_CHUNKS.  Accumulation is fp32.  Results are
 * deterministic run to run on a given device and schedule.  Keys outside a
 * chunk's range are never used (NaN there does not leak into the output).
 */
wf_status wf_chunk_attn_fwd(const wf_kv_cache *cache, const void *q, int32_t q_dtype, void *o,
                            float *lse, int32_t num_chunks, const int32_t *q_off,
                            const int64_t *kv_begin, const int64_t *kv_end, float softmax_scale,
                            void *workspace, uint64_t workspace_bytes, void *stream);

/* Attention kernels and schedules, as reported by wf_chunk_attn_plan(). */
typedef enum wf_attn_kernel {
  WF_KERNEL_F32 = 0,         /* fp32 Q and cache: fp32 MFMA                       */
  WF_KERNEL_STAGED_BF16 = 1, /* bf16 cache, pages < 64 tokens (or >= 4 GiB)       */
  WF_KERNEL_STAGED_FP8 = 2,  /* E4M3FN cache dequantised to bf16 on the way in    */
  WF_KERNEL_DMA_BF16 = 3,    /* bf16 cache, pages >= 64: LDS-DMA, bf16 MFMA        */
  WF_KERNEL_DMA_FP8 = 4      /* E4M3FN cache, pages >= 64: LDS-DMA, fp8 MFMA       */
} wf_attn_kernel;

typedef enum wf_attn_schedule {
  WF_SCHED_PER_TILE = 0, /* one workgroup per (query tile, head)              */
  WF_SCHED_SPLIT = 1     /* key-range parts + tails, merged by log-sum-exp     */
} wf_attn_schedule;

typedef struct wf_attn_plan {
  int32_t kernel;          /* wf_attn_kernel                                  */
  int32_t schedule;        /* wf_attn_schedule                                */
  int32_t grid;            /* workgroups of the attention launch              */
  int32_t items;           /* query tiles x heads                             */
  int32_t rows_per_item;   /* query rows per tile                             */
  int32_t parts;           /* split: key parts per item (1 otherwise)         */
  int32_t tail_tiles;      /* split: key tiles per tail part (0: no tails)    */
  int32_t tails_per_block; /* split: tail parts per tail workgroup            */
} wf_attn_plan;

/*
 * The launch wf_chunk_attn_fwd would make for these arguments, without
 * making it: kernel, schedule and grid (a host query, so that callers and
 * benchmarks can state which path ran).  Arguments as for
 * wf_chunk_attn_fwd; workspace_bytes is the size of the workspace that
 * would be passed (0 = none).  Validates the cache and the chunk tables like
 * wf_chunk_attn_fwd; with workspace_bytes > 0 it queries the current HIP
 * device (WF_ERR_HIP without one).  Enqueues nothing.
 */
wf_status wf_chunk_attn_plan(const wf_kv_cache *cache, int32_t q_dtype, int32_t num_chunks,
                             const int32_t *q_off, const int64_t *kv_begin, const int64_t *kv_end,
                             uint64_t workspace_bytes, wf_attn_plan *plan);

/*
 * Workspace bytes wf_chunk_attn_fwd needs for the balanced schedule on the
 * current HIP device for caches like `cache` (depends on head_dim and the
 * device's compute-unit count only; 0 when the cache's dtype does not use
 * one).  Host only.
 */
wf_status wf_chunk_attn_workspace_bytes(const wf_kv_cache *cache, uint64_t *bytes);

/*
 * Allocation-free variant of wf_chunk_attn_fwd, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results and errors as
 * wf_chunk_attn_fwd without a workspace argument: where the split schedule
 * applies, its partial results go to a scratch array inside the library (one
 * per GPU, WF_NOALLOC_SCRATCH_BYTES, held until the process ends) instead of
 * a caller workspace.  A call whose split schedule needs more than that is
 * rejected with WF_ERR_CAPACITY before anything is enqueued.  Calls on one GPU
 * share its array: calls that may overlap on one GPU (other streams, other
 * host threads) must be ordered by the caller, or they race.  Nothing is
 * allocated, freed or synchronised.
 */
#define WF_NOALLOC_SCRATCH_BYTES (72u << 20)
wf_status wf_chunk_attn_fwd_noalloc(const wf_kv_cache *cache, const void *q, int32_t q_dtype, void *o,
                                    float *lse, int32_t num_chunks, const int32_t *q_off,
                                    const int64_t *kv_begin, const int64_t *kv_end, float softmax_scale,
                                    void *stream);

/* Text of the last non-OK status on this thread ("" if none). */
const char *wf_last_error(void);

/* Library version string. */
const char *wf_version(void);

#ifdef __cplusplus
}
#endif

#endif /* WF_CHUNK_ATTN_H */
