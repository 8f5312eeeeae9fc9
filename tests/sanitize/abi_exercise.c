/* Drives every host-side path of the C ABI that needs no GPU: cache checks,
 * argument validation, attention planning (all kernels and chunk shapes) and
 * evict metadata.  Built with the sanitizers against api.cpp and host stubs
 * of the launchers (every launch ends in WF_ERR_HIP).  Exit 0 when every
 * status matches; a sanitizer report aborts. */
#include <stdio.h>
#include <stdint.h>
#include <string.h>
#include "wf_chunk_attn.h"
#include "wf_stream_copy.h"

static int failures = 0;
#define EXPECT(call, want)                                                          \
  do {                                                                              \
    wf_status got_ = (call);                                                        \
    if (got_ != (want)) {                                                           \
      printf("line %d: %s -> %d, want %d (%s)\n", __LINE__, #call, (int)got_,      \
             (int)(want), wf_last_error());                                         \
      ++failures;                                                                   \
    }                                                                               \
  } while (0)

/* Device addresses are only compared and offset on the host, never
 * dereferenced: distinct, far-apart fake addresses stand in for buffers. */
#define KBUF ((void *)(uintptr_t)0x100000000000ull)
#define VBUF ((void *)(uintptr_t)0x200000000000ull)
#define QBUF ((char *)(uintptr_t)0x300000000000ull)
#define OBUF ((char *)(uintptr_t)0x400000000000ull)
#define KSC ((float *)(uintptr_t)0x500000000000ull)
#define VSC ((float *)(uintptr_t)0x600000000000ull)
static int32_t table[21];

static wf_kv_cache make_cache(int dtype, int P, int T, int H, int D) {
  wf_kv_cache c;
  memset(&c, 0, sizeof(c));
  c.k = KBUF;
  c.v = VBUF;
  c.k_scale = dtype == WF_FP8_E4M3 ? KSC : NULL;
  c.v_scale = dtype == WF_FP8_E4M3 ? VSC : NULL;
  for (int i = 0; i < T; ++i) table[i] = (5 * i + 3) % T; /* a permutation (gcd(5, T) = 1) */
  c.page_table = table;
  c.table_len = T;
  c.num_pages = T;
  c.page_size = P;
  c.num_heads = H;
  c.head_dim = D;
  c.kv_dtype = dtype;
  c.start = 0;
  c.end = (int64_t)P * T;
  return c;
}

int main(void) {
  printf("%s\n", wf_version());
  /* cache checks */
  wf_kv_cache c = make_cache(WF_BF16, 1560, 21, 12, 128);
  EXPECT(wf_kv_cache_check(&c), WF_OK);
  uint64_t kvb = 0, scb = 0;
  EXPECT(wf_kv_cache_bytes(&c, &kvb, &scb), WF_OK);
  if (kvb != 1560ull * 21 * 12 * 128 * 2 || scb != 0) { /* bytes of K (= of V) */ printf("kv bytes %llu\n", (unsigned long long)kvb); ++failures; }
  EXPECT(wf_kv_cache_check(NULL), WF_ERR_INVALID_ARG);
  wf_kv_cache bad = c;
  bad.k = NULL;
  EXPECT(wf_kv_cache_check(&bad), WF_ERR_INVALID_ARG);
  bad = c;
  bad.head_dim = 96;
  EXPECT(wf_kv_cache_check(&bad), WF_ERR_UNSUPPORTED);
  bad = c;
  bad.page_size = 0;
  EXPECT(wf_kv_cache_check(&bad), WF_ERR_UNSUPPORTED);
  bad = c;
  bad.table_len = WF_MAX_TABLE_LEN + 1;
  EXPECT(wf_kv_cache_check(&bad), WF_ERR_INVALID_ARG);
  bad = c;
  bad.start = 5;
  bad.end = 4;
  EXPECT(wf_kv_cache_check(&bad), WF_ERR_INVALID_ARG);
  bad = c;
  table[3] = 99; /* page outside the pool */
  EXPECT(wf_kv_cache_check(&bad), WF_ERR_INVALID_ARG);
  c = make_cache(WF_BF16, 1560, 21, 12, 128);

  /* planning: the Wan round (one chunk over the full window), a 1F1C wave of
   * three chunks, and a ragged small case */
  wf_attn_plan plan;
  int32_t q1[2] = {0, 4680};
  int64_t b1[1] = {0}, e1[1] = {32760};
  EXPECT(wf_chunk_attn_plan(&c, WF_BF16, 1, q1, b1, e1, 0, &plan), WF_OK);
  if (plan.kernel != WF_KERNEL_DMA_BF16 || plan.items != 19 * 12) { printf("plan %d %d\n", plan.kernel, plan.items); ++failures; }
  int32_t q3[4] = {0, 4680, 9360, 14040};
  int64_t b3[3] = {0, 0, 9360}, e3[3] = {23400, 28080, 32760};
  EXPECT(wf_chunk_attn_plan(&c, WF_BF16, 3, q3, b3, e3, 0, &plan), WF_OK);
  int32_t qr[4] = {0, 37, 37, 301};
  int64_t br[3] = {5, 0, 100}, er[3] = {6395, 1, 32760};
  EXPECT(wf_chunk_attn_plan(&c, WF_BF16, 3, qr, br, er, 0, &plan), WF_OK);
  /* a workspace needs the device */
  EXPECT(wf_chunk_attn_plan(&c, WF_BF16, 1, q1, b1, e1, 1u << 26, &plan), WF_ERR_HIP);
  /* invalid tables */
  EXPECT(wf_chunk_attn_plan(&c, WF_BF16, 0, q1, b1, e1, 0, &plan), WF_ERR_INVALID_ARG);
  EXPECT(wf_chunk_attn_plan(&c, WF_BF16, WF_MAX_CHUNKS + 1, q1, b1, e1, 0, &plan), WF_ERR_INVALID_ARG);
  int32_t qd[2] = {10, 20};
  EXPECT(wf_chunk_attn_plan(&c, WF_BF16, 1, qd, b1, e1, 0, &plan), WF_ERR_INVALID_ARG);
  int64_t be[1] = {100}, ee[1] = {100};
  EXPECT(wf_chunk_attn_plan(&c, WF_BF16, 1, q1, be, ee, 0, &plan), WF_ERR_RANGE);
  int64_t eo[1] = {32761};
  EXPECT(wf_chunk_attn_plan(&c, WF_BF16, 1, q1, b1, eo, 0, &plan), WF_ERR_RANGE);
  EXPECT(wf_chunk_attn_plan(&c, WF_F32, 1, q1, b1, e1, 0, &plan), WF_ERR_UNSUPPORTED);
  EXPECT(wf_chunk_attn_plan(&c, WF_BF16, 1, NULL, b1, e1, 0, &plan), WF_ERR_INVALID_ARG);

  /* attention: validation, then the launch (stubbed) */
  EXPECT(wf_chunk_attn_fwd(&c, NULL, WF_BF16, OBUF, NULL, 1, q1, b1, e1, 0.f, NULL, 0, NULL), WF_ERR_INVALID_ARG);
  EXPECT(wf_chunk_attn_fwd(&c, QBUF, WF_BF16, QBUF, NULL, 1, q1, b1, e1, 0.f, NULL, 0, NULL), WF_ERR_INVALID_ARG);
  EXPECT(wf_chunk_attn_fwd(&c, QBUF, WF_BF16, OBUF, NULL, 1, q1, b1, e1, 0.f, NULL, 0, NULL), WF_ERR_HIP);
  EXPECT(wf_chunk_attn_fwd(&c, QBUF, WF_BF16, OBUF, NULL, 3, q3, b3, e3, 0.125f, NULL, 0, NULL), WF_ERR_HIP);
  EXPECT(wf_chunk_attn_fwd(&c, QBUF, WF_BF16, OBUF, NULL, 1, q1, b1, e1, 0.f, OBUF + 1, 1u << 20, NULL),
         WF_ERR_INVALID_ARG); /* misaligned workspace */

  /* fp8 cache: plan and staged (small pages) paths */
  wf_kv_cache c8 = make_cache(WF_FP8_E4M3, 1560, 21, 40, 128);
  EXPECT(wf_kv_cache_check(&c8), WF_OK);
  EXPECT(wf_chunk_attn_plan(&c8, WF_BF16, 1, q1, b1, e1, 0, &plan), WF_OK);
  if (plan.kernel != WF_KERNEL_DMA_FP8) { printf("fp8 plan kernel %d\n", plan.kernel); ++failures; }
  wf_kv_cache c40 = make_cache(WF_FP8_E4M3, 40, 21, 2, 64);
  int64_t bs[1] = {3}, es[1] = {801};
  int32_t qs[2] = {0, 70};
  EXPECT(wf_chunk_attn_plan(&c40, WF_BF16, 1, qs, bs, es, 0, &plan), WF_OK);
  if (plan.kernel != WF_KERNEL_STAGED_FP8) { printf("staged plan kernel %d\n", plan.kernel); ++failures; }
  wf_kv_cache cf = make_cache(WF_F32, 64, 3, 2, 64);
  int64_t bf[1] = {0}, ef[1] = {192};
  int32_t qf[2] = {0, 64};
  EXPECT(wf_chunk_attn_plan(&cf, WF_F32, 1, qf, bf, ef, 0, &plan), WF_OK);
  if (plan.kernel != WF_KERNEL_F32) { printf("f32 plan kernel %d\n", plan.kernel); ++failures; }
  EXPECT(wf_chunk_attn_fwd(&cf, QBUF, WF_F32, OBUF, NULL, 1, qf, bf, ef, 0.f, NULL, 0, NULL), WF_ERR_HIP);

  /* append / evict */
  wf_kv_cache ca = make_cache(WF_BF16, 1560, 21, 12, 128);
  ca.end = 4680;
  EXPECT(wf_kv_append(&ca, 4680, 4680, QBUF, OBUF, NULL, NULL, NULL), WF_ERR_HIP);
  if (ca.end != 4680) { printf("append changed end on failure\n"); ++failures; }
  EXPECT(wf_kv_append(&ca, 9361, 10, QBUF, OBUF, NULL, NULL, NULL), WF_ERR_RANGE);
  EXPECT(wf_kv_append(&ca, 4680, 40000, QBUF, OBUF, NULL, NULL, NULL), WF_ERR_CAPACITY);
  EXPECT(wf_kv_append(&ca, 4680, 10, NULL, OBUF, NULL, NULL, NULL), WF_ERR_INVALID_ARG);
  EXPECT(wf_kv_append(&ca, 4680, 0, QBUF, OBUF, NULL, NULL, NULL), WF_OK);
  EXPECT(wf_kv_evict(&ca, 1560, 0, NULL), WF_OK);
  if (ca.start != 1560) { printf("evict start %lld\n", (long long)ca.start); ++failures; }
  EXPECT(wf_kv_evict(&ca, 5000, 0, NULL), WF_ERR_RANGE);
  EXPECT(wf_kv_evict(&ca, 1560, WF_EVICT_POISON, NULL), WF_ERR_HIP);
  EXPECT(wf_stream_copy(QBUF, OBUF, 0, NULL), WF_OK);
  EXPECT(wf_stream_copy(QBUF, OBUF, 24, NULL), WF_ERR_INVALID_ARG);
  EXPECT(wf_stream_copy(QBUF, QBUF, 32, NULL), WF_ERR_INVALID_ARG);
  EXPECT(wf_stream_copy(QBUF, OBUF, 32, NULL), WF_ERR_HIP); /* valid: reaches the (stub) launch */
  EXPECT(wf_kv_append_quantize(&c8, 32760, 1560, QBUF, OBUF, NULL), WF_ERR_CAPACITY);
  EXPECT(wf_kv_append_quantize(&c8, 0, 1560, QBUF, OBUF, NULL), WF_ERR_HIP); /* overwrite in place */
  wf_kv_cache cq = make_cache(WF_FP8_E4M3, 1560, 21, 40, 128);
  cq.end = 0;
  EXPECT(wf_kv_append_quantize(&cq, 0, 1000, QBUF, OBUF, NULL), WF_ERR_INVALID_ARG);
  EXPECT(wf_kv_append_quantize(&cq, 0, 1560, QBUF, OBUF, NULL), WF_ERR_HIP);
  uint64_t wsb = 0;
  EXPECT(wf_chunk_attn_workspace_bytes(&c, &wsb), WF_ERR_HIP);
  printf(failures ? "FAILED %d\n" : "OK\n", failures);
  return failures ? 1 : 0;
}
