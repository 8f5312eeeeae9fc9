// Host side of the C ABI declared in include/wf_chunk_attn.h: argument
// validation, cache metadata, chunk scheduling and kernel launch.
//
// Every check runs before anything is enqueued, so a non-OK status leaves the
// device and the cache metadata untouched.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "copy_ref.h"
#include "wf_internal.h"

namespace {

thread_local std::string g_err;

wf_status fail(wf_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

wf_status ok() {
  g_err.clear();
  return WF_OK;
}

}  // namespace

wf_status wf::set_error(wf_status s, const char* msg) {
  g_err = msg;
  return s;
}

namespace {

int esize_of(int32_t dt) {
  switch (dt) {
    case WF_F32: return 4;
    case WF_BF16: return 2;
    case WF_FP8_E4M3: return 1;
    default: return 0;
  }
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlap(const void* a, uint64_t na, const void* b, uint64_t nb) {
  if (na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Structural checks of a cache description (not the live window).
wf_status check_layout(const wf_kv_cache* c) {
  if (c == nullptr) return fail(WF_ERR_INVALID_ARG, "cache is NULL");
  const int es = esize_of(c->kv_dtype);
  if (es == 0) return fail(WF_ERR_UNSUPPORTED, "kv_dtype %d is not F32, BF16 or FP8_E4M3", c->kv_dtype);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(WF_ERR_UNSUPPORTED, "head_dim %d not built (64 or 128)", c->head_dim);
  if (c->num_heads < 1 || c->num_heads > 4096)
    return fail(WF_ERR_INVALID_ARG, "num_heads %d out of range [1, 4096]", c->num_heads);
  if (c->page_size < 8 || c->page_size % 8 != 0)
    return fail(WF_ERR_UNSUPPORTED, "page_size %d must be a positive multiple of 8", c->page_size);
  if (c->table_len < 1 || c->table_len > WF_MAX_TABLE_LEN)
    return fail(WF_ERR_INVALID_ARG, "table_len %d out of range [1, %d]", c->table_len, WF_MAX_TABLE_LEN);
  if (c->num_pages < c->table_len)
    return fail(WF_ERR_INVALID_ARG, "num_pages %d < table_len %d", c->num_pages, c->table_len);
  if ((int64_t)c->table_len * c->page_size >= (int64_t)1 << 30)
    return fail(WF_ERR_UNSUPPORTED, "capacity table_len*page_size must stay below 2^30 tokens");
  if (c->page_table == nullptr) return fail(WF_ERR_INVALID_ARG, "page_table is NULL");
  std::vector<char> seen(c->num_pages, 0);
  for (int i = 0; i < c->table_len; ++i) {
    const int32_t pg = c->page_table[i];
    if (pg < 0 || pg >= c->num_pages)
      return fail(WF_ERR_INVALID_ARG, "page_table[%d] = %d outside [0, %d)", i, pg, c->num_pages);
    if (seen[pg]) return fail(WF_ERR_INVALID_ARG, "page_table names page %d twice", pg);
    seen[pg] = 1;
  }
  if (c->k == nullptr || c->v == nullptr) return fail(WF_ERR_INVALID_ARG, "cache k/v pointer is NULL");
  if (!aligned(c->k, 16) || !aligned(c->v, 16))
    return fail(WF_ERR_INVALID_ARG, "cache k/v pointers must be 16-byte aligned");
  if (c->kv_dtype == WF_FP8_E4M3) {
    if (c->k_scale == nullptr || c->v_scale == nullptr)
      return fail(WF_ERR_INVALID_ARG, "E4M3FN cache needs k_scale and v_scale");
    if (!aligned(c->k_scale, 4) || !aligned(c->v_scale, 4))
      return fail(WF_ERR_INVALID_ARG, "scale pointers must be 4-byte aligned");
  }
  const uint64_t kvb = (uint64_t)c->num_pages * c->num_heads * c->page_size * c->head_dim * es;
  if (overlap(c->k, kvb, c->v, kvb)) return fail(WF_ERR_INVALID_ARG, "cache k and v buffers overlap");
  return WF_OK;
}

wf_status check_window(const wf_kv_cache* c) {
  const int64_t cap = (int64_t)c->table_len * c->page_size;
  if (c->start < 0 || c->end < c->start || c->end > c->start + cap)
    return fail(WF_ERR_INVALID_ARG, "window [%lld, %lld) invalid for capacity %lld", (long long)c->start,
                (long long)c->end, (long long)cap);
  return WF_OK;
}

uint64_t kv_bytes_of(const wf_kv_cache* c) {
  return (uint64_t)c->num_pages * c->num_heads * c->page_size * c->head_dim * esize_of(c->kv_dtype);
}

wf::PageMap page_map(const wf_kv_cache* c, int64_t base) {
  wf::PageMap m;
  m.base_slot = (int32_t)((base / c->page_size) % c->table_len);
  m.base_off = (int32_t)(base % c->page_size);
  return m;
}

}  // namespace

extern "C" {

const char* wf_last_error(void) { return g_err.c_str(); }

const char* wf_version(void) { return "wf_chunk_attn 0.1 gfx950"; }

wf_status wf_kv_cache_check(const wf_kv_cache* c) {
  wf_status s = check_layout(c);
  if (s != WF_OK) return s;
  s = check_window(c);
  if (s != WF_OK) return s;
  return ok();
}

wf_status wf_kv_cache_bytes(const wf_kv_cache* c, uint64_t* kv_bytes, uint64_t* scale_bytes) {
  if (c == nullptr || kv_bytes == nullptr || scale_bytes == nullptr)
    return fail(WF_ERR_INVALID_ARG, "NULL argument");
  const int es = esize_of(c->kv_dtype);
  if (es == 0) return fail(WF_ERR_UNSUPPORTED, "kv_dtype %d unknown", c->kv_dtype);
  if (c->num_pages < 1 || c->num_heads < 1 || c->page_size < 1 || c->head_dim < 1)
    return fail(WF_ERR_INVALID_ARG, "sizes must be positive");
  *kv_bytes = kv_bytes_of(c);
  const uint64_t nblk = (c->page_size + WF_SCALE_BLOCK - 1) / WF_SCALE_BLOCK;
  *scale_bytes = c->kv_dtype == WF_FP8_E4M3 ? (uint64_t)c->num_pages * c->num_heads * nblk * 4 : 0;
  return ok();
}

wf_status wf_kv_append(wf_kv_cache* c, int64_t pos, int32_t n, const void* k_new, const void* v_new,
                       const float* k_scale_new, const float* v_scale_new, void* stream) {
  wf_status s = check_layout(c);
  if (s != WF_OK) return s;
  if ((s = check_window(c)) != WF_OK) return s;
  if (n < 0) return fail(WF_ERR_INVALID_ARG, "n = %d is negative", n);
  if (pos < c->start || pos > c->end)
    return fail(WF_ERR_RANGE, "append position %lld outside [start %lld, end %lld]", (long long)pos,
                (long long)c->start, (long long)c->end);
  const int64_t cap = (int64_t)c->table_len * c->page_size;
  if (pos + n > c->start + cap)
    return fail(WF_ERR_CAPACITY, "append [%lld, %lld) overruns live tokens (start %lld, capacity %lld)",
                (long long)pos, (long long)(pos + n), (long long)c->start, (long long)cap);
  if (n == 0) return ok();
  if (k_new == nullptr || v_new == nullptr) return fail(WF_ERR_INVALID_ARG, "k_new/v_new is NULL");
  if (!aligned(k_new, 16) || !aligned(v_new, 16))
    return fail(WF_ERR_INVALID_ARG, "k_new/v_new must be 16-byte aligned");
  const int es = esize_of(c->kv_dtype);
  const uint64_t nb = (uint64_t)n * c->num_heads * c->head_dim * es;
  const uint64_t kvb = kv_bytes_of(c);
  if (overlap(k_new, nb, c->k, kvb) || overlap(k_new, nb, c->v, kvb) || overlap(v_new, nb, c->k, kvb) ||
      overlap(v_new, nb, c->v, kvb))
    return fail(WF_ERR_INVALID_ARG, "new K/V overlap the cache buffers");
  const int nblk = (c->page_size + WF_SCALE_BLOCK - 1) / WF_SCALE_BLOCK;
  if (c->kv_dtype == WF_FP8_E4M3) {
    if (pos % c->page_size != 0 || n % c->page_size != 0)
      return fail(WF_ERR_INVALID_ARG, "E4M3FN appends must be whole pages (pos %lld, n %d, page %d)",
                  (long long)pos, n, c->page_size);
    if (k_scale_new == nullptr || v_scale_new == nullptr)
      return fail(WF_ERR_INVALID_ARG, "E4M3FN append needs k_scale_new and v_scale_new");
    if (!aligned(k_scale_new, 4) || !aligned(v_scale_new, 4))
      return fail(WF_ERR_INVALID_ARG, "scale pointers must be 4-byte aligned");
  }
  wf::AppendParams p;
  std::memset(&p, 0, sizeof(p));
  p.k_new = k_new;
  p.v_new = v_new;
  p.ks_new = c->kv_dtype == WF_FP8_E4M3 ? k_scale_new : nullptr;
  p.vs_new = c->kv_dtype == WF_FP8_E4M3 ? v_scale_new : nullptr;
  p.k = c->k;
  p.v = c->v;
  p.ks = c->k_scale;
  p.vs = c->v_scale;
  p.n = n;
  p.H = c->num_heads;
  p.D = c->head_dim;
  p.P = c->page_size;
  p.T = c->table_len;
  p.nblk = nblk;
  p.esize = es;
  p.lead = (int32_t)(pos % c->page_size);
  p.map = page_map(c, pos - p.lead);
  const int64_t tpp = (c->page_size + 63) / 64;
  p.div_tpp = wf::make_fastdiv((uint32_t)tpp);
  p.divH = wf::make_fastdiv((uint32_t)c->num_heads);
  p.divT = wf::make_fastdiv((uint32_t)c->table_len);
  std::memcpy(p.table, c->page_table, sizeof(int32_t) * c->table_len);
  const int64_t npages = ((int64_t)p.lead + n + c->page_size - 1) / c->page_size;
  if (npages * tpp * c->num_heads >= ((int64_t)1 << 31) || (int64_t)p.lead + n + 64 >= ((int64_t)1 << 31))
    return fail(WF_ERR_UNSUPPORTED, "append of %d tokens needs too many tiles", n);
  const int ntiles = (int)(npages * tpp);
  hipError_t e = wf::launch_append(p, ntiles, (hipStream_t)stream);
  if (e != hipSuccess) return fail(WF_ERR_HIP, "append launch failed: %s", hipGetErrorString(e));
  c->end = std::max(c->end, pos + n);
  return ok();
}

wf_status wf_kv_append_quantize(wf_kv_cache* c, int64_t pos, int32_t n, const void* k_new, const void* v_new,
                                void* stream) {
  wf_status s = check_layout(c);
  if (s != WF_OK) return s;
  if ((s = check_window(c)) != WF_OK) return s;
  if (c->kv_dtype != WF_FP8_E4M3) return fail(WF_ERR_UNSUPPORTED, "wf_kv_append_quantize needs an E4M3FN cache");
  if (n < 0) return fail(WF_ERR_INVALID_ARG, "n = %d is negative", n);
  if (pos < c->start || pos > c->end)
    return fail(WF_ERR_RANGE, "append position %lld outside [start %lld, end %lld]", (long long)pos,
                (long long)c->start, (long long)c->end);
  const int64_t cap = (int64_t)c->table_len * c->page_size;
  if (pos + n > c->start + cap)
    return fail(WF_ERR_CAPACITY, "append [%lld, %lld) overruns live tokens (start %lld, capacity %lld)",
                (long long)pos, (long long)(pos + n), (long long)c->start, (long long)cap);
  if (pos % c->page_size != 0 || n % c->page_size != 0)
    return fail(WF_ERR_INVALID_ARG, "quantising appends must be whole pages (pos %lld, n %d, page %d)",
                (long long)pos, n, c->page_size);
  if (n == 0) return ok();
  if (k_new == nullptr || v_new == nullptr) return fail(WF_ERR_INVALID_ARG, "k_new/v_new is NULL");
  if (!aligned(k_new, 16) || !aligned(v_new, 16))
    return fail(WF_ERR_INVALID_ARG, "k_new/v_new must be 16-byte aligned");
  const uint64_t nb = (uint64_t)n * c->num_heads * c->head_dim * 2;
  const uint64_t kvb = kv_bytes_of(c);
  if (overlap(k_new, nb, c->k, kvb) || overlap(k_new, nb, c->v, kvb) || overlap(v_new, nb, c->k, kvb) ||
      overlap(v_new, nb, c->v, kvb))
    return fail(WF_ERR_INVALID_ARG, "new K/V overlap the cache buffers");
  wf::QuantAppendParams p;
  std::memset(&p, 0, sizeof(p));
  p.k_new = k_new;
  p.v_new = v_new;
  p.k = c->k;
  p.v = c->v;
  p.ks = c->k_scale;
  p.vs = c->v_scale;
  p.npages = n / c->page_size;
  p.H = c->num_heads;
  p.D = c->head_dim;
  p.P = c->page_size;
  p.T = c->table_len;
  p.nblk = (c->page_size + WF_SCALE_BLOCK - 1) / WF_SCALE_BLOCK;
  p.base_slot = (int32_t)((pos / c->page_size) % c->table_len);
  std::memcpy(p.table, c->page_table, sizeof(int32_t) * c->table_len);
  if ((int64_t)p.npages * p.nblk >= ((int64_t)1 << 31))
    return fail(WF_ERR_UNSUPPORTED, "append of %d tokens needs too many blocks", n);
  hipError_t e = wf::launch_quant_append(p, (hipStream_t)stream);
  if (e != hipSuccess) return fail(WF_ERR_HIP, "quantising append launch failed: %s", hipGetErrorString(e));
  c->end = std::max(c->end, pos + n);
  return ok();
}

wf_status wf_stream_copy(const void* src, void* dst, uint64_t bytes, void* stream) {
  if (bytes == 0) return ok();
  if (src == nullptr || dst == nullptr) return fail(WF_ERR_INVALID_ARG, "stream copy: null pointer");
  if (bytes % 16 != 0 || ((uintptr_t)src | (uintptr_t)dst) % 16 != 0)
    return fail(WF_ERR_INVALID_ARG, "stream copy: size and pointers must be multiples of 16 bytes");
  const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
  if (a < b + bytes && b < a + bytes) return fail(WF_ERR_INVALID_ARG, "stream copy: buffers overlap");
  hipError_t e = wf::launch_stream_copy(src, dst, (int64_t)(bytes / 16), (hipStream_t)stream);
  if (e != hipSuccess) return fail(WF_ERR_HIP, "stream copy launch failed: %s", hipGetErrorString(e));
  return ok();
}

wf_status wf_kv_evict(wf_kv_cache* c, int32_t n, uint32_t flags, void* stream) {
  wf_status s = check_layout(c);
  if (s != WF_OK) return s;
  if ((s = check_window(c)) != WF_OK) return s;
  if (n < 0 || (int64_t)n > c->end - c->start)
    return fail(WF_ERR_RANGE, "cannot evict %d tokens from a window of %lld", n, (long long)(c->end - c->start));
  if (flags & ~WF_EVICT_POISON) return fail(WF_ERR_INVALID_ARG, "unknown evict flags 0x%x", flags);
  if ((flags & WF_EVICT_POISON) && n > 0) {
    wf::PoisonParams p;
    std::memset(&p, 0, sizeof(p));
    p.k = c->k;
    p.v = c->v;
    p.n = n;
    p.H = c->num_heads;
    p.D = c->head_dim;
    p.P = c->page_size;
    p.T = c->table_len;
    p.esize = esize_of(c->kv_dtype);
    p.map = page_map(c, c->start);
    p.divP = wf::make_fastdiv((uint32_t)c->page_size);
    p.divT = wf::make_fastdiv((uint32_t)c->table_len);
    std::memcpy(p.table, c->page_table, sizeof(int32_t) * c->table_len);
    hipError_t e = wf::launch_poison(p, (hipStream_t)stream);
    if (e != hipSuccess) return fail(WF_ERR_HIP, "poison launch failed: %s", hipGetErrorString(e));
  }
  c->start += n;
  return ok();
}

// Split schedule for the DMA kernel (see wf::SplitSched).  Used when every
// chunk has the same number S of key tiles and there are fewer items than
// resident blocks: each item's keys are cut into m parts (m items x parts fill
// the resident blocks, parts of at least kMinPart key tiles), and the blocks
// still idle take the last b key tiles of q parts each, b chosen so that A and
// B blocks finish together.  B parts are used only when they take at least
// 1 / (kMaxQ + 1) of a part: a smaller share does not pay for the extra
// prologues and partial results, and on a power-limited chip idle CUs are
// not free capacity (measured: 228 of 256 CUs busy ran at a 3 % higher clock
// than 254).  Returns false when the plain one-block-per-item schedule is used.
static bool plan_split(wf::AttnParams& p, int items, int resident) {
  constexpr int kMinPart = 32;  // key tiles per part
  constexpr int kMinB = 8;      // key tiles per B part
  constexpr int kMaxQ = 5;      // B parts per B block
  constexpr int kMaxParts = 8;  // the merge kernel holds 2 * kMaxParts partials per row
  const int S = p.chunk[0].nsteps;
  for (int i = 1; i < p.num_chunks; ++i)
    if (p.chunk[i].nsteps != S) return false;
  if (items >= resident) return false;
  wf::SplitSched sp;
  sp.S = S;
  sp.n = items;
  sp.tiles = items / p.H;
  sp.m = std::max(1, std::min({resident / items, S / kMinPart, kMaxParts}));
  const int na = items * sp.m;
  const int spare = resident - na;
  sp.b = 0;
  sp.q = 1;
  if (spare > 0) {
    sp.q = (na + spare - 1) / spare;
    sp.b = (S / sp.m) / (sp.q + 1);
    if (sp.b < kMinB || sp.q > kMaxQ) sp.b = 0;
  }
  if (sp.m == 1 && sp.b == 0) return false;
  p.sp = sp;
  return true;
}

wf_status wf_chunk_attn_workspace_bytes(const wf_kv_cache* c, uint64_t* bytes) {
  wf_status s = check_layout(c);
  if (s != WF_OK) return s;
  if (bytes == nullptr) return fail(WF_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = 0;
  if (c->kv_dtype == WF_F32) return ok();
  int blocks = 0;
  hipError_t e = c->kv_dtype == WF_BF16 ? wf::attn_dma_resident_blocks(c->head_dim, &blocks)
                                        : wf::attn_fp8_resident_blocks(c->head_dim, &blocks);
  if (e != hipSuccess) return fail(WF_ERR_HIP, "device query failed: %s", hipGetErrorString(e));
  *bytes = (uint64_t)2 * blocks * wf::ws_slot_floats(c->head_dim) * sizeof(float);
  return ok();
}

// Validation of the chunk tables and the whole launch plan of an attention
// call: kernel, item table, schedule and grid.  Needs the device (resident
// workgroup count) only when a workspace is given.  Fills p except for the
// q / o / lse / ws pointers.
static wf_status plan_attention(const wf_kv_cache* c, int32_t q_dtype, int32_t num_chunks, const int32_t* q_off,
                                const int64_t* kv_begin, const int64_t* kv_end, float softmax_scale,
                                uint64_t workspace_bytes, bool scratch_mode, wf::AttnParams& p, wf_attn_plan& L) {
  wf_status s = check_layout(c);
  if (s != WF_OK) return s;
  if ((s = check_window(c)) != WF_OK) return s;
  const int kvd = c->kv_dtype;
  const bool pair_ok = (q_dtype == WF_F32 && kvd == WF_F32) || (q_dtype == WF_BF16 && kvd == WF_BF16) ||
                       (q_dtype == WF_BF16 && kvd == WF_FP8_E4M3);
  if (!pair_ok)
    return fail(WF_ERR_UNSUPPORTED, "(q_dtype %d, kv_dtype %d) not built: use (F32,F32), (BF16,BF16) or "
                "(BF16,FP8_E4M3)", q_dtype, kvd);
  if (num_chunks < 1 || num_chunks > WF_MAX_CHUNKS)
    return fail(WF_ERR_INVALID_ARG, "num_chunks %d out of range [1, %d]", num_chunks, WF_MAX_CHUNKS);
  if (q_off == nullptr || kv_begin == nullptr || kv_end == nullptr)
    return fail(WF_ERR_INVALID_ARG, "chunk tables must not be NULL");
  if (q_off[0] != 0) return fail(WF_ERR_INVALID_ARG, "q_off[0] must be 0");
  for (int i = 0; i < num_chunks; ++i) {
    if (q_off[i + 1] < q_off[i]) return fail(WF_ERR_INVALID_ARG, "q_off must be non-decreasing (chunk %d)", i);
    if (!(c->start <= kv_begin[i] && kv_begin[i] < kv_end[i] && kv_end[i] <= c->end))
      return fail(WF_ERR_RANGE, "chunk %d key range [%lld, %lld) empty or outside the live window [%lld, %lld)",
                  i, (long long)kv_begin[i], (long long)kv_end[i], (long long)c->start, (long long)c->end);
  }
  const int64_t nq = q_off[num_chunks];
  if (nq * c->num_heads >= ((int64_t)1 << 31))
    return fail(WF_ERR_UNSUPPORTED, "too many query rows (%lld x %d heads)", (long long)nq, c->num_heads);
  if (!(std::isfinite(softmax_scale))) return fail(WF_ERR_INVALID_ARG, "softmax_scale is not finite");

  std::memset(&p, 0, sizeof(p));
  std::memset(&L, 0, sizeof(L));
  p.k = c->k;
  p.v = c->v;
  p.ks = c->k_scale;
  p.vs = c->v_scale;
  p.nq = (int32_t)nq;
  p.H = c->num_heads;
  p.P = c->page_size;
  p.T = c->table_len;
  p.nblk = (c->page_size + WF_SCALE_BLOCK - 1) / WF_SCALE_BLOCK;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)c->head_dim);
  p.scale_log2 = (float)((double)scale * 1.4426950408889634);
  p.divP = wf::make_fastdiv((uint32_t)c->page_size);
  p.divT = wf::make_fastdiv((uint32_t)c->table_len);
  std::memcpy(p.table, c->page_table, sizeof(int32_t) * c->table_len);
  // The DMA kernels address a key tile as at most two page runs with 32-bit
  // byte offsets: they take caches with pages of at least one tile (64 keys)
  // and under 4 GiB.  Everything else goes to the register-staged kernel.
  const uint64_t kvb = kv_bytes_of(c);
  const bool use_dma = kvd == WF_BF16 && c->page_size >= 64 && kvb < ((uint64_t)1 << 32);
  bool use_fp8 = kvd == WF_FP8_E4M3 && c->page_size >= 64 && kvb < ((uint64_t)1 << 32);
  for (int i = 0; i < num_chunks && use_fp8; ++i)
    use_fp8 = (kv_begin[i] % 8) + (kv_end[i] - kv_begin[i]) <= (int64_t)8 * wf::kFp8MaxGroups;
  L.kernel = q_dtype == WF_F32 ? WF_KERNEL_F32
             : use_dma        ? WF_KERNEL_DMA_BF16
             : use_fp8        ? WF_KERNEL_DMA_FP8
             : kvd == WF_BF16 ? WF_KERNEL_STAGED_BF16
                              : WF_KERNEL_STAGED_FP8;

  // Longest-processing-time-first order: chunks with the most (query x key) work are issued first.
  std::vector<int> order;
  for (int i = 0; i < num_chunks; ++i)
    if (q_off[i + 1] > q_off[i]) order.push_back(i);
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
    const int64_t wa = (int64_t)(q_off[a + 1] - q_off[a]) * (kv_end[a] - kv_begin[a]);
    const int64_t wb = (int64_t)(q_off[b + 1] - q_off[b]) * (kv_end[b] - kv_begin[b]);
    return wa > wb;
  });
  const bool dma = L.kernel == WF_KERNEL_DMA_BF16 || L.kernel == WF_KERNEL_DMA_FP8;
  const int block_m = q_dtype == WF_F32 ? wf::kBlockMF32 : dma ? wf::kBlockMDma : wf::kBlockMStaged;
  int64_t items = 0;
  int nc = 0;
  for (int i : order) {
    wf::ChunkDesc& d = p.chunk[nc++];
    d.q_begin = q_off[i];
    d.q_len = q_off[i + 1] - q_off[i];
    d.ntiles = (d.q_len + block_m - 1) / block_m;
    d.item0 = (int32_t)items;
    d.lead = (int32_t)(kv_begin[i] % 8);
    d.nkeys = (int32_t)(kv_end[i] - kv_begin[i]);
    d.map = page_map(c, kv_begin[i] - d.lead);
    d.nsteps = (int32_t)((d.lead + d.nkeys + 63) / 64);
    items += (int64_t)d.ntiles * c->num_heads;
  }
  p.num_chunks = nc;
  p.num_items = (int32_t)items;
  L.items = (int32_t)items;
  L.rows_per_item = block_m;
  L.grid = (int32_t)items;
  L.schedule = WF_SCHED_PER_TILE;
  L.parts = 1;
  L.tails_per_block = 0;
  L.tail_tiles = 0;
  if (items == 0 || !dma || workspace_bytes == 0) return ok();

  int resident = 0;
  hipError_t e = L.kernel == WF_KERNEL_DMA_BF16 ? wf::attn_dma_resident_blocks(c->head_dim, &resident)
                                                : wf::attn_fp8_resident_blocks(c->head_dim, &resident);
  if (e != hipSuccess) return fail(WF_ERR_HIP, "device query failed: %s", hipGetErrorString(e));
  const uint64_t slot_bytes = (uint64_t)wf::ws_slot_floats(c->head_dim) * sizeof(float);
  const uint64_t need = (uint64_t)2 * resident * slot_bytes;
  if (!scratch_mode && workspace_bytes < need)
    return fail(WF_ERR_INVALID_ARG, "workspace of %llu bytes is smaller than the %llu required",
                (unsigned long long)workspace_bytes, (unsigned long long)need);
  if (plan_split(p, (int)items, resident)) {
    // Slots written: A parts n m, and as many B parts when tails are taken.
    const uint64_t used = (uint64_t)(p.sp.b > 0 ? 2 : 1) * p.sp.n * p.sp.m * slot_bytes;
    if (scratch_mode && used > workspace_bytes)
      return fail(WF_ERR_CAPACITY, "the split schedule of this call needs %llu bytes of scratch; the "
                  "allocation-free entry point holds %llu", (unsigned long long)used,
                  (unsigned long long)workspace_bytes);
    L.schedule = WF_SCHED_SPLIT;
    L.parts = p.sp.m;
    L.tail_tiles = p.sp.b;
    L.tails_per_block = p.sp.b > 0 ? p.sp.q : 0;
    L.grid = p.sp.n * p.sp.m + (p.sp.b > 0 ? (p.sp.n * p.sp.m + p.sp.q - 1) / p.sp.q : 0);
  }
  return ok();
}

wf_status wf_chunk_attn_plan(const wf_kv_cache* c, int32_t q_dtype, int32_t num_chunks, const int32_t* q_off,
                             const int64_t* kv_begin, const int64_t* kv_end, uint64_t workspace_bytes,
                             wf_attn_plan* plan) {
  if (plan == nullptr) return fail(WF_ERR_INVALID_ARG, "plan is NULL");
  wf::AttnParams p;
  wf_attn_plan L;
  wf_status s = plan_attention(c, q_dtype, num_chunks, q_off, kv_begin, kv_end, 0.f, workspace_bytes, false, p, L);
  if (s != WF_OK) return s;
  *plan = L;
  return ok();
}

wf_status wf_chunk_attn_fwd(const wf_kv_cache* c, const void* q, int32_t q_dtype, void* o, float* lse,
                            int32_t num_chunks, const int32_t* q_off, const int64_t* kv_begin,
                            const int64_t* kv_end, float softmax_scale, void* workspace,
                            uint64_t workspace_bytes, void* stream) {
  return wf::attn_fwd_impl(c, q, q_dtype, o, lse, num_chunks, q_off, kv_begin, kv_end, softmax_scale, workspace,
                           workspace_bytes, false, stream);
}

}  // extern "C"

// Attention with a caller workspace (scratch_mode false) or the library's own
// scratch array (scratch_mode true: the split schedule may use up to
// workspace_bytes of it; no minimum size is required).
wf_status wf::attn_fwd_impl(const wf_kv_cache* c, const void* q, int32_t q_dtype, void* o, float* lse,
                            int32_t num_chunks, const int32_t* q_off, const int64_t* kv_begin,
                            const int64_t* kv_end, float softmax_scale, void* workspace, uint64_t workspace_bytes,
                            bool scratch_mode, void* stream) {
  if ((workspace == nullptr) != (workspace_bytes == 0))
    return fail(WF_ERR_INVALID_ARG, "workspace and workspace_bytes must both be set or both be 0");
  if (workspace != nullptr && !aligned(workspace, 256))
    return fail(WF_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  wf::AttnParams p;
  wf_attn_plan L;
  wf_status s = plan_attention(c, q_dtype, num_chunks, q_off, kv_begin, kv_end, softmax_scale, workspace_bytes,
                               scratch_mode, p, L);
  if (s != WF_OK) return s;
  const int64_t nq = p.nq;
  if (nq == 0) return ok();
  if (q == nullptr || o == nullptr) return fail(WF_ERR_INVALID_ARG, "q/o is NULL");
  if (!aligned(q, 16) || !aligned(o, 16)) return fail(WF_ERR_INVALID_ARG, "q/o must be 16-byte aligned");
  if (lse != nullptr && !aligned(lse, 4)) return fail(WF_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  const uint64_t qb = (uint64_t)nq * c->num_heads * c->head_dim * esize_of(q_dtype);
  const uint64_t kvb = kv_bytes_of(c);
  if (overlap(o, qb, q, qb) || overlap(o, qb, c->k, kvb) || overlap(o, qb, c->v, kvb))
    return fail(WF_ERR_INVALID_ARG, "o overlaps q or the cache");
  const uint64_t lb = lse != nullptr ? (uint64_t)nq * c->num_heads * 4 : 0;
  if (lse != nullptr) {
    if (overlap(lse, lb, o, qb) || overlap(lse, lb, q, qb) || overlap(lse, lb, c->k, kvb) ||
        overlap(lse, lb, c->v, kvb))
      return fail(WF_ERR_INVALID_ARG, "lse overlaps q, o or the cache");
  }
  if (workspace != nullptr) {
    if (overlap(workspace, workspace_bytes, q, qb) || overlap(workspace, workspace_bytes, o, qb) ||
        overlap(workspace, workspace_bytes, c->k, kvb) || overlap(workspace, workspace_bytes, c->v, kvb) ||
        (lse != nullptr && overlap(workspace, workspace_bytes, lse, lb)))
      return fail(WF_ERR_INVALID_ARG, "workspace overlaps another argument");
  }
  if (L.items == 0) return ok();
  p.q = q;
  p.o = o;
  p.lse = lse;
  if (L.schedule == WF_SCHED_SPLIT) p.ws = (float*)workspace;

  hipError_t e;
  switch (L.kernel) {
    case WF_KERNEL_F32: e = wf::launch_attn_f32(p, c->head_dim, (hipStream_t)stream); break;
    case WF_KERNEL_DMA_BF16: e = wf::launch_attn_bf16_dma(p, c->head_dim, L.grid, (hipStream_t)stream); break;
    case WF_KERNEL_DMA_FP8: e = wf::launch_attn_fp8_dma(p, c->head_dim, L.grid, (hipStream_t)stream); break;
    case WF_KERNEL_STAGED_BF16: e = wf::launch_attn_bf16_staged(p, c->head_dim, (hipStream_t)stream); break;
    default: e = wf::launch_attn_fp8kv(p, c->head_dim, (hipStream_t)stream); break;
  }
  if (e == hipSuccess && p.ws != nullptr) e = wf::launch_attn_merge(p, c->head_dim, (hipStream_t)stream);
  if (e != hipSuccess) return fail(WF_ERR_HIP, "attention launch failed: %s", hipGetErrorString(e));
  return ok();
}


