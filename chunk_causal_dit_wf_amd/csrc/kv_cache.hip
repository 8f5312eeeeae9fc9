// KV-cache append (page scatter) and evict-poison kernels for gfx950.
//
// Append writes a new chunk's K/V rows into the paged ring.  The operation is
// the cache write of KV-cached streaming generation: each new chunk's K/V
// enters the per-layer cache, and the timestep-0 re-run rewrites it with clean
// K/V (scope-causal-forcing README, "How It Works", steps 1-2; Wave Forcing
// abstract, cache-refresh stages).  It is a pure byte copy; the only work is
// the address mapping and, for V, the per-page transpose into the
// [head][dim][token] layout the attention kernel consumes.
//
// Roofline: HBM bandwidth.  Algorithmic bytes per token and head are
// 2 (K, V) * 2 (read + write) * D * esize.
#include "wf_internal.h"

namespace wf {

namespace {

constexpr int kTile = 64;      // tokens per block (8 groups of 8)
constexpr int kThreads = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// The new rows are read exactly once: nontemporal loads keep them from
// displacing cached lines (measured 19 % faster than plain loads on gfx950).
__device__ __forceinline__ uint4 load_stream(const char* a) {
  const u32x4 x = __builtin_nontemporal_load((const u32x4*)a);
  return make_uint4(x[0], x[1], x[2], x[3]);
}

__device__ __forceinline__ void locate(const PageMap& m, const FastDiv& divP, const FastDiv& divT,
                                       const int32_t* table, uint32_t rel, int32_t& page,
                                       int32_t& off) {
  uint32_t x = (uint32_t)m.base_off + rel;
  uint32_t pg = fastdiv(x, divP);
  off = (int32_t)(x - pg * divP.d);
  uint32_t s = (uint32_t)m.base_slot + pg;
  s -= fastdiv(s, divT) * divT.d;
  page = table[s];
}

// One block = one tile of one head.  Tiles are 64-token segments aligned to
// page offsets (the last tile of a page may be shorter), so a tile never
// leaves its page and the page is looked up once per block.  Every load of a
// thread is issued before its first store, so each thread keeps 2 * NR
// 16-byte loads in flight.
template <int ESIZE, int D>
__global__ __launch_bounds__(kThreads) void append_kernel(const AppendParams p) {
  constexpr int ROWB = D * ESIZE;           // bytes per token row of one head
  constexpr int CH = ROWB / 16;             // 16-byte chunks per row
  constexpr int CW = ROWB / 4;              // dwords per row
  constexpr int LSTRIDE = CW + 1;           // LDS row stride in dwords (conflict-free columns)
  constexpr int NR = kTile * CH / kThreads; // chunks per thread, per tensor
  static_assert(NR >= 1 && (kTile * CH) % kThreads == 0, "tile does not split evenly over the block");
  __shared__ uint32_t tile[kTile * LSTRIDE];

  const int tid = threadIdx.x;
  // Heads vary fastest along the grid: the blocks in flight together read one
  // contiguous stretch of the token-major source and write one page.
  const uint32_t bx = blockIdx.x;
  const uint32_t x = fastdiv(bx, p.divH);
  const int h = (int)(bx - x * (uint32_t)p.H);
  const uint32_t pk = fastdiv(x, p.div_tpp);             // page of the append (0: the page holding pos)
  const int t = (int)(x - pk * p.div_tpp.d);             // tile inside that page
  const int page_rel = (int)pk * p.P;                    // position of the page's first token
  const int off0 = kTile * t;                            // page offset of the tile's first token
  const int rel_lo = page_rel + off0;
  const int lo = max(rel_lo, p.lead);                    // valid positions [lo, hi)
  const int hi = min(min(rel_lo + kTile, page_rel + p.P), p.lead + p.n);
  if (lo >= hi) return;
  uint32_t slot = (uint32_t)p.map.base_slot + pk;
  slot -= fastdiv(slot, p.divT) * p.divT.d;
  const int64_t ph = (int64_t)p.table[slot] * p.H + h;   // (page, head) block of the cache

  const int64_t tok0 = (int64_t)(rel_lo - p.lead);       // index in k_new/v_new of the tile's first row
  const char* ksrc = (const char*)p.k_new + (tok0 * p.H + h) * ROWB;
  const char* vsrc = (const char*)p.v_new + (tok0 * p.H + h) * ROWB;
  char* kdst = (char*)p.k + (ph * p.P + off0) * ROWB;
  const uint32_t src_stride = (uint32_t)p.H * ROWB;

  uint4 kv[NR], vv[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int idx = tid + kThreads * r;
    const int tok = idx / CH, ch = idx % CH;
    const int rel = rel_lo + tok;
    kv[r] = vv[r] = make_uint4(0u, 0u, 0u, 0u);
    if (rel >= lo && rel < hi) {
      const uint32_t so = (uint32_t)tok * src_stride + ch * 16;
      kv[r] = load_stream(ksrc + so);
      vv[r] = load_stream(vsrc + so);
    }
  }
  // K rows: straight 16-byte copies into [page][h][off][D]; V rows staged in LDS.
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int idx = tid + kThreads * r;
    const int tok = idx / CH, ch = idx % CH;
    const int rel = rel_lo + tok;
    if (rel >= lo && rel < hi) {
      *(uint4*)(kdst + tok * ROWB + ch * 16) = kv[r];
      uint32_t* tl = tile + tok * LSTRIDE + ch * 4;
      tl[0] = vv[r].x; tl[1] = vv[r].y; tl[2] = vv[r].z; tl[3] = vv[r].w;
    }
  }
  // E4M3FN scales: appends are whole pages, so the first tile of page pk copies
  // that page's scales of head h.
  if (ESIZE == 1 && p.ks_new != nullptr && t == 0) {
    for (int b = tid; b < p.nblk; b += kThreads) {
      const int64_t s = ((int64_t)pk * p.H + h) * p.nblk + b;
      const int64_t d = ph * p.nblk + b;
      p.ks[d] = p.ks_new[s];
      p.vs[d] = p.vs_new[s];
    }
  }
  __syncthreads();

  // V: each lane owns (dword column c, token group g).  8 consecutive lanes
  // hold the 8 groups of one column, so they write one contiguous run of
  // 64 tokens of a [h][d][P] row.
  char* vdst = (char*)p.v + (ph * D * p.P + off0) * ESIZE;
  for (int idx = tid; idx < 8 * CW; idx += kThreads) {
    const int g = idx & 7, c = idx >> 3;
    const int relg = rel_lo + 8 * g;
    if (relg + 8 <= lo || relg >= hi) continue;
    uint32_t w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = tile[(8 * g + j) * LSTRIDE + c];
    const bool full = relg >= lo && relg + 8 <= hi;
    constexpr int NDW = 4 / ESIZE;  // d values per dword
#pragma unroll
    for (int b = 0; b < NDW; ++b) {
      const int d = c * NDW + b;
      char* vd = vdst + ((int64_t)d * p.P + 8 * g) * ESIZE;
      if constexpr (ESIZE == 4) {
        if (full) {
          *(uint4*)vd = make_uint4(w[0], w[1], w[2], w[3]);
          *(uint4*)(vd + 16) = make_uint4(w[4], w[5], w[6], w[7]);
        } else {
          for (int j = 0; j < 8; ++j)
            if (relg + j >= lo && relg + j < hi) ((uint32_t*)vd)[j] = w[j];
        }
      } else if constexpr (ESIZE == 2) {
        uint32_t e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) e[j] = b ? (w[j] >> 16) : (w[j] & 0xFFFFu);
        if (full) {
          *(uint4*)vd = make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16),
                                   e[6] | (e[7] << 16));
        } else {
          for (int j = 0; j < 8; ++j)
            if (relg + j >= lo && relg + j < hi) ((uint16_t*)vd)[j] = (uint16_t)e[j];
        }
      } else {
        uint32_t e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) e[j] = (w[j] >> (8 * b)) & 0xFFu;
        if (full) {
          *(uint2*)vd = make_uint2(e[0] | (e[1] << 8) | (e[2] << 16) | (e[3] << 24),
                                   e[4] | (e[5] << 8) | (e[6] << 16) | (e[7] << 24));
        } else {
          for (int j = 0; j < 8; ++j)
            if (relg + j >= lo && relg + j < hi) ((uint8_t*)vd)[j] = (uint8_t)e[j];
        }
      }
    }
  }
}

// Quantising append.  One block = one 128-token scale block of one new page
// and one head.  K and V rows (bf16) are read once into registers:
//   amax = max |x| over the block (fp32, exact), scale = amax / 448 and
//   r = 448 / amax (correctly rounded divisions; 1, 1 for an all-zero block),
//   code = e4m3(x * r): fp32 multiply, then v_cvt_pk_fp8_f32 (round to
//   nearest even, saturating at 448).
// K codes go straight to the page rows; V codes are transposed through LDS
// into the page's V^T rows.
constexpr int kQBlock = WF_SCALE_BLOCK;  // tokens per scale block

__device__ __forceinline__ float block_max(float x, float* red) {
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) m = fmaxf(m, red[w]);
  return m;
}

// 8 bf16 values times r -> 8 e4m3 codes (one 64-bit word).
__device__ __forceinline__ uint2 quant8(uint4 raw, float r) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  uint32_t out[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float a0 = __uint_as_float(w[2 * h] << 16) * r, a1 = __uint_as_float(w[2 * h] & 0xFFFF0000u) * r;
    const float a2 = __uint_as_float(w[2 * h + 1] << 16) * r, a3 = __uint_as_float(w[2 * h + 1] & 0xFFFF0000u) * r;
    uint32_t v = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
    out[h] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a2, a3, (int)v, true);
  }
  return make_uint2(out[0], out[1]);
}

__device__ __forceinline__ float absmax8(uint4 raw) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    m = fmaxf(m, fmaxf(fabsf(__uint_as_float(w[i] << 16)), fabsf(__uint_as_float(w[i] & 0xFFFF0000u))));
  return m;
}

template <int D>
__global__ __launch_bounds__(kThreads) void quant_append_kernel(const QuantAppendParams p) {
  constexpr int CH = D / 8;                  // 8-element chunks per row
  constexpr int NR = kQBlock * CH / kThreads;  // chunks per thread
  constexpr int VSTRIDE = kQBlock + 8;       // LDS bytes per V^T row (8-byte aligned rows)
  __shared__ float red[kThreads / 64];
  __shared__ __align__(16) uint8_t vt[D * VSTRIDE];
  const int tid = threadIdx.x;
  const int h = blockIdx.y;
  const int j = blockIdx.x / p.nblk;          // new page
  const int b = blockIdx.x - j * p.nblk;      // scale block inside the page
  const int t0 = kQBlock * b;
  const int nt = min(kQBlock, p.P - t0);      // tokens in this block
  int slot = p.base_slot + j;
  slot -= (slot / p.T) * p.T;
  const int64_t ph = (int64_t)p.table[slot] * p.H + h;
  const int64_t row0 = (int64_t)j * p.P + t0;  // first new row of the block
  const uint32_t src_stride = (uint32_t)p.H * D * 2;
  const char* ksrc = (const char*)p.k_new + (row0 * p.H + h) * D * 2;
  const char* vsrc = (const char*)p.v_new + (row0 * p.H + h) * D * 2;

  uint4 kr[NR], vr[NR];
  float km = 0.f, vm = 0.f;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int idx = tid + kThreads * r, t = idx / CH, c = idx % CH;
    kr[r] = vr[r] = make_uint4(0u, 0u, 0u, 0u);
    if (t < nt) {
      kr[r] = *(const uint4*)(ksrc + (uint32_t)t * src_stride + c * 16);
      vr[r] = *(const uint4*)(vsrc + (uint32_t)t * src_stride + c * 16);
    }
    km = fmaxf(km, absmax8(kr[r]));
    vm = fmaxf(vm, absmax8(vr[r]));
  }
  km = block_max(km, red);
  __syncthreads();
  vm = block_max(vm, red);
  const float kscale = km > 0.f ? __fdiv_rn(km, 448.f) : 1.f, kr_ = km > 0.f ? __fdiv_rn(448.f, km) : 1.f;
  const float vscale = vm > 0.f ? __fdiv_rn(vm, 448.f) : 1.f, vr_ = vm > 0.f ? __fdiv_rn(448.f, vm) : 1.f;
  if (tid == 0) {
    p.ks[ph * p.nblk + b] = kscale;
    p.vs[ph * p.nblk + b] = vscale;
  }
  char* kdst = (char*)p.k + (ph * p.P + t0) * D;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int idx = tid + kThreads * r, t = idx / CH, c = idx % CH;
    const uint2 kq = quant8(kr[r], kr_);
    const uint2 vq = quant8(vr[r], vr_);
    if (t < nt) *(uint2*)(kdst + (uint32_t)t * D + c * 8) = kq;
    const uint8_t* vb = (const uint8_t*)&vq;
#pragma unroll
    for (int e = 0; e < 8; ++e) vt[(c * 8 + e) * VSTRIDE + t] = vb[e];
  }
  __syncthreads();
  // V^T rows: for each dim d, nt consecutive bytes at page offset t0.
  char* vdst = (char*)p.v + ph * (int64_t)D * p.P + t0;
  const int words = (nt + 7) / 8;  // 8-byte words per row (nt is a multiple of 8)
  for (int idx = tid; idx < D * words; idx += kThreads) {
    const int d = idx / words, w = idx - d * words;
    *(uint2*)(vdst + (int64_t)d * p.P + 8 * w) = *(const uint2*)(vt + d * VSTRIDE + 8 * w);
  }
}

// Overwrite evicted rows with NaN codes (test aid).  Block = one token, all heads.
template <int ESIZE>
__global__ __launch_bounds__(kThreads) void poison_kernel(const PoisonParams p) {
  __shared__ int32_t table[WF_MAX_TABLE_LEN];
  for (int i = threadIdx.x; i < p.T; i += kThreads) table[i] = p.table[i];
  __syncthreads();
  const int tok = blockIdx.x;
  int32_t page, off;
  locate(p.map, p.divP, p.divT, table, (uint32_t)tok, page, off);
  for (int e = threadIdx.x; e < p.H * p.D; e += kThreads) {
    const int h = e / p.D, d = e - h * p.D;
    const int64_t ki = (((int64_t)page * p.H + h) * p.P + off) * p.D + d;
    const int64_t vi = (((int64_t)page * p.H + h) * p.D + d) * p.P + off;
    if constexpr (ESIZE == 4) {
      ((uint32_t*)p.k)[ki] = 0x7FC00000u;
      ((uint32_t*)p.v)[vi] = 0x7FC00000u;
    } else if constexpr (ESIZE == 2) {
      ((uint16_t*)p.k)[ki] = 0x7FC0u;
      ((uint16_t*)p.v)[vi] = 0x7FC0u;
    } else {
      ((uint8_t*)p.k)[ki] = 0x7Fu;
      ((uint8_t*)p.v)[vi] = 0x7Fu;
    }
  }
}

template <int ESIZE>
hipError_t launch_append_e(const AppendParams& p, int ntiles, hipStream_t s) {
  dim3 grid((uint32_t)ntiles * (uint32_t)p.H);
  if (p.D == 128)
    hipLaunchKernelGGL((append_kernel<ESIZE, 128>), grid, dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((append_kernel<ESIZE, 64>), grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_append(const QuantAppendParams& p, hipStream_t s) {
  const dim3 grid(p.npages * p.nblk, p.H);
  if (p.D == 128)
    hipLaunchKernelGGL(quant_append_kernel<128>, grid, dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL(quant_append_kernel<64>, grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_append(const AppendParams& p, int ntiles, hipStream_t s) {
  switch (p.esize) {
    case 4: return launch_append_e<4>(p, ntiles, s);
    case 2: return launch_append_e<2>(p, ntiles, s);
    default: return launch_append_e<1>(p, ntiles, s);
  }
}

hipError_t launch_poison(const PoisonParams& p, hipStream_t s) {
  dim3 grid(p.n);
  switch (p.esize) {
    case 4: hipLaunchKernelGGL(poison_kernel<4>, grid, dim3(kThreads), 0, s, p); break;
    case 2: hipLaunchKernelGGL(poison_kernel<2>, grid, dim3(kThreads), 0, s, p); break;
    default: hipLaunchKernelGGL(poison_kernel<1>, grid, dim3(kThreads), 0, s, p); break;
  }
  return hipGetLastError();
}

}  // namespace wf
