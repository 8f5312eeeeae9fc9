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
