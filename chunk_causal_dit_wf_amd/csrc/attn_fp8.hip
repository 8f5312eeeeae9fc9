// Chunk-wise causal attention over an E4M3FN KV cache with fp8 MFMA (gfx950).
//
// Operation (Wave Forcing abstract; hellomarvisaitoday Wave Forcing article,
// first paragraph): the query rows of chunk c attend to the logical keys
// [kv_begin[c], kv_end[c]) of a paged ring KV cache whose K and V are stored
// as OCP E4M3FN codes with one fp32 scale per (page, head, 128-token block):
//   K[j] = decode(k8[j]) * ks(j),  V[j] = decode(v8[j]) * vs(j).
//
// Both products run on V_MFMA_F32_32X32X64_F8F6F4 (e4m3 x e4m3, fp32
// accumulate), twice the bf16 rate:
//   S^T = K8 Q8^T: Q is quantised in the kernel, one scale per query row
//       (sq = amax / 448), as two E4M3FN terms: hi = e4m3(q / sq) and
//       lo = e4m3(q / sq - hi), both multiplied by the same K fragment into
//       one accumulator.  hi + lo carries q to within 2^-8 |q| + 2^-10 sq
//       (bf16-like precision), so scores keep the accuracy of a bf16 Q at
//       the cost of one more fp8 MFMA per 64-dim block.  The score is
//       acc * ks(key) * sq.
//   O^T += V8^T P8^T: P is quantised to e4m3 after folding in the V scale,
//       P'(key) = P(key) * 1.75 * vs(key) / vs_max, where vs_max is the
//       largest V scale of the segment's key range and 1.75 = 448 / 2^8, so
//       that P' <= 448 while P <= 2^8.  O = O_acc * vs_max / 1.75.
// Per-key factors are per 8-key group: a lane's 16 keys of a 32-key
// half-tile are two groups, so every factor is a per-register constant, and
// the V factor rides in the exponent's bias (no extra VALU per element).
// The row sums are taken from the fp32 P' before quantisation, weighted back
// by 2^-bias per group.
//
// Schedule: the two-group ping-pong of the bf16 LDS-DMA kernel.  One
// workgroup = 8 waves (2 per SIMD) = 256 query rows of one head of one
// chunk; waves 0-3 (group 0) and 4-7 (group 1) run the same program one phase
// apart, so while one wave of a SIMD issues the matrix products of a 64-key
// tile (phase M), the other runs the softmax of its next tile on the vector
// unit (phase V).  Every phase ends with a workgroup barrier; the wave in
// phase V runs at the higher wave priority (prio).  Fragment reads of a steady
// phase M run three products ahead of their use.
//   M(t): S(t+1) = K(t+1) Q^T (hi and lo terms, 4 KS MFMAs) and
//         O^T += V(t)^T P(t) (D / 32 MFMAs).  On steady tiles the first step
//         of the softmax, x = S f + c - m, runs between the P V products:
//         vector work moved out of phase V, the longer one.
//   V(t): the wave's share of the tile loads, then P'(t+1) = exp2(x) (e4m3
//         packing, group sums): the reference point m of the online softmax
//         moves only when a lane's sum of P' exceeds 448 (then every P' could
//         still saturate), to the exact row maximum, with O and l rescaled;
//         the common path takes no row maximum.
// Tiles stream through a ring of three LDS stages (stage t in slot
// (t + 1) % 3 holds K(t+1) and V(t)^T), filled by buffer LDS-DMA: group 1
// loads K tiles four tiles ahead, group 0 V^T tiles two tiles ahead.  K rows
// are padded to D + 16 bytes and permuted so that a lane half holds 16
// consecutive keys; V^T rows hold 64 keys plus 16 bytes.  V^T columns of keys
// outside the chunk's range are zeroed in LDS (0 * NaN would poison P V).
//
// Roofline: dense fp8 MFMA.  Algorithmic flops per visible (query, key) pair
// and head are 4 * head_dim.
#include <utility>

#include "attn_common.h"

namespace wf {
namespace {
namespace dma8 {

constexpr int NW = 8;          // waves per workgroup
constexpr int NTD = 64 * NW;   // threads per workgroup
constexpr int NG = 4;          // waves per group (one per SIMD)
constexpr int BMD = 32 * NW;   // query rows per workgroup
constexpr int TK = kTileKeys;  // keys per tile
constexpr float kPScale = 1.75f;
constexpr float kE4M3Max = 448.f;
static_assert(BMD == kBlockMDma, "host and kernel disagree on the block size");

typedef int i32x4 __attribute__((ext_vector_type(4)));

template <int D>
struct Geo {
  static constexpr int KROW = D + 16;                     // LDS bytes per K row (padded)
  static constexpr int KDMA = (TK * KROW + 1023) / 1024;  // 16-byte DMA instructions per K tile
  static constexpr int KTILE = KDMA * 1024;
  static constexpr int VROW = TK + 16;                    // LDS bytes per V^T row (padded)
  static constexpr int VDMA = (D * VROW + 1023) / 1024;   // 16-byte DMA instructions per V^T tile
  static constexpr int VTILE = VDMA * 1024;
  static constexpr int V4DMA = (D * VROW + 255) / 256;    // 4-byte DMA instructions per V^T tile
  static constexpr int KPW = (KDMA + NG - 1) / NG;        // K instructions per group-1 wave
  static constexpr int VPW = (VDMA + NG - 1) / NG;        // V instructions per group-0 wave
  static constexpr int PW = KPW > VPW ? KPW : VPW;        // DMA instructions per wave and tile
  static constexpr int V4PW = (V4DMA + NG - 1) / NG;      // 4-byte V instructions per wave (page break)
  static constexpr int KS = D / 64;                       // 64-deep k-blocks of Q K^T
  static constexpr int DB = D / 32;                       // 32-row d-blocks of P V
};

// Every wave issues exactly PW 16-byte DMA instructions per in-page tile: wave
// gw of a group takes instructions gw, gw + 4, ... of the tile and repeats its
// first one (same source, destination and bytes) where it runs out.
template <int D>
__device__ __forceinline__ int inst_of(int group, int gw, int r) {
  const int n = gw + NG * r;
  return n < (group == 1 ? Geo<D>::KDMA : Geo<D>::VDMA) ? n : gw;
}

// Per-lane source offsets (relative to the tile's first key in its page) and,
// for K, the tile-relative key of the lane's chunk (page select at a break).
template <int D>
struct Plan {
  uint32_t off[Geo<D>::PW];
  int32_t key[Geo<D>::PW];
};

template <int D>
__device__ __forceinline__ Plan<D> make_plan(int group, int gw, int lane, int P) {
  using G = Geo<D>;
  Plan<D> pl;
#pragma unroll
  for (int r = 0; r < G::PW; ++r) {
    const int n = inst_of<D>(group, gw, r);
    const int y = 1024 * n + 16 * lane;
    if (group == 1) {
      const int row = y / G::KROW, pc = (y % G::KROW) / 16;
      const bool data = row < TK && pc < D / 16;
      const int q = row & 31;  // row inside its 32-key half: key 16 h + 4 j + i at row 8 j + 4 h + i
      const int key = (row & 32) + 16 * ((q >> 2) & 1) + 4 * (q >> 3) + (q & 3);
      pl.key[r] = data ? key : 0;
      pl.off[r] = data ? (uint32_t)(key * D + pc * 16) : 0u;
    } else {
      const int d = y / G::VROW, pc = (y % G::VROW) / 16;
      const bool data = d < D && pc < 4;
      pl.key[r] = 0;
      pl.off[r] = data ? (uint32_t)(d * P + pc * 16) : 0u;
    }
  }
  return pl;
}

// Buffer resource over a whole cache (K or V): raw addressing, byte offsets
// below 2^32 (the host sends only caches under 4 GiB here).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t cache_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0xFFFFFFFFu, 0x00020000);
}

// LDS-DMA through a buffer resource: lane L's bytes at voff + soff land at
// lds + 16 L (or + 4 L).
__device__ __forceinline__ void dma16b(__amdgpu_buffer_rsrc_t rs, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void dma4b(__amdgpu_buffer_rsrc_t rs, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 4, voff, 0u, 0, 0);
}

// DMA the K tile (64 keys) at cursor c into kt (group 1).  A 16-byte chunk is
// part of one key's row, so at a page break each lane selects its page.
template <int D>
__device__ __forceinline__ void dma_k(const AttnParams& p, __amdgpu_buffer_rsrc_t rs, const Cursor& c,
                                      const Plan<D>& pl, char* kt, int gw) {
  using G = Geo<D>;
  if (p.P - c.off >= TK) {
    const uint32_t soff = __builtin_amdgcn_readfirstlane(c.k0 + (uint32_t)c.off * D);
#pragma unroll
    for (int r = 0; r < G::PW; ++r) dma16b(rs, kt + 1024 * inst_of<D>(1, gw, r), pl.off[r], soff);
    return;
  }
  const RunGeom g = run_geom<D, 1>(p, c);
#pragma unroll
  for (int r = 0; r < G::PW; ++r)
    dma16b(rs, kt + 1024 * inst_of<D>(1, gw, r), (pl.key[r] < g.split ? g.kb0 : g.kb1) + pl.off[r], 0u);
}

// DMA the V^T tile (64 keys) at cursor c into vt (group 0).  A 16-byte chunk
// holds 16 keys of one V^T row and can straddle a page break (pages are
// multiples of 8 keys), so the tile that crosses a page moves in 4-byte
// pieces (4 keys, never straddling): V4PW instructions instead of PW.
template <int D>
__device__ __forceinline__ void dma_v(const AttnParams& p, __amdgpu_buffer_rsrc_t rs, const Cursor& c,
                                      const Plan<D>& pl, char* vt, int gw, int lane) {
  using G = Geo<D>;
  if (p.P - c.off >= TK) {
    const uint32_t soff = __builtin_amdgcn_readfirstlane(c.v0 + (uint32_t)c.off);
#pragma unroll
    for (int r = 0; r < G::PW; ++r) dma16b(rs, vt + 1024 * inst_of<D>(0, gw, r), pl.off[r], soff);
    return;
  }
  const RunGeom g = run_geom<D, 1>(p, c);
  // Per-lane offsets are recomputed here (an opaque copy of the lane index keeps
  // the compiler from holding them in registers across the tile loop).
  int ln = lane;
  asm volatile("" : "+v"(ln));
#pragma unroll
  for (int r = 0; r < G::V4PW; ++r) {
    const int n = min(gw + NG * r, G::V4DMA - 1);  // the last wave repeats the final piece
    const int y = 256 * n + 4 * ln;
    const int d = y / G::VROW, b = y - d * G::VROW;
    const bool data = d < D && b < TK;
    const uint32_t off = data ? (b < g.split ? g.vb0 : g.vb1) + (uint32_t)(d * p.P + b) : g.vb0;
    dma4b(rs, vt + 256 * n, off);
  }
}

// Zero the keys of V^T tile t (in LDS) that lie outside [lo, hi) (all threads).
template <int D>
__device__ __forceinline__ void zero_v_outside(char* vt, int t, int lo, int hi) {
  for (int idx = threadIdx.x; idx < D * 4; idx += NTD) {
    const int d = idx >> 2, c = idx & 3;
    const int rel = t * TK + 16 * c;
    if (rel >= lo && rel + 16 <= hi) continue;
    // Keys rel + e with e in [ka, kb) stay; their bytes are kept by a mask
    // built from the bit range (no per-key compares: sixteen per-lane key
    // constants would be hoisted out of the tile loop and spilled).
    const int ka = min(max(lo - rel, 0), 16), kb = min(max(hi - rel, 0), 16);
    const uint32_t keep = kb > ka ? (((1u << kb) - 1u) & ~((1u << ka) - 1u)) : 0u;
    uint4* a = (uint4*)(vt + d * Geo<D>::VROW + 16 * c);
    const uint4 v = *a;
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t n = (keep >> (4 * q)) & 0xFu;        // bit j: byte j of word q stays
      w[q] &= ((n * 0x00204081u) & 0x01010101u) * 0xFFu;  // bit j -> byte j
    }
    *a = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Wave priority on the SIMD: the wave in its softmax phase (a long vector
// stream) issues ahead of the wave in its matrix phase (one product per
// 32-64 cycles, which tolerates a late issue).  At equal priority the older
// wave of each SIMD's pair issued first in both of its phases, and the other
// group's phases ran 10-20 % longer (per-phase cycle stamps of an
// instrumented build); with it the Wan-round kernel runs about 3 % faster,
// the 14B fp8 one about 1 %.
__device__ __forceinline__ void prio(int level) {
  __builtin_amdgcn_sched_barrier(0);
  if (level) __builtin_amdgcn_s_setprio(1); else __builtin_amdgcn_s_setprio(0);
  __builtin_amdgcn_sched_barrier(0);
}

// Workgroup barrier that leaves outstanding loads in flight (each wave waits
// for its own DMA before it); scheduling barriers keep each phase's
// instructions on their side.
__device__ __forceinline__ void barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// 32 bytes (two 16-byte LDS reads) as an MFMA fp8 operand.
__device__ __forceinline__ i32x8 lds16x2(const char* a, int gap) {
  const i32x4 lo = *(const i32x4*)a;
  const i32x4 hi = *(const i32x4*)(a + gap);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
// K fragment of half h, k-block kb: LDS row 32 h + lq, dims 64 kb + 32 hf + [0, 32) (kx covers lq, hf).
template <int D>
__device__ __forceinline__ i32x8 k_frag(const char* kt, int kx, int h, int kb) {
  return lds16x2(kt + h * 32 * Geo<D>::KROW + kx + 64 * kb, 16);
}
// V fragment of d-block db: V^T row 32 db + lq, keys 16 hf + [0, 16) and 32 + 16 hf + [0, 16).
template <int D>
__device__ __forceinline__ i32x8 v_frag(const char* vt, int vx, int db) {
  return lds16x2(vt + vx + db * 32 * Geo<D>::VROW, 32);
}

__device__ __forceinline__ f32x16 mfma8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma8z(const i32x8& a, const i32x8& b) {
  f32x16 z;
#pragma unroll
  for (int e = 0; e < 16; ++e) z[e] = 0.f;
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, z, 0, 0, 0, 0, 0, 0);
}

// f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>), unrolled at compile time.
template <typename F, int... I>
__device__ __forceinline__ void static_for_seq(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_seq(f, std::make_integer_sequence<int, N>{});
}

// Per-key factors of the 8-key groups a lane holds in one tile: group
// 4 h + 2 hf + j (half h, j = 0, 1).  tab[g] = (ks, c, 2^-c, 0): K scale, V
// bias c = log2(1.75 vs / vs_max) and its weight for the row sum.
struct Factors {
  float f[4], c[4], w[4];  // index 2 h + j
};
__device__ __forceinline__ Factors factors(const float4* tab, int t, int hf, float qs) {
  Factors F;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float4 e = tab[8 * t + 4 * h + 2 * hf + j];
      F.f[2 * h + j] = e.x * qs;
      F.c[2 * h + j] = e.y;
      F.w[2 * h + j] = e.z;
    }
  return F;
}

// Phase M of one 64-key tile.  QK: S(t+1) = K(t+1) (Qhi + Qlo)^T from the K
// tile at kt into s[0] (keys 0..31) and s[1] (32..63).  PV: O^T += V(t)^T
// P'(t) from the V^T tile at vt.  Order per k-block kb: the hi products of
// both halves, PV product 2 kb, the lo products of both halves, PV product
// 2 kb + 1 (D / 32 = 2 D / 64 PV products in all).  Each accumulator's
// products are at least two MFMAs apart.  Every index is a compile-time
// constant.
//
// XPRE (steady tiles, both products): every Q K^T product first, then the
// P V products, then -- while those run on the matrix pipe -- the first step
// of the softmax, x = S f_q + c_q - m, in place in s (F: the factors of the
// tile of S, m: the current reference point).  This moves a quarter of the
// softmax's vector work from phase V, which is the longer one, into phase M.
template <int D, bool QK, bool PV, bool XPRE = false>
__device__ __forceinline__ void m_phase(f32x16 (&s)[2], f32x16 (&o)[D / 32], const i32x8 (&qh)[D / 64],
                                        const i32x8 (&ql)[D / 64], const i32x8& p8, const char* kt,
                                        const char* vt, int kx, int vx, const Factors* F = nullptr,
                                        float m = 0.f) {
  constexpr int KS = D / 64;
  constexpr int DB = D / 32;
  static_assert(DB == 2 * KS, "two PV products per k-block");
  static_assert(!XPRE || (QK && PV), "XPRE needs both products");
  if constexpr (XPRE) {
    // Products in issue order: Q K^T (half h, k-block kb, term) as
    // [hi h0, hi h1, lo h0, lo h1] per kb, then the DB P V products.  Every
    // fragment read is issued PF products before the product that first uses it.
    constexpr int NQ = 4 * KS;
    constexpr int NL = 2 * KS + DB;  // fragment reads: K (h, kb) in kb-major order, then V (db)
    constexpr int PF = 3;
    i32x8 kf[2][KS];
    i32x8 vf[DB];
    auto first_use = [](int j) { return j < 2 * KS ? 4 * (j / 2) + j % 2 : NQ + (j - 2 * KS); };
    auto issue_for = [&](auto I) {  // the reads due before product I
      constexpr int i = decltype(I)::value;
      static_for<NL>([&](auto J) {
        constexpr int j = decltype(J)::value;
        constexpr int due = first_use(j) - PF;
        if constexpr ((i == 0 && due <= 0) || (i > 0 && due == i)) {
          if constexpr (j < 2 * KS)
            kf[j % 2][j / 2] = k_frag<D>(kt, kx, j % 2, j / 2);
          else
            vf[j - 2 * KS] = v_frag<D>(vt, vx, j - 2 * KS);
        }
      });
    };
    float cm[4];
    // With four P V products the first three are each followed by the x of
    // PER elements of S (the last product then runs while the phase ends);
    // with two, each by 16.  Either way no x reads s[h] sooner than two
    // products after the last Q K^T product into s[h]: a VALU read closer to
    // such a product has returned its old value on this hardware, although
    // the compiler's wait states allow it.
    constexpr int PER = DB > 2 ? (32 + DB - 2) / (DB - 1) : 32 / DB;
    static_for<NQ + DB>([&](auto I) {
      constexpr int i = decltype(I)::value;
      issue_for(I);
      if constexpr (i < NQ) {
        constexpr int kb = i / 4, h = i % 2;
        if constexpr ((i % 4) >= 2)
          s[h] = mfma8(kf[h][kb], ql[kb], s[h]);
        else if constexpr (kb == 0)
          s[h] = mfma8z(kf[h][kb], qh[0]);
        else
          s[h] = mfma8(kf[h][kb], qh[kb], s[h]);
        if constexpr (i == NQ - 1) {
#pragma unroll
          for (int q = 0; q < 4; ++q) cm[q] = F->c[q] - m;
        }
      } else {
        constexpr int db = i - NQ;
        o[db] = mfma8(vf[db], p8, o[db]);
        static_for<PER>([&](auto E) {
          constexpr int k = PER * db + decltype(E)::value;
          if constexpr (k < 32) {
            constexpr int h = k / 16, e = k % 16;
            s[h][e] = __builtin_fmaf(s[h][e], F->f[2 * h + e / 8], cm[2 * h + e / 8]);
          }
        });
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  } else if constexpr (QK) {
    i32x8 fa = k_frag<D>(kt, kx, 0, 0), fb = k_frag<D>(kt, kx, 1, 0);
    i32x8 fv;
    if constexpr (PV) fv = v_frag<D>(vt, vx, 0);
    static_for<KS>([&](auto KB) {
      constexpr int kb = decltype(KB)::value;
      if constexpr (kb == 0) {
        s[0] = mfma8z(fa, qh[0]);
        s[1] = mfma8z(fb, qh[0]);
      } else {
        s[0] = mfma8(fa, qh[kb], s[0]);
        s[1] = mfma8(fb, qh[kb], s[1]);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (PV) {
        const i32x8 f = fv;
        fv = v_frag<D>(vt, vx, 2 * kb + 1);
        o[2 * kb] = mfma8(f, p8, o[2 * kb]);
        __builtin_amdgcn_sched_barrier(0);
      }
      s[0] = mfma8(fa, ql[kb], s[0]);
      if constexpr (kb + 1 < KS) fa = k_frag<D>(kt, kx, 0, kb + 1);
      s[1] = mfma8(fb, ql[kb], s[1]);
      if constexpr (kb + 1 < KS) fb = k_frag<D>(kt, kx, 1, kb + 1);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (PV) {
        const i32x8 f = fv;
        if constexpr (kb + 1 < KS) fv = v_frag<D>(vt, vx, 2 * kb + 2);
        o[2 * kb + 1] = mfma8(f, p8, o[2 * kb + 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    });
  } else if constexpr (PV) {
    i32x8 fv = v_frag<D>(vt, vx, 0);
    static_for<DB>([&](auto DBI) {
      constexpr int db = decltype(DBI)::value;
      const i32x8 f = fv;
      if constexpr (db + 1 < DB) fv = v_frag<D>(vt, vx, db + 1);
      o[db] = mfma8(f, p8, o[db]);
      __builtin_amdgcn_sched_barrier(0);
    });
  }
  // Keep the products in this phase (nothing may sink them past the barrier
  // into the phase that uses them).
  if constexpr (QK) asm volatile("" : "+v"(s[0]), "+v"(s[1]));
  if constexpr (PV) {
#pragma unroll
    for (int db = 0; db < DB; ++db) asm volatile("" : "+v"(o[db]));
  }
}

// Phase V: P'(t+1) from the raw products S(t+1) (both 32-key halves, 32
// elements per lane; element e of half h is key kb + 32 h + 16 hf + e of the
// segment, scale group q = 2 h + e / 8):
//   x = S f_q + c_q - m (f_q = ks sq scale log2(e), c_q the V bias), -inf
//   outside [lo, hi) with MASK, kept in place of S;  P' = exp2(x), packed to
//   E4M3FN into p8 one group at a time;  l += sum over groups 2^-c_q sum P'.
// The reference point m moves only when some lane's sum of P' exceeds 448 (an
// element could then exceed e4m3's range): then the row maximum is taken, O
// and l are rescaled exactly, x is shifted by the move and P' formed again.
// FIRST: the first tile of a segment sets m from its own row maxima.
// XPRE: s already holds x (computed in phase M; no mask, not the first tile).
template <int D, bool MASK, bool FIRST, bool XPRE = false>
__device__ __forceinline__ void v_phase(f32x16 (&s)[2], i32x8& p8, f32x16 (&o)[D / 32], float& m, float& l,
                                        const Factors& F, int kb, int lo, int hi, int hf) {
  static_assert(!XPRE || (!MASK && !FIRST), "x is formed in phase M only for unmasked, later tiles");
  // Key of element e of half h, from an opaque copy of hf (per-element key
  // offsets would otherwise be precomputed once and held in registers).
  int k0 = kb + 16 * hf;
  if constexpr (MASK) asm volatile("" : "+v"(k0));
  auto valid = [&](int h, int e) {
    const int key = k0 + 32 * h + e;
    return key >= lo && key < hi;
  };
  if constexpr (FIRST) {
    // Row maximum of S f_q (f_q >= 0: K scales and the Q scale are non-negative).
    float a = -INFINITY;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float v = s[h][e] * F.f[2 * h + e / 8];
        if constexpr (MASK) v = valid(h, e) ? v : -INFINITY;
        a = fmaxf(a, v);
      }
    m = half_max(a);
    l = 0.f;
  }
  if constexpr (!XPRE) {
    float cm[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) cm[q] = F.c[q] - m;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float x = __builtin_fmaf(s[h][e], F.f[2 * h + e / 8], cm[2 * h + e / 8]);
        if constexpr (MASK) x = valid(h, e) ? x : -INFINITY;
        s[h][e] = x;
      }
  }
  // P' of group q: exp2, sum, pack into dwords 2 q and 2 q + 1 of p8 (dword w
  // holds keys 4 w .. 4 w + 3 of the lane's 32: 16 of half 0, then 16 of half
  // 1, matching the V^T fragment of the P V product).
  float g[4];
  auto form = [&]() {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int h = q >> 1, e0 = 8 * (q & 1);
      float pe[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) pe[i] = __builtin_amdgcn_exp2f(s[h][e0 + i]);
      g[q] = ((pe[0] + pe[1]) + (pe[2] + pe[3])) + ((pe[4] + pe[5]) + (pe[6] + pe[7]));
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        // Both halves of the dword are written; the old value only fills the
        // half each conversion keeps (the register's own, so no zeroing move).
        uint32_t v = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(pe[4 * w], pe[4 * w + 1], p8[2 * q + w], false);
        v = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(pe[4 * w + 2], pe[4 * w + 3], (int)v, true);
        p8[2 * q + w] = (int)v;
      }
    }
  };
  form();
  const float lsum = (g[0] + g[1]) + (g[2] + g[3]);
  if (!FIRST && __builtin_expect(__builtin_amdgcn_ballot_w64(!(lsum <= kE4M3Max)) != 0, 0)) {
    asm volatile("");  // a real branch: the recomputation must not be executed speculatively
    // Row maximum of S f_q = x - c_q + m.
    float a = -INFINITY;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 16; ++e) a = fmaxf(a, s[h][e] - F.c[2 * h + e / 8]);
    const float m_new = fmaxf(m, half_max(a) + m);
    const float shift = m - m_new;  // <= 0
    const float alpha = __builtin_amdgcn_exp2f(shift);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[h][e] += shift;
    form();
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) l = __builtin_fmaf(g[q], F.w[q], l);
  // Keep the softmax in this phase.
  asm volatile("" : "+v"(p8), "+v"(l));
}

// LDS stages: K tile and V^T tile of each of the three ring slots.
struct Ring {
  char *k0, *k1, *k2, *v0, *v1, *v2;
  float4* tab;
  template <int S>
  __device__ __forceinline__ char* k() const { return S == 0 ? k0 : S == 1 ? k1 : k2; }
  template <int S>
  __device__ __forceinline__ char* v() const { return S == 0 ? v0 : S == 1 ? v1 : v2; }
};

template <int N>
using IC = std::integral_constant<int, N>;

// One query tile (item) of chunk cd over its 64-key tiles [j0, j1); slot < 0
// writes O (and LSE), slot >= 0 the partial result for the merge kernel.
template <int D>
__device__ __forceinline__ void segment(const AttnParams& p, const ChunkDesc& cd, int qt, int head, int j0,
                                        int j1, int slot, const Ring& rg, const Plan<D>& plan, int wave,
                                        int lane) {
  using G = Geo<D>;
  constexpr int KS = G::KS;
  constexpr int DB = G::DB;
  const int group = wave >> 2;
  const int gw = wave & 3;
  const int lq = lane & 31;
  const int hf = lane >> 5;
  const int qrow = qt * BMD + wave * 32 + lq;
  const int row = cd.q_begin + qrow;
  const bool row_ok = qrow < cd.q_len;
  const int base = TK * j0;
  const int lo = max(cd.lead - base, 0);
  const int hi = min(cd.lead + cd.nkeys, TK * j1) - base;
  const int nt = (hi + TK - 1) / TK;  // >= 1
  const int ngroups = (hi + 7) / 8;   // groups holding keys of the segment; the table runs to 8 nt
  const int kx = lq * G::KROW + 32 * hf;
  const int vx = lq * G::VROW + 16 * hf;
  bool pend = false;  // whether this wave's latest batch of loads is in flight

  // Prologue loads: group 1 K(0), K(1), K(2) -> slots 0, 1, 2; group 0 V(0) -> slot 1.
  Cursor cur = cursor_at<D>(p, cd, head, base);
  const __amdgpu_buffer_rsrc_t rs = cache_rsrc(group == 1 ? p.k : p.v);
  if (group == 1) {
    dma_k<D>(p, rs, cur, plan, rg.k<0>(), gw);
    advance<D>(p, head, cur, TK);
    if (nt > 1) dma_k<D>(p, rs, cur, plan, rg.k<1>(), gw);
    advance<D>(p, head, cur, TK);
    if (nt > 2) dma_k<D>(p, rs, cur, plan, rg.k<2>(), gw);
    advance<D>(p, head, cur, TK);
  } else {
    dma_v<D>(p, rs, cur, plan, rg.v<1>(), gw, lane);
    advance<D>(p, head, cur, TK);
  }

  // Scale table: entry g = (ks, c, 2^-c) of keys [8 g, 8 g + 8) of the segment,
  // with c = log2(1.75 vs / vs_max) (clamped: zero or tiny V scales only make P'
  // underflow; l stays exact).
  __shared__ float red[NW];
  float vmax = 0.f;
  for (int g = ngroups + threadIdx.x; g < 8 * nt; g += NTD) rg.tab[g] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int g = threadIdx.x; g < ngroups; g += NTD) {
    const uint32_t x = (uint32_t)cd.map.base_off + (uint32_t)(base + 8 * g);
    const uint32_t pg = fastdiv(x, p.divP);
    const uint32_t off = x - pg * p.divP.d;
    uint32_t sl = (uint32_t)cd.map.base_slot + pg;
    sl -= fastdiv(sl, p.divT) * p.divT.d;
    const int64_t bi = ((int64_t)p.table[sl] * p.H + head) * p.nblk + off / WF_SCALE_BLOCK;
    const float vs = p.vs[bi];
    rg.tab[g] = make_float4(p.ks[bi], vs, 0.f, 0.f);
    vmax = fmaxf(vmax, vs);
  }
  for (int sh = 32; sh > 0; sh >>= 1) vmax = fmaxf(vmax, __shfl_xor(vmax, sh));
  if (lane == 0) red[wave] = vmax;
  __syncthreads();
  vmax = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) vmax = fmaxf(vmax, red[w]);
  const float cmin = __log2f(kPScale) - 24.f;
  for (int g = threadIdx.x; g < 8 * nt; g += NTD) {
    const float4 e = rg.tab[g];
    const float c = fmaxf((vmax > 0.f && e.y > 0.f) ? __log2f(kPScale * e.y / vmax) : cmin, cmin);
    rg.tab[g] = make_float4(e.x, c, __builtin_amdgcn_exp2f(-c), 0.f);
  }

  // Q row -> two e4m3 terms with one scale per row: lane (lq, hf) holds dims
  // 64 kb + 32 hf + [0, 32) of its row.  x = q * 448 / amax; hi = e4m3(x);
  // lo = e4m3(x - hi) (the residual, exact in fp32).
  i32x8 qh[KS], ql[KS];
  float qs;
  {
    const __bf16* qp = (const __bf16*)p.q + ((int64_t)row * p.H + head) * D;
    f32x4 qv[KS][8];
    float amax = 0.f;
#pragma unroll
    for (int kb = 0; kb < KS; ++kb)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint4 raw = make_uint4(0, 0, 0, 0);
        if (row_ok) raw = *(const uint4*)(qp + 64 * kb + 32 * hf + 8 * c);
        const bf16x8 b = __builtin_bit_cast(bf16x8, raw);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = (float)b[e];
          qv[kb][2 * c + e / 4][e % 4] = v;
          amax = fmaxf(amax, fabsf(v));
        }
      }
    amax = half_max(amax);
    const float inv = amax > 0.f ? kE4M3Max / amax : 1.f;
    qs = (amax > 0.f ? amax / kE4M3Max : 1.f) * p.scale_log2;
#pragma unroll
    for (int kb = 0; kb < KS; ++kb)
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const float x0 = qv[kb][w][0] * inv, x1 = qv[kb][w][1] * inv;
        const float x2 = qv[kb][w][2] * inv, x3 = qv[kb][w][3] * inv;
        uint32_t v = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
        v = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, (int)v, true);
        qh[kb][w] = (int)v;
        const f32x2 h01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(v, 1.0f, false);
        const f32x2 h23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(v, 1.0f, true);
        uint32_t u = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x0 - h01[0], x1 - h01[1], 0, false);
        u = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x2 - h23[0], x3 - h23[1], (int)u, true);
        ql[kb][w] = (int)u;
      }
  }
  f32x16 o[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[b][i] = 0.f;
  f32x16 s[2];
  i32x8 p8;
  float m = -INFINITY, l = 0.f;

  auto end_phase = [&]() {
    if (pend)
      wait_vmcnt<G::PW>();
    else
      wait_vmcnt<0>();
    barrier();
  };
  // Loads issued at the start of phase V(t) (t >= -1): group 0 V(t+2) -> slot
  // t % 3 (vdst), group 1 K(t+4) -> slot (t+1) % 3 (kdst).  The previous batch
  // is complete first (a CU stalls LDS-DMA issue beyond about 40 loads in flight).
  auto loads = [&](int t, char* vdst, char* kdst) {
    wait_vmcnt<0>();
    if (group == 0) {
      pend = t + 2 < nt;
      if (pend) dma_v<D>(p, rs, cur, plan, vdst, gw, lane);
    } else {
      pend = t + 4 < nt;
      if (pend) dma_k<D>(p, rs, cur, plan, kdst, gw);
    }
    advance<D>(p, head, cur, TK);
    asm volatile("" ::"s"(cur.k1), "s"(cur.v1));
  };
  auto vedge = [&](int t) { return (t == 0 && lo > 0) || TK * (t + 1) > hi; };
  auto zero_v = [&](char* vt, int t) {
    zero_v_outside<D>(vt, t, lo, hi);
    wait_lgkm0();
    barrier();
  };

  wait_vmcnt<0>();
  barrier();                   // tiles of the prologue and the scale table are in LDS
  if (group == 1) barrier();   // group 1 runs one phase behind
  // M(-1): S(0) from K(0) in slot 0.
  m_phase<D, true, false>(s, o, qh, ql, p8, rg.k<0>(), rg.v<0>(), kx, vx);
  end_phase();
  if (group == 1 && vedge(0)) zero_v(rg.v<1>(), 0);
  // V(-1)
  prio(1);  // the softmax wave issues first on its SIMD
  loads(-1, rg.v<2>(), rg.k<0>());
  v_phase<D, true, true>(s, p8, o, m, l, factors(rg.tab, 0, hf, qs), 0, lo, hi, hf);
  prio(0);
  end_phase();
  if (group == 0 && vedge(0)) zero_v(rg.v<1>(), 0);

  // Tile t uses stage t in slot (t + 1) % 3; the loop is unrolled by three so
  // every slot is a compile-time constant.  steady(t) needs t + 2 < nt;
  // edge_step(t) is tile nt - 2; tile nt - 1 follows the switch.
  auto steady = [&](auto rho_tag, int t) {
    constexpr int rho = decltype(rho_tag)::value;
    constexpr int sl = (rho + 1) % 3;
    const Factors F = factors(rg.tab, t + 1, hf, qs);
    m_phase<D, true, true, true>(s, o, qh, ql, p8, rg.k<sl>(), rg.v<sl>(), kx, vx, &F, m);
    end_phase();
    prio(1);  // the softmax wave issues first on its SIMD
    loads(t, rg.v<rho>(), rg.k<sl>());
    v_phase<D, false, false, true>(s, p8, o, m, l, factors(rg.tab, t + 1, hf, qs), 0, lo, hi, hf);
    prio(0);
    end_phase();
  };
  auto edge_step = [&](auto rho_tag, int t) {
    constexpr int rho = decltype(rho_tag)::value;
    constexpr int sl = (rho + 1) % 3;
    constexpr int sn = (rho + 2) % 3;  // slot of stage t + 1
    m_phase<D, true, true>(s, o, qh, ql, p8, rg.k<sl>(), rg.v<sl>(), kx, vx);
    end_phase();
    const bool ze = vedge(t + 1);
    if (group == 1 && ze) zero_v(rg.v<sn>(), t + 1);
    prio(1);  // the softmax wave issues first on its SIMD
    loads(t, rg.v<rho>(), rg.k<sl>());
    v_phase<D, true, false>(s, p8, o, m, l, factors(rg.tab, t + 1, hf, qs), TK * (t + 1), lo, hi, hf);
    prio(0);
    end_phase();
    if (group == 0 && ze) zero_v(rg.v<sn>(), t + 1);
  };
  int t = 0;
  for (; t + 4 < nt; t += 3) {
    steady(IC<0>{}, t);
    steady(IC<1>{}, t + 1);
    steady(IC<2>{}, t + 2);
  }
  switch (nt - t) {  // 1 .. 4 tiles left, t % 3 == 0
    case 1:
      break;
    case 2:
      edge_step(IC<0>{}, t);
      break;
    case 3:
      steady(IC<0>{}, t);
      edge_step(IC<1>{}, t + 1);
      break;
    default:
      steady(IC<0>{}, t);
      steady(IC<1>{}, t + 1);
      edge_step(IC<2>{}, t + 2);
      break;
  }
  // Tile nt - 1: its P V product alone, from slot nt % 3 (one code path for
  // every tile count).  Its accumulators are read by plain VALU code right
  // after, so the wave sleeps until the products have left the matrix pipe:
  // copies taken 20 wait states after issue (the count the compiler allows)
  // returned the old accumulator when this phase had a path of its own.
  {
    const int sl = nt % 3;
    const char* vt = sl == 0 ? rg.v0 : sl == 1 ? rg.v1 : rg.v2;
    m_phase<D, false, true>(s, o, qh, ql, p8, rg.k0, vt, kx, vx);
    __builtin_amdgcn_s_sleep(2);
    end_phase();
  }
  if (group == 0) barrier();  // matches group 1's last M phase

  const float lt = half_sum(l);
  const float vfac = vmax / kPScale;  // O = O_acc * vs_max / 1.75
  if (slot < 0) {
    const float inv = vfac / lt;
    if (row_ok) {
      __bf16* orow = (__bf16*)p.o + ((int64_t)row * p.H + head) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x4 v = {(__bf16)(o[db][4 * g + 0] * inv), (__bf16)(o[db][4 * g + 1] * inv),
                      (__bf16)(o[db][4 * g + 2] * inv), (__bf16)(o[db][4 * g + 3] * inv)};
          *(bf16x4*)(orow + db * 32 + 8 * g + 4 * hf) = v;
        }
      if (p.lse != nullptr && hf == 0) p.lse[(int64_t)head * p.nq + row] = (m + __log2f(lt)) * kLn2;
    }
  } else if (row_ok) {
    float* ws = p.ws + (int64_t)slot * ws_slot_floats(D);
    const int r = wave * 32 + lq;
    float* orow = ws + (int64_t)r * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(f32x4*)(orow + db * 32 + 8 * g + 4 * hf) = {o[db][4 * g + 0] * vfac, o[db][4 * g + 1] * vfac,
                                                       o[db][4 * g + 2] * vfac, o[db][4 * g + 3] * vfac};
    if (hf == 0) {
      ws[BMD * D + r] = m;
      ws[BMD * D + BMD + r] = lt;
    }
  }
  __syncthreads();  // the next segment rebuilds the scale table and refills the ring
}

template <int D>
__global__ __launch_bounds__(NTD, 2) void attn_fwd_fp8_kernel(const AttnParams p) {
  using G = Geo<D>;
  __shared__ __align__(1024) char k0[G::KTILE];
  __shared__ __align__(1024) char k1[G::KTILE];
  __shared__ __align__(1024) char k2[G::KTILE];
  __shared__ __align__(1024) char v0[G::VTILE];
  __shared__ __align__(1024) char v1[G::VTILE];
  __shared__ __align__(1024) char v2[G::VTILE];
  __shared__ __align__(16) float4 tab[kFp8MaxGroups + 2];
  const Ring rg{k0, k1, k2, v0, v1, v2, tab};
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const Plan<D> plan = make_plan<D>(wave >> 2, wave & 3, lane, p.P);
  walk_segments(p, (int)blockIdx.x, [&](int item, int j0, int j1, int slot) {
    const Item it = decode_item(p, item);
    segment<D>(p, p.chunk[it.c], it.qt, it.head, j0, j1, slot, rg, plan, wave, lane);
  });
}

}  // namespace dma8
}  // namespace

hipError_t launch_attn_fp8_dma(const AttnParams& p, int head_dim, int grid, hipStream_t s) {
  if (head_dim == 128)
    hipLaunchKernelGGL(dma8::attn_fwd_fp8_kernel<128>, dim3(grid), dim3(dma8::NTD), 0, s, p);
  else
    hipLaunchKernelGGL(dma8::attn_fwd_fp8_kernel<64>, dim3(grid), dim3(dma8::NTD), 0, s, p);
  return hipGetLastError();
}

hipError_t attn_fp8_resident_blocks(int head_dim, int* blocks) {
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess)
    e = head_dim == 128
            ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, dma8::attn_fwd_fp8_kernel<128>, dma8::NTD, 0)
            : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, dma8::attn_fwd_fp8_kernel<64>, dma8::NTD, 0);
  *blocks = cus * (per_cu > 0 ? per_cu : 1);
  return e;
}

}  // namespace wf
