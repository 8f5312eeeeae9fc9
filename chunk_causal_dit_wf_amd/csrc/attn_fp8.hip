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
//       largest V scale of the block's key range and 1.75 maps the largest
//       P between rescales (2^8) onto e4m3's 448.  O = O_acc * vs_max / 1.75.
// Per-key factors are per 8-key group: a lane's 16 keys of a 32-key
// half-tile are two groups, so every factor is a per-register constant, and
// the V factor rides in the exponent's bias (no extra VALU per element).
// The row sums are taken from the fp32 P' before quantisation.
//
// Structure as the bf16 LDS-DMA kernel: 8 waves x 32 query rows per
// workgroup; K tiles (64 keys, rows padded to D + 16 bytes, keys permuted so a
// lane half holds 16 consecutive keys) and V^T tiles (D rows of 64 keys plus
// 16 bytes) double-buffered through LDS by LDS-DMA; one barrier per tile.
// Step j: S[j+1] = K[j+1] Q^T alongside P[j] = exp(S[j]); then
// O += V[j] P[j] alongside the row maxima of S[j+1] and the lazy rescale.
//
// Roofline: dense fp8 MFMA.  Algorithmic flops per visible (query, key) pair
// and head are 4 * head_dim.
#include <utility>

#include "attn_common.h"

namespace wf {
namespace {
namespace dma8 {

constexpr int NW = 8;         // waves per workgroup
constexpr int NTD = 64 * NW;  // threads per workgroup
constexpr int BMD = 32 * NW;  // query rows per workgroup
constexpr int TK = kTileKeys;  // keys per tile
constexpr float kPScale = 1.75f;
constexpr float kE4M3Max = 448.f;
static_assert(BMD == kBlockMDma, "host and kernel disagree on the block size");

template <int D>
struct Geo {
  static constexpr int KROW = D + 16;                     // LDS bytes per K row (padded)
  static constexpr int KDMA = (TK * KROW + 1023) / 1024;  // 16-byte DMA instructions per K tile
  static constexpr int KTILE = KDMA * 1024;
  static constexpr int VROW = TK + 16;                    // LDS bytes per V^T row (padded)
  static constexpr int VDMA = (D * VROW + 1023) / 1024;   // 16-byte DMA instructions per V^T tile
  static constexpr int VTILE = VDMA * 1024;
  static constexpr int V4DMA = (D * VROW + 255) / 256;    // 4-byte DMA instructions per V^T tile
  static constexpr int KPW = (KDMA + NW - 1) / NW;
  static constexpr int VPW = (VDMA + NW - 1) / NW;
  static constexpr int V4PW = (V4DMA + NW - 1) / NW;
  static constexpr int KS = D / 64;  // 64-deep k-blocks of Q K^T
  static constexpr int DB = D / 32;  // 32-row d-blocks of P V
};

// Per-lane constants of this wave's 16-byte DMA instructions (see the bf16
// kernel): source offset relative to the run base and the run-relative key.
template <int D>
struct Plan {
  uint32_t koff[Geo<D>::KPW];
  int32_t kkey[Geo<D>::KPW];
  uint32_t voff[Geo<D>::VPW];
};

template <int D>
__device__ __forceinline__ Plan<D> make_plan(int wave, int lane, int P) {
  using G = Geo<D>;
  Plan<D> pl;
#pragma unroll
  for (int r = 0; r < G::KPW; ++r) {
    const int y = 1024 * (wave + NW * r) + 16 * lane;
    const int row = y / G::KROW, pc = (y % G::KROW) / 16;
    const bool data = row < TK && pc < D / 16;
    const int q = row & 31;  // row inside its 32-key half: key 16 h + 4 j + i at row 8 j + 4 h + i
    const int key = (row & 32) + 16 * ((q >> 2) & 1) + 4 * (q >> 3) + (q & 3);
    pl.kkey[r] = data ? key : 0;
    pl.koff[r] = data ? (uint32_t)(key * D + pc * 16) : 0u;
  }
#pragma unroll
  for (int r = 0; r < G::VPW; ++r) {
    const int y = 1024 * (wave + NW * r) + 16 * lane;
    const int d = y / G::VROW, pc = (y % G::VROW) / 16;
    const bool data = d < D && pc < 4;
    pl.voff[r] = data ? (uint32_t)(d * P + pc * 16) : 0u;
  }
  return pl;
}

// DMA the K tile at cursor c (64 keys) into kbuf.  Runs inside one page add
// the run base to the plan offset; a run that crosses a page selects its page
// per lane (a 16-byte chunk is part of one key's row, so it never straddles).
template <int D>
__device__ __forceinline__ void dma_k(const AttnParams& p, const Cursor& c, const Plan<D>& pl, char* kbuf,
                                      int wave) {
  using G = Geo<D>;
  if (p.P - c.off >= TK) {
    const uint32_t soff = c.k0 + (uint32_t)c.off * D;
#pragma unroll
    for (int r = 0; r < G::KPW; ++r)
      if ((NW - 1) + NW * r < G::KDMA || wave + NW * r < G::KDMA)
        dma16((const char*)p.k + (soff + pl.koff[r]), kbuf + 1024 * (wave + NW * r));
    return;
  }
  const RunGeom g = run_geom<D, 1>(p, c);
#pragma unroll
  for (int r = 0; r < G::KPW; ++r)
    if (wave + NW * r < G::KDMA)
      dma16((const char*)p.k + ((pl.kkey[r] < g.split ? g.kb0 : g.kb1) + pl.koff[r]),
            kbuf + 1024 * (wave + NW * r));
}

// DMA the V^T tile at cursor c (64 keys) into vbuf.  A 16-byte chunk holds 16
// keys of one V^T row and can straddle a page break (pages are multiples of
// 8 keys), so a run that crosses a page (one tile per page) moves in 4-byte
// pieces, each of which stays inside one page.
template <int D>
__device__ __forceinline__ void dma_v(const AttnParams& p, const Cursor& c, const Plan<D>& pl, char* vbuf,
                                      int wave, int lane) {
  using G = Geo<D>;
  if (p.P - c.off >= TK) {
    const uint32_t soff = c.v0 + (uint32_t)c.off;
#pragma unroll
    for (int r = 0; r < G::VPW; ++r)
      if ((NW - 1) + NW * r < G::VDMA || wave + NW * r < G::VDMA)
        dma16((const char*)p.v + (soff + pl.voff[r]), vbuf + 1024 * (wave + NW * r));
    return;
  }
  const RunGeom g = run_geom<D, 1>(p, c);
  for (int r = 0; r < G::V4PW; ++r) {
    const int ins = wave + NW * r;
    if (ins < G::V4DMA) {
      const int y = 256 * ins + 4 * lane;
      const int d = y / G::VROW, b = y - d * G::VROW;
      const bool data = d < D && b < TK;
      const uint32_t off = data ? (b < g.split ? g.vb0 : g.vb1) + (uint32_t)(d * p.P + b) : g.vb0;
      dma4((const char*)p.v + off, vbuf + 256 * ins);
    }
  }
}

// Zero the keys of V^T tile t (in LDS) that lie outside [lo, hi).
template <int D>
__device__ __forceinline__ void zero_v_outside(char* vbuf, int t, int lo, int hi) {
  for (int idx = threadIdx.x; idx < D * 4; idx += NTD) {
    const int d = idx >> 2, c = idx & 3;
    const int rel = t * TK + 16 * c;
    if (rel >= lo && rel + 16 <= hi) continue;
    uint32_t w[4];
    uint4* a = (uint4*)(vbuf + d * Geo<D>::VROW + 16 * c);
    const uint4 v = *a;
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (!(rel + e >= lo && rel + e < hi)) w[e >> 2] &= ~(0xFFu << (8 * (e & 3)));
    *a = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Scale factors of one 32-key half-tile for this lane (its keys are two 8-key
// groups A, B): score factor f = ks * sq * scale * log2(e), and the bias of the
// exponent cb = log2(1.75 vs / vs_max).
struct HalfScale {
  float fa, fb, ca, cb;
};

__device__ __forceinline__ HalfScale half_scale(const float2* table, int group, float qs) {
  const f32x4 t = *(const f32x4*)(table + group);  // groups group, group + 1
  HalfScale h;
  h.fa = t[0] * qs;
  h.ca = t[1];
  h.fb = t[2] * qs;
  h.cb = t[3];
  return h;
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>), unrolled at compile time.
template <typename F, int... I>
__device__ __forceinline__ void static_for_seq(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_seq(f, std::make_integer_sequence<int, N>{});
}

// 32 bytes (two 16-byte LDS reads) as an MFMA fp8 operand.
__device__ __forceinline__ i32x8 lds32(const char* a) {
  const i32x4 lo = *(const i32x4*)a;
  const i32x4 hi = *(const i32x4*)(a + 16);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ i32x8 lds16x2(const char* a, int gap) {
  const i32x4 lo = *(const i32x4*)a;
  const i32x4 hi = *(const i32x4*)(a + gap);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// MFMA i of a tile's S^T: half-tile i / KS, k-block i % KS.  A operand: 32
// bytes of LDS row 32 (i / KS) + lq at dims 64 (i % KS) + 32 hf (kx covers lq, hf).
template <int D>
__device__ __forceinline__ i32x8 k_frag(const char* kbuf, int kx, int i) {
  return lds32(kbuf + (i / Geo<D>::KS) * 32 * Geo<D>::KROW + kx + 64 * (i % Geo<D>::KS));
}
// PV MFMA db: A operand = V^T row 32 db + lq, keys 16 hf + [0, 16) and 32 + 16 hf + [0, 16).
template <int D>
__device__ __forceinline__ i32x8 v_frag(const char* vbuf, int vx, int db) {
  return lds16x2(vbuf + vx + db * 32 * Geo<D>::VROW, 32);
}

// S^T of one tile in one go (prologue): halves a (keys 0..31) and b (32..63).
template <int D>
__device__ __forceinline__ void qk_tile(const char* kbuf, int kx, const i32x8 (&q8)[Geo<D>::KS],
                                        const i32x8 (&q8lo)[Geo<D>::KS], f32x16& sa, f32x16& sb) {
  constexpr int KS = Geo<D>::KS;
#pragma unroll
  for (int i = 0; i < 16; ++i) sa[i] = sb[i] = 0.f;
#pragma unroll
  for (int i = 0; i < 2 * KS; ++i) {
    f32x16& acc = i < KS ? sa : sb;
    const i32x8 kf = k_frag<D>(kbuf, kx, i);
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf, q8[i % KS], acc, 0, 0, 0, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf, q8lo[i % KS], acc, 0, 0, 0, 0, 0, 0);
  }
}

// Scaled, masked scores of a half-tile in place and their row max (edge tiles).
__device__ __forceinline__ float mask_half(f32x16& acc, const HalfScale& h, int key0, int lo, int hi) {
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int key = key0 + i;
    const float sv = acc[i] * (i < 8 ? h.fa : h.fb);
    acc[i] = (key >= lo && key < hi) ? sv : -INFINITY;
    mx = fmaxf(mx, acc[i]);
  }
  return mx;
}

// P' of elements [E0, E0 + EN) of a half-tile (EN = 8 or 16, one or two scale
// groups): exponent, e4m3 packing into pk (dword (E0 + e) / 4 of the half),
// and the row-sum contribution.  fa, fb: score factors of the two groups (1
// when acc already holds scaled scores).
template <int E0, int EN>
__device__ __forceinline__ void p_group(const f32x16& acc, const HalfScale& h, float fa, float fb, float m,
                                        uint32_t* pk, float& l) {
#pragma unroll
  for (int g = E0 / 8; g < (E0 + EN) / 8; ++g) {
    const float f = g == 0 ? fa : fb;
    const float c = g == 0 ? h.ca : h.cb;
    const float bias = c - m;
    float e[8], sum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      e[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[8 * g + i], f, bias));
      sum += e[i];
    }
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      uint32_t v = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(e[4 * w], e[4 * w + 1], 0, false);
      v = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(e[4 * w + 2], e[4 * w + 3], (int)v, true);
      pk[2 * g + w] = v;
    }
    l = __builtin_fmaf(sum, __builtin_amdgcn_exp2f(-c), l);
  }
}

// Raw maximum of elements [E0, E0 + EN) of a half-tile (unmasked tiles).
template <int E0, int EN>
__device__ __forceinline__ float raw_max(const f32x16& acc) {
  float m0 = fmaxf(acc[E0], acc[E0 + 1]), m1 = fmaxf(acc[E0 + 2], acc[E0 + 3]);
#pragma unroll
  for (int i = E0 + 4; i < E0 + EN; i += 2) {
    m0 = fmaxf(m0, acc[i]);
    m1 = fmaxf(m1, acc[i + 1]);
  }
  return fmaxf(m0, m1);
}

struct Bufs {
  char *k0, *k1, *v0, *v1;
  float2* scales;
};

// One query tile (item) of chunk cd over its 64-key tiles [j0, j1); slot < 0
// writes O (and LSE), slot >= 0 the partial result for the merge kernel.
template <int D>
__device__ __forceinline__ void segment(const AttnParams& p, const ChunkDesc& cd, int qt, int head, int j0,
                                        int j1, int slot, const Bufs& bf, const Plan<D>& plan, int wave,
                                        int lane) {
  using G = Geo<D>;
  constexpr int KS = G::KS, DB = G::DB;
  const int lq = lane & 31;
  const int hf = lane >> 5;
  const int qrow = qt * BMD + wave * 32 + lq;
  const int row = cd.q_begin + qrow;
  const bool row_ok = qrow < cd.q_len;
  const int base = TK * j0;
  const int lo = max(cd.lead - base, 0);
  const int hi = min(cd.lead + cd.nkeys, TK * j1) - base;
  const int nt = (hi + TK - 1) / TK;
  const int ngroups = (hi + 7) / 8;  // groups holding keys of the segment; the table runs to 8 nt

  // K tiles 0, 1 and V tile 0 in flight while the scale table and Q are built.
  Cursor kcur = cursor_at<D>(p, cd, head, base), vcur = kcur;
  dma_k<D>(p, kcur, plan, bf.k0, wave);
  advance<D>(p, head, kcur, TK);
  if (nt > 1) dma_k<D>(p, kcur, plan, bf.k1, wave);
  advance<D>(p, head, kcur, TK);
  dma_v<D>(p, vcur, plan, bf.v0, wave, lane);
  advance<D>(p, head, vcur, TK);

  // Scale table: entry g = (ks, vs) of keys [8 g, 8 g + 8) of the segment, then
  // (ks, log2(1.75 vs / vs_max)).
  __shared__ float red[NW];
  float vmax = 0.f;
  for (int g = ngroups + threadIdx.x; g < 8 * nt; g += NTD) bf.scales[g] = make_float2(0.f, 0.f);
  for (int g = threadIdx.x; g < ngroups; g += NTD) {
    const uint32_t x = (uint32_t)cd.map.base_off + (uint32_t)(base + 8 * g);
    const uint32_t pg = fastdiv(x, p.divP);
    const uint32_t off = x - pg * p.divP.d;
    uint32_t s = (uint32_t)cd.map.base_slot + pg;
    s -= fastdiv(s, p.divT) * p.divT.d;
    const int64_t bi = ((int64_t)p.table[s] * p.H + head) * p.nblk + off / WF_SCALE_BLOCK;
    const float vs = p.vs[bi];
    bf.scales[g] = make_float2(p.ks[bi], vs);
    vmax = fmaxf(vmax, vs);
  }
  for (int o = 32; o > 0; o >>= 1) vmax = fmaxf(vmax, __shfl_xor(vmax, o));
  if (lane == 0) red[wave] = vmax;
  __syncthreads();
  vmax = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) vmax = fmaxf(vmax, red[w]);
  const float cmin = __log2f(kPScale) - 24.f;  // zero or tiny V scales: P' underflows, l stays exact
  for (int g = threadIdx.x; g < 8 * nt; g += NTD) {
    const float2 e = bf.scales[g];
    const float c = (vmax > 0.f && e.y > 0.f) ? __log2f(kPScale * e.y / vmax) : cmin;
    bf.scales[g] = make_float2(e.x, fmaxf(c, cmin));
  }

  // Q row -> two e4m3 terms with one scale per row: lane (lq, hf) holds dims
  // 64 s + 32 hf + [0, 32) of its row.  x = q * 448 / amax; hi = e4m3(x);
  // lo = e4m3(x - hi) (the residual, exact in fp32).
  i32x8 q8[KS], q8lo[KS];
  float qs;
  {
    const __bf16* qp = (const __bf16*)p.q + ((int64_t)row * p.H + head) * D;
    f32x4 qv[KS][8];
    float amax = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint4 raw = make_uint4(0, 0, 0, 0);
        if (row_ok) raw = *(const uint4*)(qp + 64 * s + 32 * hf + 8 * c);
        const bf16x8 b = __builtin_bit_cast(bf16x8, raw);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = (float)b[e];
          qv[s][2 * c + e / 4][e % 4] = v;
          amax = fmaxf(amax, fabsf(v));
        }
      }
    amax = half_max(amax);
    const float inv = amax > 0.f ? kE4M3Max / amax : 1.f;
    qs = (amax > 0.f ? amax / kE4M3Max : 1.f) * p.scale_log2;
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const float x0 = qv[s][w][0] * inv, x1 = qv[s][w][1] * inv;
        const float x2 = qv[s][w][2] * inv, x3 = qv[s][w][3] * inv;
        uint32_t v = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
        v = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, (int)v, true);
        q8[s][w] = (int)v;
        const f32x2 h01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(v, 1.0f, false);
        const f32x2 h23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(v, 1.0f, true);
        uint32_t u = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x0 - h01[0], x1 - h01[1], 0, false);
        u = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x2 - h23[0], x3 - h23[1], (int)u, true);
        q8lo[s][w] = (int)u;
      }
  }
  f32x16 o[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[b][i] = 0.f;
  float l = 0.f;

  const int kx = lq * G::KROW + 32 * hf;  // K row lq, dims 32 hf + [0, 32) of each k-block
  const int vx = lq * G::VROW + 16 * hf;  // V^T row lq, keys 16 hf + [0, 16)
  wait_vmcnt<0>();
  __syncthreads();  // tile 0 and the scale table are in LDS
  if (lo > 0 || TK > hi) {
    zero_v_outside<D>(bf.v0, 0, lo, hi);
    __syncthreads();
  }
  // S[0], scaled and masked (tile 0 holds key lo < 8, so its row maxima are finite)
  f32x16 s0a, s0b, s1a, s1b;
  qk_tile<D>(bf.k0, kx, q8, q8lo, s0a, s0b);
  HalfScale h0a = half_scale(bf.scales, 2 * hf, qs), h0b = half_scale(bf.scales, 4 + 2 * hf, qs), h1a, h1b;
  float m = half_max(fmaxf(mask_half(s0a, h0a, 16 * hf, lo, hi), mask_half(s0b, h0b, 32 + 16 * hf, lo, hi)));
  __syncthreads();  // k0 is free for tile 2

  // Step j.  EVEN: S[j] in s0*, S[j+1] computed into s1* (odd j: the other
  // way).  sc: S[j] holds scaled, masked scores (tile 0, the last tile);
  // mn: tile j+1 is the last tile and is masked when its maxima are taken.
  // Both are runtime flags that select factors or take a short uniform
  // branch, so each parity is instantiated once (more instances of the
  // staged step exhaust the register file).
  //   [A] stage i: MFMA i of S[j+1] = K[j+1] Q^T (its fragment read one stage
  //       ahead) and P' of one 8-key group of S[j] (exp, e4m3 pack, row sum);
  //   [B] stage d: MFMA d of O += V[j] P[j] and the raw maxima of one group
  //       of S[j+1]; then the lazy rescale.
  bool sc = true;
  auto step = [&](auto even_tag, int j) {
    constexpr bool even = decltype(even_tag)::value;
    constexpr int NA = 2 * KS;   // QK MFMAs per tile
    constexpr int EA = 32 / NA;  // S[j] elements per [A] stage
    constexpr int EB = 32 / DB;  // S[j+1] elements per [B] stage
    f32x16& ca = even ? s0a : s1a;
    f32x16& cb = even ? s0b : s1b;
    f32x16& na = even ? s1a : s0a;
    f32x16& nb = even ? s1b : s0b;
    HalfScale& hca = even ? h0a : h1a;
    HalfScale& hcb = even ? h0b : h1b;
    HalfScale& hna = even ? h1a : h0a;
    HalfScale& hnb = even ? h1b : h0b;
    char* const kc = even ? bf.k1 : bf.k0;  // K[j+1]
    char* const kf = even ? bf.k0 : bf.k1;  // receives K[j+2]
    char* const vc = even ? bf.v0 : bf.v1;  // V[j]
    char* const vf = even ? bf.v1 : bf.v0;  // receives V[j+1]
    int wv = wave;
    asm volatile("" : "+s"(wv));
    if (j + 2 < nt) dma_k<D>(p, kcur, plan, kf, wv);
    advance<D>(p, head, kcur, TK);
    if (j + 1 < nt) dma_v<D>(p, vcur, plan, vf, wv, lane);
    advance<D>(p, head, vcur, TK);
    if (j > 0 && TK * j + TK > hi) {
      zero_v_outside<D>(vc, j, lo, hi);
      __syncthreads();
    }
    // The last step also computes an S[j+1] (from the stale K buffer, unused):
    // guarding it would keep two versions of the score registers alive.
    const bool more = j + 1 < nt;
    const bool mn = more && TK * (j + 1) + TK > hi;
    const float faa = sc ? 1.f : hca.fa, fab = sc ? 1.f : hca.fb;
    const float fba = sc ? 1.f : hcb.fa, fbb = sc ? 1.f : hcb.fb;
    uint32_t pk[8];
    i32x8 fr[2];
    fr[0] = k_frag<D>(kc, kx, 0);
    static_for<NA>([&](auto I) {
      constexpr int i = decltype(I)::value;
      if constexpr (i + 1 < NA) fr[(i + 1) & 1] = k_frag<D>(kc, kx, i + 1);
      f32x16& acc = i < KS ? na : nb;
      if constexpr (i % KS == 0) {
        f32x16 z;
#pragma unroll
        for (int e = 0; e < 16; ++e) z[e] = 0.f;
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fr[i & 1], q8[0], z, 0, 0, 0, 0, 0, 0);
      } else {
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fr[i & 1], q8[i % KS], acc, 0, 0, 0, 0, 0, 0);
      }
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fr[i & 1], q8lo[i % KS], acc, 0, 0, 0, 0, 0, 0);
      constexpr int e0 = EA * i;
      if constexpr (e0 < 16)
        p_group<e0 % 16, EA>(ca, hca, faa, fab, m, pk, l);
      else
        p_group<e0 % 16, EA>(cb, hcb, fba, fbb, m, pk + 4, l);
      asm volatile("" : "+v"(l));
      __builtin_amdgcn_sched_barrier(0);
    });
    i32x8 p8;
#pragma unroll
    for (int w = 0; w < 8; ++w) p8[w] = (int)pk[w];
    if (more) {
      hna = half_scale(bf.scales, 8 * (j + 1) + 2 * hf, qs);
      hnb = half_scale(bf.scales, 8 * (j + 1) + 4 + 2 * hf, qs);
    }
    float gm[4];  // raw maxima of the 8-key groups of S[j+1]: (half a: A, B), (half b: A, B)
    fr[0] = v_frag<D>(vc, vx, 0);
    static_for<DB>([&](auto I) {
      constexpr int d = decltype(I)::value;
      if constexpr (d + 1 < DB) fr[(d + 1) & 1] = v_frag<D>(vc, vx, d + 1);
      o[d] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fr[d & 1], p8, o[d], 0, 0, 0, 0, 0, 0);
#pragma unroll
      for (int g = EB * d / 8; g < EB * (d + 1) / 8; ++g) {
        gm[g] = g < 2 ? (g == 0 ? raw_max<0, 8>(na) : raw_max<8, 8>(na))
                      : (g == 2 ? raw_max<0, 8>(nb) : raw_max<8, 8>(nb));
      }
      asm volatile("" : "+v"(o[d]));
      __builtin_amdgcn_sched_barrier(0);
    });
    if (more) {
      float mx;
      if (mn)
        mx = fmaxf(mask_half(na, hna, TK * (j + 1) + 16 * hf, lo, hi),
                   mask_half(nb, hnb, TK * (j + 1) + 32 + 16 * hf, lo, hi));
      else
        mx = fmaxf(fmaxf(gm[0] * hna.fa, gm[1] * hna.fb), fmaxf(gm[2] * hnb.fa, gm[3] * hnb.fb));
      mx = half_max(mx);
      maybe_rescale<D>(mx, m, l, o);
    }
    sc = mn;
    wait_vmcnt<0>();
    __syncthreads();
  };
  for (int j = 0; j < nt; j += 2) {
    step(std::true_type{}, j);
    if (j + 1 < nt) step(std::false_type{}, j + 1);
  }

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
  __syncthreads();  // the next segment rebuilds the scale table
}

template <int D>
__global__ __launch_bounds__(NTD, 2) void attn_fwd_fp8_kernel(const AttnParams p) {
  using G = Geo<D>;
  __shared__ __align__(1024) char k0[G::KTILE];
  __shared__ __align__(1024) char k1[G::KTILE];
  __shared__ __align__(1024) char v0[G::VTILE];
  __shared__ __align__(1024) char v1[G::VTILE];
  __shared__ __align__(16) float2 scales[kFp8MaxGroups + 2];
  const Bufs bf{k0, k1, v0, v1, scales};
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const Plan<D> plan = make_plan<D>(wave, lane, p.P);
  walk_segments(p, (int)blockIdx.x, [&](int item, int j0, int j1, int slot) {
    const Item it = decode_item(p, item);
    segment<D>(p, p.chunk[it.c], it.qt, it.head, j0, j1, slot, bf, plan, wave, lane);
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
