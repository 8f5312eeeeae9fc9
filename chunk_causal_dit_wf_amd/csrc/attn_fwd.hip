// Chunk-wise causal attention forward for gfx950 (MI355X).
//
// Operation (Wave Forcing abstract; hellomarvisaitoday Wave Forcing article,
// first paragraph): the query rows of chunk c attend to the logical keys
// [kv_begin[c], kv_end[c]) of a paged ring KV cache -- their own chunk
// (bidirectional) plus the earlier, possibly still-noisy chunks.  Softmax is
// evaluated online (flash style), an exact re-association of
//   O = softmax(scale * Q K^T) V.
//
// Work decomposition.  One workgroup = 4 waves = 128 query rows of one head
// of one chunk; each wave owns 32 rows.  Keys stream through LDS in tiles of
// 64, double-buffered: the global loads of tile j+1 are in flight while tile
// j is consumed.  Tiles are aligned to 8 logical positions, so only the first
// and last tile of a chunk carry masked keys (block-causal tile skipping: no
// tile outside [kv_begin, kv_end) is ever loaded).
//
// MFMA formulation.  The wave computes S^T = K Q^T with
// V_MFMA_F32_32X32X16_BF16 (A = K tile rows from LDS, B = the wave's Q rows
// held in VGPRs).  In the 32x32 accumulator a lane holds one query column and
// 16 key rows, so the row max and row sum are in-lane reductions plus one
// exchange between the two 32-lane halves (v_permlane32_swap).  The same
// registers, converted to bf16, are directly the B operand of
// O^T += V^T P^T, whose A operand (V^T rows: 8 keys of one head dim) is read
// from the transposed V pages.  Key order inside each 16-key group of the
// V^T LDS tile is permuted (bits 2 and 3 of the key index swapped) so the 8
// keys a lane needs are one 16-byte LDS read.
//
// Roofline: dense MFMA.  Algorithmic flops per visible (query, key) pair and
// head are 4 * head_dim (2 for Q K^T, 2 for P V).
#include "attn_common.h"

namespace wf {

namespace {

constexpr int BN = kTileKeys;      // keys per LDS tile
constexpr int BM = kBlockMF32;     // query rows per workgroup (fp32 and staged kernels)
constexpr int NT = 256;            // threads per workgroup (fp32 and staged kernels)
static_assert(kBlockMF32 == kBlockMStaged, "fp32 and staged kernels share BM");
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

// Keep bf16 element e of v only where bit e of m is set.
__device__ __forceinline__ uint4 mask_bf16x8(uint4 v, uint32_t m) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (!((m >> e) & 1u)) w[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
  return make_uint4(w[0], w[1], w[2], w[3]);
}

namespace staged {

// ---------------------------------------------------------------------------
// bf16 Q with bf16 or E4M3FN K/V: register-staged tile loads.  Serves E4M3FN
// caches (converted to bf16 on the way into LDS) and bf16 caches the DMA
// kernel below does not take (pages under 64 tokens, caches of 4 GiB or more).
//
// LDS holds two K tiles and two V^T tiles (bf16).  Rows are padded by 16
// bytes (K: 64 keys x (2D+16) B; V^T: D dims x (128+16) B) so that the 8 (or
// 16) lanes an LDS cycle serves hit distinct banks and every fragment access
// is a fixed immediate offset from one per-lane base address.  Inside each
// 16-key group of a V^T row the keys are stored in the order the P^T operand
// consumes them (bits 2 and 3 of the key index swapped).
//
// Software pipeline (one barrier per 64-key tile).  Iteration j:
//   issue global loads of K[j+2] and V[j+1];
//   S[j+1] = K[j+1] Q^T  (MFMA, independent of ...)
//   softmax(S[j]) -> P[j] (VALU), so the two interleave;
//   O^T += V^T[j] P^T[j] (MFMA);
//   write K[j+2], V[j+1] into the LDS buffers freed by iteration j-1.
// ---------------------------------------------------------------------------
template <int D, bool FP8KV>
struct Geo {
  static constexpr int ESZ = FP8KV ? 1 : 2;       // cache bytes per element
  static constexpr int KROW = 2 * D + 16;         // LDS bytes per K row
  static constexpr int KTILE = BN * KROW;
  static constexpr int VROW = 2 * BN + 16;        // LDS bytes per V^T row
  static constexpr int VTILE = D * VROW;
  static constexpr int LDS = 2 * KTILE + 2 * VTILE;
  static constexpr int KCH = D / 8;               // 8-element chunks per K row
  static constexpr int KPASS = NT / KCH;          // keys per loader pass
  static constexpr int KITEMS = BN / KPASS;       // K chunks per thread
  static constexpr int VPASS = NT / 8;            // V^T rows per loader pass
  static constexpr int VITEMS = D / VPASS;        // V 8-key groups per thread
};

// Register staging of one tile's K (or V) slice owned by this thread.
template <int N>
struct Stage {
  uint4 w[N];    // bf16 payload, or E4M3FN codes in .x/.y
  float sc[N];   // E4M3FN block scale (1 otherwise)
  uint8_t m[N];  // per-element validity (8 keys / 8 dims); 0xFF = all valid
};

// Per-tile page geometry (uniform): page and offset of the tile's first key.
struct TilePos {
  int32_t page0, off0;
  bool fast;  // all keys valid and inside one page
};

__device__ __forceinline__ TilePos tile_pos(const AttnParams& p, const ChunkDesc& cd, const int32_t* table,
                                            int t) {
  TilePos tp;
  const int rel0 = t * BN;
  locate(cd.map, p.divP, p.divT, table, (uint32_t)rel0, tp.page0, tp.off0);
  tp.fast = rel0 >= cd.lead && rel0 + BN <= cd.lead + cd.nkeys && tp.off0 + BN <= p.P;
  return tp;
}

template <int D, bool FP8KV>
__device__ __forceinline__ void load_k(Stage<Geo<D, FP8KV>::KITEMS>& st, const AttnParams& p,
                                       const ChunkDesc& cd, const int32_t* table, int head, int t) {
  using G = Geo<D, FP8KV>;
  const int tid = threadIdx.x;
  const int kq = tid / G::KCH, ch = tid - kq * G::KCH;
  const TilePos tp = tile_pos(p, cd, table, t);
  const uint8_t* kb = (const uint8_t*)p.k;
  if (tp.fast) {
    const uint8_t* base = kb + (((int64_t)tp.page0 * p.H + head) * p.P + tp.off0) * (D * G::ESZ);
    const int64_t sbase = ((int64_t)tp.page0 * p.H + head) * p.nblk;
#pragma unroll
    for (int r = 0; r < G::KITEMS; ++r) {
      const int key = kq + r * G::KPASS;
      const uint8_t* a = base + key * (D * G::ESZ) + ch * (8 * G::ESZ);
      if constexpr (FP8KV) {
        const uint2 raw = *(const uint2*)a;
        st.w[r] = make_uint4(raw.x, raw.y, 0, 0);
        st.sc[r] = p.ks[sbase + ((tp.off0 + key) >> 7)];
      } else {
        st.w[r] = *(const uint4*)a;
        st.sc[r] = 1.f;
      }
      st.m[r] = 0xFF;
    }
    return;
  }
  const int lo = cd.lead, hi = cd.lead + cd.nkeys;
#pragma unroll
  for (int r = 0; r < G::KITEMS; ++r) {
    const int key = kq + r * G::KPASS;
    const int rel = t * BN + key;
    st.w[r] = make_uint4(0, 0, 0, 0);
    st.sc[r] = 1.f;
    st.m[r] = 0;
    if (rel >= lo && rel < hi) {
      int32_t page = tp.page0, off = tp.off0 + key;
      if (off >= p.P) locate(cd.map, p.divP, p.divT, table, (uint32_t)rel, page, off);
      const int64_t row = ((int64_t)page * p.H + head) * p.P + off;
      const uint8_t* a = kb + row * (D * G::ESZ) + ch * (8 * G::ESZ);
      if constexpr (FP8KV) {
        const uint2 raw = *(const uint2*)a;
        st.w[r] = make_uint4(raw.x, raw.y, 0, 0);
        st.sc[r] = p.ks[((int64_t)page * p.H + head) * p.nblk + (off >> 7)];
      } else {
        st.w[r] = *(const uint4*)a;
      }
      st.m[r] = 0xFF;
    }
  }
}

template <int D, bool FP8KV>
__device__ __forceinline__ void load_v(Stage<Geo<D, FP8KV>::VITEMS>& st, const AttnParams& p,
                                       const ChunkDesc& cd, const int32_t* table, int head, int t) {
  using G = Geo<D, FP8KV>;
  const int tid = threadIdx.x;
  const int vd = tid >> 3, a8 = tid & 7;
  const TilePos tp = tile_pos(p, cd, table, t);
  const uint8_t* vb = (const uint8_t*)p.v;
  const int rel = t * BN + 8 * a8;
  int32_t page = tp.page0, off = tp.off0 + 8 * a8;
  uint8_t m = 0xFF;
  if (!tp.fast) {
    const int lo = cd.lead, hi = cd.lead + cd.nkeys;
    m = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) m |= (uint8_t)((rel + e >= lo && rel + e < hi) ? 1u << e : 0u);
    if (off >= p.P) locate(cd.map, p.divP, p.divT, table, (uint32_t)rel, page, off);
  }
  const uint8_t* base = vb + (((int64_t)page * p.H + head) * D * p.P + off) * G::ESZ;
  float sc = 1.f;
  if constexpr (FP8KV) {
    if (m) sc = p.vs[((int64_t)page * p.H + head) * p.nblk + (off >> 7)];
  }
#pragma unroll
  for (int r = 0; r < G::VITEMS; ++r) {
    const int d = vd + r * G::VPASS;
    st.w[r] = make_uint4(0, 0, 0, 0);
    st.sc[r] = sc;
    st.m[r] = m;
    if (m) {
      const uint8_t* a = base + (int64_t)d * p.P * G::ESZ;
      if constexpr (FP8KV) {
        const uint2 raw = *(const uint2*)a;
        st.w[r] = make_uint4(raw.x, raw.y, 0, 0);
      } else {
        st.w[r] = *(const uint4*)a;
      }
    }
  }
}

// E4M3FN pairs -> bf16 pairs times a float32 block scale.  The hardware
// conversion (v_cvt_scalef32_pk_f32_fp8, OCP E4M3FN on gfx950) applies its own
// scale operand as a power of two, so it is given 1.0 (exact) and the block
// scale is a separate fp32 multiply.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(f32x2 f, float scale) {
  bf16x2 b = {(__bf16)(f[0] * scale), (__bf16)(f[1] * scale)};
  return __builtin_bit_cast(uint32_t, b);
}
__device__ __forceinline__ uint4 fp8x8_to_bf16x8(uint4 raw, float scale) {
  return make_uint4(pack_bf16x2(__builtin_amdgcn_cvt_scalef32_pk_f32_fp8(raw.x, 1.0f, false), scale),
                    pack_bf16x2(__builtin_amdgcn_cvt_scalef32_pk_f32_fp8(raw.x, 1.0f, true), scale),
                    pack_bf16x2(__builtin_amdgcn_cvt_scalef32_pk_f32_fp8(raw.y, 1.0f, false), scale),
                    pack_bf16x2(__builtin_amdgcn_cvt_scalef32_pk_f32_fp8(raw.y, 1.0f, true), scale));
}
__device__ __forceinline__ uint4 mask_bf16x8(uint4 v, uint32_t m) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (!((m >> e) & 1u)) w[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
  return make_uint4(w[0], w[1], w[2], w[3]);
}

template <int D, bool FP8KV>
__device__ __forceinline__ void store_k(const Stage<Geo<D, FP8KV>::KITEMS>& st, char* kbuf) {
  using G = Geo<D, FP8KV>;
  const int tid = threadIdx.x;
  const int kq = tid / G::KCH, ch = tid - kq * G::KCH;
  char* base = kbuf + kq * G::KROW + ch * 16;
#pragma unroll
  for (int r = 0; r < G::KITEMS; ++r) {
    uint4 v = st.w[r];
    if constexpr (FP8KV) v = fp8x8_to_bf16x8(v, st.sc[r]);
    *(uint4*)(base + r * G::KPASS * G::KROW) = v;
  }
}

template <int D, bool FP8KV>
__device__ __forceinline__ void store_v(const Stage<Geo<D, FP8KV>::VITEMS>& st, char* vbuf) {
  using G = Geo<D, FP8KV>;
  const int tid = threadIdx.x;
  const int vd = tid >> 3, a8 = tid & 7;
  // keys 8a..8a+3 -> 16-byte chunk (a & ~1), keys 8a+4..8a+7 -> chunk (a | 1); byte 8*(a & 1)
  char* base = vbuf + vd * G::VROW + ((a8 & ~1) << 4) + ((a8 & 1) << 3);
#pragma unroll
  for (int r = 0; r < G::VITEMS; ++r) {
    uint4 v = st.w[r];
    if constexpr (FP8KV) v = fp8x8_to_bf16x8(v, st.sc[r]);
    if (st.m[r] != 0xFF) v = mask_bf16x8(v, st.m[r]);
    char* row = base + r * G::VPASS * G::VROW;
    *(uint2*)row = make_uint2(v.x, v.y);
    *(uint2*)(row + 16) = make_uint2(v.z, v.w);
  }
}

template <int D, bool FP8KV>
__device__ __forceinline__ void qk_tile(f32x16 (&s)[2], const char* kbuf, const bf16x8 (&qf)[D / 16],
                                        int lane_off) {
  using G = Geo<D, FP8KV>;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
#pragma unroll
    for (int i = 0; i < 16; ++i) s[b][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const bf16x8 kf = *(const bf16x8*)(kbuf + lane_off + b * 32 * G::KROW + ks * 32);
      s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[b], 0, 0, 0);
    }
  }
}


template <int D>
__device__ __forceinline__ void softmax_tile(f32x16 (&s)[2], bf16x8 (&pf)[2][2], f32x16 (&o)[D / 32], float& m,
                                             float& l, float scale_log2, int rel0, int lo, int hi, int hf) {
  if (rel0 < lo || rel0 + BN > hi) {
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int rel = rel0 + b * 32 + 8 * (i >> 2) + 4 * hf + (i & 3);
        if (rel < lo || rel >= hi) s[b][i] = -INFINITY;
      }
  }
  float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[b][i]);
  mx = half_max(mx) * scale_log2;
  // Exact lazy rescaling: the reference point m only moves when the running
  // maximum exceeds it by more than the threshold; O and l always share m.
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
  const float nm = -m;
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  const bf16x2v ones = {(__bf16)1.0f, (__bf16)1.0f};
  float l0 = 0.f, l1 = 0.f;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 8; r += 2) {
        const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][8 * u + r], scale_log2, nm));
        const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][8 * u + r + 1], scale_log2, nm));
        const bf16x2v pk = {(__bf16)e0, (__bf16)e1};
        pf[b][u][r] = pk[0];
        pf[b][u][r + 1] = pk[1];
        if (r & 2)
          l1 = __builtin_amdgcn_fdot2_f32_bf16(pk, ones, l1, false);
        else
          l0 = __builtin_amdgcn_fdot2_f32_bf16(pk, ones, l0, false);
      }
  l += l0 + l1;
}

template <int D, bool FP8KV>
__device__ __forceinline__ void pv_tile(f32x16 (&o)[D / 32], const char* vbuf, const bf16x8 (&pf)[2][2],
                                        int lane_off) {
  using G = Geo<D, FP8KV>;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bf16x8 vf = *(const bf16x8*)(vbuf + lane_off + db * 32 * G::VROW + (4 * b + 2 * u) * 16);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[b][u], o[db], 0, 0, 0);
      }
}

template <int D, bool FP8KV>
__global__ __launch_bounds__(NT, 2) void attn_fwd_bf16_kernel(const AttnParams p) {
  using G = Geo<D, FP8KV>;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  extern __shared__ __align__(16) char smem[];
  __shared__ int32_t table[WF_MAX_TABLE_LEN];
  char* kbuf0 = smem;
  char* kbuf1 = smem + G::KTILE;
  char* vbuf0 = smem + 2 * G::KTILE;
  char* vbuf1 = vbuf0 + G::VTILE;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lq = lane & 31;  // query column owned by this lane
  const int hf = lane >> 5;  // 32-lane half

  for (int i = tid; i < p.T; i += NT) table[i] = p.table[i];

  const Item it = decode_item(p, blockIdx.x);
  const ChunkDesc cd = p.chunk[it.c];
  const int head = it.head;
  const int qrow = it.qt * BM + wave * 32 + lq;
  const int row = cd.q_begin + qrow;
  const bool row_ok = qrow < cd.q_len;
  const int lo = cd.lead, hi = cd.lead + cd.nkeys;
  const int nt = (hi + BN - 1) / BN;
  const int k_lane = lq * G::KROW + hf * 16;
  const int v_lane = lq * G::VROW + hf * 16;

  bf16x8 qf[KS];
  {
    const __bf16* qp = (const __bf16*)p.q + ((int64_t)row * p.H + head) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (row_ok) v = *(const uint4*)(qp + ks * 16 + hf * 8);
      qf[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }
  f32x16 o[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[b][i] = 0.f;
  float m = -INFINITY, l = 0.f;

  __syncthreads();  // page table
  Stage<G::KITEMS> sk;
  Stage<G::VITEMS> sv;
  load_k<D, FP8KV>(sk, p, cd, table, head, 0);
  load_v<D, FP8KV>(sv, p, cd, table, head, 0);
  store_k<D, FP8KV>(sk, kbuf0);
  store_v<D, FP8KV>(sv, vbuf0);
  if (nt > 1) {
    load_k<D, FP8KV>(sk, p, cd, table, head, 1);
    store_k<D, FP8KV>(sk, kbuf1);
  }
  __syncthreads();

  f32x16 sa[2], sb[2];
  bf16x8 pf[2][2];
  qk_tile<D, FP8KV>(sa, kbuf0, qf, k_lane);

  // One pipeline step; `even` selects the buffer parity at compile time.
  auto step = [&](auto even_tag, f32x16(&s_cur)[2], f32x16(&s_next)[2], int j) {
    constexpr bool even = decltype(even_tag)::value;
    char* kb_next = even ? kbuf1 : kbuf0;  // holds K[j+1]
    char* kb_free = even ? kbuf0 : kbuf1;  // receives K[j+2]
    char* vb_cur = even ? vbuf0 : vbuf1;   // holds V[j]
    char* vb_free = even ? vbuf1 : vbuf0;  // receives V[j+1]
    const bool has1 = j + 1 < nt, has2 = j + 2 < nt;
    if (has2) load_k<D, FP8KV>(sk, p, cd, table, head, j + 2);
    if (has1) load_v<D, FP8KV>(sv, p, cd, table, head, j + 1);
    if (has1) qk_tile<D, FP8KV>(s_next, kb_next, qf, k_lane);
    softmax_tile<D>(s_cur, pf, o, m, l, p.scale_log2, j * BN, lo, hi, hf);
    pv_tile<D, FP8KV>(o, vb_cur, pf, v_lane);
    if (has2) store_k<D, FP8KV>(sk, kb_free);
    if (has1) store_v<D, FP8KV>(sv, vb_free);
    __syncthreads();
  };
  for (int j = 0; j < nt; j += 2) {
    step(std::true_type{}, sa, sb, j);
    if (j + 1 < nt) step(std::false_type{}, sb, sa, j + 1);
  }

  const float lt = half_sum(l);
  const float inv = 1.f / lt;
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
}

}  // namespace staged

// ---------------------------------------------------------------------------
// bf16 kernel with LDS-DMA tile loads (bf16 cache, pages >= 64 tokens,
// cache < 4 GiB).
//
// One workgroup = 8 waves (2 per SIMD) = 256 query rows of one head of one
// chunk; each wave owns 32 rows and keeps its Q^T fragments in VGPRs.  The 8
// waves share every K/V tile.
//
// Tiles reach LDS through global_load_lds_dwordx4 (16 bytes per lane, written
// to LDS at base + 16 * lane), so no VGPRs stage them.  Rows are padded by 16
// bytes (K: 2D+16 bytes, V^T: 144 bytes) so that the 16 lanes one LDS cycle
// serves hit distinct banks and every fragment read is an immediate offset
// from one per-lane base; DMA lanes that land on padding load a dummy chunk.
//   K half-tile [32 rows][D] bf16: LDS row r holds key pi(r) of the half-tile,
//     pi(8 j + 4 h + i) = 16 h + 4 j + i.  The MFMA A operand of lane l is
//     LDS row l % 32, so in the S^T accumulator lane-half h holds the 16
//     consecutive keys 16 h .. 16 h + 15 of the half-tile.
//   V^T tile [D][64 keys] bf16, keys in natural order.  Because of pi the 8
//     keys one P^T operand slot group needs are contiguous: one 16-byte LDS
//     read per MFMA, and V^T rows are plain 16-byte DMA chunks.
//
// Pipeline.  The key range is walked in 32-key half-steps q; one barrier per
// 64-key tile j (half-steps 2j, 2j+1).  Entering half-step q the wave holds
// S[q] (masked) and a reference maximum m within 2^8 of S[q]'s row maxima,
// with O and l relative to m:
//   [A] S[q+1] = K[q+1] Q^T (MFMA)  ||  P[q] = exp2(S[q] - m), row sums
//   [B] O^T += V^T[q] P^T[q] (MFMA) ||  mask S[q+1], row max of S[q+1]
//   [C] rare exact rescale when a row max of S[q+1] exceeds m by more than 8
// At the start of tile j the DMA for K half-tiles 2j+3, 2j+4 (ring of four)
// and V tile j+1 (double buffer) is issued into buffers the previous tile
// freed; V tile j's keys outside the chunk's range are zeroed first if it is
// an edge tile (0 * NaN would poison P V); the tile ends with a wait for its
// DMA and a barrier.
// ---------------------------------------------------------------------------
namespace dma {

constexpr int NW = 8;         // waves per workgroup
constexpr int NTD = 64 * NW;  // threads per workgroup
constexpr int BMD = 32 * NW;  // query rows per workgroup
constexpr int HK = 32;        // keys per K half-tile
static_assert(BMD == kBlockMDma, "host and kernel disagree on the DMA kernel block size");

template <int D>
struct Geo {
  static constexpr int KROW = 2 * D + 16;                 // LDS bytes per K row (padded)
  static constexpr int KCH = D / 8;                       // 16-byte data chunks per K row
  static constexpr int KDMA = (HK * KROW + 1023) / 1024;  // DMA instructions per K half-tile
  static constexpr int KHALF = KDMA * 1024;               // LDS bytes per K half-tile buffer
  static constexpr int VROW = 2 * BN + 16;                // LDS bytes per V^T row (padded)
  static constexpr int VDMA = (D * VROW + 1023) / 1024;   // DMA instructions per V^T tile
  static constexpr int VTILE = VDMA * 1024;               // LDS bytes per V^T tile buffer
  static constexpr int KPW = (KDMA + NW - 1) / NW;        // max K instructions per wave
  static constexpr int VPW = (VDMA + NW - 1) / NW;        // max V instructions per wave
};

// Per-lane constants of this wave's DMA instructions: source byte offset
// relative to the run geometry base and the run-relative key of the 16-byte
// chunk (for the page-break select).  Wave w issues instructions w, w + NW, ...
// of each K half-tile and V^T tile.  Lanes that land on row padding (or past
// the last row) load the run's first chunk, a valid address, into the slack.
template <int D>
struct DmaPlan {
  uint32_t koff[Geo<D>::KPW];
  int32_t kkey[Geo<D>::KPW];
  uint32_t voff[Geo<D>::VPW];
  int32_t vkey[Geo<D>::VPW];
};

template <int D>
__device__ __forceinline__ DmaPlan<D> make_plan(int wave, int lane, int P) {
  using G = Geo<D>;
  DmaPlan<D> pl;
#pragma unroll
  for (int r = 0; r < G::KPW; ++r) {
    const int y = 1024 * (wave + NW * r) + 16 * lane;  // LDS byte inside the K half-tile buffer
    const int row = y / G::KROW, pc = (y % G::KROW) / 16;
    const bool data = row < HK && pc < G::KCH;
    const int key = 16 * ((row >> 2) & 1) + 4 * (row >> 3) + (row & 3);  // pi(row)
    pl.kkey[r] = data ? key : 0;
    pl.koff[r] = data ? (uint32_t)(key * 2 * D + pc * 16) : 0u;
  }
#pragma unroll
  for (int r = 0; r < G::VPW; ++r) {
    const int y = 1024 * (wave + NW * r) + 16 * lane;  // LDS byte inside the V^T tile buffer
    const int d = y / G::VROW, pc = (y % G::VROW) / 16;
    const bool data = d < D && pc < 8;
    pl.vkey[r] = data ? pc * 8 : 0;
    pl.voff[r] = data ? (uint32_t)(d * P * 2 + pc * 16) : 0u;
  }
  return pl;
}

// DMA the K half-tile at cursor c (32 keys) into khalf.  Runs inside one page
// (all but about one in P / 32) add the run's byte base to the lane's plan
// offset; a run that crosses a page selects its page per lane.  Sources are
// the cache base plus one 32-bit offset per lane (the scalar-base form of the
// load).
template <int D>
__device__ __forceinline__ void dma_k(const AttnParams& p, const Cursor& c, const DmaPlan<D>& pl, char* khalf,
                                      int wave) {
  using G = Geo<D>;
  if (p.P - c.off >= HK) {
    const uint32_t soff = c.k0 + (uint32_t)c.off * (2 * D);
#pragma unroll
    for (int r = 0; r < G::KPW; ++r)
      if ((NW - 1) + NW * r < G::KDMA || wave + NW * r < G::KDMA)
        dma16((const char*)p.k + (soff + pl.koff[r]), khalf + 1024 * (wave + NW * r));
    return;
  }
  const RunGeom g = run_geom<2 * D, 2>(p, c);
#pragma unroll
  for (int r = 0; r < G::KPW; ++r)
    if (wave + NW * r < G::KDMA)
      dma16((const char*)p.k + ((pl.kkey[r] < g.split ? g.kb0 : g.kb1) + pl.koff[r]),
            khalf + 1024 * (wave + NW * r));
}

// DMA the V^T tile at cursor c (64 keys) into vbuf (same scheme as dma_k).
template <int D>
__device__ __forceinline__ void dma_v(const AttnParams& p, const Cursor& c, const DmaPlan<D>& pl, char* vbuf,
                                      int wave) {
  using G = Geo<D>;
  if (p.P - c.off >= BN) {
    const uint32_t soff = c.v0 + (uint32_t)c.off * 2;
#pragma unroll
    for (int r = 0; r < G::VPW; ++r)
      if ((NW - 1) + NW * r < G::VDMA || wave + NW * r < G::VDMA)
        dma16((const char*)p.v + (soff + pl.voff[r]), vbuf + 1024 * (wave + NW * r));
    return;
  }
  const RunGeom g = run_geom<2 * D, 2>(p, c);
#pragma unroll
  for (int r = 0; r < G::VPW; ++r)
    if (wave + NW * r < G::VDMA)
      dma16((const char*)p.v + ((pl.vkey[r] < g.split ? g.vb0 : g.vb1) + pl.voff[r]),
            vbuf + 1024 * (wave + NW * r));
}

// Zero the keys of V^T tile t (in LDS) that lie outside [lo, hi).
template <int D>
__device__ __forceinline__ void zero_v_outside(char* vbuf, int t, int lo, int hi) {
  for (int idx = threadIdx.x; idx < D * 8; idx += NTD) {
    const int d = idx >> 3, c = idx & 7;
    const int rel = t * BN + 8 * c;
    if (rel >= lo && rel + 8 <= hi) continue;
    uint32_t m = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) m |= (rel + e >= lo && rel + e < hi) ? 1u << e : 0u;
    uint4* a = (uint4*)(vbuf + d * Geo<D>::VROW + 16 * c);
    *a = mask_bf16x8(*a, m);
  }
}

// One 32-key half-step as explicitly ordered stages.  Stage i of [A] issues
// the LDS read of the K fragment two stages ahead, one MFMA of the S[q+1]
// chain (k-step i), and exponent / bf16 packing / row sum for two elements of
// S[q].  Stage i of [B] issues the V fragment read two stages ahead, one O^T
// MFMA (d block i % DB, P slot group i / DB), and masking + row max for two
// elements of S[q+1].  Stages are separated by scheduling barriers and each
// stage's VALU results are pinned with empty asm statements, so at most three
// fragments are live and every MFMA is followed by independent VALU work.
// kx / vx are this lane's LDS byte offsets of its K row chunk (k-step 0) and
// of its V^T row chunk (d block 0, slot group 0).
template <int D, bool MASK>
__device__ __forceinline__ float half_step(const f32x16& s_cur, f32x16& s_next, f32x16 (&o)[D / 32],
                                           const bf16x8 (&qf)[D / 16], const char* khalf, const char* vtile,
                                           int kx, int vx, float m, float& l,
                                           float sl2, int key_next0, int lo, int hi, int hf) {
  constexpr int NA = D / 16;        // QK^T MFMAs (k-steps) per half-step
  constexpr int NB = 2 * (D / 32);  // PV MFMAs per half-step
  constexpr int DB = D / 32;
  constexpr int EA = 16 / NA;       // S[q] elements per [A] stage
  constexpr int EB = 16 / NB;       // S[q+1] elements per [B] stage
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  const bf16x2v ones = {(__bf16)1.0f, (__bf16)1.0f};
  const float nm = -m;
  bf16x8 pf[2];
  bf16x8 frag[3];
  float lsum[2] = {0.f, 0.f};
  auto kaddr = [&](int ks) { return (const bf16x8*)(khalf + kx + 32 * ks); };
  frag[0] = *kaddr(0);
  frag[1] = *kaddr(1);
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    if (i + 2 < NA) frag[(i + 2) % 3] = *kaddr(i + 2);
    if (i == 0) {
      f32x16 z;
#pragma unroll
      for (int e = 0; e < 16; ++e) z[e] = 0.f;
      s_next = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag[0], qf[0], z, 0, 0, 0);
    } else {
      s_next = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag[i % 3], qf[i], s_next, 0, 0, 0);
    }
#pragma unroll
    for (int e = EA * i; e < EA * (i + 1); e += 2) {
      const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[e], sl2, nm));
      const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[e + 1], sl2, nm));
      const bf16x2v pk = {(__bf16)e0, (__bf16)e1};
      pf[e >> 3][e & 7] = pk[0];
      pf[e >> 3][(e & 7) + 1] = pk[1];
      lsum[(e >> 1) & 1] = __builtin_amdgcn_fdot2_f32_bf16(pk, ones, lsum[(e >> 1) & 1], false);
    }
    asm volatile("" : "+v"(lsum[0]), "+v"(lsum[1]));
    __builtin_amdgcn_sched_barrier(0);
  }
  l += lsum[0] + lsum[1];
  auto vaddr = [&](int i) { return (const bf16x8*)(vtile + vx + 16 * (i / DB) + (i % DB) * 32 * Geo<D>::VROW); };
  frag[0] = *vaddr(0);
  frag[1] = *vaddr(1);
  float mx[2] = {-INFINITY, -INFINITY};
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    if (i + 2 < NB) frag[(i + 2) % 3] = *vaddr(i + 2);
    o[i % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag[i % 3], pf[i / DB], o[i % DB], 0, 0, 0);
#pragma unroll
    for (int e = EB * i; e < EB * (i + 1); e += 2) {
      float a0 = s_next[e], a1 = s_next[e + 1];
      if constexpr (MASK) {
        const int key = key_next0 + 16 * hf + e;  // key of S^T element e
        a0 = (key >= lo && key < hi) ? a0 : -INFINITY;
        a1 = (key + 1 >= lo && key + 1 < hi) ? a1 : -INFINITY;
        s_next[e] = a0;
        s_next[e + 1] = a1;
      }
      mx[(e >> 1) & 1] = fmaxf(mx[(e >> 1) & 1], fmaxf(a0, a1));
    }
    asm volatile("" : "+v"(mx[0]), "+v"(mx[1]));
    __builtin_amdgcn_sched_barrier(0);
  }
  return half_max(fmaxf(mx[0], mx[1])) * sl2;
}

// LDS buffers of the DMA kernel.  K half-tiles form a ring of four, V^T tiles
// are double-buffered.  They are separate __shared__ objects (see the kernel)
// so the compiler can tell that DMA into one buffer does not alias reads of
// another.
struct Bufs {
  char *kh0, *kh1, *kh2, *kh3, *vbuf0, *vbuf1;
};

// One query tile (item) of chunk cd over its 64-key tiles [j0, j1).  slot < 0:
// the segment is the whole key range and the block writes O (and LSE);
// otherwise it stores its unnormalised partial result in workspace slot
// `slot` for the merge kernel.
template <int D>
__device__ __forceinline__ void segment(const AttnParams& p, const ChunkDesc& cd, int qt, int head, int j0,
                                        int j1, int slot, const Bufs& bf, const DmaPlan<D>& plan, int wave,
                                        int lane) {
  using G = Geo<D>;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  char* const kh0 = bf.kh0;
  char* const kh1 = bf.kh1;
  char* const kh2 = bf.kh2;
  char* const kh3 = bf.kh3;
  char* const vbuf0 = bf.vbuf0;
  char* const vbuf1 = bf.vbuf1;
  const int lq = lane & 31;  // query column owned by this lane
  const int hf = lane >> 5;  // 32-lane half
  const int qrow = qt * BMD + wave * 32 + lq;
  const int row = cd.q_begin + qrow;
  const bool row_ok = qrow < cd.q_len;
  // Keys relative to the segment's first tile (logical base kv_begin - lead + 64 j0).
  const int base = BN * j0;
  const int lo = max(cd.lead - base, 0);
  const int hi = min(cd.lead + cd.nkeys, BN * j1) - base;
  const int nt = (hi + BN - 1) / BN;  // 64-key tiles
  const int nh = (hi + HK - 1) / HK;  // 32-key half-tiles
  const float sl2 = p.scale_log2;
  const int kx = lq * G::KROW + 16 * hf;             // K row lq, chunk hf (k-step 0)
  const int vx0 = lq * G::VROW + 16 * (2 * hf);      // V^T row lq, keys 16 hf .. (first half of a tile)
  const int vx1 = lq * G::VROW + 16 * (4 + 2 * hf);  // ... keys 32 + 16 hf .. (second half)

  // K half-tiles 0..2 and V tile 0 in flight while Q is fetched
  Cursor kcur = cursor_at<2 * D>(p, cd, head, base), vcur = kcur;
  dma_k<D>(p, kcur, plan, kh0, wave);
  advance<2 * D>(p, head, kcur, HK);
  if (nh > 1) dma_k<D>(p, kcur, plan, kh1, wave);
  advance<2 * D>(p, head, kcur, HK);
  if (nh > 2) dma_k<D>(p, kcur, plan, kh2, wave);
  advance<2 * D>(p, head, kcur, HK);
  dma_v<D>(p, vcur, plan, vbuf0, wave);
  advance<2 * D>(p, head, vcur, BN);

  bf16x8 qf[KS];
  {
    const __bf16* qp = (const __bf16*)p.q + ((int64_t)row * p.H + head) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (row_ok) v = *(const uint4*)(qp + ks * 16 + hf * 8);
      qf[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }
  f32x16 o[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[b][i] = 0.f;
  float l = 0.f;

  wait_vmcnt<0>();
  __syncthreads();
  if (lo > 0 || BN > hi) {  // tile 0 is an edge tile
    zero_v_outside<D>(vbuf0, 0, lo, hi);
    __syncthreads();
  }
  // S of half-tile 0 (it holds key lo < 8, so its row maxima are finite)
  f32x16 sa, sb;
#pragma unroll
  for (int i = 0; i < 16; ++i) sa[i] = 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const bf16x8 kf = *(const bf16x8*)(kh0 + kx + 32 * ks);
    sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sa, 0, 0, 0);
  }
  float m;
  {
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = 16 * hf + i;
      sa[i] = (key >= lo && key < hi) ? sa[i] : -INFINITY;
      mx = fmaxf(mx, sa[i]);
    }
    m = half_max(mx) * sl2;
  }
  __syncthreads();  // kh0 is free for half-tile 4

  // Tile step j: half-steps 2j (S in sa) and 2j+1 (S in sb).  EVEN selects
  // the ring parity: even j reads K halves in kh1, kh2 and refills kh3, kh0;
  // odd j reads kh3, kh0 and refills kh1, kh2.  M0 / M1: half-tiles 2j+1 /
  // 2j+2 need masking.
  auto step = [&](auto even_tag, auto m0_tag, auto m1_tag, int j) {
    constexpr bool even = decltype(even_tag)::value;
    char* const k_a = even ? kh1 : kh3;   // half-tile 2j+1
    char* const k_b = even ? kh2 : kh0;   // half-tile 2j+2
    char* const k_f0 = even ? kh3 : kh1;  // receives half-tile 2j+3
    char* const k_f1 = even ? kh0 : kh2;  // receives half-tile 2j+4
    char* const vb_cur = even ? vbuf0 : vbuf1;
    char* const vb_free = even ? vbuf1 : vbuf0;
    // The wave index passes through an empty asm so that the LDS destinations
    // (one per buffer and instruction) are formed at their use instead of being
    // hoisted into long-lived scalar registers.
    int wv = wave;
    asm volatile("" : "+s"(wv));
    if (2 * j + 3 < nh) dma_k<D>(p, kcur, plan, k_f0, wv);
    advance<2 * D>(p, head, kcur, HK);
    if (2 * j + 4 < nh) dma_k<D>(p, kcur, plan, k_f1, wv);
    advance<2 * D>(p, head, kcur, HK);
    if (j + 1 < nt) dma_v<D>(p, vcur, plan, vb_free, wv);
    advance<2 * D>(p, head, vcur, BN);
    if (j > 0 && 64 * j + 64 > hi) {  // edge tile (tile 0 was handled before the loop)
      zero_v_outside<D>(vb_cur, j, lo, hi);
      __syncthreads();
    }
    float mx = half_step<D, decltype(m0_tag)::value>(sa, sb, o, qf, k_a, vb_cur, kx, vx0, m, l,
                                                     sl2, (2 * j + 1) * HK, lo, hi, hf);
    if (2 * j + 1 < nh) {
      maybe_rescale<D>(mx, m, l, o);
      mx = half_step<D, decltype(m1_tag)::value>(sb, sa, o, qf, k_b, vb_cur, kx, vx1, m, l,
                                                 sl2, (2 * j + 2) * HK, lo, hi, hf);
      if (2 * j + 2 < nh) maybe_rescale<D>(mx, m, l, o);
    }
    wait_vmcnt<0>();
    __syncthreads();
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  // Half-tiles q >= 1 need masking iff they reach past hi (lo < 8 only affects
  // half-tile 0, masked before the loop): iff q >= qe.
  const int qe = hi / HK;
  auto dispatch = [&](auto even_tag, int j) {
    if (2 * j + 2 < qe)
      step(even_tag, F_{}, F_{}, j);
    else
      step(even_tag, T_{}, T_{}, j);
  };
  for (int j = 0; j < nt; j += 2) {
    dispatch(T_{}, j);
    if (j + 1 < nt) dispatch(F_{}, j + 1);
  }

  const float lt = half_sum(l);
  if (slot < 0) {
    const float inv = 1.f / lt;
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
        *(f32x4*)(orow + db * 32 + 8 * g + 4 * hf) = {o[db][4 * g + 0], o[db][4 * g + 1], o[db][4 * g + 2],
                                                       o[db][4 * g + 3]};
    if (hf == 0) {
      ws[BMD * D + r] = m;
      ws[BMD * D + BMD + r] = lt;
    }
  }
}

template <int D>
__global__ __launch_bounds__(NTD, 2) void attn_fwd_dma_kernel(const AttnParams p) {
  using G = Geo<D>;
  __shared__ __align__(1024) char kh0[G::KHALF];
  __shared__ __align__(1024) char kh1[G::KHALF];
  __shared__ __align__(1024) char kh2[G::KHALF];
  __shared__ __align__(1024) char kh3[G::KHALF];
  __shared__ __align__(1024) char vbuf0[G::VTILE];
  __shared__ __align__(1024) char vbuf1[G::VTILE];
  const Bufs bf{kh0, kh1, kh2, kh3, vbuf0, vbuf1};

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const DmaPlan<D> plan = make_plan<D>(wave, lane, p.P);

  walk_segments(p, (int)blockIdx.x, [&](int item, int j0, int j1, int slot) {
    const Item it = decode_item(p, item);
    segment<D>(p, p.chunk[it.c], it.qt, it.head, j0, j1, slot, bf, plan, wave, lane);
  });
}

// Merge the partial results of the split schedule: for each row,
// O = sum_k 2^(m_k - M) O_k / sum_k 2^(m_k - M) l_k with M = max_k m_k (the
// log-sum-exp combination of attention over disjoint key sets).  One block
// per (item, kMergeRows rows); the item's partials are its m A parts (slots
// part * n + item) and, if b > 0, its m B parts.
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(const AttnParams p) {
  constexpr int C4 = D / 4;            // float4 columns per row
  constexpr int RPP = 256 / C4;        // rows per pass
  constexpr int MAXP = 16;             // partials held in registers
  const SplitSched& sp = p.sp;
  const int nrb = BMD / kMergeRows;
  const int item = blockIdx.x / nrb;
  const int r0 = (blockIdx.x - item * nrb) * kMergeRows;
  const Item it = decode_item(p, item);
  const ChunkDesc& cd = p.chunk[it.c];
  const int na = sp.n * sp.m;
  const int np = sp.b > 0 ? 2 * sp.m : sp.m;
  int slots[MAXP];
#pragma unroll
  for (int k = 0; k < MAXP; ++k) {
    const int part = k % sp.m;
    slots[k] = k >= np ? 0 : k < sp.m ? part * sp.n + item : na + b_index(p, item, part);
  }
  const int tid = threadIdx.x;
  const int c4 = tid % C4;
  const int64_t sf = ws_slot_floats(D);
  for (int r = r0 + tid / C4; r < r0 + kMergeRows; r += RPP) {
    const int qrow = it.qt * BMD + r;
    if (qrow >= cd.q_len) break;
    float mk[MAXP];
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < MAXP; ++k) {
      mk[k] = k < np ? p.ws[slots[k] * sf + BMD * D + r] : -INFINITY;
      M = fmaxf(M, mk[k]);
    }
    float L = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < MAXP; ++k) {
      if (k >= np) break;
      const float* ws = p.ws + slots[k] * sf;
      const float w = __builtin_amdgcn_exp2f(mk[k] - M);
      L += w * ws[BMD * D + BMD + r];
      const f32x4 v = *(const f32x4*)(ws + (int64_t)r * D + 4 * c4);
      acc += w * v;
    }
    const float inv = 1.f / L;
    const int row = cd.q_begin + qrow;
    bf16x4 ov = {(__bf16)(acc[0] * inv), (__bf16)(acc[1] * inv), (__bf16)(acc[2] * inv), (__bf16)(acc[3] * inv)};
    *(bf16x4*)((__bf16*)p.o + ((int64_t)row * p.H + it.head) * D + 4 * c4) = ov;
    if (p.lse != nullptr && c4 == 0) p.lse[(int64_t)it.head * p.nq + row] = (M + __log2f(L)) * kLn2;
  }
}

}  // namespace dma

// ---------------------------------------------------------------------------
// fp32 kernel (tight-tolerance path): V_MFMA_F32_32X32X2_F32, 32-key tiles,
// single-buffered.  Same S^T formulation as the bf16 kernel.
// ---------------------------------------------------------------------------
constexpr int BN32 = 32;

template <int D>
__global__ __launch_bounds__(NT) void attn_fwd_f32_kernel(const AttnParams p) {
  constexpr int KS = D / 2;
  constexpr int DB = D / 32;
  constexpr int KST = D + 2;       // LDS K row stride (floats)
  constexpr int VST = BN32 + 1;    // LDS V^T row stride (floats)
  __shared__ float ks_lds[BN32 * KST];
  __shared__ float vt_lds[D * VST];
  __shared__ int32_t table[WF_MAX_TABLE_LEN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lq = lane & 31;
  const int hf = lane >> 5;
  for (int i = tid; i < p.T; i += NT) table[i] = p.table[i];

  const Item it = decode_item(p, blockIdx.x);
  const ChunkDesc cd = p.chunk[it.c];
  const int head = it.head;
  const int row = cd.q_begin + it.qt * BM + wave * 32 + lq;
  const bool row_ok = (it.qt * BM + wave * 32 + lq) < cd.q_len;
  const int lo = cd.lead, hi = cd.lead + cd.nkeys;
  const int nt = (hi + BN32 - 1) / BN32;

  float qf[KS];
  {
    const float* qrow = (const float*)p.q + ((int64_t)row * p.H + head) * D;
#pragma unroll
    for (int k = 0; k < KS; ++k) qf[k] = row_ok ? qrow[2 * k + hf] : 0.f;
  }
  f32x16 o[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[b][i] = 0.f;
  float m = -INFINITY, l = 0.f;
  __syncthreads();

  for (int j = 0; j < nt; ++j) {
    const int rel0 = j * BN32;
    // K rows: BN32 keys x D floats
    for (int idx = tid; idx < BN32 * D; idx += NT) {
      const int key = idx / D, d = idx - key * D;
      const int rel = rel0 + key;
      float v = 0.f;
      if (rel >= lo && rel < hi) {
        int32_t page, off;
        locate(cd.map, p.divP, p.divT, table, (uint32_t)rel, page, off);
        v = ((const float*)p.k)[(((int64_t)page * p.H + head) * p.P + off) * D + d];
      }
      ks_lds[key * KST + d] = v;
    }
    // V^T rows: D dims x BN32 keys
    for (int idx = tid; idx < BN32 * D; idx += NT) {
      const int d = idx / BN32, key = idx - d * BN32;
      const int rel = rel0 + key;
      float v = 0.f;
      if (rel >= lo && rel < hi) {
        int32_t page, off;
        locate(cd.map, p.divP, p.divT, table, (uint32_t)rel, page, off);
        v = ((const float*)p.v)[(((int64_t)page * p.H + head) * D + d) * p.P + off];
      }
      vt_lds[d * VST + key] = v;
    }
    __syncthreads();

    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
    for (int k = 0; k < KS; ++k)
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(ks_lds[lq * KST + 2 * k + hf], qf[k], s, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int rel = rel0 + 8 * (i >> 2) + 4 * hf + (i & 3);
      if (rel < lo || rel >= hi) s[i] = -INFINITY;
    }
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = half_max(mx);
    const float m_new = fmaxf(m, mx * p.scale_log2);
    const float alpha = exp2f(m - m_new);
    m = m_new;
    float rs = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s[i] = exp2f(__builtin_fmaf(s[i], p.scale_log2, -m_new));
      rs += s[i];
    }
    l = l * alpha + rs;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
      const int d = db * 32 + lq;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 8 * (i >> 2) + 4 * hf + (i & 3);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vt_lds[d * VST + key], s[i], o[db], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  const float lt = half_sum(l);
  if (row_ok) {
    float* orow = (float*)p.o + ((int64_t)row * p.H + head) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v = {o[db][4 * g] / lt, o[db][4 * g + 1] / lt, o[db][4 * g + 2] / lt, o[db][4 * g + 3] / lt};
        *(f32x4*)(orow + db * 32 + 8 * g + 4 * hf) = v;
      }
    if (p.lse != nullptr && hf == 0) p.lse[(int64_t)head * p.nq + row] = (m + log2f(lt)) * kLn2;
  }
}


template <int D, bool FP8KV>
hipError_t launch_staged_t(const AttnParams& p, hipStream_t s) {
  const size_t lds = staged::Geo<D, FP8KV>::LDS;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&staged::attn_fwd_bf16_kernel<D, FP8KV>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((staged::attn_fwd_bf16_kernel<D, FP8KV>), dim3(p.num_items), dim3(NT), lds, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16_dma(const AttnParams& p, int head_dim, int grid, hipStream_t s) {
  if (head_dim == 128)
    hipLaunchKernelGGL(dma::attn_fwd_dma_kernel<128>, dim3(grid), dim3(dma::NTD), 0, s, p);
  else
    hipLaunchKernelGGL(dma::attn_fwd_dma_kernel<64>, dim3(grid), dim3(dma::NTD), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_attn_merge(const AttnParams& p, int head_dim, hipStream_t s) {
  const dim3 grid(p.num_items * (kBlockMDma / kMergeRows));
  if (head_dim == 128)
    hipLaunchKernelGGL(dma::attn_merge_kernel<128>, grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(dma::attn_merge_kernel<64>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t attn_dma_resident_blocks(int head_dim, int* blocks) {
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess)
    e = head_dim == 128
            ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, dma::attn_fwd_dma_kernel<128>, dma::NTD, 0)
            : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, dma::attn_fwd_dma_kernel<64>, dma::NTD, 0);
  *blocks = cus * (per_cu > 0 ? per_cu : 1);
  return e;
}

hipError_t launch_attn_bf16_staged(const AttnParams& p, int head_dim, hipStream_t s) {
  return head_dim == 128 ? launch_staged_t<128, false>(p, s) : launch_staged_t<64, false>(p, s);
}

hipError_t launch_attn_fp8kv(const AttnParams& p, int head_dim, hipStream_t s) {
  return head_dim == 128 ? launch_staged_t<128, true>(p, s) : launch_staged_t<64, true>(p, s);
}

hipError_t launch_attn_f32(const AttnParams& p, int head_dim, hipStream_t s) {
  if (head_dim == 128)
    hipLaunchKernelGGL(attn_fwd_f32_kernel<128>, dim3(p.num_items), dim3(NT), 0, s, p);
  else
    hipLaunchKernelGGL(attn_fwd_f32_kernel<64>, dim3(p.num_items), dim3(NT), 0, s, p);
  return hipGetLastError();
}

}  // namespace wf
