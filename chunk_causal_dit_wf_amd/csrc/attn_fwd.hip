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
// bf16 kernel with LDS-DMA tile loads (bf16 cache, pages >= 64 tokens, cache
// < 4 GiB), two-group ping-pong schedule.
//
// One workgroup = 8 waves (2 per SIMD) = 256 query rows of one head of one
// chunk; each wave owns 32 rows and keeps its Q^T fragments in VGPRs.  Waves
// 0-3 (group 0) and 4-7 (group 1) put one wave on each SIMD (waves w and w+4
// share one), and the two groups run the same program one phase apart: while
// one wave of a SIMD issues the matrix products of a 64-key tile (phase M),
// the other computes the softmax of its next tile on the vector unit (phase
// V).  Every phase ends with a workgroup barrier, so the offset never drifts
// and the matrix unit of each SIMD always has one wave feeding it; the wave
// in phase V runs at the higher wave priority (prio).
//
// Per 64-key tile t and wave:
//   M(t): S(t+1) = K(t+1) Q^T (two 32-key halves, 16 MFMAs) and
//         O^T += V(t)^T P(t) (16 MFMAs); fragment reads run ahead in LDS.
//   V(t): issue this wave's share of the tile loads, then x = S(t+1) sl2 - m,
//         the guard (largest x), P(t+1) = exp2(x) in bf16, and -- only when
//         some x exceeds 11 -- the exact rescale; then the row sums of
//         P(t+1) on the matrix unit (4 16x16x32 selector products, which the
//         SIMD's matrix pipe runs between the other wave's products).
//
// LDS layout.  Rows are padded by 16 bytes (K: 2D+16 bytes, V^T: 144 bytes)
// so that the lanes one LDS cycle serves hit distinct banks and every
// fragment read is an immediate offset from one per-lane base.
//   K half-tile [32 rows][D] bf16: LDS row r holds key pi(r) of the half,
//     pi(8 j + 4 h + i) = 16 h + 4 j + i.  The MFMA A operand of lane l is
//     LDS row l % 32, so in the S^T accumulator lane-half h holds the 16
//     consecutive keys 16 h .. 16 h + 15 of the half.
//   V^T tile [D][64 keys] bf16, keys in natural order.  Because of pi the 8
//     keys one P^T operand needs are contiguous: one 16-byte LDS read per
//     MFMA, and V^T rows are plain 16-byte DMA chunks.
// Tiles stream through a ring of three LDS stages; stage t (slot (t+1) % 3)
// holds K(t+1) and V(t)^T.  Loads are buffer LDS-DMA (16 bytes per lane,
// written to LDS at base + 16 * lane; padding lanes load a dummy chunk).
// Group 1 loads K tiles four tiles ahead, group 0 V^T tiles two tiles ahead,
// at the start of their V phases, so the loads' latency is covered before
// the wave reads LDS again.  A stage is complete once every wave has waited
// for its own loads into it and passed a barrier.  V tiles with keys outside
// the chunk's range (0 * NaN would poison P V) are zeroed in LDS behind one
// extra barrier.
// ---------------------------------------------------------------------------
namespace pp {

constexpr int NW = 8;          // waves per workgroup
constexpr int NTD = 64 * NW;   // threads per workgroup
constexpr int NG = 4;          // waves per group (one per SIMD)
constexpr int BMD = 32 * NW;   // query rows per workgroup
constexpr int HK = 32;         // keys per K half-tile
static_assert(BMD == kBlockMDma, "host and kernel disagree on the DMA kernel block size");

template <int D>
struct Geo {
  static constexpr int KROW = 2 * D + 16;                 // LDS bytes per K row (padded)
  static constexpr int KCH = D / 8;                       // 16-byte data chunks per K row
  static constexpr int KDMA = (HK * KROW + 1023) / 1024;  // DMA instructions per K half-tile
  static constexpr int KHALF = KDMA * 1024;               // LDS bytes per K half-tile
  static constexpr int KTILE = 2 * KHALF;                 // LDS bytes per K tile
  static constexpr int KN = 2 * KDMA;                     // DMA instructions per K tile
  static constexpr int VROW = 2 * BN + 16;                // LDS bytes per V^T row (padded)
  static constexpr int VDMA = (D * VROW + 1023) / 1024;   // DMA instructions per V^T tile
  static constexpr int VTILE = VDMA * 1024;               // LDS bytes per V^T tile
  static constexpr int KPW = (KN + NG - 1) / NG;          // K instructions per group-1 wave (max)
  static constexpr int VPW = (VDMA + NG - 1) / NG;        // V instructions per group-0 wave (max)
  static constexpr int PW = KPW > VPW ? KPW : VPW;  // DMA instructions per wave and tile
};

// Every wave issues exactly PW DMA instructions per tile: wave gw of a group
// takes instructions gw, gw + 4, ... of the tile, and repeats its first one
// (same source, same destination, same bytes) where it runs out.  The fixed
// count lets every wait for a tile be a compile-time vmcnt.
template <int D>
__device__ __forceinline__ int inst_of(int group, int gw, int r) {
  const int n = gw + NG * r;
  return n < (group == 1 ? Geo<D>::KN : Geo<D>::VDMA) ? n : gw;
}

// Per-lane source byte offsets of this wave's DMA instructions, relative to
// the tile's first key in its page.  Padding lanes load the tile's first
// chunk.  The tile-relative key of a lane's chunk (needed only when a tile
// crosses a page) is recomputed from the lane instead of being kept.
template <int D>
struct Plan {
  uint32_t off[Geo<D>::PW];
};

// K instruction n, lane: tile-relative key of the lane's 16-byte chunk and
// its byte offset (row pi(key) of half n / KDMA, 16-byte chunk pc).
template <int D>
__device__ __forceinline__ void k_chunk(int n, int lane, int& key, uint32_t& off) {
  using G = Geo<D>;
  const int half = n / G::KDMA, rr = n - half * G::KDMA;
  const int y = 1024 * rr + 16 * lane;
  const int row = y / G::KROW, pc = (y % G::KROW) / 16;
  const bool data = row < HK && pc < G::KCH;
  const int k = HK * half + 16 * ((row >> 2) & 1) + 4 * (row >> 3) + (row & 3);  // pi(row)
  key = data ? k : 0;
  off = data ? (uint32_t)(k * 2 * D + pc * 16) : 0u;
}

// V^T instruction n, lane: key of the lane's chunk and its byte offset (row d
// of the V^T block, keys 8 pc .. 8 pc + 7).
template <int D>
__device__ __forceinline__ void v_chunk(int n, int lane, int P, int& key, uint32_t& off) {
  using G = Geo<D>;
  const int y = 1024 * n + 16 * lane;
  const int d = y / G::VROW, pc = (y % G::VROW) / 16;
  const bool data = d < D && pc < 8;
  key = data ? pc * 8 : 0;
  off = data ? (uint32_t)(d * P * 2 + pc * 16) : 0u;
}

template <int D>
__device__ __forceinline__ Plan<D> make_plan(int group, int gw, int lane, int P) {
  Plan<D> pl;
#pragma unroll
  for (int r = 0; r < Geo<D>::PW; ++r) {
    int key;
    if (group == 1)
      k_chunk<D>(inst_of<D>(1, gw, r), lane, key, pl.off[r]);
    else
      v_chunk<D>(inst_of<D>(0, gw, r), lane, P, key, pl.off[r]);
  }
  return pl;
}

// Buffer resource over a whole cache (K or V): raw addressing, byte offsets
// below 2^32 (the DMA kernels take caches under 4 GiB).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t cache_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0xFFFFFFFFu, 0x00020000);
}

// LDS-DMA through a buffer resource: lane L's 16 bytes at byte voff + soff of
// the resource land at lds + 16 L.  (The buffer form keeps the compiler's
// wait tracking exact for LDS reads issued while such loads are in flight.)
__device__ __forceinline__ void dma16b(__amdgpu_buffer_rsrc_t rs, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

// DMA the K tile (64 keys) at cursor c into kt (group 1).
template <int D>
__device__ __forceinline__ void dma_k(const AttnParams& p, __amdgpu_buffer_rsrc_t rs, const Cursor& c,
                                      const Plan<D>& pl, char* kt, int gw) {
  using G = Geo<D>;
  auto dst = [&](int r) {
    const int n = inst_of<D>(1, gw, r);
    const int half = n / G::KDMA;
    return kt + half * G::KHALF + 1024 * (n - half * G::KDMA);
  };
  if (p.P - c.off >= BN) {
    const uint32_t soff = __builtin_amdgcn_readfirstlane(c.k0 + (uint32_t)c.off * (2 * D));  // uniform
#pragma unroll
    for (int r = 0; r < G::PW; ++r) dma16b(rs, dst(r), pl.off[r], soff);
    return;
  }
  const RunGeom g = run_geom<2 * D, 2>(p, c);
  const int lane = __lane_id();
#pragma unroll
  for (int r = 0; r < G::PW; ++r) {
    int key;
    uint32_t off;
    k_chunk<D>(inst_of<D>(1, gw, r), lane, key, off);
    dma16b(rs, dst(r), (key < g.split ? g.kb0 : g.kb1) + off, 0u);
  }
}

// DMA the V^T tile (64 keys) at cursor c into vt (group 0).
template <int D>
__device__ __forceinline__ void dma_v(const AttnParams& p, __amdgpu_buffer_rsrc_t rs, const Cursor& c,
                                      const Plan<D>& pl, char* vt, int gw) {
  using G = Geo<D>;
  auto dst = [&](int r) { return vt + 1024 * inst_of<D>(0, gw, r); };
  if (p.P - c.off >= BN) {
    const uint32_t soff = __builtin_amdgcn_readfirstlane(c.v0 + (uint32_t)c.off * 2);  // uniform
#pragma unroll
    for (int r = 0; r < G::PW; ++r) dma16b(rs, dst(r), pl.off[r], soff);
    return;
  }
  const RunGeom g = run_geom<2 * D, 2>(p, c);
  const int lane = __lane_id();
#pragma unroll
  for (int r = 0; r < G::PW; ++r) {
    int key;
    uint32_t off;
    v_chunk<D>(inst_of<D>(0, gw, r), lane, p.P, key, off);
    dma16b(rs, dst(r), (key < g.split ? g.vb0 : g.vb1) + off, 0u);
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

// Workgroup barrier that leaves outstanding loads in flight: the caller
// orders the LDS data itself (each wave waits for its own DMA before the
// barrier).  The empty asm statements keep the compiler from moving memory
// accesses across it, the scheduling barriers keep the phases' instructions
// on their side of it.
__device__ __forceinline__ void barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// s_waitcnt lgkmcnt(0) alone (LDS writes done before a barrier).
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Zero the keys of V^T tile t (in LDS) that lie outside [lo, hi) (all threads).
template <int D>
__device__ __forceinline__ void zero_v_outside(char* vt, int t, int lo, int hi) {
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));  // keep the per-lane keys below out of the tile loop's registers
  for (int idx = tid; idx < D * 8; idx += NTD) {
    const int d = idx >> 3, c = idx & 7;
    const int rel = t * BN + 8 * c;
    if (rel >= lo && rel + 8 <= hi) continue;
    uint32_t m = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) m |= (rel + e >= lo && rel + e < hi) ? 1u << e : 0u;
    uint4* a = (uint4*)(vt + d * Geo<D>::VROW + 16 * c);
    *a = mask_bf16x8(*a, m);
  }
}

// Row sums on the matrix unit.  A 16x16x32 bf16 product reads a P fragment
// of the 32x32x16 P V product as its B operand: lane L holds keys
// 8 (L / 32) + j of query L % 32, which that product takes as k = 8 (L / 16) + j
// of column L % 16.  With the selector A = rows 0 and 1 of ones over the
// k-blocks of queries L % 16 and L % 16 + 16 (lanes 0, 32 and 17, 49), output
// row 0 / row 1 of column n is the sum of P over the fragment's 16 keys for
// query n / n + 16: lanes 0..15 accumulate l in lacc[0] (query L) and lacc[1]
// (query L + 16), summed from the same bf16 P the P V product multiplies.
__device__ __forceinline__ bf16x8 row_sum_selector(int lane) {
  const bool one = lane == 0 || lane == 32 || lane == 17 || lane == 49;
  bf16x8 a;
#pragma unroll
  for (int j = 0; j < 8; ++j) a[j] = one ? (__bf16)1.0f : (__bf16)0.0f;
  return a;
}

// Phase M of one 64-key tile.  QK: S(t+1) = K(t+1) Q^T from the K tile at kt
// (two halves into s[0], s[1]).  PV: O^T += V(t)^T P(t) from the V tile at vt.
// kx / vx: this lane's LDS byte offsets of its K row chunk and of its V^T row
// chunk.  Fragment reads run DIST products ahead of their use.
template <int D, bool QK, bool PV>
__device__ __forceinline__ void m_phase(f32x16 (&s)[2], f32x16 (&o)[D / 32], const bf16x8 (&qf)[D / 16],
                                        const bf16x8 (&pf)[4], const char* kt, const char* vt, int kx, int vx,
                                        f32x4& lacc) {
  using G = Geo<D>;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  static_assert(4 * DB == 2 * KS, "two PV products per k-step");
  // Products in issue order: per k-step ks, [S_a(ks), S_b(ks)] then [PV(2ks), PV(2ks+1)].
  constexpr int PER = (QK ? 2 : 0) + (PV ? 2 : 0);
  constexpr int N = PER * KS;
  constexpr int DIST = 3;
  auto is_qk = [&](int i) { return QK && (i % PER) < 2; };
  auto frag = [&](int i) -> bf16x8 {
    const int ks = i / PER, r = i % PER;
    if (is_qk(i)) return *(const bf16x8*)(kt + r * G::KHALF + kx + 32 * ks);
    const int j = 2 * ks + (r - (QK ? 2 : 0));  // PV product j: key step j / DB, d block j % DB
    const int kk = j / DB, db = j % DB;
    const int half = kk >> 1, k = kk & 1;
    return *(const bf16x8*)(vt + vx + 16 * (4 * half + k) + db * 32 * G::VROW);
  };
  bf16x8 fr[DIST + 1];
#pragma unroll
  for (int i = 0; i < DIST; ++i) fr[i] = frag(i);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (i + DIST < N) fr[(i + DIST) % (DIST + 1)] = frag(i + DIST);
    const bf16x8 f = fr[i % (DIST + 1)];
    const int ks = i / PER, r = i % PER;
    if (is_qk(i)) {
      if (ks == 0) {
        f32x16 z;
#pragma unroll
        for (int e = 0; e < 16; ++e) z[e] = 0.f;
        s[r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, qf[0], z, 0, 0, 0);
      } else {
        s[r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, qf[ks], s[r], 0, 0, 0);
      }
    } else {
      const int j = 2 * ks + (r - (QK ? 2 : 0));
      o[j % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, pf[j / DB], o[j % DB], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // Keep the products in this phase (nothing may sink them past the barrier
  // into the phase that uses them).
  if constexpr (QK) asm volatile("" : "+v"(s[0]), "+v"(s[1]));
  if constexpr (PV) {
#pragma unroll
    for (int db = 0; db < DB; ++db) asm volatile("" : "+v"(o[db]));
    // The row sums are taken in phase V, but pinning them here as well
    // measured 1-2 % faster than leaving them free.
    asm volatile("" : "+v"(lacc));
  }
}

// Phase V: softmax of S(t+1) (both 32-key halves, 32 elements per lane).
//
// The reference point m of the online softmax is moved only when needed: P is
// formed with the current m, x = S sl2 - m, and only if some x exceeds 11 (a
// p above 2^11) is the row maximum taken and O and the row sums rescaled
// exactly before P is formed again.  Every p stays at most 2^11 (no overflow;
// bf16 keeps its relative precision), and the common path needs no exact
// maximum: the guard is a max3 tree over x, which does not wait for the
// exponentials.  The row sums of the new P are taken on the matrix unit at
// the end of the phase (row_sum_selector).  FIRST: the first tile of a segment sets m from its own
// row maxima.  MASK: keys outside [lo, hi) (tile-relative key kb + ...) are
// set to -inf first.  Each step is applied to all 32 elements before the next:
// independent instructions cover each other's latency.
template <int D, bool MASK, bool FIRST>
__device__ __forceinline__ void v_phase(f32x16 (&s)[2], bf16x8 (&pf)[4], f32x16 (&o)[D / 32], float& m,
                                        f32x4& lacc, const bf16x8& sel, float sl2, int kb, int lo, int hi,
                                        int hf) {
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  if constexpr (MASK) {
    // Element e of half h holds key kb + HK h + 16 hf + e.  The lane's part
    // 16 hf is made opaque here so that the compiler keeps the 32 per-element
    // keys inside this (rare) block instead of hoisting them out of the tile
    // loop into registers it would then spill.
    int lane_key = 16 * hf;
    asm volatile("" : "+v"(lane_key));
    const int lo_r = lo - kb, hi_r = hi - kb;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = lane_key + (HK * h + e);
        s[h][e] = (key >= lo_r && key < hi_r) ? s[h][e] : -INFINITY;
      }
  }
  auto row_max = [&]() {
    float mx[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int h = q >> 1, e0 = 8 * (q & 1);
      float a = fmaxf(s[h][e0], fmaxf(s[h][e0 + 1], s[h][e0 + 2]));
      a = fmaxf(a, fmaxf(s[h][e0 + 3], s[h][e0 + 4]));
      a = fmaxf(a, fmaxf(s[h][e0 + 5], s[h][e0 + 6]));
      mx[q] = fmaxf(a, s[h][e0 + 7]);
    }
    return half_max(fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]))) * sl2;
  };
  // P = exp2(x), x = S sl2 - m, into pf; returns this lane's largest x.
  auto form_p = [&]() {
    const float nm = -m;
    float e[2][16];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int k = 0; k < 16; ++k) e[h][k] = __builtin_fmaf(s[h][k], sl2, nm);
    __builtin_amdgcn_sched_barrier(0);
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 32; i += 2) mx = fmaxf(fmaxf(e[i >> 4][i & 15], e[i >> 4][(i & 15) + 1]), mx);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int k = 0; k < 16; ++k) e[h][k] = __builtin_amdgcn_exp2f(e[h][k]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int k = 0; k < 16; k += 2) {
        const bf16x2v pk = {(__bf16)e[h][k], (__bf16)e[h][k + 1]};
        pf[2 * h + (k >> 3)][k & 7] = pk[0];
        pf[2 * h + (k >> 3)][(k & 7) + 1] = pk[1];
      }
    return mx;
  };
  if constexpr (FIRST) m = row_max();
  const float mx = form_p();
  if (!FIRST && __builtin_expect(__builtin_amdgcn_ballot_w64(!(mx <= 11.f)) != 0, 0)) {
    asm volatile("");  // a real branch: the recomputation must not be executed speculatively
    const float m_new = fmaxf(m, row_max());
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    m = m_new;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
    // lacc[0] of lane L < 16 is relative to row L's m, lacc[1] to row L + 16's.
    const float alpha_hi = __shfl_down(alpha, 16);
    lacc[0] *= alpha;
    lacc[1] *= alpha_hi;
    form_p();
  }
  // Row sums of the new P on the matrix unit (row_sum_selector).
#pragma unroll
  for (int q = 0; q < 4; ++q) lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, pf[q], lacc, 0, 0, 0);
  // Keep the softmax in this phase.
  asm volatile("" : "+v"(pf[0]), "+v"(pf[1]), "+v"(pf[2]), "+v"(pf[3]), "+v"(lacc));
}

// LDS stages: K tile and V^T tile of each of the three ring slots, as
// separate __shared__ objects (see the kernel).
struct Ring {
  char *k0, *k1, *k2, *v0, *v1, *v2;
  template <int S>
  __device__ __forceinline__ char* k() const { return S == 0 ? k0 : S == 1 ? k1 : k2; }
  template <int S>
  __device__ __forceinline__ char* v() const { return S == 0 ? v0 : S == 1 ? v1 : v2; }
};

template <int N>
using IC = std::integral_constant<int, N>;

// One query tile (item) of chunk cd over its 64-key tiles [j0, j1); slot as
// in the other DMA kernel (< 0: final output, else a partial-result slot).
template <int D>
__device__ __forceinline__ void segment(const AttnParams& p, const ChunkDesc& cd, int qt, int head, int j0,
                                        int j1, int slot, const Ring& rg, const Plan<D>& plan, int wave,
                                        int lane) {
  using G = Geo<D>;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  const int group = wave >> 2;  // wave-uniform
  const int gw = wave & 3;
  const int lq = lane & 31;
  const int hf = lane >> 5;
  const int qrow = qt * BMD + wave * 32 + lq;
  const int row = cd.q_begin + qrow;
  const bool row_ok = qrow < cd.q_len;
  const int base = BN * j0;
  const int lo = max(cd.lead - base, 0);
  const int hi = min(cd.lead + cd.nkeys, BN * j1) - base;
  const int nt = (hi + BN - 1) / BN;  // >= 1
  const float sl2 = p.scale_log2;
  const int kx = lq * G::KROW + 16 * hf;
  const int vx = lq * G::VROW + 16 * (2 * hf);
  // Whether this wave's latest batch of loads (PW instructions) is in flight.
  bool pend = false;

  // Prologue loads: group 1 K(0) -> slot 0, K(1) -> slot 1, K(2) -> slot 2;
  // group 0 V(0) -> slot 1.  Then the query fragments.
  Cursor cur = cursor_at<2 * D>(p, cd, head, base);
  const __amdgpu_buffer_rsrc_t rs = cache_rsrc(group == 1 ? p.k : p.v);
  if (group == 1) {
    dma_k<D>(p, rs, cur, plan, rg.k<0>(), gw);
    advance<2 * D>(p, head, cur, BN);
    if (nt > 1) dma_k<D>(p, rs, cur, plan, rg.k<1>(), gw);
    advance<2 * D>(p, head, cur, BN);
    if (nt > 2) dma_k<D>(p, rs, cur, plan, rg.k<2>(), gw);
    advance<2 * D>(p, head, cur, BN);
  } else {
    dma_v<D>(p, rs, cur, plan, rg.v<1>(), gw);
    advance<2 * D>(p, head, cur, BN);
  }
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
  f32x16 s[2];
  bf16x8 pf[4];
  float m = -INFINITY;
  f32x4 lacc = {0.f, 0.f, 0.f, 0.f};
  const bf16x8 sel = row_sum_selector(lane);

  auto end_phase = [&]() {
    if (pend)
      wait_vmcnt<G::PW>();
    else
      wait_vmcnt<0>();
    barrier();
  };
  // Loads issued at the start of phase V(t) (t >= -1), before its vector
  // work covers their latency (an LDS read after an LDS-DMA load of the same
  // wave waits for that load): group 0 V(t+2) -> slot t % 3 (vdst), group 1
  // K(t+4) -> slot (t+1) % 3 (kdst).
  auto loads = [&](int t, char* vdst, char* kdst) {
    // The previous batch (issued two phases ago) is complete before the next
    // one is issued: a CU stalls the issue of LDS-DMA loads once about 40 are
    // in flight, so each wave keeps at most one batch outstanding.
    wait_vmcnt<0>();
    if (group == 0) {
      pend = t + 2 < nt;
      if (pend) dma_v<D>(p, rs, cur, plan, vdst, gw);
    } else {
      pend = t + 4 < nt;
      if (pend) dma_k<D>(p, rs, cur, plan, kdst, gw);
    }
    advance<2 * D>(p, head, cur, BN);
    // Consume the page-table read now: a scalar load still in flight would
    // make every LDS wait of the next phase a full wait.
    asm volatile("" ::"s"(cur.k1), "s"(cur.v1));
  };

  // Zero the keys of V tile t (stage t, slot sl) outside [lo, hi) in LDS: P is
  // zero there, but the cache may hold NaN.  Both groups do it at the same
  // barrier: group 1 after its M(t-1), group 0 after its V(t-1).
  auto vedge = [&](int t) { return (t == 0 && lo > 0) || BN * (t + 1) > hi; };
  auto zero_v = [&](char* vt, int t) {
    zero_v_outside<D>(vt, t, lo, hi);
    wait_lgkm0();
    barrier();
  };

  wait_vmcnt<0>();
  barrier();
  if (group == 1) barrier();  // group 1 runs one phase behind
  // M(-1): S(0) from K(0) in slot 0.
  m_phase<D, true, false>(s, o, qf, pf, rg.k<0>(), rg.v<0>(), kx, vx, lacc);
  end_phase();
  if (group == 1 && vedge(0)) zero_v(rg.v<1>(), 0);
  // V(-1)
  prio(1);  // the softmax wave issues first on its SIMD
  loads(-1, rg.v<2>(), rg.k<0>());
  v_phase<D, true, true>(s, pf, o, m, lacc, sel, sl2, 0, lo, hi, hf);
  prio(0);
  end_phase();
  if (group == 0 && vedge(0)) zero_v(rg.v<1>(), 0);

  // Tile t uses stage t in slot (t + 1) % 3.  The loop is unrolled by three
  // so that every slot is a compile-time constant (the compiler can then tell
  // the LDS-DMA targets from the buffers being read); every call site below
  // has a static ring position.  steady(t) needs t + 2 < nt: S(t+1) needs no
  // mask and V tile t+1 no zeroing.  edge_step(t) is tile nt - 2; tile nt - 1
  // follows the steps.
  auto steady = [&](auto rho_tag, int t) {
    constexpr int rho = decltype(rho_tag)::value;
    constexpr int sl = (rho + 1) % 3;
    m_phase<D, true, true>(s, o, qf, pf, rg.k<sl>(), rg.v<sl>(), kx, vx, lacc);
    end_phase();
    prio(1);  // the softmax wave issues first on its SIMD
    loads(t, rg.v<rho>(), rg.k<sl>());
    v_phase<D, false, false>(s, pf, o, m, lacc, sel, sl2, 0, lo, hi, hf);
    prio(0);
    end_phase();
  };
  auto edge_step = [&](auto rho_tag, int t) {
    constexpr int rho = decltype(rho_tag)::value;
    constexpr int sl = (rho + 1) % 3;
    constexpr int sn = (rho + 2) % 3;  // slot of stage t + 1
    m_phase<D, true, true>(s, o, qf, pf, rg.k<sl>(), rg.v<sl>(), kx, vx, lacc);
    end_phase();
    const bool ze = vedge(t + 1);
    if (group == 1 && ze) zero_v(rg.v<sn>(), t + 1);
    prio(1);  // the softmax wave issues first on its SIMD
    loads(t, rg.v<rho>(), rg.k<sl>());
    v_phase<D, true, false>(s, pf, o, m, lacc, sel, sl2, BN * (t + 1), lo, hi, hf);
    prio(0);
    end_phase();
    if (group == 0 && ze) zero_v(rg.v<sn>(), t + 1);
  };
  // Steps 0 .. nt - 3 are steady, step nt - 2 the edge step.  Each residue
  // R = (nt - 2) % 3 runs its own copy of the loop and of the steps after it.
  // (One loop shared by the four remainders spilled 424 bytes per lane where
  // the remainders joined, about 60 MB of scratch traffic per Wan-round
  // launch; with a copy per residue nothing spills.)
  auto run = [&](auto r_tag) {
    constexpr int R = decltype(r_tag)::value;
    int t = 0;
    for (; t + R + 2 < nt; t += 3) {
      steady(IC<0>{}, t);
      steady(IC<1>{}, t + 1);
      steady(IC<2>{}, t + 2);
    }
    if constexpr (R >= 1) steady(IC<0>{}, t);
    if constexpr (R >= 2) steady(IC<1>{}, t + 1);
    edge_step(IC<R>{}, t + R);
  };
  if (nt >= 2) {
    const int r = (nt - 2) % 3;
    if (r == 0)
      run(IC<0>{});
    else if (r == 1)
      run(IC<1>{});
    else
      run(IC<2>{});
  }
  // Tile nt - 1: its P V product alone, from slot nt % 3 (one code path for
  // every tile count).  The epilogue reads the accumulators with plain VALU
  // code right after, so the wave first sleeps until the products have left
  // the matrix pipe.
  {
    const int sl = nt % 3;
    const char* vt = sl == 0 ? rg.v0 : sl == 1 ? rg.v1 : rg.v2;
    m_phase<D, false, true>(s, o, qf, pf, rg.k0, vt, kx, vx, lacc);
    __builtin_amdgcn_s_sleep(2);
    end_phase();
  }
  if (group == 0) barrier();  // matches group 1's last M phase

  // Row sum of row lq: lacc[lq / 16] of lane lq % 16.
  const float l_lo = __shfl(lacc[0], lq & 15), l_hi = __shfl(lacc[1], lq & 15);
  const float lt = lq < 16 ? l_lo : l_hi;
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
__global__ __launch_bounds__(NTD, 2) void attn_fwd_pp_kernel(const AttnParams p) {
  using G = Geo<D>;
  __shared__ __align__(1024) char k0[G::KTILE];
  __shared__ __align__(1024) char k1[G::KTILE];
  __shared__ __align__(1024) char k2[G::KTILE];
  __shared__ __align__(1024) char v0[G::VTILE];
  __shared__ __align__(1024) char v1[G::VTILE];
  __shared__ __align__(1024) char v2[G::VTILE];
  const Ring rg{k0, k1, k2, v0, v1, v2};
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const Plan<D> plan = make_plan<D>(wave >> 2, wave & 3, lane, p.P);
  walk_segments(p, (int)blockIdx.x, [&](int item, int j0, int j1, int slot) {
    const Item it = decode_item(p, item);
    segment<D>(p, p.chunk[it.c], it.qt, it.head, j0, j1, slot, rg, plan, wave, lane);
  });
}

// Merge the partial results of the split schedule: for each row,
// O = sum_k 2^(m_k - M) O_k / sum_k 2^(m_k - M) l_k with M = max_k m_k (the
// log-sum-exp combination of attention over disjoint key sets).  One block
// per (item, kMergeRows rows); the item's NP partials are its m A parts
// (slots part * n + item) and, if b > 0, its m B parts.  NP is a template
// argument so that every partial's loads of a row are issued before the first
// is used.
template <int D, int NP>
__global__ __launch_bounds__(256) void attn_merge_kernel(const AttnParams p) {
  constexpr int C4 = D / 4;            // float4 columns per row
  constexpr int RPP = 256 / C4;        // rows per pass
  const SplitSched& sp = p.sp;
  const int nrb = BMD / kMergeRows;
  const int item = blockIdx.x / nrb;
  const int r0 = (blockIdx.x - item * nrb) * kMergeRows;
  const Item it = decode_item(p, item);
  const ChunkDesc& cd = p.chunk[it.c];
  const int na = sp.n * sp.m;
  int slots[NP];
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    const int part = k % sp.m;
    slots[k] = k < sp.m ? part * sp.n + item : na + b_index(p, item, part);
  }
  const int tid = threadIdx.x;
  const int c4 = tid % C4;
  const int64_t sf = ws_slot_floats(D);
  for (int r = r0 + tid / C4; r < r0 + kMergeRows; r += RPP) {
    const int qrow = it.qt * BMD + r;
    if (qrow >= cd.q_len) break;
    float mk[NP], lk[NP];
    f32x4 vk[NP];
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      const float* ws = p.ws + slots[k] * sf;
      mk[k] = ws[BMD * D + r];
      lk[k] = ws[BMD * D + BMD + r];
      vk[k] = *(const f32x4*)(ws + (int64_t)r * D + 4 * c4);
    }
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < NP; ++k) M = fmaxf(M, mk[k]);
    float L = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      const float w = __builtin_amdgcn_exp2f(mk[k] - M);
      L += w * lk[k];
      acc += w * vk[k];
    }
    const float inv = 1.f / L;
    const int row = cd.q_begin + qrow;
    bf16x4 ov = {(__bf16)(acc[0] * inv), (__bf16)(acc[1] * inv), (__bf16)(acc[2] * inv), (__bf16)(acc[3] * inv)};
    *(bf16x4*)((__bf16*)p.o + ((int64_t)row * p.H + it.head) * D + 4 * c4) = ov;
    if (p.lse != nullptr && c4 == 0) p.lse[(int64_t)it.head * p.nq + row] = (M + __log2f(L)) * kLn2;
  }
}

}  // namespace pp

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
    hipLaunchKernelGGL(pp::attn_fwd_pp_kernel<128>, dim3(grid), dim3(pp::NTD), 0, s, p);
  else
    hipLaunchKernelGGL(pp::attn_fwd_pp_kernel<64>, dim3(grid), dim3(pp::NTD), 0, s, p);
  return hipGetLastError();
}

// The merge instantiation for np partials (1 <= np <= 16: m <= 8 parts, doubled with tails).
template <int D, int NP = 1>
static hipError_t launch_merge_np(const AttnParams& p, dim3 grid, hipStream_t s, int np) {
  if constexpr (NP > 16) {
    return hipErrorInvalidValue;
  } else {
    if (np != NP) return launch_merge_np<D, NP + 1>(p, grid, s, np);
    hipLaunchKernelGGL((pp::attn_merge_kernel<D, NP>), grid, dim3(256), 0, s, p);
    return hipGetLastError();
  }
}

hipError_t launch_attn_merge(const AttnParams& p, int head_dim, hipStream_t s) {
  const dim3 grid(p.num_items * (kBlockMDma / kMergeRows));
  const int np = p.sp.b > 0 ? 2 * p.sp.m : p.sp.m;
  return head_dim == 128 ? launch_merge_np<128>(p, grid, s, np) : launch_merge_np<64>(p, grid, s, np);
}

hipError_t attn_dma_resident_blocks(int head_dim, int* blocks) {
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess)
    e = head_dim == 128
            ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, pp::attn_fwd_pp_kernel<128>, pp::NTD, 0)
            : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, pp::attn_fwd_pp_kernel<64>, pp::NTD, 0);
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
