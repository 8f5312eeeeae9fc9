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
#include "wf_internal.h"

namespace wf {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = kBlockM;   // query rows per workgroup
constexpr int BN = 64;        // keys per LDS tile
constexpr int NT = 256;       // threads per workgroup
constexpr float kLn2 = 0.69314718055994530942f;

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

// Value of the other 32-lane half (lane l <-> l ^ 32) combined with op.
__device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Work item -> (chunk, query tile, head).  Items are numbered tile-major inside
// a chunk (item = tile * H + head), so consecutive workgroups -- which the
// dispatcher spreads round-robin over the 8 XCDs -- visit different heads and
// each XCD's L2 sees a small, fixed subset of heads.
struct Item {
  int c, qt, head;
};
__device__ __forceinline__ Item decode_item(const AttnParams& p, int item) {
  int c = 0;
  while (c + 1 < p.num_chunks && item >= p.chunk[c + 1].item0) ++c;
  const int local = item - p.chunk[c].item0;
  Item it;
  it.c = c;
  it.qt = local / p.H;
  it.head = local - it.qt * p.H;
  return it;
}

// ---------------------------------------------------------------------------
// bf16 Q (and bf16 or E4M3FN K/V) kernel.
// LDS per stage: K tile [64 keys][D] bf16, 16-byte chunks XOR-swizzled by
// (key & 7); V^T tile [D][64 keys] bf16, 16-byte chunks XOR-swizzled by
// (d & 7), keys permuted inside 16-key groups.
// ---------------------------------------------------------------------------
template <int D, bool FP8KV>
struct TileLoader {
  static constexpr int KCH = D / 8;                 // 16-byte bf16 chunks per K row in LDS
  static constexpr int KITEMS = BN * KCH / NT;      // K chunks per thread
  static constexpr int VITEMS = D * (BN / 8) / NT;  // V 8-key groups per thread
  static constexpr int KBYTES = BN * D * 2;
  static constexpr int STAGE = KBYTES + D * BN * 2;
  // staged registers: bf16 payload (16 B per item) or raw fp8 (8 B per item) + scale
  uint4 kr[KITEMS];
  uint4 vr[VITEMS];
  float ksc[KITEMS];
  float vsc[VITEMS];
  uint32_t kmask;  // bit i: K item i valid
  uint32_t vfull;  // bit i: V group i fully valid
  uint32_t vpart;  // bit i: V group i partially valid (element masks below)
  uint8_t vmask[VITEMS];
};

template <int D, bool FP8KV>
__device__ __forceinline__ void load_tile(TileLoader<D, FP8KV>& L, const AttnParams& p,
                                          const ChunkDesc& cd, const int32_t* table, int head,
                                          int j) {
  using TL = TileLoader<D, FP8KV>;
  const int tid = threadIdx.x;
  const int lo = cd.lead, hi = cd.lead + cd.nkeys;
  const int rel0 = j * BN;
  // tile start page/offset (uniform)
  int32_t page0, off0;
  locate(cd.map, p.divP, p.divT, table, (uint32_t)rel0, page0, off0);
  L.kmask = 0;
#pragma unroll
  for (int r = 0; r < TL::KITEMS; ++r) {
    const int idx = tid + NT * r;
    const int key = idx / TL::KCH, ch = idx - key * TL::KCH;
    const int rel = rel0 + key;
    L.kr[r] = make_uint4(0, 0, 0, 0);
    L.ksc[r] = 1.f;
    if (rel >= lo && rel < hi) {
      int32_t page = page0, off = off0 + key;
      if (off >= p.P) locate(cd.map, p.divP, p.divT, table, (uint32_t)rel, page, off);
      const int64_t row = ((int64_t)page * p.H + head) * p.P + off;
      if constexpr (FP8KV) {
        const uint2 raw = *(const uint2*)((const uint8_t*)p.k + row * D + ch * 8);
        L.kr[r] = make_uint4(raw.x, raw.y, 0, 0);
        L.ksc[r] = p.ks[((int64_t)page * p.H + head) * p.nblk + (off >> 7)];
      } else {
        L.kr[r] = *(const uint4*)((const __bf16*)p.k + row * D + ch * 8);
      }
      L.kmask |= 1u << r;
    }
  }
  L.vfull = 0;
  L.vpart = 0;
#pragma unroll
  for (int r = 0; r < TL::VITEMS; ++r) {
    const int idx = tid + NT * r;
    const int d = idx >> 3, a = idx & 7;
    const int rel = rel0 + 8 * a;
    L.vr[r] = make_uint4(0, 0, 0, 0);
    L.vsc[r] = 1.f;
    L.vmask[r] = 0;
    if (rel + 8 > lo && rel < hi) {
      int32_t page = page0, off = off0 + 8 * a;
      if (off >= p.P) locate(cd.map, p.divP, p.divT, table, (uint32_t)rel, page, off);
      const int64_t col = (((int64_t)page * p.H + head) * D + d) * p.P + off;
      if constexpr (FP8KV) {
        const uint2 raw = *(const uint2*)((const uint8_t*)p.v + col);
        L.vr[r] = make_uint4(raw.x, raw.y, 0, 0);
        L.vsc[r] = p.vs[((int64_t)page * p.H + head) * p.nblk + (off >> 7)];
      } else {
        L.vr[r] = *(const uint4*)((const __bf16*)p.v + col);
      }
      if (rel >= lo && rel + 8 <= hi) {
        L.vfull |= 1u << r;
      } else {
        uint8_t m = 0;
        for (int e = 0; e < 8; ++e) m |= (uint8_t)((rel + e >= lo && rel + e < hi) ? 1u << e : 0u);
        L.vmask[r] = m;
        L.vpart |= 1u << r;
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

template <int D, bool FP8KV>
__device__ __forceinline__ void store_tile(const TileLoader<D, FP8KV>& L, char* stage) {
  using TL = TileLoader<D, FP8KV>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int r = 0; r < TL::KITEMS; ++r) {
    const int idx = tid + NT * r;
    const int key = idx / TL::KCH, ch = idx - key * TL::KCH;
    uint4 v = L.kr[r];
    if constexpr (FP8KV) v = fp8x8_to_bf16x8(v, L.ksc[r]);
    *(uint4*)(stage + key * (D * 2) + ((ch ^ (key & 7)) << 4)) = v;
  }
  char* vt = stage + TL::KBYTES;
#pragma unroll
  for (int r = 0; r < TL::VITEMS; ++r) {
    const int idx = tid + NT * r;
    const int d = idx >> 3, a = idx & 7;
    uint4 v = L.vr[r];
    if constexpr (FP8KV) v = fp8x8_to_bf16x8(v, L.vsc[r]);
    if ((L.vpart >> r) & 1u) {
      const uint32_t m = L.vmask[r];
      uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (!((m >> e) & 1u)) w[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
      v = make_uint4(w[0], w[1], w[2], w[3]);
    }
    // keys 8a..8a+3 -> chunk (a & ~1), keys 8a+4..8a+7 -> chunk (a | 1); byte offset 8*(a & 1)
    const int sw = d & 7;
    char* row = vt + d * (BN * 2) + ((a & 1) << 3);
    *(uint2*)(row + (((a & ~1) ^ sw) << 4)) = make_uint2(v.x, v.y);
    *(uint2*)(row + (((a | 1) ^ sw) << 4)) = make_uint2(v.z, v.w);
  }
}

template <int D, bool FP8KV>
__global__ __launch_bounds__(NT, 2) void attn_fwd_bf16_kernel(const AttnParams p) {
  using TL = TileLoader<D, FP8KV>;
  constexpr int KS = D / 16;   // MFMA k-steps over the head dim
  constexpr int DB = D / 32;   // 32-row blocks of O^T
  extern __shared__ __align__(16) char smem[];
  __shared__ int32_t table[WF_MAX_TABLE_LEN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lq = lane & 31;     // query column owned by this lane
  const int hf = lane >> 5;     // 32-lane half

  for (int i = tid; i < p.T; i += NT) table[i] = p.table[i];

  const Item it = decode_item(p, blockIdx.x);
  const ChunkDesc cd = p.chunk[it.c];
  const int head = it.head;
  const int row = cd.q_begin + it.qt * BM + wave * 32 + lq;  // this lane's query row
  const bool row_ok = (it.qt * BM + wave * 32 + lq) < cd.q_len;
  const int nt = (cd.lead + cd.nkeys + BN - 1) / BN;

  // Q^T fragments (B operand): lane holds 8 consecutive dims of its row per k-step.
  bf16x8 qf[KS];
  {
    const __bf16* qrow = (const __bf16*)p.q + ((int64_t)row * p.H + head) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (row_ok) v = *(const uint4*)(qrow + ks * 16 + hf * 8);
      qf[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x16 o[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[b][i] = 0.f;
  float m = -INFINITY;  // running max, log2 domain
  float l = 0.f;        // running partial sum over this lane's keys

  __syncthreads();  // page table in LDS
  TL L;
  load_tile<D, FP8KV>(L, p, cd, table, head, 0);
  store_tile<D, FP8KV>(L, smem);
  __syncthreads();

  for (int j = 0; j < nt; ++j) {
    char* stage = smem + (j & 1) * TL::STAGE;
    if (j + 1 < nt) load_tile<D, FP8KV>(L, p, cd, table, head, j + 1);

    // ---- S^T = K Q^T for two 32-key blocks
    f32x16 s[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[b][i] = 0.f;
      const int key = b * 32 + lq;
      const char* krow = stage + key * (D * 2);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int ch = (2 * ks + hf) ^ (key & 7);
        const bf16x8 kf = *(const bf16x8*)(krow + (ch << 4));
        s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[b], 0, 0, 0);
      }
    }

    // ---- mask keys outside [lead, lead + nkeys) (first / last tile only)
    const int rel0 = j * BN;
    if (rel0 < cd.lead || rel0 + BN > cd.lead + cd.nkeys) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int rel = rel0 + b * 32 + 8 * (i >> 2) + 4 * hf + (i & 3);
          if (rel < cd.lead || rel >= cd.lead + cd.nkeys) s[b][i] = -INFINITY;
        }
    }

    // ---- online softmax (log2 domain)
    float mx = s[0][0];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[b][i]);
    mx = half_max(mx);
    const float m_new = fmaxf(m, mx * p.scale_log2);
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    m = m_new;
    float rs = 0.f;
    bf16x8 pf[2][2];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][8 * u + r], p.scale_log2, -m_new));
          rs += e;
          pf[b][u][r] = (__bf16)e;
        }
    l = l * alpha + rs;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][i] *= alpha;

    // ---- O^T += V^T P^T
    const char* vt = stage + TL::KBYTES;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int d = db * 32 + lq;
      const char* vrow = vt + d * (BN * 2);
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int ch = (4 * b + 2 * u + hf) ^ (d & 7);
          const bf16x8 vf = *(const bf16x8*)(vrow + (ch << 4));
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[b][u], o[db], 0, 0, 0);
        }
    }

    if (j + 1 < nt) store_tile<D, FP8KV>(L, smem + ((j + 1) & 1) * TL::STAGE);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, lse = (m + log2 l) ln 2
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
hipError_t launch_bf16_t(const AttnParams& p, hipStream_t s) {
  using TL = TileLoader<D, FP8KV>;
  const size_t lds = 2 * TL::STAGE;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&attn_fwd_bf16_kernel<D, FP8KV>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, FP8KV>), dim3(p.num_items), dim3(NT), lds, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const AttnParams& p, int head_dim, hipStream_t s) {
  return head_dim == 128 ? launch_bf16_t<128, false>(p, s) : launch_bf16_t<64, false>(p, s);
}

hipError_t launch_attn_fp8kv(const AttnParams& p, int head_dim, hipStream_t s) {
  return head_dim == 128 ? launch_bf16_t<128, true>(p, s) : launch_bf16_t<64, true>(p, s);
}

hipError_t launch_attn_f32(const AttnParams& p, int head_dim, hipStream_t s) {
  if (head_dim == 128)
    hipLaunchKernelGGL(attn_fwd_f32_kernel<128>, dim3(p.num_items), dim3(NT), 0, s, p);
  else
    hipLaunchKernelGGL(attn_fwd_f32_kernel<64>, dim3(p.num_items), dim3(NT), 0, s, p);
  return hipGetLastError();
}

}  // namespace wf
