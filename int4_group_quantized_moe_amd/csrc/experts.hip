// Expert kernels of the MoE layer: fused int4/int8 group-dequant gate/up GEMV
// with SiLU*up, dequant down GEMV with the weighted combine, token->expert
// bucketing, residual + RMSNorm, and the device packer of expert blobs.
//
// Quantisation: MLX-style int4/int8 group quantisation with byte-addressed
// blobs and 64-bit offsets (page "Paquets Swiftlet 80B Qwen ..." on xix.ai,
// last paragraph); w = scale * q + bias per group of 64 input columns.
// Each routed expert is one fixed-stride blob, so one slot index gives one
// contiguous expert (same page, 4th paragraph).
//
// The dot products use the group-affine factoring
//   sum_c (s q_c + b) x_c = s * sum_c q_c x_c + b * sum_c x_c,
// so codes are never turned into weights.  With bf16 activations the int
// codes are widened to fp16 by OR-ing them into the mantissa of 1024.0
// (0x6400 | q == 1024 + q exactly, and 0x6400 | (q << 4) == 1024 + 16 q), and
// the products are taken two at a time with v_dot2_f32_f16 against fp16
// activations prepared once per token; the 1024 * x terms are removed with a
// per-chunk correction.  fp32 activations keep an exact fp32 path.
#include "moe_internal.h"

namespace moe {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c,
                                false);
}

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const _Float16 l = (_Float16)lo, h = (_Float16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, l) | ((uint32_t)__builtin_bit_cast(uint16_t, h) << 16);
}

__device__ __forceinline__ float f16_lo(uint32_t p) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(p & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t p) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(p >> 16));
}

// Columns covered by one lane's 16 code bytes.
template <int BITS>
constexpr int chunk_cols() { return BITS == 4 ? 32 : 16; }

// ---------------------------------------------------------------------------
// Per-token activation staging in LDS.
//
// BF16 path: xp holds, per chunk of chunk_cols columns, the fp16 pairs in the
// order the code unpacking produces them; cs holds per chunk
// (1024 * sum of the staged fp16 values, sum of the effective x values).
//   int4, chunk of 32 columns, dword j (columns 8j..8j+7):
//     [x0, x4], [x1/16, x5/16], [x2, x6], [x3/16, x7/16]
//   int8, chunk of 16 columns: [x0, x1], [x2, x3], ... (8 dwords)
// F32 path: xs holds x as fp32; cs.y the chunk sum of x.
template <int BITS, int ACT>
struct XStage {
  static constexpr int kCC = chunk_cols<BITS>();
  // dwords of staged activations per token
  static __host__ __device__ constexpr int dwords(int H) {
    return ACT == MOE_ACT_F32 ? H : H / 2;
  }
  static __host__ __device__ constexpr int bytes(int H) {
    return dwords(H) * 4 + (H / kCC) * 8;
  }
};

template <int BITS, int ACT>
__device__ __forceinline__ void stage_chunk(const void* __restrict__ x, int64_t row, int ch, int H,
                                            uint32_t* xp, float2* cs) {
  constexpr int CC = chunk_cols<BITS>();
  // the chunk's CC activations with 16-byte loads (rows and chunks are
  // 16-byte aligned: H is a multiple of 64)
  const int64_t base = row * H + (int64_t)ch * CC;
  float xv[CC];
  if constexpr (ACT == MOE_ACT_F32) {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + base);
#pragma unroll
    for (int i = 0; i < CC / 4; ++i) {
      const float4 v = p[i];
      xv[4 * i] = v.x;
      xv[4 * i + 1] = v.y;
      xv[4 * i + 2] = v.z;
      xv[4 * i + 3] = v.w;
    }
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + base);
#pragma unroll
    for (int i = 0; i < CC / 8; ++i) {
      const uint4 v = p[i];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        xv[8 * i + 2 * j] = bf16_bits_to_f32(w[j] & 0xFFFFu);
        xv[8 * i + 2 * j + 1] = bf16_bits_to_f32(w[j] >> 16);
      }
    }
  }
  if constexpr (ACT == MOE_ACT_F32) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < CC; ++i) {
      xp[ch * CC + i] = __float_as_uint(xv[i]);
      s += xv[i];
    }
    cs[ch] = make_float2(0.f, s);
  } else if constexpr (BITS == 4) {
    float c = 0.f, s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float* v = xv + 8 * j;
      const uint32_t pa = pack_f16x2(v[0], v[4]);
      const uint32_t pb = pack_f16x2(v[1] * 0.0625f, v[5] * 0.0625f);
      const uint32_t pc = pack_f16x2(v[2], v[6]);
      const uint32_t pf = pack_f16x2(v[3] * 0.0625f, v[7] * 0.0625f);
      xp[ch * 16 + j * 4 + 0] = pa;
      xp[ch * 16 + j * 4 + 1] = pb;
      xp[ch * 16 + j * 4 + 2] = pc;
      xp[ch * 16 + j * 4 + 3] = pf;
      c += f16_lo(pa) + f16_hi(pa) + f16_lo(pb) + f16_hi(pb) + f16_lo(pc) + f16_hi(pc) +
           f16_lo(pf) + f16_hi(pf);
      s += f16_lo(pa) + f16_hi(pa) + f16_lo(pc) + f16_hi(pc) +
           16.0f * (f16_lo(pb) + f16_hi(pb) + f16_lo(pf) + f16_hi(pf));
    }
    cs[ch] = make_float2(1024.0f * c, s);
  } else {
    float c = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t p = pack_f16x2(xv[2 * j], xv[2 * j + 1]);
      xp[ch * 8 + j] = p;
      c += f16_lo(p) + f16_hi(p);
    }
    cs[ch] = make_float2(1024.0f * c, c);
  }
}

// sum_c q_c * x_c over one lane's 16 code bytes (32 int4 / 16 int8 codes),
// returned as (dot, correction) so that dot - correction = sum q x.
template <int BITS, int ACT>
__device__ __forceinline__ float lane_dot(const uint4 q, const uint32_t* __restrict__ xp, int gc) {
  const uint32_t d[4] = {q.x, q.y, q.z, q.w};
  float acc = 0.f;
  if constexpr (ACT == MOE_ACT_F32) {
    const float* xs = reinterpret_cast<const float*>(xp) + gc * chunk_cols<BITS>();
    if constexpr (BITS == 4) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = d[j] & 0x0F0F0F0Fu, hi = (d[j] >> 4) & 0x0F0F0F0Fu;
        const float* v = xs + 8 * j;
        acc += (float)(lo & 0xFF) * v[0] + (float)(hi & 0xFF) * v[1] +
               (float)((lo >> 8) & 0xFF) * v[2] + (float)((hi >> 8) & 0xFF) * v[3] +
               (float)((lo >> 16) & 0xFF) * v[4] + (float)((hi >> 16) & 0xFF) * v[5] +
               (float)(lo >> 24) * v[6] + (float)(hi >> 24) * v[7];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float* v = xs + 4 * j;
        acc += (float)(d[j] & 0xFF) * v[0] + (float)((d[j] >> 8) & 0xFF) * v[1] +
               (float)((d[j] >> 16) & 0xFF) * v[2] + (float)(d[j] >> 24) * v[3];
      }
    }
  } else if constexpr (BITS == 4) {
    const uint4* xq = reinterpret_cast<const uint4*>(xp + gc * 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 X = xq[j];
      const uint32_t e = d[j] >> 8;
      acc = dot2((d[j] & 0x000F000Fu) | 0x64006400u, X.x, acc);
      acc = dot2((d[j] & 0x00F000F0u) | 0x64006400u, X.y, acc);
      acc = dot2((e & 0x000F000Fu) | 0x64006400u, X.z, acc);
      acc = dot2((e & 0x00F000F0u) | 0x64006400u, X.w, acc);
    }
  } else {
    const uint4* xq = reinterpret_cast<const uint4*>(xp + gc * 8);
    const uint4 X0 = xq[0], X1 = xq[1];
    const uint32_t xs[8] = {X0.x, X0.y, X0.z, X0.w, X1.x, X1.y, X1.z, X1.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc = dot2(__builtin_amdgcn_perm(0x64646464u, d[j], 0x04010400u), xs[2 * j], acc);
      acc = dot2(__builtin_amdgcn_perm(0x64646464u, d[j], 0x04030402u), xs[2 * j + 1], acc);
    }
  }
  return acc;
}

// ---------------------------------------------------------------------------
// gate/up: one workgroup = one 16-row tile of one work item (a (token, j)
// pair at small batch, or an expert bucket).  4 waves split the k-blocks;
// lane l owns row l/4 and chunk l%4 of each k-block.

constexpr int kGuTokens = 4;  // tokens per LDS staging round
constexpr int kGemvSlots = 1024;  // workgroups of the grid-stride bucketed GEMV kernels
// The down GEMV's items are one 16-row output tile of one bucket (H/16 per
// bucket): 2048 workgroups (8 per CU, no dynamic LDS) take a few small
// buckets in one round.
constexpr int kDownSlots = 2048;

struct GuItem {
  const uint8_t* blob;
  int n;          // tokens
  int start;      // bucket start position
  int tile_limit; // tiles of this blob
  int kind;       // 0 decode pair, 1 bucket, 2 shared
  int t;          // decode: token
  int64_t hrow;   // decode: h row
};

#define MOE_GATEUP_PARAMS                                                                   \
  const void* __restrict__ x, const int32_t* __restrict__ topk_idx,                          \
      const uint8_t* __restrict__ slab, const int32_t* __restrict__ slot_table, int64_t stride, \
      const uint8_t* __restrict__ shared_blob, const int32_t* __restrict__ counts,           \
      const int32_t* __restrict__ offsets, const int32_t* __restrict__ pairs,                \
      float* __restrict__ h, int T, int H, int E, int k, int I, int Is, int64_t gu_unit_r,     \
      int64_t gu_tile_r, int64_t gu_unit_s, int64_t gu_tile_s, int bucketed, int has_shared,   \
      int min_rows
#define MOE_GATEUP_ARGS                                                                        \
  x, topk_idx, slab, slot_table, stride, shared_blob, counts, offsets, pairs, h, T, H, E, k, I, \
      Is, gu_unit_r, gu_tile_r, gu_unit_s, gu_tile_s, bucketed, has_shared, min_rows

template <int BITS, int ACT>
__device__ __forceinline__ void gateup_item(MOE_GATEUP_PARAMS, int tile, int item) {
  constexpr int GPK = BITS == 4 ? 2 : 1;
  constexpr int CC = chunk_cols<BITS>();
  extern __shared__ uint8_t smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  // resolve the work item
  const uint8_t* blob;
  int n, start = 0, inter, kind, t_dec = 0;
  int64_t unit_b, tile_b, hbase;
  if (!bucketed) {
    const int t = item / (k + has_shared), j = item % (k + has_shared);
    t_dec = t;
    n = 1;
    if (j < k) {
      const int e = topk_idx[(int64_t)t * k + j];
      blob = slab + (int64_t)slot_table[e] * stride;
      inter = I;
      unit_b = gu_unit_r;
      tile_b = gu_tile_r;
      hbase = ((int64_t)t * k + j) * I;
      kind = 0;
    } else {
      blob = shared_blob;
      inter = Is;
      unit_b = gu_unit_s;
      tile_b = gu_tile_s;
      hbase = (int64_t)T * k * I + (int64_t)t * Is;
      kind = 0;
    }
  } else if (item < E) {
    n = counts[item];
    if (n == 0 || n >= min_rows) return;  // empty, or on the MFMA grouped GEMMs
    start = offsets[item];
    blob = slab + (int64_t)slot_table[item] * stride;
    inter = I;
    unit_b = gu_unit_r;
    tile_b = gu_tile_r;
    hbase = 0;
    kind = 1;
  } else {
    n = T;
    if (n >= min_rows) return;
    blob = shared_blob;
    inter = Is;
    unit_b = gu_unit_s;
    tile_b = gu_tile_s;
    hbase = (int64_t)T * k * I;
    kind = 2;
  }
  if (tile * kRowTile >= inter) return;

  const int stage_bytes = XStage<BITS, ACT>::bytes(H);
  const int n_kb = H / (kRowBytes * (8 / BITS));
  float* red = reinterpret_cast<float*>(smem + kGuTokens * stage_bytes);  // [4][kGuTokens][16][2]
  const int row = lane >> 2, c4 = lane & 3;
  const uint8_t* tbase = blob + (int64_t)tile * tile_b;
  const int sbg_off = 2 * kCodeBlockBytes + (row * GPK + (c4 * CC) / kGroup) * 4;
  const int sbu_off = sbg_off + kRowTile * GPK * 4;

  // The wave's first KU k-blocks of codes are requested before the tokens
  // are staged, so the two memory round trips overlap (the staging barrier
  // waits for both).  KU covers H = 2048; larger H runs the rest in a loop.
  constexpr int KU = BITS == 4 ? 4 : 8;
  for (int t0 = 0; t0 < n; t0 += kGuTokens) {
    const int nt = min(kGuTokens, n - t0);
    uint4 qg[KU], qu[KU];
    uint32_t sbg[KU], sbu[KU];
#pragma unroll
    for (int i = 0; i < KU; ++i) {
      const int kb = wave + 4 * i;
      if (kb < n_kb) {
        const uint8_t* unit = tbase + (int64_t)kb * unit_b;
        qg[i] = *reinterpret_cast<const uint4*>(unit + lane * 16);
        qu[i] = *reinterpret_cast<const uint4*>(unit + kCodeBlockBytes + lane * 16);
        sbg[i] = *reinterpret_cast<const uint32_t*>(unit + sbg_off);
        sbu[i] = *reinterpret_cast<const uint32_t*>(unit + sbu_off);
      }
    }
    if (t0 > 0) __syncthreads();  // the previous round's staging and sums are read
    {
      // every chunk of the round's tokens at once: thread i stages chunk
      // i % nchunk of token i / nchunk
      const int nchunk = H / chunk_cols<BITS>();
      for (int i = threadIdx.x; i < nt * nchunk; i += blockDim.x) {
        const int tt = i / nchunk, ch = i - tt * nchunk;
        int tok;
        if (kind == 0) tok = t_dec;
        else if (kind == 1) tok = pairs[start + t0 + tt] / k;
        else tok = t0 + tt;
        uint8_t* st = smem + tt * stage_bytes;
        stage_chunk<BITS, ACT>(x, tok, ch, H, reinterpret_cast<uint32_t*>(st),
                               reinterpret_cast<float2*>(st + XStage<BITS, ACT>::dwords(H) * 4));
      }
    }
    __syncthreads();
    float g[kGuTokens], u[kGuTokens];
#pragma unroll
    for (int tt = 0; tt < kGuTokens; ++tt) g[tt] = u[tt] = 0.f;
    auto kblock = [&](int kb, const uint4& cg, const uint4& cu, uint32_t wg, uint32_t wu) {
      const float sg = bf16_bits_to_f32(wg & 0xFFFFu), bg = bf16_bits_to_f32(wg >> 16);
      const float su = bf16_bits_to_f32(wu & 0xFFFFu), bu = bf16_bits_to_f32(wu >> 16);
      const int gc = kb * 4 + c4;
#pragma unroll
      for (int tt = 0; tt < kGuTokens; ++tt) {
        if (tt < nt) {
          const uint8_t* st = smem + tt * stage_bytes;
          const uint32_t* xp = reinterpret_cast<const uint32_t*>(st);
          const float2 cs =
              reinterpret_cast<const float2*>(st + XStage<BITS, ACT>::dwords(H) * 4)[gc];
          const float pg = lane_dot<BITS, ACT>(cg, xp, gc) - cs.x;
          const float pu = lane_dot<BITS, ACT>(cu, xp, gc) - cs.x;
          g[tt] += sg * pg + bg * cs.y;
          u[tt] += su * pu + bu * cs.y;
        }
      }
    };
#pragma unroll
    for (int i = 0; i < KU; ++i) {
      const int kb = wave + 4 * i;
      if (kb < n_kb) kblock(kb, qg[i], qu[i], sbg[i], sbu[i]);
    }
    for (int kb = wave + 4 * KU; kb < n_kb; kb += 4) {
      const uint8_t* unit = tbase + (int64_t)kb * unit_b;
      kblock(kb, *reinterpret_cast<const uint4*>(unit + lane * 16),
             *reinterpret_cast<const uint4*>(unit + kCodeBlockBytes + lane * 16),
             *reinterpret_cast<const uint32_t*>(unit + sbg_off),
             *reinterpret_cast<const uint32_t*>(unit + sbu_off));
    }
    // reduce the 4 lanes of a row, then the 4 waves
#pragma unroll
    for (int tt = 0; tt < kGuTokens; ++tt) {
      g[tt] = quad_sum(g[tt]);
      u[tt] = quad_sum(u[tt]);
      if (c4 == 0) {
        red[((wave * kGuTokens + tt) * kRowTile + row) * 2 + 0] = g[tt];
        red[((wave * kGuTokens + tt) * kRowTile + row) * 2 + 1] = u[tt];
      }
    }
    __syncthreads();
    if (threadIdx.x < nt * kRowTile) {
      const int tt = threadIdx.x / kRowTile, r = threadIdx.x % kRowTile;
      float gs = 0.f, us = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        gs += red[((w * kGuTokens + tt) * kRowTile + r) * 2 + 0];
        us += red[((w * kGuTokens + tt) * kRowTile + r) * 2 + 1];
      }
      int64_t hrow;
      if (kind == 0) hrow = hbase;
      else if (kind == 1) hrow = (int64_t)(start + t0 + tt) * inter;
      else hrow = hbase + (int64_t)(t0 + tt) * inter;
      h[hrow + tile * kRowTile + r] = silu_f32(gs) * us;
    }
  }
}

// Small batch: grid (tiles, T*(k+has_shared)) work items.  Bucketed: a
// grid-stride loop over (bucket, tile) pairs of the buckets listed in
// small_list (those not on the MFMA grouped GEMMs), so that no workgroup is
// launched for an empty or MFMA-handled bucket.
template <int BITS, int ACT>
__global__ __launch_bounds__(256) void gateup_kernel(MOE_GATEUP_PARAMS,
                                                     const int32_t* __restrict__ small_list,
                                                     const int32_t* __restrict__ n_small,
                                                     int tiles) {
  if (!bucketed) {
    gateup_item<BITS, ACT>(MOE_GATEUP_ARGS, blockIdx.x, blockIdx.y);
    return;
  }
  const int total = *n_small * tiles;
  for (int q = blockIdx.x; q < total; q += gridDim.x) {
    gateup_item<BITS, ACT>(MOE_GATEUP_ARGS, q % tiles, small_list[q / tiles]);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// down + combine at small batch: one workgroup = one 16-row tile of the
// output of one token; it walks the token's k routed items and the shared
// item, so the weighted sum is formed in a fixed order without atomics.

template <int BITS>
__device__ __forceinline__ float lane_dot_h(const uint4 q, const float* __restrict__ hv,
                                            float& hsum) {
  const uint32_t d[4] = {q.x, q.y, q.z, q.w};
  float acc = 0.f;
  if constexpr (BITS == 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 a = *reinterpret_cast<const float4*>(hv + 8 * j);
      const float4 b = *reinterpret_cast<const float4*>(hv + 8 * j + 4);
      const uint32_t lo = d[j] & 0x0F0F0F0Fu, hi = (d[j] >> 4) & 0x0F0F0F0Fu;
      acc += (float)(lo & 0xFF) * a.x + (float)(hi & 0xFF) * a.y +
             (float)((lo >> 8) & 0xFF) * a.z + (float)((hi >> 8) & 0xFF) * a.w +
             (float)((lo >> 16) & 0xFF) * b.x + (float)((hi >> 16) & 0xFF) * b.y +
             (float)(lo >> 24) * b.z + (float)(hi >> 24) * b.w;
      hsum += (a.x + a.y) + (a.z + a.w) + (b.x + b.y) + (b.z + b.w);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 a = *reinterpret_cast<const float4*>(hv + 4 * j);
      acc += (float)(d[j] & 0xFF) * a.x + (float)((d[j] >> 8) & 0xFF) * a.y +
             (float)((d[j] >> 16) & 0xFF) * a.z + (float)(d[j] >> 24) * a.w;
      hsum += (a.x + a.y) + (a.z + a.w);
    }
  }
  return acc;
}

template <int BITS, int ACT>
__global__ __launch_bounds__(256) void down_decode_kernel(
    const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_w,
    const float* __restrict__ gamma, const uint8_t* __restrict__ slab,
    const int32_t* __restrict__ slot_table, int64_t stride, const uint8_t* __restrict__ shared_blob,
    const float* __restrict__ h, void* __restrict__ out, int T, int H, int k, int I, int Is,
    int64_t d_off_r, int64_t d_unit_r, int64_t d_tile_r, int64_t d_off_s, int64_t d_unit_s,
    int64_t d_tile_s, int has_shared) {
  constexpr int GPK = BITS == 4 ? 2 : 1;
  constexpr int CC = chunk_cols<BITS>();
  constexpr int KBC = kRowBytes * (8 / BITS);
  __shared__ float red[4][kRowTile];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tile = blockIdx.x, t = blockIdx.y;
  const int row = lane >> 2, c4 = lane & 3;
  const int sb_off = kCodeBlockBytes + (row * GPK + (c4 * CC) / kGroup) * 4;
  const int nkb_r = I / KBC, nkb_s = has_shared ? Is / KBC : 0;
  const int n_units = k * nkb_r + nkb_s;
  float acc = 0.f;
  for (int u = wave; u < n_units; u += 4) {
    const uint8_t* unit;
    const float* hv;
    float w;
    int kb;
    if (u < k * nkb_r) {
      const int j = u / nkb_r;
      kb = u - j * nkb_r;
      const int e = topk_idx[(int64_t)t * k + j];
      unit = slab + (int64_t)slot_table[e] * stride + d_off_r + (int64_t)tile * d_tile_r +
             (int64_t)kb * d_unit_r;
      hv = h + ((int64_t)t * k + j) * I;
      w = topk_w[(int64_t)t * k + j];
    } else {
      kb = u - k * nkb_r;
      unit = shared_blob + d_off_s + (int64_t)tile * d_tile_s + (int64_t)kb * d_unit_s;
      hv = h + (int64_t)T * k * I + (int64_t)t * Is;
      w = gamma[t];
    }
    const uint4 q = *reinterpret_cast<const uint4*>(unit + lane * 16);
    const uint32_t sb = *reinterpret_cast<const uint32_t*>(unit + sb_off);
    float hsum = 0.f;
    const float p = lane_dot_h<BITS>(q, hv + kb * KBC + c4 * CC, hsum);
    acc += w * (bf16_bits_to_f32(sb & 0xFFFFu) * p + bf16_bits_to_f32(sb >> 16) * hsum);
  }
  acc = quad_sum(acc);
  if (c4 == 0) red[wave][row] = acc;
  __syncthreads();
  if (threadIdx.x < kRowTile) {
    const float v = (red[0][threadIdx.x] + red[1][threadIdx.x]) +
                    (red[2][threadIdx.x] + red[3][threadIdx.x]);
    store_act<ACT>(out, (int64_t)t * H + tile * kRowTile + threadIdx.x, v);
  }
}

// ---------------------------------------------------------------------------
// batched: down per expert bucket, writing weighted per-(token, j) partial
// rows; a combine kernel then sums each token's k+1 partials in order.

constexpr int kDownTok = 4;  // tokens per round of the bucketed down GEMV

#define MOE_DOWNB_PARAMS                                                                     \
  const float* __restrict__ topk_w, const float* __restrict__ gamma,                           \
      const uint8_t* __restrict__ slab, const int32_t* __restrict__ slot_table, int64_t stride, \
      const uint8_t* __restrict__ shared_blob, const int32_t* __restrict__ counts,           \
      const int32_t* __restrict__ offsets, const int32_t* __restrict__ pairs,                \
      const float* __restrict__ h, float* __restrict__ partial, int T, int H, int E, int k,    \
      int I, int Is, int64_t d_off_r, int64_t d_unit_r, int64_t d_tile_r, int64_t d_off_s,     \
      int64_t d_unit_s, int64_t d_tile_s, int min_rows
#define MOE_DOWNB_ARGS                                                                       \
  topk_w, gamma, slab, slot_table, stride, shared_blob, counts, offsets, pairs, h, partial, T, \
      H, E, k, I, Is, d_off_r, d_unit_r, d_tile_r, d_off_s, d_unit_s, d_tile_s, min_rows

template <int BITS>
__device__ __forceinline__ void down_bucket_item(MOE_DOWNB_PARAMS, float (*red)[kDownTok][kRowTile],
                                                 int tile, int item) {
  constexpr int GPK = BITS == 4 ? 2 : 1;
  constexpr int CC = chunk_cols<BITS>();
  constexpr int KBC = kRowBytes * (8 / BITS);
  constexpr int kTok = kDownTok;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = lane >> 2, c4 = lane & 3;
  const int sb_off = kCodeBlockBytes + (row * GPK + (c4 * CC) / kGroup) * 4;
  const uint8_t* tbase;
  int n, start = 0, inter, nkb;
  int64_t unit_b;
  const bool shared = item >= E;
  if (!shared) {
    n = counts[item];
    if (n == 0 || n >= min_rows) return;  // empty, or on the MFMA grouped GEMMs
    start = offsets[item];
    inter = I;
    tbase = slab + (int64_t)slot_table[item] * stride + d_off_r + (int64_t)tile * d_tile_r;
    unit_b = d_unit_r;
  } else {
    n = T;
    if (n >= min_rows) return;
    inter = Is;
    tbase = shared_blob + d_off_s + (int64_t)tile * d_tile_s;
    unit_b = d_unit_s;
  }
  nkb = inter / KBC;
  for (int t0 = 0; t0 < n; t0 += kTok) {
    const int nt = min(kTok, n - t0);
    // the destination of this thread's output (token, slot, weight), read
    // while the codes load
    int otok = 0, oj = 0;
    float ow = 0.f;
    if (threadIdx.x < nt * kRowTile) {
      const int tt = threadIdx.x / kRowTile;
      if (!shared) {
        const int p = pairs[start + t0 + tt];
        otok = p / k;
        oj = p - otok * k;
        ow = topk_w[p];
      } else {
        otok = t0 + tt;
        oj = k;
        ow = gamma[otok];
      }
    }
    float acc[kTok];
#pragma unroll
    for (int tt = 0; tt < kTok; ++tt) acc[tt] = 0.f;
    for (int kb = wave; kb < nkb; kb += 4) {
      const uint8_t* unit = tbase + (int64_t)kb * unit_b;
      const uint4 q = *reinterpret_cast<const uint4*>(unit + lane * 16);
      const uint32_t sb = *reinterpret_cast<const uint32_t*>(unit + sb_off);
      const float s = bf16_bits_to_f32(sb & 0xFFFFu), b = bf16_bits_to_f32(sb >> 16);
#pragma unroll
      for (int tt = 0; tt < kTok; ++tt) {
        if (tt < nt) {
          const float* hv = shared ? h + (int64_t)T * k * I + (int64_t)(t0 + tt) * Is
                                   : h + (int64_t)(start + t0 + tt) * I;
          float hsum = 0.f;
          const float p = lane_dot_h<BITS>(q, hv + kb * KBC + c4 * CC, hsum);
          acc[tt] += s * p + b * hsum;
        }
      }
    }
#pragma unroll
    for (int tt = 0; tt < kTok; ++tt) {
      acc[tt] = quad_sum(acc[tt]);
      if (c4 == 0) red[wave][tt][row] = acc[tt];
    }
    __syncthreads();
    if (threadIdx.x < nt * kRowTile) {
      const int tt = threadIdx.x / kRowTile, r = threadIdx.x % kRowTile;
      const float v = (red[0][tt][r] + red[1][tt][r]) + (red[2][tt][r] + red[3][tt][r]);
      partial[((int64_t)otok * (k + 1) + oj) * H + tile * kRowTile + r] = ow * v;
    }
    __syncthreads();
  }
}

template <int BITS>
__global__ __launch_bounds__(256) void down_bucket_kernel(MOE_DOWNB_PARAMS,
                                                          const int32_t* __restrict__ small_list,
                                                          const int32_t* __restrict__ n_small,
                                                          int tiles) {
  __shared__ float red[4][kDownTok][kRowTile];
  const int total = *n_small * tiles;
  for (int q = blockIdx.x; q < total; q += gridDim.x) {
    down_bucket_item<BITS>(MOE_DOWNB_ARGS, red, q % tiles, small_list[q / tiles]);
    __syncthreads();
  }
}

template <int ACT>
__device__ __forceinline__ float4 load_act4v(const void* p, int64_t i) {
  if constexpr (ACT == MOE_ACT_F32) {
    return *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p) + i);
  } else {
    const uint2 q = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(p) + i);
    return make_float4(bf16_bits_to_f32(q.x & 0xFFFFu), bf16_bits_to_f32(q.x >> 16),
                       bf16_bits_to_f32(q.y & 0xFFFFu), bf16_bits_to_f32(q.y >> 16));
  }
}
template <int ACT>
__device__ __forceinline__ void store_act4v(void* p, int64_t i, float4 v) {
  if constexpr (ACT == MOE_ACT_F32) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(p) + i) = v;
  } else {
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p) + i) =
        make_uint2((uint32_t)f32_to_bf16_bits(v.x) | ((uint32_t)f32_to_bf16_bits(v.y) << 16),
                   (uint32_t)f32_to_bf16_bits(v.z) | ((uint32_t)f32_to_bf16_bits(v.w) << 16));
  }
}
template <int ACT>
__device__ __forceinline__ float round_act1(float v) {
  if constexpr (ACT == MOE_ACT_F32) return v;
  else return bf16_bits_to_f32(f32_to_bf16_bits(v));
}

// out[t] = sum over the token's k routed slots and the shared slot of the
// weighted partial rows, in slot order, rounded to the act dtype.  One
// workgroup per token; thread i holds columns 8 (i + 256 r) .. +7, so that
// at hidden <= 2048 every load of a thread is in flight at once (one memory
// round trip per token).  With epi >= 1 it also adds the residual, x_res[t] =
// act(x_res[t] + out[t]), and with epi == 2 writes the next layer's input
// act(rmsnorm(x_res[t])) (unit weight), so a chain needs no separate launch
// between layers.  NJ = the most slots a call has (k + 1 <= NJ).  F16P: the
// partial rows are fp16 with a power-of-two scale 2^e per row and 64-column
// block, the exponents a byte each at byte offset e_off (the grouped GEMMs'
// down kernel); the scale is undone exactly before the same fp32 sum.
template <int ACT, int NJ, bool F16P>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ partial,
                                                      void* __restrict__ out, int H, int k,
                                                      int has_shared, void* __restrict__ x_res,
                                                      void* __restrict__ x_hat, float eps,
                                                      int epi, int64_t e_off) {
  constexpr int kR = MOE_MAX_HIDDEN / 2048;
  __shared__ float wsum[4];
  const int t = blockIdx.x;
  const int nj = k + has_shared;
  const int64_t base = (int64_t)t * H;
  float4 v[kR][2];
  float ss = 0.f;
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    const int c = (r * 256 + (int)threadIdx.x) * 8;
    if (c >= H) continue;
    float4 p[NJ][2];
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      if (j < nj) {
        const int64_t row = (int64_t)t * (k + 1) + j;
        if constexpr (F16P) {
          const uint4 q = *reinterpret_cast<const uint4*>(
              reinterpret_cast<const uint16_t*>(partial) + row * H + c);
          const int e = reinterpret_cast<const int8_t*>(partial)[e_off + row * (H / 64) + c / 64];
          const float sc = __uint_as_float((uint32_t)(127 + e) << 23);  // 2^e
          const uint32_t w[4] = {q.x, q.y, q.z, q.w};
          float f[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            f[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xFFFFu)) * sc;
            f[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16)) * sc;
          }
          p[j][0] = make_float4(f[0], f[1], f[2], f[3]);
          p[j][1] = make_float4(f[4], f[5], f[6], f[7]);
        } else {
          const float4* src = reinterpret_cast<const float4*>(partial + row * H + c);
          p[j][0] = src[0];
          p[j][1] = src[1];
        }
      }
    // the residual columns requested with the partial rows (one round trip)
    float4 xr[2];
    if (epi >= 1)
#pragma unroll
      for (int h = 0; h < 2; ++h) xr[h] = load_act4v<ACT>(x_res, base + c + 4 * h);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        if (j < nj) {
          a.x += p[j][h].x;
          a.y += p[j][h].y;
          a.z += p[j][h].z;
          a.w += p[j][h].w;
        }
      }
      store_act4v<ACT>(out, base + c + 4 * h, a);
      if (epi >= 1) {
        v[r][h] = make_float4(round_act1<ACT>(xr[h].x + round_act1<ACT>(a.x)),
                              round_act1<ACT>(xr[h].y + round_act1<ACT>(a.y)),
                              round_act1<ACT>(xr[h].z + round_act1<ACT>(a.z)),
                              round_act1<ACT>(xr[h].w + round_act1<ACT>(a.w)));
        store_act4v<ACT>(x_res, base + c + 4 * h, v[r][h]);
        ss += (v[r][h].x * v[r][h].x + v[r][h].y * v[r][h].y) +
              (v[r][h].z * v[r][h].z + v[r][h].w * v[r][h].w);
      }
    }
  }
  if (epi < 2) return;
  ss = warp_sum(ss);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
  const float inv = 1.0f / sqrtf(tot / (float)H + eps);
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    const int c = (r * 256 + (int)threadIdx.x) * 8;
    if (c < H)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        store_act4v<ACT>(x_hat, base + c + 4 * h,
                         make_float4(v[r][h].x * inv, v[r][h].y * inv, v[r][h].z * inv,
                                     v[r][h].w * inv));
  }
}

// ---------------------------------------------------------------------------
// token -> expert bucketing: stable by token.  Each 64-token block builds a
// per-expert 64-bit mask of the tokens that chose the expert; ranks inside a
// block are popcounts of the mask below the token, so the order is
// deterministic without sorting.

__global__ __launch_bounds__(64) void bucket_mask_kernel(const int32_t* __restrict__ topk_idx,
                                                         uint64_t* __restrict__ masks, int T,
                                                         int E, int k) {
  __shared__ unsigned long long m[MOE_MAX_EXPERTS];
  const int b = blockIdx.x, lane = threadIdx.x;
  for (int e = lane; e < E; e += 64) m[e] = 0ull;
  __syncthreads();
  const int t = b * 64 + lane;
  if (t < T)
    for (int j = 0; j < k; ++j) atomicOr(&m[topk_idx[(int64_t)t * k + j]], 1ull << lane);
  __syncthreads();
  for (int e = lane; e < E; e += 64) masks[(int64_t)b * E + e] = m[e];
}

// Per-expert counts and bucket offsets (exclusive scan over experts), the
// per-block write offsets, and the list of buckets the GEMV kernels take:
// experts with 1 .. min_rows-1 tokens, and the shared expert (bucket E) when
// T < min_rows.  One workgroup of 1024 threads (E <= 1024).  With tiles !=
// nullptr (E + has_shared <= 1024) it also builds the grouped GEMMs' tile
// list as the tile-list kernel does (bucket E the shared expert's T rows,
// each bucket of at least tile_min entries cut into tiles of mt rows).  When the block
// masks fit one round of loads per thread, Q = 1024 / E' threads share an
// expert (E' = 256, 512 or 1024 expert slots), each reading a run of at most
// 16 consecutive blocks; else one thread per expert reads them in rounds.
__global__ __launch_bounds__(1024) void bucket_scan_kernel(const uint64_t* __restrict__ masks,
                                                           int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ blkoff,
                                                           int32_t* __restrict__ small_list,
                                                           int32_t* __restrict__ n_small, int T,
                                                           int E, int k, int nblk, int min_rows,
                                                           int has_shared,
                                                           int32_t* __restrict__ tiles,
                                                           int32_t* __restrict__ ntiles,
                                                           int max_tiles, int mt, int tile_min) {
  __shared__ int wsum[16], wsmall[16];
  __shared__ int cqs[1024];  // one round: count of thread (q, e)'s run, at q * EP + e
  __shared__ int exl[1024];  // one round: expert e's bucket offset
  const int e = threadIdx.x, lane = e & 63, wave = e >> 6;
  constexpr int kU = 16;  // block masks in flight per thread and round
  // one round: Q threads per expert, thread (q, eq) = q * EP + eq reads blocks
  // q * BQ .. q * BQ + BQ - 1 of expert eq; the per-block counts kept a byte each
  const int Q = E <= 256 ? 4 : (E <= 512 ? 2 : 1), EP = 1024 / Q;
  const int q = e / EP, eq = e % EP, BQ = (nblk + Q - 1) / Q;
  const bool one_round = BQ <= kU;
  uint32_t pq[kU / 4] = {};
  // with at most kPackedBlocks blocks the per-block counts are kept, a byte
  // each, for the offsets below (no second read of the masks)
  constexpr int kPackedBlocks = 64;
  const bool packed = nblk <= kPackedBlocks;
  uint32_t pc[kPackedBlocks / 4] = {};
  int c = 0;
  if (one_round) {
    int cv = 0;
    if (eq < E) {
      // every load unconditional (past the run: the last block again, not counted)
      uint64_t m[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) m[u] = masks[(int64_t)min(q * BQ + u, nblk - 1) * E + eq];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int n = (u < BQ && q * BQ + u < nblk) ? __popcll(m[u]) : 0;
        cv += n;
        pq[u >> 2] |= (uint32_t)n << (8 * (u & 3));
      }
    }
    cqs[e] = cv;
    __syncthreads();
    if (e < E)
      for (int j = 0; j < Q; ++j) c += cqs[j * EP + e];
  } else if (e < E && packed) {
#pragma unroll
    for (int r = 0; r < kPackedBlocks / kU; ++r) {
      uint64_t m[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int b = r * kU + u;
        m[u] = b < nblk ? masks[(int64_t)b * E + e] : 0ull;
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int b = r * kU + u, n = __popcll(m[u]);
        c += n;
        pc[b >> 2] |= (uint32_t)n << (8 * (b & 3));
      }
    }
  } else if (e < E) {
    for (int b0 = 0; b0 < nblk; b0 += kU) {
      uint64_t m[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) m[u] = b0 + u < nblk ? masks[(int64_t)(b0 + u) * E + e] : 0ull;
#pragma unroll
      for (int u = 0; u < kU; ++u) c += __popcll(m[u]);
    }
  }
  // inclusive scans inside the wave: token counts, and small-bucket flags
  const int sm = (e < E && c > 0 && c < min_rows) ? 1 : 0;
  int v = c, vs = sm;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off, 64), os = __shfl_up(vs, off, 64);
    if (lane >= off) {
      v += o;
      vs += os;
    }
  }
  if (lane == 63) {
    wsum[wave] = v;
    wsmall[wave] = vs;
  }
  __syncthreads();
  int wbase = 0, sbase = 0;
  for (int w = 0; w < wave; ++w) {
    wbase += wsum[w];
    sbase += wsmall[w];
  }
  const int excl = wbase + v - c;
  if (sm) small_list[sbase + vs - 1] = e;
  if (e < E) {
    counts[e] = c;
    offsets[e] = excl;
  }
  if (one_round) {
    // thread (q, eq): its run of blocks starts after the runs of q' < q
    if (e < E) exl[e] = excl;
    __syncthreads();
    if (eq < E) {
      int run = exl[eq];
      for (int j = 0; j < q; ++j) run += cqs[j * EP + eq];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int b = q * BQ + u;
        if (u < BQ && b < nblk) {
          blkoff[(int64_t)b * E + eq] = run;
          run += (pq[u >> 2] >> (8 * (u & 3))) & 0xFFu;
        }
      }
    }
  } else if (e < E) {
    int run = excl;
    if (packed) {
#pragma unroll
      for (int b = 0; b < kPackedBlocks; ++b) {
        if (b < nblk) {
          blkoff[(int64_t)b * E + e] = run;
          run += (pc[b >> 2] >> (8 * (b & 3))) & 0xFFu;
        }
      }
    }
    for (int b0 = 0; !packed && b0 < nblk; b0 += kU) {
      uint64_t m[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) m[u] = b0 + u < nblk ? masks[(int64_t)(b0 + u) * E + e] : 0ull;
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if (b0 + u < nblk) {
          blkoff[(int64_t)(b0 + u) * E + e] = run;
          run += __popcll(m[u]);
        }
      }
    }
  }
  if (tiles != nullptr) {
    const int nb = e < E ? c : (e == E && has_shared ? T : 0);
    const int ct = nb >= tile_min ? (nb + mt - 1) / mt : 0;
    int tv = ct;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(tv, off, 64);
      if (lane >= off) tv += o;
    }
    __shared__ int tsum[16];
    if (lane == 63) tsum[wave] = tv;
    __syncthreads();
    int tb = 0;
    for (int w = 0; w < wave; ++w) tb += tsum[w];
    if (e == 1023) *ntiles = min(tb + tv, max_tiles);
    const int tbase = tb + tv - ct;
    for (int i = 0; i < ct; ++i) {
      const int t = tbase + i;
      if (t < max_tiles) {
        tiles[2 * t] = e;
        tiles[2 * t + 1] = i * mt;
      }
    }
  }
  if (e == 1023) {
    int ns = 0;
    for (int w = 0; w < 16; ++w) ns += wsmall[w];
    if (has_shared && T < min_rows) small_list[ns++] = E;
    *n_small = ns;
    counts[E] = T;
    offsets[E] = T * k;
  }
}

__global__ __launch_bounds__(64) void bucket_scatter_kernel(const int32_t* __restrict__ topk_idx,
                                                            const uint64_t* __restrict__ masks,
                                                            const int32_t* __restrict__ blkoff,
                                                            int32_t* __restrict__ pairs, int T,
                                                            int E, int k) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int t = b * 64 + lane;
  if (t >= T) return;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int j = 0; j < k; ++j) {
    const int e = topk_idx[(int64_t)t * k + j];
    const uint64_t m = masks[(int64_t)b * E + e];
    pairs[blkoff[(int64_t)b * E + e] + __popcll(m & below)] = t * k + j;
  }
}

// One token block (T <= 64) and E < 1024: the mask, scan and scatter of the
// three kernels above in one workgroup of 1024 threads, with the masks in
// LDS, the same arithmetic and so the same outputs; with tiles != nullptr
// also the grouped GEMMs' tile list (buckets 0..E, bucket E the shared
// expert's T rows, each of at least tile_min entries cut into tiles of mt
// rows), as the tile-list kernel builds it.  Thread e owns expert e, thread
// t < T token t.
__global__ __launch_bounds__(1024) void bucket_small_kernel(
    const int32_t* __restrict__ topk_idx, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ pairs, int32_t* __restrict__ small_list,
    int32_t* __restrict__ n_small, int32_t* __restrict__ tiles, int32_t* __restrict__ ntiles,
    int max_tiles, int mt, int tile_min, int T, int E, int k, int min_rows, int has_shared) {
  __shared__ unsigned long long m[MOE_MAX_EXPERTS];
  __shared__ int excl_l[MOE_MAX_EXPERTS];
  __shared__ int wsum[16], wsmall[16];
  const int e = threadIdx.x, lane = e & 63, wave = e >> 6;
  if (e < E) m[e] = 0ull;
  __syncthreads();
  if (e < T)
    for (int j = 0; j < k; ++j) atomicOr(&m[topk_idx[(int64_t)e * k + j]], 1ull << e);
  __syncthreads();
  const int c = e < E ? __popcll(m[e]) : 0;
  const int sm = (e < E && c > 0 && c < min_rows) ? 1 : 0;
  int v = c, vs = sm;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off, 64), os = __shfl_up(vs, off, 64);
    if (lane >= off) {
      v += o;
      vs += os;
    }
  }
  if (lane == 63) {
    wsum[wave] = v;
    wsmall[wave] = vs;
  }
  __syncthreads();
  int wbase = 0, sbase = 0;
  for (int w = 0; w < wave; ++w) {
    wbase += wsum[w];
    sbase += wsmall[w];
  }
  const int excl = wbase + v - c;
  if (sm) small_list[sbase + vs - 1] = e;
  if (e < E) {
    counts[e] = c;
    offsets[e] = excl;
    excl_l[e] = excl;
  }
  if (e == 1023) {
    int ns = 0;
    for (int w = 0; w < 16; ++w) ns += wsmall[w];
    if (has_shared && T < min_rows) small_list[ns++] = E;
    *n_small = ns;
    counts[E] = T;
    offsets[E] = T * k;
  }
  if (tiles != nullptr) {
    const int nb = e < E ? c : (e == E && has_shared ? T : 0);
    const int ct = nb >= tile_min ? (nb + mt - 1) / mt : 0;
    int tv = ct;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(tv, off, 64);
      if (lane >= off) tv += o;
    }
    __syncthreads();  // every thread has read wsum
    if (lane == 63) wsum[wave] = tv;
    __syncthreads();
    int tb = 0;
    for (int w = 0; w < wave; ++w) tb += wsum[w];
    if (e == 1023) *ntiles = min(tb + tv, max_tiles);
    const int tbase = tb + tv - ct;
    for (int i = 0; i < ct; ++i) {
      const int t = tbase + i;
      if (t < max_tiles) {
        tiles[2 * t] = e;
        tiles[2 * t + 1] = i * mt;
      }
    }
  }
  __syncthreads();
  if (e < T) {
    const uint64_t below = (e == 0) ? 0ull : (~0ull >> (64 - e));
    for (int j = 0; j < k; ++j) {
      const int ee = topk_idx[(int64_t)e * k + j];
      pairs[excl_l[ee] + __popcll(m[ee] & below)] = e * k + j;
    }
  }
}

// ---------------------------------------------------------------------------
// residual + RMSNorm (unit weight)

// Eight consecutive activations (16-byte aligned: rows start at multiples of
// H, a multiple of 64) as fp32, and back with RNE rounding to the act dtype.
template <int ACT>
__device__ __forceinline__ void load_act8(const void* p, int64_t i, float (&v)[8]) {
  if constexpr (ACT == MOE_ACT_F32) {
    const float4 a = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p) + i);
    const float4 b = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p) + i + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint4 q = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p) + i);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = bf16_bits_to_f32(w[j] & 0xFFFFu);
      v[2 * j + 1] = bf16_bits_to_f32(w[j] >> 16);
    }
  }
}
template <int ACT>
__device__ __forceinline__ void store_act8(void* p, int64_t i, const float (&v)[8]) {
  if constexpr (ACT == MOE_ACT_F32) {
    float* d = reinterpret_cast<float*>(p) + i;
    *reinterpret_cast<float4*>(d) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(d + 4) = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = (uint32_t)f32_to_bf16_bits(v[2 * j]) | ((uint32_t)f32_to_bf16_bits(v[2 * j + 1]) << 16);
    *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(p) + i) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}
template <int ACT>
__device__ __forceinline__ float round_act(float v) {
  if constexpr (ACT == MOE_ACT_F32) return v;
  else return bf16_bits_to_f32(f32_to_bf16_bits(v));
}

// One workgroup per token; thread i holds elements 8 (i + 256 r) .. +7 for
// r < 4 (H <= 8192) in registers, so x is read once: the residual sum (x +
// out, rounded to the act dtype and stored back), its sum of squares, and
// the normalised row.
// The same as rmsnorm_kernel with one wave per row, four rows per workgroup,
// for H = 512 NC: lane l holds chunks l, l + 64, ... of 8 values, every load
// of a row in flight together; the sum of squares in lane order, then across
// the wave.
template <int ACT, int NC>
__global__ __launch_bounds__(256) void rmsnorm_row_kernel(void* __restrict__ x,
                                                          const void* __restrict__ out,
                                                          void* __restrict__ x_hat, int T, int H,
                                                          float eps, int do_norm) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (t >= T) return;
  const int64_t base = (int64_t)t * H;
  float v[NC][8], o[NC][8];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    load_act8<ACT>(x, base + 8 * (lane + 64 * i), v[i]);
    if (out != nullptr) load_act8<ACT>(out, base + 8 * (lane + 64 * i), o[i]);
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    if (out != nullptr) {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[i][j] = round_act<ACT>(v[i][j] + o[i][j]);
      store_act8<ACT>(x, base + 8 * (lane + 64 * i), v[i]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) ss += v[i][j] * v[i][j];
  }
  if (!do_norm) return;
  const float inv = 1.0f / sqrtf(warp_sum(ss) / (float)H + eps);
#pragma unroll
  for (int i = 0; i < NC; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[i][j] *= inv;
    store_act8<ACT>(x_hat, base + 8 * (lane + 64 * i), v[i]);
  }
}

template <int ACT>
__global__ __launch_bounds__(256) void rmsnorm_kernel(void* __restrict__ x,
                                                      const void* __restrict__ out,
                                                      void* __restrict__ x_hat, int H, float eps,
                                                      int do_norm) {
  constexpr int kR = MOE_MAX_HIDDEN / (256 * 8);
  __shared__ float wsum[4];
  const int t = blockIdx.x;
  const int64_t base = (int64_t)t * H;
  float v[kR][8];
  float o[kR][8];
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    const int c = (r * 256 + (int)threadIdx.x) * 8;
    if (c < H) {
      load_act8<ACT>(x, base + c, v[r]);
      if (out != nullptr) load_act8<ACT>(out, base + c, o[r]);
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    const int c = (r * 256 + (int)threadIdx.x) * 8;
    if (c < H) {
      if (out != nullptr) {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[r][j] = round_act<ACT>(v[r][j] + o[r][j]);
        store_act8<ACT>(x, base + c, v[r]);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) ss += v[r][j] * v[r][j];
    }
  }
  if (!do_norm) return;
  ss = warp_sum(ss);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
  const float inv = 1.0f / sqrtf(tot / (float)H + eps);
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    const int c = (r * 256 + (int)threadIdx.x) * 8;
    if (c < H) {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[r][j] *= inv;
      store_act8<ACT>(x_hat, base + c, v[r]);
    }
  }
}

// ---------------------------------------------------------------------------
// device packer: one workgroup per (tile, k-block) unit of one section.

template <int BITS>
__device__ __forceinline__ uint4 pack_codes16(const uint8_t* __restrict__ q) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t v = 0;
    if constexpr (BITS == 4) {
#pragma unroll
      for (int b = 0; b < 8; ++b) v |= (uint32_t)(q[8 * i + b] & 15u) << (4 * b);
    } else {
#pragma unroll
      for (int b = 0; b < 4; ++b) v |= (uint32_t)q[4 * i + b] << (8 * b);
    }
    w[i] = v;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

template <int BITS>
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ qa,
                                                   const uint8_t* __restrict__ qb,
                                                   const uint16_t* __restrict__ sba,
                                                   const uint16_t* __restrict__ sbb,
                                                   uint8_t* __restrict__ dst, int rows, int cols,
                                                   int64_t unit_bytes, int64_t tile_bytes,
                                                   int two) {
  constexpr int GPK = BITS == 4 ? 2 : 1;
  constexpr int CC = chunk_cols<BITS>();
  constexpr int KBC = kRowBytes * (8 / BITS);
  const int nkb = cols / KBC;
  const int tile = blockIdx.x / nkb, kb = blockIdx.x % nkb;
  const int G = cols / kGroup;
  uint8_t* unit = dst + (int64_t)tile * tile_bytes + (int64_t)kb * unit_bytes;
  const int i = threadIdx.x;
  const int ncode = two ? 128 : 64;
  if (i < ncode) {
    const int which = i >> 6, l = i & 63;
    const int r = tile * kRowTile + (l >> 2);
    const int c = kb * KBC + (l & 3) * CC;
    const uint8_t* q = (which ? qb : qa) + (int64_t)r * cols + c;
    *reinterpret_cast<uint4*>(unit + which * kCodeBlockBytes + l * 16) = pack_codes16<BITS>(q);
  } else if (i < ncode + (two ? 2 : 1) * kRowTile * GPK) {
    const int s = i - ncode;
    const int which = s / (kRowTile * GPK), idx = s % (kRowTile * GPK);
    const int rl = idx / GPK, gi = idx % GPK;
    const int r = tile * kRowTile + rl, g = kb * GPK + gi;
    const uint16_t* sb = which ? sbb : sba;
    const uint32_t sc = sb[(int64_t)r * G + g];
    const uint32_t bi = sb[(int64_t)rows * G + (int64_t)r * G + g];
    uint8_t* p = unit + (two ? 2 : 1) * kCodeBlockBytes + which * kRowTile * GPK * 4 +
                 (rl * GPK + gi) * 4;
    *reinterpret_cast<uint32_t*>(p) = sc | (bi << 16);
  }
}

template <int BITS, int ACT>
hipError_t launch_experts_t(const ExpertArgs& a, hipStream_t s) {
  const WsPlan& P = a.plan;
  float* h = reinterpret_cast<float*>(a.ws + P.h);
  int32_t* counts = reinterpret_cast<int32_t*>(a.ws + P.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(a.ws + P.offsets);
  int32_t* pairs = reinterpret_cast<int32_t*>(a.ws + P.pairs);
  const int hs = a.has_shared ? 1 : 0;
  const int Is = a.has_shared ? a.Ls.inter : 0;
  const int tiles_gu = max(a.L.n_tiles_gu, a.has_shared ? a.Ls.n_tiles_gu : 0);
  const size_t lds_gu =
      (size_t)kGuTokens * XStage<BITS, ACT>::bytes(a.H) + sizeof(float) * 4 * kGuTokens * kRowTile * 2;
  hipError_t e;
  if (!P.bucketed) {
    hipLaunchKernelGGL((gateup_kernel<BITS, ACT>), dim3(tiles_gu, a.T * (a.k + hs)), dim3(256),
                       lds_gu, s, a.x, a.topk_idx, a.slab, a.slot_table, a.stride, a.shared_blob,
                       counts, offsets, pairs, h, a.T, a.H, a.E, a.k, a.L.inter, Is, a.L.gu_unit,
                       a.L.gu_tile, a.Ls.gu_unit, a.Ls.gu_tile, 0, hs, 0, nullptr, nullptr,
                       0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((down_decode_kernel<BITS, ACT>), dim3(a.L.n_tiles_d, a.T), dim3(256), 0, s,
                       a.topk_idx, a.topk_w, a.gamma, a.slab, a.slot_table, a.stride,
                       a.shared_blob, h, a.out, a.T, a.H, a.k, a.L.inter, Is, a.L.d_off,
                       a.L.d_unit, a.L.d_tile, a.Ls.d_off, a.Ls.d_unit, a.Ls.d_tile, hs);
    return hipGetLastError();
  }
  uint64_t* masks = reinterpret_cast<uint64_t*>(a.ws + P.masks);
  int32_t* blkoff = reinterpret_cast<int32_t*>(a.ws + P.blkoff);
  float* partial = reinterpret_cast<float*>(a.ws + P.partial);
  const int nblk = (a.T + 63) / 64;
  int32_t* small_list = reinterpret_cast<int32_t*>(a.ws + P.small);
  int32_t* n_small = reinterpret_cast<int32_t*>(a.ws + P.nsmall);
  int32_t* tiles = reinterpret_cast<int32_t*>(a.ws + P.tiles);
  int32_t* ntiles = reinterpret_cast<int32_t*>(a.ws + P.ntiles);
  // buckets below the MFMA threshold (all of them without the MFMA path)
  const int min_rows = a.mfma ? kMfmaMinRows : 0x7FFFFFFF;
  // one token block: buckets (and the MFMA tile list) in one launch
  const bool small_batch = nblk == 1 && a.E < 1024;
  const bool one_block =
      a.mfma && small_batch && batched_supported(a.act, a.T, a.H, a.L.inter, Is, a.has_shared);
  // larger batches: the scan builds the MFMA tile list where every bucket has a thread
  const bool scan_tiles = a.mfma && !small_batch && a.E + hs <= 1024;
  if (small_batch) {
    hipLaunchKernelGGL(bucket_small_kernel, dim3(1), dim3(1024), 0, s, a.topk_idx, counts,
                       offsets, pairs, small_list, n_small, a.mfma ? tiles : nullptr, ntiles,
                       P.max_tiles, kMfmaTileRows, kMfmaMinRows, a.T, a.E, a.k, min_rows, hs);
  } else {
    hipLaunchKernelGGL(bucket_mask_kernel, dim3(nblk), dim3(64), 0, s, a.topk_idx, masks, a.T,
                       a.E, a.k);
    hipLaunchKernelGGL(bucket_scan_kernel, dim3(1), dim3(1024), 0, s, masks, counts, offsets,
                       blkoff, small_list, n_small, a.T, a.E, a.k, nblk, min_rows, hs,
                       scan_tiles ? tiles : nullptr, ntiles, P.max_tiles, kMfmaTileRows,
                       kMfmaMinRows);
    hipLaunchKernelGGL(bucket_scatter_kernel, dim3(nblk), dim3(64), 0, s, a.topk_idx, masks,
                       blkoff, pairs, a.T, a.E, a.k);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.mfma) {
    PrefillArgs pa{};
    pa.x = reinterpret_cast<const uint16_t*>(a.x);
    pa.pairs = pairs;
    pa.counts = counts;
    pa.offsets = offsets;
    pa.topk_w = a.topk_w;
    pa.gamma = a.gamma;
    pa.slab = a.slab;
    pa.slot_table = a.slot_table;
    pa.stride = a.stride;
    pa.shared_blob = a.shared_blob;
    pa.h = reinterpret_cast<uint16_t*>(h);
    pa.partial = partial;
    pa.out = a.out;
    pa.tiles = tiles;
    pa.ntiles = ntiles;
    pa.tiles_ready = small_batch || scan_tiles;
    pa.x16 = reinterpret_cast<uint16_t*>(a.ws + P.x16);
    pa.xe = reinterpret_cast<int32_t*>(a.ws + P.xe);
    pa.x16_ready = a.x16_ready;
    pa.max_tiles = P.max_tiles;
    pa.L = a.L;
    pa.Ls = a.Ls;
    pa.T = a.T;
    pa.H = a.H;
    pa.E = a.E;
    pa.k = a.k;
    pa.I = a.L.inter;
    pa.Is = Is;
    pa.bits = a.bits;
    pa.has_shared = a.has_shared;
    pa.min_rows = kMfmaMinRows;
    if ((e = one_block ? launch_batched(pa, s) : launch_prefill(pa, s)) != hipSuccess) return e;
  }
  // the bucketed GEMVs own the buckets below the MFMA threshold (none when
  // every bucket of at least one token runs on the grouped GEMMs)
  if (min_rows > 1) {
    hipLaunchKernelGGL((gateup_kernel<BITS, ACT>), dim3(kGemvSlots), dim3(256), lds_gu, s,
                       a.x, a.topk_idx, a.slab, a.slot_table, a.stride, a.shared_blob, counts,
                       offsets, pairs, h, a.T, a.H, a.E, a.k, a.L.inter, Is, a.L.gu_unit,
                       a.L.gu_tile, a.Ls.gu_unit, a.Ls.gu_tile, 1, hs, min_rows, small_list,
                       n_small, tiles_gu);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((down_bucket_kernel<BITS>), dim3(kDownSlots), dim3(256), 0, s,
                       a.topk_w, a.gamma, a.slab, a.slot_table, a.stride, a.shared_blob, counts,
                       offsets, pairs, h, partial, a.T, a.H, a.E, a.k, a.L.inter, Is, a.L.d_off,
                       a.L.d_unit, a.L.d_tile, a.Ls.d_off, a.Ls.d_unit, a.Ls.d_tile, min_rows,
                       small_list, n_small, a.L.n_tiles_d);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // the grouped GEMMs of large batches write fp16 partial rows (their down
  // kernel's epilogue), every other path fp32
  const bool f16p = a.mfma && !one_block;
  const int64_t e_off = (int64_t)a.T * (a.k + 1) * a.H * 2;
#define MOE_COMBINE(NJ, F16P)                                                                 \
  hipLaunchKernelGGL((combine_kernel<ACT, NJ, F16P>), dim3(a.T), dim3(256), 0, s, partial, a.out, \
                     a.H, a.k, hs, a.x_res, a.x_hat_next, a.eps, a.epi, e_off)
  if constexpr (ACT == MOE_ACT_BF16) {
    if (f16p) {
      if (a.k + hs <= 12) MOE_COMBINE(12, true);
      else MOE_COMBINE(MOE_MAX_TOP_K + 1, true);
      return hipGetLastError();
    }
  }
  if (a.k + hs <= 12) MOE_COMBINE(12, false);
  else MOE_COMBINE(MOE_MAX_TOP_K + 1, false);
#undef MOE_COMBINE
  return hipGetLastError();
}

}  // namespace

hipError_t launch_experts(const ExpertArgs& a, hipStream_t s) {
  if (a.bits == 4)
    return a.act == MOE_ACT_F32 ? launch_experts_t<4, MOE_ACT_F32>(a, s)
                                : launch_experts_t<4, MOE_ACT_BF16>(a, s);
  return a.act == MOE_ACT_F32 ? launch_experts_t<8, MOE_ACT_F32>(a, s)
                              : launch_experts_t<8, MOE_ACT_BF16>(a, s);
}

hipError_t launch_rmsnorm(void* x, const void* out, void* x_hat, int T, int H, int act, float eps,
                          bool do_norm, hipStream_t s) {
  // one wave per row where H is 1024, 2048 or 4096
  const int nc = H % 512 == 0 ? H / 512 : 0;
  if (nc == 2 || nc == 4 || nc == 8) {
    const dim3 grid((unsigned)((T + 3) / 4));
    const int dn = do_norm ? 1 : 0;
#define MOE_RMS_ROW(A, NC)                                                                        \
  hipLaunchKernelGGL((rmsnorm_row_kernel<A, NC>), grid, dim3(256), 0, s, x, out, x_hat, T, H, eps, dn)
#define MOE_RMS_ROW_NC(A)   \
  if (nc == 2)              \
    MOE_RMS_ROW(A, 2);      \
  else if (nc == 4)         \
    MOE_RMS_ROW(A, 4);      \
  else                      \
    MOE_RMS_ROW(A, 8)
    if (act == MOE_ACT_F32) {
      MOE_RMS_ROW_NC(MOE_ACT_F32);
    } else {
      MOE_RMS_ROW_NC(MOE_ACT_BF16);
    }
#undef MOE_RMS_ROW_NC
#undef MOE_RMS_ROW
    return hipGetLastError();
  }
  if (act == MOE_ACT_F32)
    hipLaunchKernelGGL(rmsnorm_kernel<MOE_ACT_F32>, dim3(T), dim3(256), 0, s, x, out, x_hat, H, eps,
                       do_norm ? 1 : 0);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<MOE_ACT_BF16>, dim3(T), dim3(256), 0, s, x, out, x_hat, H,
                       eps, do_norm ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_pack_device(const BlobLayout& L, int n, const uint8_t* qg, const uint8_t* qu,
                              const uint8_t* qd, const uint16_t* sbg, const uint16_t* sbu,
                              const uint16_t* sbd, uint8_t* slab, int64_t stride,
                              const int64_t* slots_host, hipStream_t s) {
  const int64_t H = L.hidden, I = L.inter;
  for (int i = 0; i < n; ++i) {
    uint8_t* blob = slab + slots_host[i] * stride;
    const int64_t qoff = (int64_t)i * I * H;
    const int64_t sgu = (int64_t)i * 2 * I * (H / kGroup);
    const int64_t sdd = (int64_t)i * 2 * H * (I / kGroup);
    const dim3 g_gu(L.n_tiles_gu * L.n_kb_gu), g_d(L.n_tiles_d * L.n_kb_d);
    if (L.bits == 4) {
      hipLaunchKernelGGL(pack_kernel<4>, g_gu, dim3(256), 0, s, qg + qoff, qu + qoff, sbg + sgu,
                         sbu + sgu, blob + L.gu_off, (int)I, (int)H, L.gu_unit, L.gu_tile, 1);
      hipLaunchKernelGGL(pack_kernel<4>, g_d, dim3(256), 0, s, qd + qoff, nullptr, sbd + sdd,
                         nullptr, blob + L.d_off, (int)H, (int)I, L.d_unit, L.d_tile, 0);
    } else {
      hipLaunchKernelGGL(pack_kernel<8>, g_gu, dim3(256), 0, s, qg + qoff, qu + qoff, sbg + sgu,
                         sbu + sgu, blob + L.gu_off, (int)I, (int)H, L.gu_unit, L.gu_tile, 1);
      hipLaunchKernelGGL(pack_kernel<8>, g_d, dim3(256), 0, s, qd + qoff, nullptr, sbd + sdd,
                         nullptr, blob + L.d_off, (int)H, (int)I, L.d_unit, L.d_tile, 0);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace moe
