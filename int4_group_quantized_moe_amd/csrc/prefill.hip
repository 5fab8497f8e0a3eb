// Prefill / large-batch path: grouped GEMMs on the MFMA matrix cores.
//
// When many tokens share an expert (a prefill chunk routes ~T*k/E tokens to
// each expert) the expert FFN is a dense contraction: per expert e with its
// bucket of n_e tokens,
//   G|U = X_e [n_e x H] . [Wg_e | Wu_e]^T,  h = silu(G) * U,
//   Y_e = h [n_e x I] . Wd_e^T,  out[t] += w_{t,j} Y_e[t]
// and the shared expert is the same with all T tokens.  The pages call prefill
// the bottleneck for long contexts (page "Swiftlet: 在 Mac 和 iPhone 上執行 ..."
// on agentlenshq.com, section "社群觀點"); the weights are MLX-style
// group-quantised int4/int8 (page "Paquets Swiftlet 80B Qwen ..." on xix.ai,
// last paragraph).
//
// Both GEMMs run on v_mfma_f32_32x32x16_bf16 with fp32 accumulation, and no
// operand is rounded on its way into the matrix cores:
//  * weights enter as their integer codes, which bf16 holds exactly (int4 as
//    1 + q/16, int8 as q); the group's bf16 scale is applied in fp32 to the
//    group's code sums, and the group's bias multiplies the group sum of the
//    activations (w = s q + b factors as s * sum(q x) + b * sum(x));
//  * the gate/up input x_hat is bf16 already; the down input h is carried
//    as a pair of bf16 parts (hi + lo, 16 significant bits) and multiplied
//    twice.
// Dequantising to bf16 instead (s*q + b rounded, and h rounded to bf16)
// would add ~2^-9 relative error per weight and per h value.
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kMT = 128;          // rows (bucket entries) per tile
constexpr int kLdsRow = kGroup + 8;  // padded LDS row of one group (bf16 elements)

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Order of the 8 K positions inside one MFMA operand chunk.  int4: the chunk
// built from one 32-bit word of codes (codes c0..c7, nibble i = code i) holds
// (c0,c4,c1,c5,c2,c6,c3,c7), which takes two instructions per pair to form;
// the activations are permuted the same way so that the products pair up.
// int8: natural order.
template <int BITS>
__device__ __forceinline__ u32x4 permute_chunk(u32x4 v) {
  if constexpr (BITS == 4) {
    return u32x4{__builtin_amdgcn_perm(v.z, v.x, 0x05040100u),
                 __builtin_amdgcn_perm(v.z, v.x, 0x07060302u),
                 __builtin_amdgcn_perm(v.w, v.y, 0x05040100u),
                 __builtin_amdgcn_perm(v.w, v.y, 0x07060302u)};
  } else {
    return v;
  }
}

// Exact bf16 operands from integer codes.  int4: the nibble goes into
// mantissa bits 3..6 of 1.0, giving 1 + q/16 exactly; int8: the float of the
// byte has at most 8 significant bits, so its upper half is q exactly.
__device__ __forceinline__ u32x4 code_frag4(uint32_t d) {
  constexpr uint32_t M = 0x00780078u, O = 0x3F803F80u;
  return u32x4{((d << 3) & M) | O, ((d >> 1) & M) | O, ((d >> 5) & M) | O, ((d >> 9) & M) | O};
}
__device__ __forceinline__ uint32_t hi_halves(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}
__device__ __forceinline__ u32x4 code_frag8(uint32_t d0, uint32_t d1) {
  return u32x4{hi_halves((float)(d0 & 0xFFu), (float)((d0 >> 8) & 0xFFu)),
               hi_halves((float)((d0 >> 16) & 0xFFu), (float)(d0 >> 24)),
               hi_halves((float)(d1 & 0xFFu), (float)((d1 >> 8) & 0xFFu)),
               hi_halves((float)((d1 >> 16) & 0xFFu), (float)(d1 >> 24))};
}

// One lane's codes of one weight row for one group: 32 consecutive codes
// (16 bytes of int4, 32 bytes of int8).
template <int BITS>
struct LaneCodes {
  uint4 q[BITS / 4];
  __device__ __forceinline__ void load(const uint8_t* p) {
#pragma unroll
    for (int i = 0; i < BITS / 4; ++i) q[i] = reinterpret_cast<const uint4*>(p)[i];
  }
  // MFMA B operand of K step ks (codes 8ks .. 8ks+7 of the 32)
  __device__ __forceinline__ u32x4 frag(int ks) const {
    if constexpr (BITS == 4) {
      const uint32_t d = ks == 0 ? q[0].x : ks == 1 ? q[0].y : ks == 2 ? q[0].z : q[0].w;
      return code_frag4(d);
    } else {
      const uint4& v = q[ks >> 1];
      return (ks & 1) ? code_frag8(v.z, v.w) : code_frag8(v.x, v.y);
    }
  }
};

// Per-group fp32 scale applied to the code sums, and the bias coefficient of
// the group sum of the activations: with codes staged as 1 + q/16 (int4),
//   sum_k (s q_k + b) x_k = 16 s * sum_k (1 + q_k/16) x_k + (b - 16 s) * sum_k x_k,
// and with plain codes (int8) the pair is (s, b).
template <int BITS>
__device__ __forceinline__ float code_scale(uint32_t sb) {
  const float s = bf16_bits_to_f32(sb & 0xFFFFu);
  return BITS == 4 ? 16.0f * s : s;
}
template <int BITS>
__device__ __forceinline__ float bias_coef(uint32_t sb) {
  const float s = bf16_bits_to_f32(sb & 0xFFFFu), b = bf16_bits_to_f32(sb >> 16);
  return BITS == 4 ? b - 16.0f * s : b;
}

// fp32 -> (hi, lo) bf16 pair with hi + lo = v to 16 significant bits.
__device__ __forceinline__ void split_bf16(float v, uint32_t& hi, uint32_t& lo) {
  hi = f32_to_bf16_bits(v);
  lo = f32_to_bf16_bits(v - bf16_bits_to_f32(hi));
}
__device__ __forceinline__ void split8(const float v[8], u32x4& hi, u32x4& lo) {
  uint32_t h[8], l[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) split_bf16(v[i], h[i], l[i]);
  hi = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
  lo = u32x4{l[0] | (l[1] << 16), l[2] | (l[3] << 16), l[4] | (l[5] << 16), l[6] | (l[7] << 16)};
}

// Address of a weight row's codes and (scale, bias) words inside a blob
// section of 16-row tiles and 64-byte-per-row k-blocks; `mat` selects the
// gate (0) or up (1) matrix of a gate/up unit (nmat = 2) or the down matrix
// (nmat = 1).
template <int BITS>
struct RowAddr {
  static constexpr int GPK = kRowBytes * (8 / BITS) / kGroup;  // groups per k-block
  static constexpr int GBYTES = kGroup * BITS / 8;             // code bytes per group
  const uint8_t* codes;  // row's codes in k-block 0, plus this lane's half
  const uint8_t* sb;     // row's (scale, bias) words in k-block 0
  int64_t unit_b;
  __device__ __forceinline__ RowAddr(const uint8_t* sec, int64_t unit, int64_t tile, int nmat,
                                     int mat, int row, int half)
      : unit_b(unit) {
    const uint8_t* t = sec + (int64_t)(row / kRowTile) * tile;
    codes = t + mat * kCodeBlockBytes + (row % kRowTile) * kRowBytes + half * (GBYTES / 2);
    sb = t + nmat * kCodeBlockBytes + mat * kRowTile * GPK * 4 + (row % kRowTile) * GPK * 4;
  }
  __device__ __forceinline__ const uint8_t* group_codes(int g) const {
    return codes + (int64_t)(g / GPK) * unit_b + (g % GPK) * GBYTES;
  }
  __device__ __forceinline__ uint32_t group_sb(int g) const {
    return *reinterpret_cast<const uint32_t*>(sb + (int64_t)(g / GPK) * unit_b + (g % GPK) * 4);
  }
};

// Bias term of a tile: C[m][n] += sum_g beta_g[n] * S_g[m], where S_g[m] is
// the group sum of the activations of row m, as one more small MFMA product
// over the group index (K = groups, padded to 16) with both operands split
// into bf16 hi/lo parts (hi*hi + hi*lo + lo*hi).
template <int BITS>
__device__ __forceinline__ void bias_mfma(const float* const srow[2], const RowAddr<BITS> wr[2],
                                          int G, int half, f32x16 C[2][2]) {
#pragma unroll 1
  for (int j = 0; j < (G + 15) / 16; ++j) {
    u32x4 ah[2], al[2], bh[2], bl[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int g = 16 * j + 8 * half + i;
        v[i] = (srow[mb] != nullptr && g < G) ? srow[mb][g] : 0.f;
      }
      split8(v, ah[mb], al[mb]);
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int g = 16 * j + 8 * half + i;
        v[i] = g < G ? bias_coef<BITS>(wr[nb].group_sb(g)) : 0.f;
      }
      split8(v, bh[nb], bl[nb]);
    }
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        C[mb][nb] = mfma(ah[mb], bh[nb], C[mb][nb]);
        if constexpr (BITS == 4) C[mb][nb] = mfma(ah[mb], bl[nb], C[mb][nb]);
        C[mb][nb] = mfma(al[mb], bh[nb], C[mb][nb]);
      }
  }
}

struct TileInfo {
  int e;        // expert, or E for the shared expert
  int m0;       // first row of the tile inside the bucket
  int rows;     // valid rows (<= kMT)
  int base;     // bucket position of row 0 (routed) or token of row 0 (shared)
};

__device__ __forceinline__ TileInfo get_tile(const int32_t* tiles, const int32_t* counts,
                                             const int32_t* offsets, int t, int E) {
  TileInfo ti;
  ti.e = tiles[2 * t];
  ti.m0 = tiles[2 * t + 1];
  ti.rows = min(kMT, counts[ti.e] - ti.m0);
  ti.base = ti.e == E ? ti.m0 : offsets[ti.e] + ti.m0;  // token (shared) or bucket position
  return ti;
}

// ---------------------------------------------------------------------------
// tile list: every expert bucket of at least min_rows tokens (and the shared
// expert's T tokens as bucket E) cut into tiles of kMT rows.  One workgroup.

__global__ __launch_bounds__(1024) void tile_list_kernel(const int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ tiles,
                                                         int32_t* __restrict__ ntiles, int E,
                                                         int has_shared, int max_tiles,
                                                         int min_rows) {
  __shared__ int wsum[16];
  __shared__ int carry_s;
  __shared__ int tbase[MOE_MAX_EXPERTS + 2];
  const int n_b = E + has_shared;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int carry = 0;
  // exclusive scan of the per-bucket tile counts, 1024 buckets per pass
  for (int b0 = 0; b0 < n_b; b0 += 1024) {
    const int b = b0 + threadIdx.x;
    const int nb = b < n_b ? counts[b] : 0;
    const int c = nb >= min_rows ? (nb + kMT - 1) / kMT : 0;
    int v = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(v, off, 64);
      if (lane >= off) v += o;
    }
    if (lane == 63) wsum[wave] = v;
    __syncthreads();
    int wb = carry;
    for (int w = 0; w < wave; ++w) wb += wsum[w];
    if (b < n_b) tbase[b] = wb + v - c;
    if (threadIdx.x == 1023) carry_s = wb + v;
    __syncthreads();
    carry = carry_s;
    __syncthreads();
  }
  const int total = min(carry, max_tiles);
  if (threadIdx.x == 0) *ntiles = total;
  for (int b = threadIdx.x; b < n_b; b += 1024) {
    const int c = counts[b] >= min_rows ? (counts[b] + kMT - 1) / kMT : 0;
    for (int i = 0; i < c; ++i) {
      const int t = tbase[b] + i;
      if (t < max_tiles) {
        tiles[2 * t] = b;
        tiles[2 * t + 1] = i * kMT;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// per-group sums of the activations: xsum[t][g] = sum of x[t][64g .. 64g+63]

__global__ __launch_bounds__(256) void group_sum_kernel(const uint16_t* __restrict__ x,
                                                        float* __restrict__ xsum, int T, int H) {
  const int G = H / kGroup;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)T * G) return;
  const uint4* p = reinterpret_cast<const uint4*>(x + (i / G) * H + (i % G) * kGroup);
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kGroup / 8; ++c) {
    const uint4 v = p[c];
    s += (bf16_bits_to_f32(v.x & 0xFFFFu) + bf16_bits_to_f32(v.x >> 16)) +
         (bf16_bits_to_f32(v.y & 0xFFFFu) + bf16_bits_to_f32(v.y >> 16)) +
         (bf16_bits_to_f32(v.z & 0xFFFFu) + bf16_bits_to_f32(v.z >> 16)) +
         (bf16_bits_to_f32(v.w & 0xFFFFu) + bf16_bits_to_f32(v.w >> 16));
  }
  xsum[i] = s;
}

// ---------------------------------------------------------------------------
// Shared tile structure of both GEMMs.  A workgroup computes a 128-row x
// 128-column tile; wave (wm, wn) = (wave / 2, wave % 2) owns rows
// 64 wm .. 64 wm + 63 (two 32-row blocks mb) and two 32-column blocks nb.
// K runs one quantisation group (64) per stage: the activation rows of the
// group are staged in LDS (double-buffered, next stage's loads in flight
// during the MFMAs); each lane reads its weight row's 32 codes of the group
// straight from memory into registers (lane half 0: codes 0..31, half 1:
// 32..63) and expands them to exact bf16 operands.  Per group the code sums
// go into a fresh accumulator that is then scaled into the tile:
//   C += scale_g[n] * acc_g,
// and the bias terms are added at the end by bias_mfma.

// gate/up: grid (max(I, Is)/64, tiles).  Tile columns: 64 gate rows and the
// 64 up rows of the same h columns; wave wn holds h columns n0 + 32 wn ..
// n0 + 32 wn + 31 as block 0 (gate) and block 1 (up).  Writes per row the
// 64 h values as bf16 (hi, lo) pairs in the K order the down GEMM stages,
// and the row's group sum of h.

template <int BITS>
__global__ __launch_bounds__(256) void prefill_gateup_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ xsum,
    const int32_t* __restrict__ pairs, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ ntiles, const uint8_t* __restrict__ slab,
    const int32_t* __restrict__ slot_table, int64_t stride, const uint8_t* __restrict__ shared_blob,
    uint16_t* __restrict__ h, float* __restrict__ hsum, int T, int H, int E, int k, int I, int Is,
    int64_t gu_unit_r, int64_t gu_tile_r, int64_t gu_unit_s, int64_t gu_tile_s) {
  // two stages of 128 activation rows x 64 K; reused as the fp32 h tile
  __shared__ __align__(16) uint16_t A[2 * kMT * kLdsRow];
  __shared__ int32_t rowsrc[kMT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31, half = lane >> 5;
  if ((int)blockIdx.y >= *ntiles) return;
  const TileInfo ti = get_tile(tiles, counts, offsets, blockIdx.y, E);
  const bool shared = ti.e == E;
  const int inter = shared ? Is : I;
  const int n0 = blockIdx.x * kGroup;
  if (n0 >= inter) return;
  const uint8_t* sec = shared ? shared_blob : slab + (int64_t)slot_table[ti.e] * stride;
  const int64_t unit_b = shared ? gu_unit_s : gu_unit_r, tile_b = shared ? gu_tile_s : gu_tile_r;
  if (tid < kMT) {
    int src = -1;
    if (tid < ti.rows) src = shared ? ti.base + tid : pairs[ti.base + tid] / k;
    rowsrc[tid] = src;
  }
  __syncthreads();
  // staging role: row sr, K half sc (32 columns = 4 chunks of 8)
  const int sr = tid >> 1, sc = tid & 1;
  const int ssrc = rowsrc[sr];
  const uint16_t* xrow = x + (int64_t)(ssrc >= 0 ? ssrc : 0) * H + sc * 32;
  const RowAddr<BITS> wr[2] = {RowAddr<BITS>(sec, unit_b, tile_b, 2, 0, n0 + 32 * wn + l32, half),
                               RowAddr<BITS>(sec, unit_b, tile_b, 2, 1, n0 + 32 * wn + l32, half)};
  const int G = H / kGroup;

  uint4 ra[4];
  LaneCodes<BITS> cn[2];
  uint32_t sbn[2];
  auto load_stage = [&](int g) {
    if (ssrc >= 0) {
      const uint4* p = reinterpret_cast<const uint4*>(xrow + g * kGroup);
#pragma unroll
      for (int q = 0; q < 4; ++q) ra[q] = p[q];
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) ra[q] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      cn[nb].load(wr[nb].group_codes(g));
      sbn[nb] = wr[nb].group_sb(g);
    }
  };
  auto store_stage = [&](int buf) {
    uint16_t* dst = A + buf * kMT * kLdsRow + sr * kLdsRow + sc * 32;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 v = ra[q];
      const u32x4 p = permute_chunk<BITS>(u32x4{v.x, v.y, v.z, v.w});
      *reinterpret_cast<u32x4*>(dst + 8 * q) = p;
    }
  };

  f32x16 C[2][2];
  const f32x16 zero = {};
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) C[mb][nb] = zero;

  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int g = 0; g < G; ++g) {
    const LaneCodes<BITS> cc[2] = {cn[0], cn[1]};
    const float scl[2] = {code_scale<BITS>(sbn[0]), code_scale<BITS>(sbn[1])};
    if (g + 1 < G) load_stage(g + 1);
    const uint16_t* As = A + (g & 1) * kMT * kLdsRow;
    f32x16 acc[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = zero;
#pragma unroll
    for (int ks = 0; ks < kGroup / 16; ++ks) {
      u32x4 a[2], b[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        a[mb] = *reinterpret_cast<const u32x4*>(As + (64 * wm + 32 * mb + l32) * kLdsRow +
                                                32 * half + 8 * ks);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) b[nb] = cc[nb].frag(ks);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma(a[mb], b[nb], acc[mb][nb]);
    }
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) C[mb][nb][r] += scl[nb] * acc[mb][nb][r];
    if (g + 1 < G) store_stage((g + 1) & 1);
    __syncthreads();
  }

  // bias terms from the group sums of the activation rows
  {
    const float* srow[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int src = rowsrc[64 * wm + 32 * mb + l32];
      srow[mb] = src >= 0 ? xsum + (int64_t)src * G : nullptr;
    }
    bias_mfma<BITS>(srow, wr, G, half, C);
  }

  // epilogue: h = silu(g) * u into an fp32 LDS tile [128][64 + 4]
  constexpr int HS = kGroup + 4;
  float* ht = reinterpret_cast<float*>(A);
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 64 * wm + 32 * mb + 8 * (r / 4) + 4 * half + (r % 4);
      const float gv = C[mb][0][r], uv = C[mb][1][r];
      ht[m * HS + 32 * wn + l32] = gv / (1.0f + __expf(-gv)) * uv;
    }
  __syncthreads();
  // row sr, columns 32 sc .. 32 sc + 31: group sum and (hi, lo) parts
  float v[32];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const float4 t = *reinterpret_cast<const float4*>(ht + sr * HS + 32 * sc + 4 * q);
    v[4 * q] = t.x;
    v[4 * q + 1] = t.y;
    v[4 * q + 2] = t.z;
    v[4 * q + 3] = t.w;
  }
  float part = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) part += v[i];
  const float other = __shfl_xor(part, 1, 64);
  const float total = sc == 0 ? part + other : other + part;
  if (sr < ti.rows) {
    const int gi = n0 / kGroup;
    int64_t hrow, srow_i;
    if (shared) {
      hrow = (int64_t)T * k * 2 * I + (int64_t)(ti.base + sr) * 2 * Is;
      srow_i = (int64_t)T * k * (I / kGroup) + (int64_t)(ti.base + sr) * (Is / kGroup) + gi;
    } else {
      hrow = (int64_t)(ti.base + sr) * 2 * I;
      srow_i = (int64_t)(ti.base + sr) * (I / kGroup) + gi;
    }
    if (sc == 0) hsum[srow_i] = total;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      u32x4 hi, lo;
      split8(v + 8 * q, hi, lo);
      *reinterpret_cast<u32x4*>(h + hrow + n0 + 32 * sc + 8 * q) = permute_chunk<BITS>(hi);
      *reinterpret_cast<u32x4*>(h + hrow + inter + n0 + 32 * sc + 8 * q) = permute_chunk<BITS>(lo);
    }
  }
}

// ---------------------------------------------------------------------------
// down: grid (H/128 column blocks, tiles).  A = h as (hi, lo) bf16 parts, two
// MFMAs per K step.  Writes the weighted expert output of every bucket entry
// to partial[(t*(k+1) + j) * H + col] (fp32; the shared expert is j = k).

template <int BITS>
__global__ __launch_bounds__(256) void prefill_down_kernel(
    const uint16_t* __restrict__ h, const float* __restrict__ hsum,
    const int32_t* __restrict__ pairs, const float* __restrict__ topk_w,
    const float* __restrict__ gamma, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ ntiles, const uint8_t* __restrict__ slab,
    const int32_t* __restrict__ slot_table, int64_t stride, const uint8_t* __restrict__ shared_blob,
    float* __restrict__ partial, int T, int H, int E, int k, int I, int Is, int64_t d_off_r,
    int64_t d_unit_r, int64_t d_tile_r, int64_t d_off_s, int64_t d_unit_s, int64_t d_tile_s) {
  __shared__ __align__(16) uint16_t Ah[2 * kMT * kLdsRow];
  __shared__ __align__(16) uint16_t Al[2 * kMT * kLdsRow];
  __shared__ __align__(16) float HS[2 * kMT];  // group sums of the staged h rows
  __shared__ int32_t rowdst[kMT];
  __shared__ float roww[kMT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31, half = lane >> 5;
  if ((int)blockIdx.y >= *ntiles) return;
  const TileInfo ti = get_tile(tiles, counts, offsets, blockIdx.y, E);
  const bool shared = ti.e == E;
  const int inter = shared ? Is : I;
  const int n0 = blockIdx.x * 128;
  const uint8_t* sec = shared ? shared_blob + d_off_s
                              : slab + (int64_t)slot_table[ti.e] * stride + d_off_r;
  const int64_t unit_b = shared ? d_unit_s : d_unit_r, tile_b = shared ? d_tile_s : d_tile_r;
  if (tid < kMT) {
    int dst = -1;
    float wv = 0.f;
    if (tid < ti.rows) {
      if (shared) {
        const int t = ti.base + tid;
        dst = t * (k + 1) + k;
        wv = gamma[t];
      } else {
        const int p = pairs[ti.base + tid];
        dst = (p / k) * (k + 1) + (p % k);
        wv = topk_w[p];
      }
    }
    rowdst[tid] = dst;
    roww[tid] = wv;
  }
  const int G = inter / kGroup;
  // h rows and group-sum rows of the tile
  const int64_t hbase = shared ? (int64_t)T * k * 2 * I + (int64_t)ti.base * 2 * Is
                               : (int64_t)ti.base * 2 * I;
  const int64_t sbase = shared ? (int64_t)T * k * (I / kGroup) + (int64_t)ti.base * G
                               : (int64_t)ti.base * G;
  const int sr = tid >> 1, sc = tid & 1;
  const bool srow_ok = sr < ti.rows;
  const uint16_t* hrow = h + hbase + (int64_t)(srow_ok ? sr : 0) * 2 * inter + 32 * sc;
  const RowAddr<BITS> wr[2] = {
      RowAddr<BITS>(sec, unit_b, tile_b, 1, 0, n0 + 64 * wn + l32, half),
      RowAddr<BITS>(sec, unit_b, tile_b, 1, 0, n0 + 64 * wn + 32 + l32, half)};

  uint4 rh[4], rl[4];
  LaneCodes<BITS> cn[2];
  uint32_t sbn[2];
  float rs = 0.f;
  auto load_stage = [&](int g) {
    if (tid < ti.rows) rs = hsum[sbase + (int64_t)tid * G + g];
    if (srow_ok) {
      const uint4* ph = reinterpret_cast<const uint4*>(hrow + g * kGroup);
      const uint4* pl = reinterpret_cast<const uint4*>(hrow + inter + g * kGroup);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        rh[q] = ph[q];
        rl[q] = pl[q];
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        rh[q] = make_uint4(0, 0, 0, 0);
        rl[q] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      cn[nb].load(wr[nb].group_codes(g));
      sbn[nb] = wr[nb].group_sb(g);
    }
  };
  auto store_stage = [&](int buf) {
    const int o = buf * kMT * kLdsRow + sr * kLdsRow + sc * 32;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      *reinterpret_cast<uint4*>(Ah + o + 8 * q) = rh[q];
      *reinterpret_cast<uint4*>(Al + o + 8 * q) = rl[q];
    }
    if (tid < kMT) HS[buf * kMT + tid] = rs;
  };

  f32x16 C[2][2];
  const f32x16 zero = {};
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) C[mb][nb] = zero;


  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int g = 0; g < G; ++g) {
    const LaneCodes<BITS> cc[2] = {cn[0], cn[1]};
    const float scl[2] = {code_scale<BITS>(sbn[0]), code_scale<BITS>(sbn[1])};
    const float bco[2] = {bias_coef<BITS>(sbn[0]), bias_coef<BITS>(sbn[1])};
    if (g + 1 < G) load_stage(g + 1);
    const int so = (g & 1) * kMT * kLdsRow;
    f32x16 acc[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = zero;
#pragma unroll
    for (int ks = 0; ks < kGroup / 16; ++ks) {
      u32x4 ah[2], al[2], b[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int o = so + (64 * wm + 32 * mb + l32) * kLdsRow + 32 * half + 8 * ks;
        ah[mb] = *reinterpret_cast<const u32x4*>(Ah + o);
        al[mb] = *reinterpret_cast<const u32x4*>(Al + o);
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) b[nb] = cc[nb].frag(ks);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma(ah[mb], b[nb], acc[mb][nb]);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma(al[mb], b[nb], acc[mb][nb]);
    }
    // C += scale * code sums + bias * (group sum of the row's h)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      float4 hv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        hv[q] = *reinterpret_cast<const float4*>(HS + (g & 1) * kMT + 64 * wm + 32 * mb + 8 * q +
                                                 4 * half);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float4 t = hv[r / 4];
          const float hsv = (r % 4) == 0 ? t.x : (r % 4) == 1 ? t.y : (r % 4) == 2 ? t.z : t.w;
          C[mb][nb][r] += scl[nb] * acc[mb][nb][r] + bco[nb] * hsv;
        }
    }
    if (g + 1 < G) store_stage((g + 1) & 1);
    __syncthreads();
  }


#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = 64 * wm + 32 * mb + 8 * (r / 4) + 4 * half + (r % 4);
        const int dst = rowdst[m];
        if (dst >= 0)
          partial[(int64_t)dst * H + n0 + 64 * wn + 32 * nb + l32] = roww[m] * C[mb][nb][r];
      }
}

template <int BITS>
hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t s) {
  const int hs = a.has_shared ? 1 : 0;
  hipLaunchKernelGGL(tile_list_kernel, dim3(1), dim3(1024), 0, s, a.counts, a.tiles, a.ntiles,
                     a.E, hs, a.max_tiles, a.min_rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int G = a.H / kGroup;
  const int64_t nsum = (int64_t)a.T * G;
  hipLaunchKernelGGL(group_sum_kernel, dim3((unsigned)((nsum + 255) / 256)), dim3(256), 0, s, a.x,
                     a.xsum, a.T, a.H);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int nbg = (max(a.I, a.Is) + kGroup - 1) / kGroup;
  hipLaunchKernelGGL((prefill_gateup_kernel<BITS>), dim3(nbg, a.max_tiles), dim3(256), 0, s, a.x,
                     a.xsum, a.pairs, a.counts, a.offsets, a.tiles, a.ntiles, a.slab, a.slot_table,
                     a.stride, a.shared_blob, a.h, a.hsum, a.T, a.H, a.E, a.k, a.I, a.Is,
                     a.L.gu_unit, a.L.gu_tile, a.Ls.gu_unit, a.Ls.gu_tile);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((prefill_down_kernel<BITS>), dim3(a.H / 128, a.max_tiles), dim3(256), 0, s,
                     a.h, a.hsum, a.pairs, a.topk_w, a.gamma, a.counts, a.offsets, a.tiles,
                     a.ntiles, a.slab, a.slot_table, a.stride, a.shared_blob, a.partial, a.T, a.H,
                     a.E, a.k, a.I, a.Is, a.L.d_off, a.L.d_unit, a.L.d_tile, a.Ls.d_off,
                     a.Ls.d_unit, a.Ls.d_tile);
  if ((e = hipGetLastError()) != hipSuccess) return e;
return hipSuccess;
}

}  // namespace

int prefill_max_tiles(int T, int E, int k, bool has_shared) {
  // sum over buckets of ceil(n_b / kMT) <= sum(n_b) / kMT + number of buckets
  const int64_t rows = (int64_t)T * k + (has_shared ? T : 0);
  return (int)(rows / kMT + E + (has_shared ? 1 : 0) + 1);
}

bool prefill_supported(int act, int H, int I, int Is, bool has_shared) {
  if (act != MOE_ACT_BF16) return false;
  if (H % 128 != 0 || I % kGroup != 0 || (has_shared && Is % kGroup != 0)) return false;
  return true;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
  return a.bits == 4 ? launch_prefill_t<4>(a, s) : launch_prefill_t<8>(a, s);
}

}  // namespace moe
