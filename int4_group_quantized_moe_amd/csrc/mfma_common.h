// MFMA helpers shared by the grouped-GEMM kernels (prefill.hip: tiles of up
// to 128 bucket rows with LDS-staged operands; batched.hip: one token block
// of at most 64 rows).  Device code only; each including file gets its own
// internal copy.
#pragma once

#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kMT = kMfmaTileRows;  // rows (bucket entries) per tile
constexpr int kPersistSlots = 1024;  // workgroups of the persistent GEMM grids (multiple of 8)
constexpr int kLdsRow = kGroup + 8;  // padded LDS row of one group (bf16 elements)

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f32x16 mfma_f16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Exact fp16 operands from integer codes, in the permuted K order of the
// down GEMM.  int4: word d of 8 codes becomes the fp16 pairs (q0, q4),
// (q1, q5), (q2, q6), (q3, q7), each 1 + q/16 (the nibble in mantissa bits
// 6..9 of 1.0): 8 instructions.  int8: each word of 4 codes becomes (q0, q2),
// (q1, q3): 1024 + q by a mask into the mantissa of 1024.0, then 1024
// subtracted in packed fp16, both exact.
__device__ __forceinline__ u32x4 code_frag4_f16(uint32_t d) {
  constexpr uint32_t M = 0x03C003C0u, O = 0x3C003C00u;
  return u32x4{((d << 6) & M) | O, ((d << 2) & M) | O, ((d >> 2) & M) | O, ((d >> 6) & M) | O};
}
__device__ __forceinline__ uint32_t byte_pair_f16(uint32_t d) {
  const f16x2 v = __builtin_bit_cast(f16x2, (d & 0x00FF00FFu) | 0x64006400u) - (f16x2){1024, 1024};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ u32x4 code_frag8_f16(uint32_t d0, uint32_t d1) {
  return u32x4{byte_pair_f16(d0), byte_pair_f16(d0 >> 8), byte_pair_f16(d1), byte_pair_f16(d1 >> 8)};
}
// Position, in the natural K order of an 8-value chunk, of the value the
// down GEMM's fp16 operands hold at slot j (the order the expansions above
// produce).
template <int BITS>
__device__ __forceinline__ constexpr int dn_perm(int j) {
  return BITS == 4 ? (j >> 1) + 4 * (j & 1) : (j & 4) + ((j & 3) >> 1) + 2 * (j & 1);
}

// Exact bf16 operands from integer codes, in natural K order.  int4: the
// nibble goes into mantissa bits 3..6 of 1.0, giving 1 + q/16 exactly (a
// 32-bit word of 8 codes becomes 4 bf16 pairs with 12 instructions); int8:
// the float of the byte has at most 8 significant bits, so its upper half is
// q exactly.
__device__ __forceinline__ u32x4 code_frag4(uint32_t d) {
  constexpr uint32_t M = 0x78787878u, O = 0x3F803F80u;
  const uint32_t lo = (d << 3) & M;  // codes 0,2,4,6 in bits 3..6 of bytes 0..3
  const uint32_t hi = (d >> 1) & M;  // codes 1,3,5,7
  return u32x4{__builtin_amdgcn_perm(hi, lo, 0x0C040C00u) | O,
               __builtin_amdgcn_perm(hi, lo, 0x0C050C01u) | O,
               __builtin_amdgcn_perm(hi, lo, 0x0C060C02u) | O,
               __builtin_amdgcn_perm(hi, lo, 0x0C070C03u) | O};
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
  RowAddr() = default;
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
  __device__ __forceinline__ const uint8_t* group_sb_ptr(int g) const {
    return sb + (int64_t)(g / GPK) * unit_b + (g % GPK) * 4;
  }
  __device__ __forceinline__ uint32_t group_sb(int g) const {
    return *reinterpret_cast<const uint32_t*>(group_sb_ptr(g));
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
    // all loads first (clamped indices, so they are unconditional), then
    // the selects: one wait for the whole batch
    float va[2][8];
    uint32_t vb[2][8];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const float* p = srow[mb] != nullptr ? srow[mb] : srow[mb ^ 1];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int g = min(16 * j + 8 * half + i, G - 1);
        va[mb][i] = p != nullptr ? p[g] : 0.f;
      }
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 8; ++i) vb[nb][i] = wr[nb].group_sb(min(16 * j + 8 * half + i, G - 1));
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int g = 16 * j + 8 * half + i;
        v[i] = (srow[mb] != nullptr && g < G) ? va[mb][i] : 0.f;
      }
      split8(v, ah[mb], al[mb]);
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int g = 16 * j + 8 * half + i;
        v[i] = g < G ? bias_coef<BITS>(vb[nb][i]) : 0.f;
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

// Work-item order for the MI355X's 8 XCDs (each with its own L2): the
// hardware hands linear workgroup w to XCD w % 8, so XCD c is given the
// contiguous item range [c*per, (c+1)*per) of the (tile, column block)
// items, column block fastest, per = ceil(items / 8).  The column blocks of
// one row tile (which share its activation rows) and the row tiles of one
// expert (which share its weights) then run on the same L2.  The item count
// is only known on the device.
struct XcdItem {
  int tile, nb;
  bool valid;
};

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

}  // namespace
}  // namespace moe
