// MFMA helpers shared by the grouped-GEMM kernels (prefill.hip: tiles of up
// to 128 bucket rows; batched.hip: one token block of at most 64 rows).  Device code only; each including file gets its own
// internal copy.
#pragma once

#include "moe_internal.h"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kMT = kMfmaTileRows;  // rows (bucket entries) per tile
constexpr int kPersistSlots = 1024;  // workgroups of the persistent GEMM grids (multiple of 8)
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

// One lane's codes of one weight row for one group: 32 consecutive codes
// (16 bytes of int4, 32 bytes of int8).
template <int BITS>
struct LaneCodes {
  uint4 q[BITS / 4];
  __device__ __forceinline__ void load(const uint8_t* p) {
#pragma unroll
    for (int i = 0; i < BITS / 4; ++i) q[i] = reinterpret_cast<const uint4*>(p)[i];
  }
};

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

// (scale, bias) word -> the fp16 pairs (S, S), (B, B) of w = S c + B, with c
// the code's fp16 expansion (int4: c = 1 + q/16, so S = 16 s and B = b - 16 s;
// int8: c = q, so S = s and B = b).
template <int BITS>
__device__ __forceinline__ void sb_f16(uint32_t sb, f16x2& S2, f16x2& B2) {
  const float sc = bf16_bits_to_f32(sb & 0xFFFFu), bi = bf16_bits_to_f32(sb >> 16);
  const _Float16 S = (_Float16)(BITS == 4 ? 16.0f * sc : sc);
  const _Float16 B = (_Float16)(BITS == 4 ? bi - 16.0f * sc : bi);
  S2 = f16x2{S, S};
  B2 = f16x2{B, B};
}

// MFMA operand of K step kk: the lane's 8 weights of the step in fp16, in the
// fp16 expansion's K order (int4 (0, 4, 1, 5, 2, 6, 3, 7); int8 (0, 2, 1, 3, 4,
// 6, 5, 7) within the 8 codes).
template <int BITS>
__device__ __forceinline__ u32x4 w_frag_f16(const LaneCodes<BITS>& q, int kk, f16x2 S2, f16x2 B2) {
  u32x4 c;
  if constexpr (BITS == 4) {
    const uint32_t d = kk == 0 ? q.q[0].x : kk == 1 ? q.q[0].y : kk == 2 ? q.q[0].z : q.q[0].w;
    c = code_frag4_f16(d);
  } else {
    const uint4 v = q.q[kk >> 1];
    c = (kk & 1) ? code_frag8_f16(v.z, v.w) : code_frag8_f16(v.x, v.y);
  }
  // (each element is taken as a value before its bit cast: a bit cast applied
  // to an indexed vector element directly has been seen to read element 0)
  uint32_t r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t ci = c[i];
    r[i] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(f16x2, ci), S2, B2));
  }
  return u32x4{r[0], r[1], r[2], r[3]};
}

// 2^e as a float (|e| <= 100)
__device__ __forceinline__ float exp2i(int e) { return __uint_as_float((uint32_t)(127 + e) << 23); }

}  // namespace
}  // namespace moe
