// Internal definitions of the MoE layer library: device helpers shared by the
// kernels and the launcher interfaces (the blob layout arithmetic and the
// workspace plan are in layout.h).  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "layout.h"
#include "moe.h"

namespace moe {

// ---------------------------------------------------------------------------
// device helpers

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
// Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

template <int ACT>
__device__ __forceinline__ float load_act(const void* p, int64_t i) {
  if constexpr (ACT == MOE_ACT_F32) {
    return reinterpret_cast<const float*>(p)[i];
  } else {
    return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
  }
}

template <int ACT>
__device__ __forceinline__ void store_act(void* p, int64_t i, float v) {
  if constexpr (ACT == MOE_ACT_F32) {
    reinterpret_cast<float*>(p)[i] = v;
  } else {
    reinterpret_cast<uint16_t*>(p)[i] = f32_to_bf16_bits(v);
  }
}

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + __expf(-g)); }

// Reductions over the 4 lanes of each quad (lanes 4i .. 4i+3) with DPP quad
// permutes (no LDS round trip, unlike a shuffle).  Every lane of the quad
// gets the same bits: (v0 + v1) + (v2 + v3).
template <int CTRL>
__device__ __forceinline__ float quad_perm_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                0xF, 0xF, false));
}
__device__ __forceinline__ float quad_sum(float v) {
  v += quad_perm_f<0xB1>(v);  // lane ^ 1
  v += quad_perm_f<0x4E>(v);  // lane ^ 2
  return v;
}
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, quad_perm_f<0xB1>(v));
  v = fmaxf(v, quad_perm_f<0x4E>(v));
  return v;
}

__device__ __forceinline__ float warp_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

}  // namespace moe

// ---------------------------------------------------------------------------
// launchers (defined in the .hip files)

namespace moe {

// One wave converts a bf16 activation row of H values (H a multiple of 512)
// to fp16 after a power-of-two scale: x16 = x * 2^-e, with e the exponent of
// the row's largest magnitude minus 14 (0 for a zero row), so the largest
// value lies in [2^14, 2^15) and every bf16 value at or above 2^-28 of it
// converts exactly.  Within each chunk of 8 columns the values are stored in
// the K order of the codes' fp16 expansion: (0, 4, 1, 5, 2, 6, 3, 7) for int4
// and (0, 2, 1, 3, 4, 6, 5, 7) for int8.  Lane 0 writes e.
__device__ __forceinline__ void x16_row(const uint16_t* __restrict__ xr, uint16_t* __restrict__ x16r,
                                        int32_t* __restrict__ e_out, int H, int bits) {
  const int lane = threadIdx.x & 63;
  uint32_t m = 0;
  for (int c = lane; c < H / 8; c += 64) {
    const uint4 v = reinterpret_cast<const uint4*>(xr)[c];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) m = max(m, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  // bf16 magnitude bits: exponent field in bits 7..14
  int e = m == 0 ? 0 : (int)(m >> 7) - 127 - 14;
  e = e < -100 ? -100 : (e > 100 ? 100 : e);
  const float sc = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e
  for (int c = lane; c < H / 8; c += 64) {
    const uint4 v = reinterpret_cast<const uint4*>(xr)[c];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    _Float16 f[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = (_Float16)(bf16_bits_to_f32(w[i] & 0xFFFFu) * sc);
      f[2 * i + 1] = (_Float16)(bf16_bits_to_f32(w[i] >> 16) * sc);
    }
    // stored slot j holds natural position p(j)
    const int p4[8] = {0, 4, 1, 5, 2, 6, 3, 7}, p8[8] = {0, 2, 1, 3, 4, 6, 5, 7};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const _Float16 lo = bits == 4 ? f[p4[2 * i]] : f[p8[2 * i]];
      const _Float16 hi = bits == 4 ? f[p4[2 * i + 1]] : f[p8[2 * i + 1]];
      o[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
             ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    reinterpret_cast<uint4*>(x16r)[c] = make_uint4(o[0], o[1], o[2], o[3]);
  }
  if (lane == 0) *e_out = e;
}

struct RouterArgs {
  const void* x;
  const float* router_w;
  const float* router_bias;
  const float* shared_gate_w;
  float* logits;          // [T x (E+1)]
  int32_t* topk_idx;
  float* topk_w;
  float* gamma;           // may be null
  uint16_t* x16;          // if non-null, the top-k kernel also writes x in fp16 (x16_row)
  int32_t* xe;            //   and the rows' exponents; x16_bits selects the K order
  int x16_bits;
  int T, H, E, k, act;
};
hipError_t launch_router_topk(const RouterArgs& a, hipStream_t s);
// MOE_FLAG_DENSE_Q4: the dense blob's rows dequantised to fp32 rows [rows][H]
hipError_t launch_dense_dequant(const uint8_t* blob, int rows, int H, int64_t words_off, float* out,
                                hipStream_t s);
// The router runs as an MFMA GEMM (bf16 batches from 16 tokens, H a multiple of 64).
constexpr int kRouterMfmaMinTokens = 16;
inline bool router_uses_mfma(int act, int64_t T, int64_t H) {
  return act == MOE_ACT_BF16 && T >= kRouterMfmaMinTokens && H % 64 == 0;
}

struct ExpertArgs {
  const void* x;                 // x_hat [T x H]
  const int32_t* topk_idx;
  const float* topk_w;
  const float* gamma;            // null without shared expert
  const uint8_t* slab;
  const int32_t* slot_table;
  int64_t stride;
  const uint8_t* shared_blob;    // null without shared expert
  void* out;
  uint8_t* ws;
  WsPlan plan;
  BlobLayout L;                  // routed experts
  BlobLayout Ls;                 // shared expert
  int T, H, E, k, act, bits;
  bool has_shared;
  bool mfma;                     // large batch: grouped GEMMs on MFMA
  // Chain epilogue fused into the combine (bucketed path only): 0 none;
  // 1 x_res += out; 2 also x_hat = rmsnorm(x_res) with eps.
  int epi;
  void* x_res;
  void* x_hat_next;
  float eps;
  bool x16_ready;                // the router's top-k kernel already wrote x16 / xe
};
hipError_t launch_experts(const ExpertArgs& a, hipStream_t s);

// Grouped-GEMM (MFMA) experts for large batches, after bucketing.
struct PrefillArgs {
  const uint16_t* x;
  const int32_t* pairs;
  const int32_t* counts;         // [E+1], counts[E] = T (shared)
  const int32_t* offsets;
  const float* topk_w;
  const float* gamma;
  const uint8_t* slab;
  const int32_t* slot_table;
  int64_t stride;
  const uint8_t* shared_blob;
  uint16_t* h;                   // h rows (fp32 GEMV layout; fp16 + scales on this path)
  float* partial;                // fp32 [T*(k+1)*H]
  uint16_t* x16;                 // x in fp16 (x16_row) and the rows' exponents
  int32_t* xe;
  bool x16_ready;                // written by the router's top-k kernel
  void* out;
  int32_t* tiles;
  int32_t* ntiles;
  int max_tiles;
  int min_rows;                  // buckets with fewer tokens are left to the GEMV kernels
  bool tiles_ready;              // the tile list was built with the buckets
  BlobLayout L, Ls;
  int T, H, E, k, I, Is, bits;
  bool has_shared;
};
bool prefill_supported(int act, int64_t T, int H, int k, int I, int Is, bool has_shared);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s);
// One token block (T <= 64): the same GEMMs with every weight tile requested
// up front (batched.hip); h is written as fp32 rows of `inter` floats.
bool batched_supported(int act, int T, int H, int I, int Is, bool has_shared);
hipError_t launch_batched(const PrefillArgs& a, hipStream_t s);
// x16 / xe of a batch (one wave per row) when the router did not write them
hipError_t launch_x16(const uint16_t* x, uint16_t* x16, int32_t* xe, int T, int H, int bits,
                      hipStream_t s);
// Whether a layer call runs the grouped GEMMs on the matrix cores (bucketed
// bf16 batches; they read x16 / xe).
inline bool mfma_path(const moe_layer_desc& d) {
  const bool sh = (d.flags & MOE_FLAG_SHARED) != 0;
  return d.n_tokens > kDecodeMaxTokens &&
         prefill_supported(d.act_dtype, d.n_tokens, d.hidden, d.top_k, d.inter,
                           sh ? d.shared_inter : d.inter, sh);
}
// Whether it runs the one-token-block variant: batches of 9..64 tokens.
inline bool one_block_path(const moe_layer_desc& d) {
  const bool sh = (d.flags & MOE_FLAG_SHARED) != 0;
  const int Is = sh ? d.shared_inter : 0;
  return d.n_tokens > kDecodeMaxTokens && d.n_tokens <= kOneBlockTokens && d.n_experts < 1024 &&
         prefill_supported(d.act_dtype, d.n_tokens, d.hidden, d.top_k, d.inter, sh ? Is : d.inter,
                           sh) &&
         batched_supported(d.act_dtype, d.n_tokens, d.hidden, d.inter, Is, sh);
}

// Batch-1 bf16 decode fast path: three kernels per layer (router with an
// optional fused RMSNorm; top-k + gate/up; down + combine with an optional
// fused residual add).
struct DecodeArgs {
  const uint16_t* x_in;          // router input: residual stream (do_norm) or x_hat
  uint16_t* x_hat;               // [H] normalised input (written when do_norm)
  const float* router_w;
  const float* router_bias;
  const float* shared_gate_w;    // null without shared expert
  const uint8_t* dense;          // MOE_FLAG_DENSE_Q4: the dense blob (router_w unused), else null
  int64_t dense_words;           //   offset of its (scale, bias) words
  float* logits;                 // ws
  int32_t* idx;                  // ws routing
  float* w;
  float* gamma;
  int32_t* slots;                // ws: slab slot of each selected expert
  float* h;                      // ws
  const uint8_t* slab;
  const int32_t* slot_table;
  int64_t stride;
  const uint8_t* shared_blob;
  uint16_t* out;                 // [H]
  uint16_t* x_res;               // residual stream to update, or null
  BlobLayout L, Ls;
  int H, E, k, bits;
  float eps;
  bool do_norm, has_shared;
};
bool decode_fast_supported(int T, int act, int H, int k, int E, int bits, int I, int Is,
                           bool has_shared);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);

// Persistent decode chain (one launch for all layers, every workgroup resident).
struct ChainParams {
  uint16_t* x;                   // [H] residual stream in/out
  uint16_t* x_hat;               // [H] last layer's normalised input
  uint16_t* out;                 // [H] last layer's output
  const float* router_w;         // [L][E][H] (unused with dense)
  const float* router_bias;      // [L][E] or null
  const uint8_t* dense;          // MOE_FLAG_DENSE_Q4: layer l's dense blob at l * dense_stride
  int64_t dense_stride, dense_words;
  const uint8_t* slab;
  int64_t stride;
  const int32_t* slot_tables;    // [L][E]
  const uint8_t* shared_blobs;   // layer l at + l * shared_stride
  int64_t shared_stride;
  int L, H, E, k, I, Is, has_shared, bits_;
  float eps;
  int64_t gu_unit_r, gu_tile_r, d_off_r, d_unit_r, d_tile_r;
  int64_t gu_unit_s, gu_tile_s, d_off_s, d_unit_s, d_tile_s, sg_off;
  uint64_t* xw;                  // [H/2] exchange words (epoch | 2 x bf16)
  uint64_t* lw;                  // [E+1] exchange words (epoch | fp32 logit)
  uint64_t* hw;                  // [k*I + Is] exchange words (epoch | fp32 h)
  uint32_t* ctr;                 // last epoch used
  uint32_t* err;                 // bit 0: an exchange poll expired
  int32_t* r_idx;                // last layer's routing
  float* r_w;
  float* r_gamma;
};
int chain_grid(int device);
bool chain_supported(int nwg, int T, int act, int H, int E, int k, int bits, int I, int Is,
                     bool has_shared);
hipError_t launch_chain(const ChainParams& p, int nwg, hipStream_t s);

hipError_t launch_rmsnorm(void* x, const void* out, void* x_hat, int T, int H, int act,
                          float eps, bool do_norm, hipStream_t s);

hipError_t launch_pack_device(const BlobLayout& L, int n, const uint8_t* qg, const uint8_t* qu,
                              const uint8_t* qd, const uint16_t* sbg, const uint16_t* sbu,
                              const uint16_t* sbd, uint8_t* slab, int64_t stride,
                              const int64_t* slots_host, hipStream_t s);

}  // namespace moe
