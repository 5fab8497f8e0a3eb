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

struct RouterArgs {
  const void* x;
  const float* router_w;
  const float* router_bias;
  const float* shared_gate_w;
  float* logits;          // [T x (E+1)]
  int32_t* topk_idx;
  float* topk_w;
  float* gamma;           // may be null
  float* xsum;            // [T x H/64] group sums of x, written by the MFMA router if non-null
  int T, H, E, k, act;
};
hipError_t launch_router_topk(const RouterArgs& a, hipStream_t s);
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
  bool xsum_ready;               // the router already wrote the group sums of x
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
  uint16_t* h;                   // per row: I bf16 high parts, then I bf16 low parts
  float* xsum;                   // [T][H/64] group sums of x
  float* hsum;                   // [T*k][I/64] then [T][Is/64] group sums of h
  float* partial;                // fp32 [T*(k+1)*H]
  void* out;
  int32_t* tiles;
  int32_t* ntiles;
  int max_tiles;
  int min_rows;                  // buckets with fewer tokens are left to the GEMV kernels
  bool tiles_ready;              // the tile list was built with the buckets
  bool xsum_ready;               // xsum was written by the router
  BlobLayout L, Ls;
  int T, H, E, k, I, Is, bits;
  bool has_shared;
};
bool prefill_supported(int act, int H, int I, int Is, bool has_shared);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s);

// Batch-1 bf16 decode fast path: three kernels per layer (router with an
// optional fused RMSNorm; top-k + gate/up; down + combine with an optional
// fused residual add).
struct DecodeArgs {
  const uint16_t* x_in;          // router input: residual stream (do_norm) or x_hat
  uint16_t* x_hat;               // [H] normalised input (written when do_norm)
  const float* router_w;
  const float* router_bias;
  const float* shared_gate_w;    // null without shared expert
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

// Persistent decode chain (one cooperative launch for all layers).
struct ChainParams {
  uint16_t* x;                   // [H] residual stream in/out
  uint16_t* x_hat;               // [H] last layer's normalised input
  uint16_t* out;                 // [H] last layer's output
  const float* router_w;         // [L][E][H]
  const float* router_bias;      // [L][E] or null
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
