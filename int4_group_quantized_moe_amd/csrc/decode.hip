// Batch-1 decode fast path (bf16 activations): one MoE layer in three
// kernels, each kernel boundary being one of the three all-to-all exchanges a
// layer needs (the full input for the router, the full logits for the top-k,
// every expert's full h for the down projection).
//
//   A  decode_router_kernel   optional RMSNorm (chain step) + router GEMV and
//                             shared-gate logit; one wave per router row.
//   B  decode_gateup_kernel   exact top-k + renormalised weights (wave 0, in
//                             every workgroup) while the other waves stage the
//                             activations; then the fused dequant gate/up GEMV
//                             + SiLU*up of one 16-row tile of one expert.
//   C  decode_down_kernel     dequant down GEMV over all selected experts for
//                             8 output rows, fixed-order weighted combine,
//                             optional residual add.
//
// Routing: top-k of E experts per token with a shared expert always active
// (page "Paquets Swiftlet 80B Qwen ..." on xix.ai, 4th paragraph); weights
// are MLX-style group-quantised int4/int8 (same page, last paragraph).
#include "decode_common.h"

namespace moe {
namespace {

using namespace dec;

// ---------------------------------------------------------------------------
// A: router.  Block = one wave = one row (router rows 0..E-1, then the shared
// gate row).  With do_norm, x is the residual stream and every wave
// normalises it itself (x_hat = bf16(x / rms)); block 0 stores x_hat.  With
// Q4 the rows come from the layer's dense blob (4-bit codes, (scale, bias)
// per group of 64; the shared gate is its row E), dequantised in fp32.

template <int NIT, bool Q4>
__global__ __launch_bounds__(64) void decode_router_kernel(
    const uint16_t* __restrict__ x, uint16_t* __restrict__ x_hat, const float* __restrict__ W,
    const float* __restrict__ bias, const float* __restrict__ wsg,
    const uint8_t* __restrict__ dense, int64_t dense_words, float* __restrict__ logits, int H,
    int E, float eps, int do_norm) {
  const int lane = threadIdx.x;
  const int r = blockIdx.x;
  float4 w4[NIT];
  uint2 x4[NIT];
  if constexpr (Q4) {
    const uint8_t* crow = dense + (int64_t)r * (H / 2);
    const uint32_t* words = reinterpret_cast<const uint32_t*>(dense + dense_words) + (int64_t)r * (H / kGroup);
    uint32_t q[NIT], sb[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      q[it] = *reinterpret_cast<const uint16_t*>(crow + it * 128 + lane * 2);
      sb[it] = words[it * 4 + (lane >> 4)];
      x4[it] = *reinterpret_cast<const uint2*>(x + it * 256 + lane * 4);
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const float sc = bf16_bits_to_f32(sb[it] & 0xFFFFu), bi = bf16_bits_to_f32(sb[it] >> 16);
      w4[it] = make_float4(fmaf(sc, (float)(q[it] & 15u), bi), fmaf(sc, (float)((q[it] >> 4) & 15u), bi),
                           fmaf(sc, (float)((q[it] >> 8) & 15u), bi), fmaf(sc, (float)(q[it] >> 12), bi));
    }
  } else {
    const float* wrow = r < E ? W + (int64_t)r * H : wsg;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int c = it * 256 + lane * 4;
      w4[it] = *reinterpret_cast<const float4*>(wrow + c);
      x4[it] = *reinterpret_cast<const uint2*>(x + c);
    }
  }
  float xv[NIT][4];
  float ss = 0.f;
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    xv[it][0] = bf16_bits_to_f32(x4[it].x & 0xFFFFu);
    xv[it][1] = bf16_bits_to_f32(x4[it].x >> 16);
    xv[it][2] = bf16_bits_to_f32(x4[it].y & 0xFFFFu);
    xv[it][3] = bf16_bits_to_f32(x4[it].y >> 16);
#pragma unroll
    for (int q = 0; q < 4; ++q) ss += xv[it][q] * xv[it][q];
  }
  if (do_norm) {
    const float inv = 1.0f / sqrtf(wave_sum_dpp(ss) / (float)H + eps);
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      uint32_t b[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        b[q] = f32_to_bf16_bits(xv[it][q] * inv);
        xv[it][q] = bf16_bits_to_f32(b[q]);
      }
      if (r == 0)
        *reinterpret_cast<uint2*>(x_hat + it * 256 + lane * 4) =
            make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
    }
  }
  float acc = 0.f;
#pragma unroll
  for (int it = 0; it < NIT; ++it)
    acc += w4[it].x * xv[it][0] + w4[it].y * xv[it][1] + w4[it].z * xv[it][2] + w4[it].w * xv[it][3];
  acc = wave_sum_dpp(acc);
  if (lane == 0) logits[r] = acc + ((r < E && bias != nullptr) ? bias[r] : 0.0f);
}

// ---------------------------------------------------------------------------
// B: top-k + gate/up.  grid = (tiles, k + has_shared); block = 4 waves.
// Each wave owns k-blocks kb = wave, wave+4, ...; lane l owns row l/4 and
// the 16-byte chunk l%4 of every k-block.



template <int BITS>
__global__ __launch_bounds__(256) void decode_gateup_kernel(
    const uint16_t* __restrict__ x_hat, const float* __restrict__ logits,
    const uint8_t* __restrict__ slab, const int32_t* __restrict__ slot_table, int64_t stride,
    const uint8_t* __restrict__ shared_blob, int32_t* __restrict__ ws_idx,
    float* __restrict__ ws_w, float* __restrict__ ws_gamma, int32_t* __restrict__ ws_slot,
    float* __restrict__ h, int H, int E,
    int k, int I, int Is, int64_t gu_unit_r, int64_t gu_tile_r, int64_t gu_unit_s,
    int64_t gu_tile_s, int has_shared) {
  using C = GuCfg<BITS>;
  constexpr int CC = C::CC, GPK = C::GPK;
  __shared__ __align__(16) uint32_t xp[MOE_MAX_HIDDEN / 32 * 20];
  __shared__ float2 cs[MOE_MAX_HIDDEN / 16];
  __shared__ int32_t sel_idx[MOE_MAX_TOP_K];
  __shared__ float sel_val[MOE_MAX_TOP_K], sel_w[MOE_MAX_TOP_K], gam;
  __shared__ __align__(16) uint32_t cand_key[64];
  __shared__ __align__(16) int32_t cand_idx[64];
  __shared__ float cand_val[64];
  __shared__ float red[4][kRowTile][2];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tile = blockIdx.x, j = blockIdx.y;
  const bool is_shared = j >= k;
  const int inter = is_shared ? Is : I;
  if (tile * kRowTile >= inter) return;
  const int n_kb = H / C::KBC;
  const int row = lane >> 2, c4 = lane & 3;
  const int sbg_off = 2 * kCodeBlockBytes + (row * GPK + (c4 * CC) / kGroup) * 4;
  const int sbu_off = sbg_off + kRowTile * GPK * 4;

  uint4 qg[kMaxKbPerWave], qu[kMaxKbPerWave];
  uint32_t sg[kMaxKbPerWave], su[kMaxKbPerWave];
  auto issue = [&](const uint8_t* blob, int64_t unit_b, int64_t tile_b) {
    const uint8_t* tb = blob + (int64_t)tile * tile_b;
#pragma unroll
    for (int i = 0; i < kMaxKbPerWave; ++i) {
      const int kb = wave + 4 * i;
      if (kb < n_kb) {
        const uint8_t* unit = tb + (int64_t)kb * unit_b;
        qg[i] = *reinterpret_cast<const uint4*>(unit + lane * 16);
        qu[i] = *reinterpret_cast<const uint4*>(unit + kCodeBlockBytes + lane * 16);
        sg[i] = *reinterpret_cast<const uint32_t*>(unit + sbg_off);
        su[i] = *reinterpret_cast<const uint32_t*>(unit + sbu_off);
      }
    }
  };
  if (is_shared) issue(shared_blob, gu_unit_s, gu_tile_s);

  if (wave == 0 && !is_shared) {
    wave_topk(logits, E, k, has_shared != 0, sel_idx, sel_val, sel_w, &gam, cand_key, cand_idx,
              cand_val);
    if (tile == 0 && j == 0) {
      if (lane < k) {
        ws_idx[lane] = sel_idx[lane];
        ws_w[lane] = sel_w[lane];
      }
      if (lane == 0 && has_shared) *ws_gamma = gam;
    }
  } else if (wave == 1) {
    // stage the activations: one chunk of CC columns per lane
    const int nchunk = H / CC;
    for (int ch = lane; ch < nchunk; ch += 64) {
      const uint4* src = reinterpret_cast<const uint4*>(x_hat + ch * CC);
      float xv[CC];
#pragma unroll
      for (int q = 0; q < CC / 8; ++q) {
        const uint4 p = src[q];
        const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          xv[q * 8 + 2 * m] = bf16_bits_to_f32(w[m] & 0xFFFFu);
          xv[q * 8 + 2 * m + 1] = bf16_bits_to_f32(w[m] >> 16);
        }
      }
      if constexpr (BITS == 4) {
        float c = 0.f, s = 0.f;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float* vv = xv + 8 * jj;
          const uint32_t pa = pack_f16x2(vv[0], vv[4]);
          const uint32_t pb = pack_f16x2(vv[1] * 0.0625f, vv[5] * 0.0625f);
          const uint32_t pc = pack_f16x2(vv[2], vv[6]);
          const uint32_t pf = pack_f16x2(vv[3] * 0.0625f, vv[7] * 0.0625f);
          *reinterpret_cast<uint4*>(xp + ch * C::XS + jj * 4) = make_uint4(pa, pb, pc, pf);
          c += f16lo(pa) + f16hi(pa) + f16lo(pb) + f16hi(pb) + f16lo(pc) + f16hi(pc) + f16lo(pf) +
               f16hi(pf);
          s += f16lo(pa) + f16hi(pa) + f16lo(pc) + f16hi(pc) +
               16.0f * (f16lo(pb) + f16hi(pb) + f16lo(pf) + f16hi(pf));
        }
        cs[ch] = make_float2(1024.0f * c, s);
      } else {
        float c = 0.f;
        uint32_t pk[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          pk[jj] = pack_f16x2(xv[2 * jj], xv[2 * jj + 1]);
          c += f16lo(pk[jj]) + f16hi(pk[jj]);
        }
        *reinterpret_cast<uint4*>(xp + ch * C::XS) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
        *reinterpret_cast<uint4*>(xp + ch * C::XS + 4) = make_uint4(pk[4], pk[5], pk[6], pk[7]);
        cs[ch] = make_float2(1024.0f * c, c);
      }
    }
  }
  __syncthreads();
  if (!is_shared) {
    const int e = sel_idx[j];
    const int32_t slot = slot_table[e];
    if (tile == 0 && threadIdx.x == 0) ws_slot[j] = slot;
    issue(slab + (int64_t)slot * stride, gu_unit_r, gu_tile_r);
  }
  float g = 0.f, u = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxKbPerWave; ++i) {
    const int kb = wave + 4 * i;
    if (kb < n_kb) {
      const int gc = kb * 4 + c4;
      const float2 c = cs[gc];
      float pg = 0.f, pu = 0.f;
      const uint32_t dg[4] = {qg[i].x, qg[i].y, qg[i].z, qg[i].w};
      const uint32_t du[4] = {qu[i].x, qu[i].y, qu[i].z, qu[i].w};
      if constexpr (BITS == 4) {
        const uint4* xq = reinterpret_cast<const uint4*>(xp + gc * C::XS);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint4 X = xq[m];
          const uint32_t eg = dg[m] >> 8, eu = du[m] >> 8;
          pg = dot2((dg[m] & 0x000F000Fu) | 0x64006400u, X.x, pg);
          pu = dot2((du[m] & 0x000F000Fu) | 0x64006400u, X.x, pu);
          pg = dot2((dg[m] & 0x00F000F0u) | 0x64006400u, X.y, pg);
          pu = dot2((du[m] & 0x00F000F0u) | 0x64006400u, X.y, pu);
          pg = dot2((eg & 0x000F000Fu) | 0x64006400u, X.z, pg);
          pu = dot2((eu & 0x000F000Fu) | 0x64006400u, X.z, pu);
          pg = dot2((eg & 0x00F000F0u) | 0x64006400u, X.w, pg);
          pu = dot2((eu & 0x00F000F0u) | 0x64006400u, X.w, pu);
        }
      } else {
        const uint4* xq = reinterpret_cast<const uint4*>(xp + gc * C::XS);
        const uint4 X0 = xq[0], X1 = xq[1];
        const uint32_t xs[8] = {X0.x, X0.y, X0.z, X0.w, X1.x, X1.y, X1.z, X1.w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          pg = dot2(__builtin_amdgcn_perm(0x64646464u, dg[m], 0x04010400u), xs[2 * m], pg);
          pg = dot2(__builtin_amdgcn_perm(0x64646464u, dg[m], 0x04030402u), xs[2 * m + 1], pg);
          pu = dot2(__builtin_amdgcn_perm(0x64646464u, du[m], 0x04010400u), xs[2 * m], pu);
          pu = dot2(__builtin_amdgcn_perm(0x64646464u, du[m], 0x04030402u), xs[2 * m + 1], pu);
        }
      }
      g += bf16_bits_to_f32(sg[i] & 0xFFFFu) * (pg - c.x) + bf16_bits_to_f32(sg[i] >> 16) * c.y;
      u += bf16_bits_to_f32(su[i] & 0xFFFFu) * (pu - c.x) + bf16_bits_to_f32(su[i] >> 16) * c.y;
    }
  }
  g = quad_sum(g);
  u = quad_sum(u);
  if (c4 == 0) {
    red[wave][row][0] = g;
    red[wave][row][1] = u;
  }
  __syncthreads();
  if (threadIdx.x < kRowTile) {
    const int r = threadIdx.x;
    const float gs = (red[0][r][0] + red[1][r][0]) + (red[2][r][0] + red[3][r][0]);
    const float us = (red[0][r][1] + red[1][r][1]) + (red[2][r][1] + red[3][r][1]);
    const int64_t hrow = is_shared ? (int64_t)k * I : (int64_t)j * I;
    h[hrow + tile * kRowTile + r] = silu_f32(gs) * us;
  }
}

// ---------------------------------------------------------------------------
// C: down + combine (+ residual).  grid = H/8 workgroups of 4 waves; a
// workgroup owns 8 output rows = one half of a 16-row tile.  The work list is
// every (item, k-block) half-unit; half-wave hw (0..7) takes every 8th one.
// Lane l: row (l%32)/4 of the half tile, chunk l%4.

constexpr int kMaxDownUnitsPerHalfWave = 12;

template <int BITS>
__global__ __launch_bounds__(256) void decode_down_kernel(
    const int32_t* __restrict__ ws_slot, const float* __restrict__ ws_w,
    const float* __restrict__ ws_gamma, const uint8_t* __restrict__ slab, int64_t stride,
    const uint8_t* __restrict__ shared_blob, const float* __restrict__ h,
    uint16_t* __restrict__ out, uint16_t* __restrict__ x_res, int H, int k, int I, int Is,
    int64_t d_off_r, int64_t d_unit_r, int64_t d_tile_r, int64_t d_off_s, int64_t d_unit_s,
    int64_t d_tile_s, int has_shared) {
  using C = GuCfg<BITS>;
  constexpr int CC = C::CC, GPK = C::GPK, KBC = C::KBC;
  constexpr int CP = CC + 4;     // padded chunk stride in LDS (bank-conflict free)
  extern __shared__ float hs[];  // per chunk of CC h values: CP floats; then chunk sums
  __shared__ float red[4][2][8];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tile = blockIdx.x >> 1, half = blockIdx.x & 1;
  const int hw = wave * 2 + (lane >> 5);  // half-wave 0..7
  const int l32 = lane & 31;
  const int row8 = l32 >> 2, c4 = lane & 3;
  const int rt = half * 8 + row8;  // row inside the 16-row tile
  const int sb_off = kCodeBlockBytes + (rt * GPK + (c4 * CC) / kGroup) * 4;
  const int nkb_r = I / KBC, nkb_s = has_shared ? Is / KBC : 0;
  const int n_units = k * nkb_r + nkb_s;
  const int htot = k * I + (has_shared ? Is : 0);
  const int nchunk = htot / CC;
  float* hsum = hs + nchunk * CP;

  // weights first: slot of each selected expert (one dependent load), then
  // every unit of this half-wave
  uint4 q[kMaxDownUnitsPerHalfWave];
  uint32_t sb[kMaxDownUnitsPerHalfWave];
  float wgt[kMaxDownUnitsPerHalfWave];
#pragma unroll
  for (int i = 0; i < kMaxDownUnitsPerHalfWave; ++i) {
    const int uidx = hw + 8 * i;
    if (uidx < n_units) {
      const uint8_t* unit;
      if (uidx < k * nkb_r) {
        const int jj = uidx / nkb_r, kb = uidx - jj * nkb_r;
        unit = slab + (int64_t)ws_slot[jj] * stride + d_off_r + (int64_t)tile * d_tile_r +
               (int64_t)kb * d_unit_r;
        wgt[i] = ws_w[jj];
      } else {
        const int kb = uidx - k * nkb_r;
        unit = shared_blob + d_off_s + (int64_t)tile * d_tile_s + (int64_t)kb * d_unit_s;
        wgt[i] = *ws_gamma;
      }
      q[i] = *reinterpret_cast<const uint4*>(unit + half * 512 + l32 * 16);
      sb[i] = *reinterpret_cast<const uint32_t*>(unit + sb_off);
    }
  }
  // h into LDS, one chunk per thread, with its sum
  for (int ch = threadIdx.x; ch < nchunk; ch += 256) {
    const float4* src = reinterpret_cast<const float4*>(h + ch * CC);
    float s = 0.f;
#pragma unroll
    for (int m = 0; m < CC / 4; ++m) {
      const float4 v = src[m];
      *reinterpret_cast<float4*>(hs + ch * CP + 4 * m) = v;
      s += (v.x + v.y) + (v.z + v.w);
    }
    hsum[ch] = s;
  }
  __syncthreads();
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxDownUnitsPerHalfWave; ++i) {
    const int uidx = hw + 8 * i;
    if (uidx < n_units) {
      int jj, kb, hb;
      if (uidx < k * nkb_r) {
        jj = uidx / nkb_r;
        kb = uidx - jj * nkb_r;
        hb = jj * I;
      } else {
        jj = k;
        kb = uidx - k * nkb_r;
        hb = k * I;
      }
      const int ch = (hb + kb * KBC) / CC + c4;
      const float* hv = hs + ch * CP;
      const uint32_t d[4] = {q[i].x, q[i].y, q[i].z, q[i].w};
      float p = 0.f;
      if constexpr (BITS == 4) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const float4 a = *reinterpret_cast<const float4*>(hv + 8 * m);
          const float4 b = *reinterpret_cast<const float4*>(hv + 8 * m + 4);
          const uint32_t lo = d[m] & 0x0F0F0F0Fu, hi = (d[m] >> 4) & 0x0F0F0F0Fu;
          p += (float)(lo & 0xFF) * a.x + (float)(hi & 0xFF) * a.y +
               (float)((lo >> 8) & 0xFF) * a.z + (float)((hi >> 8) & 0xFF) * a.w +
               (float)((lo >> 16) & 0xFF) * b.x + (float)((hi >> 16) & 0xFF) * b.y +
               (float)(lo >> 24) * b.z + (float)(hi >> 24) * b.w;
        }
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const float4 a = *reinterpret_cast<const float4*>(hv + 4 * m);
          p += (float)(d[m] & 0xFF) * a.x + (float)((d[m] >> 8) & 0xFF) * a.y +
               (float)((d[m] >> 16) & 0xFF) * a.z + (float)(d[m] >> 24) * a.w;
        }
      }
      const float s = bf16_bits_to_f32(sb[i] & 0xFFFFu), b = bf16_bits_to_f32(sb[i] >> 16);
      acc += wgt[i] * (s * p + b * hsum[ch]);
    }
  }
  acc = quad_sum(acc);
  if (c4 == 0) red[wave][lane >> 5][row8] = acc;
  __syncthreads();
  if (threadIdx.x < 8) {
    const int r = threadIdx.x;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) v += red[w][0][r] + red[w][1][r];
    const int orow = tile * kRowTile + half * 8 + r;
    const uint16_t ob = f32_to_bf16_bits(v);
    out[orow] = ob;
    if (x_res != nullptr)
      x_res[orow] = f32_to_bf16_bits(bf16_bits_to_f32(x_res[orow]) + bf16_bits_to_f32(ob));
  }
}

template <int BITS>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t s) {
  const int nit = a.H / 256;
  const int rows = a.E + (a.has_shared ? 1 : 0);
#define MOE_A(N)                                                                               \
  case N:                                                                                      \
    if (a.dense != nullptr)                                                                    \
      hipLaunchKernelGGL((decode_router_kernel<N, true>), dim3(rows), dim3(64), 0, s, a.x_in,   \
                         a.x_hat, a.router_w, a.router_bias, a.shared_gate_w, a.dense,         \
                         a.dense_words, a.logits, a.H, a.E, a.eps, a.do_norm ? 1 : 0);         \
    else                                                                                       \
      hipLaunchKernelGGL((decode_router_kernel<N, false>), dim3(rows), dim3(64), 0, s, a.x_in,  \
                         a.x_hat, a.router_w, a.router_bias, a.shared_gate_w, a.dense,         \
                         a.dense_words, a.logits, a.H, a.E, a.eps, a.do_norm ? 1 : 0);         \
    break;
  switch (nit) {
    MOE_A(1) MOE_A(2) MOE_A(3) MOE_A(4) MOE_A(5) MOE_A(6) MOE_A(7) MOE_A(8)
    MOE_A(9) MOE_A(10) MOE_A(11) MOE_A(12) MOE_A(13) MOE_A(14) MOE_A(15) MOE_A(16)
    default: return hipErrorInvalidValue;
  }
#undef MOE_A
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int hsflag = a.has_shared ? 1 : 0;
  const int Is = a.has_shared ? a.Ls.inter : 0;
  const int tiles = max(a.L.n_tiles_gu, a.has_shared ? a.Ls.n_tiles_gu : 0);
  hipLaunchKernelGGL((decode_gateup_kernel<BITS>), dim3(tiles, a.k + hsflag), dim3(256), 0, s,
                     a.x_hat, a.logits, a.slab, a.slot_table, a.stride, a.shared_blob, a.idx, a.w,
                     a.gamma, a.slots, a.h, a.H, a.E, a.k, a.L.inter, Is, a.L.gu_unit, a.L.gu_tile,
                     a.Ls.gu_unit, a.Ls.gu_tile, hsflag);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int htot = a.k * a.L.inter + Is;
  const int cc = GuCfg<BITS>::CC;
  const size_t lds = sizeof(float) * (size_t)(htot / cc * (cc + 4) + htot / cc);
  hipLaunchKernelGGL((decode_down_kernel<BITS>), dim3(a.H / 8), dim3(256), lds, s, a.slots, a.w,
                     a.gamma, a.slab, a.stride, a.shared_blob, a.h, a.out, a.x_res,
                     a.H, a.k, a.L.inter, Is, a.L.d_off, a.L.d_unit, a.L.d_tile, a.Ls.d_off,
                     a.Ls.d_unit, a.Ls.d_tile, hsflag);
  return hipGetLastError();
}

}  // namespace

bool decode_fast_supported(int T, int act, int H, int k, int E, int bits, int I, int Is,
                           bool has_shared) {
  if (T != 1 || act != MOE_ACT_BF16) return false;
  if (H % 256 != 0 || H / 256 > 16) return false;
  const int kbc = kRowBytes * (8 / bits);
  if (H / kbc > 4 * kMaxKbPerWave) return false;
  const int n_units = k * (I / kbc) + (has_shared ? Is / kbc : 0);
  if (n_units > 8 * kMaxDownUnitsPerHalfWave) return false;
  const int htot = k * I + (has_shared ? Is : 0);
  const int cc = bits == 4 ? 32 : 16;
  if ((size_t)(htot / cc * (cc + 4) + htot / cc) * sizeof(float) > 60 * 1024) return false;
  (void)E;
  return true;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  return a.bits == 4 ? launch_decode_t<4>(a, s) : launch_decode_t<8>(a, s);
}

}  // namespace moe
