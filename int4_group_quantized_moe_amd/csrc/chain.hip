// Persistent batch-1 decode chain: every layer of the chain in ONE
// cooperative launch, one workgroup per compute unit.
//
// A layer needs three all-to-all exchanges (the full input before the
// router, the full logits before the top-k, every selected expert's full h
// before the down projection).  Kernel boundaries cost about as much as an
// in-kernel exchange plus a cold first load, so here the exchanges stay
// inside the kernel: each producer stores 64-bit words (epoch << 32 | payload)
// with relaxed device-scope atomics, each consumer polls them with relaxed
// device-scope atomic loads.  A word is its own ready flag (no fences, no
// counters, no contention).  The epoch is read from the workspace at start
// and advanced by workgroup 0 at the end, so graph replays never see stale
// words.  Every poll is bounded: on expiry an error bit is set and the
// workgroup carries on, so the grid always drains.
//
// Per layer l, workgroup w of NWG:
//   prefetch  router row(s) w + NWG*wave, the layer's slot table, the
//             shared expert's gate/up tiles and down units owned by w
//   A         x_l (layer 0: input buffer; else polled), RMSNorm, x_hat
//             staged for the gate/up dot products, router logits published
//   B         shared-expert gate/up tiles first; then the top-k of the
//             polled logits; the routed down units of phase C are issued;
//             routed gate/up tiles; h published
//   C         all h polled; down GEMV of 8 output rows over all selected
//             experts in a fixed order; residual add; x_{l+1} published
//
// Routing: top-k of E experts per token plus an always-active shared expert
// (page "Paquets Swiftlet 80B Qwen ..." on xix.ai, 4th paragraph); weights
// are MLX-style group-quantised int4/int8 (same page, last paragraph).
#include "decode_common.h"

namespace moe {
namespace {

using namespace dec;

constexpr uint32_t kSpinLimit = 1u << 18;
constexpr int kChainMaxExperts = 512;  // top-k over at most 8 logits per lane
template <int BITS>
constexpr int max_down_units() { return BITS == 4 ? 6 : 12; }  // per half-wave

__device__ __forceinline__ uint64_t ld_word(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_word(uint64_t* p, uint32_t ep, uint32_t payload) {
  __hip_atomic_store(p, ((uint64_t)ep << 32) | payload, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// Polls words [0, n) of `base` until each carries epoch `ep`; thread `tid`
// of a group of `gsize` threads handles words tid, tid + gsize, ...  All of a
// thread's loads of one batch are in flight together.  f(i, payload) is
// called once per word.
template <int NB, class F>
__device__ __forceinline__ void poll_words(const uint64_t* base, int n, int tid, int gsize,
                                           uint32_t ep, uint32_t* err, F&& f) {
  for (int b0 = 0; b0 < n; b0 += NB * gsize) {
    uint32_t pending = 0;
#pragma unroll
    for (int m = 0; m < NB; ++m)
      if (b0 + m * gsize + tid < n) pending |= 1u << m;
    uint64_t v[NB];
    uint32_t spins = 0;
    while (pending) {
#pragma unroll
      for (int m = 0; m < NB; ++m)
        if ((pending >> m) & 1u) v[m] = ld_word(base + b0 + m * gsize + tid);
#pragma unroll
      for (int m = 0; m < NB; ++m) {
        if (((pending >> m) & 1u) && (uint32_t)(v[m] >> 32) == ep) {
          f(b0 + m * gsize + tid, (uint32_t)v[m]);
          pending &= ~(1u << m);
        }
      }
      if (pending) {
        if (++spins > kSpinLimit) {
          atomicOr(err, 1u);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
  }
}

__device__ __forceinline__ float bf16r(float v) { return bf16_bits_to_f32(f32_to_bf16_bits(v)); }

__device__ __forceinline__ void st_u32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_u32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_u64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int BITS, int NIT>
__global__ __launch_bounds__(256, 1) void chain_kernel(ChainParams p) {
  using C = GuCfg<BITS>;
  constexpr int CC = C::CC, GPK = C::GPK, KBC = C::KBC, XS = C::XS, CP = CC + 4;
  constexpr int H = NIT * 256;
  constexpr int NKB = H / KBC;       // gate/up k-blocks
  constexpr int NKW = NKB / 4;       // k-blocks per wave
  constexpr int NCH = H / CC;        // staged activation chunks
  constexpr int kMaxDownUnits = max_down_units<BITS>();

  __shared__ __align__(16) float xs[H];
  __shared__ __align__(16) uint32_t xp[NCH * XS];
  __shared__ float2 cs[NCH];
  __shared__ float lg[kChainMaxExperts + 1];
  __shared__ int32_t slot_l[kChainMaxExperts];
  __shared__ int32_t sel_idx[MOE_MAX_TOP_K];
  __shared__ float sel_val[MOE_MAX_TOP_K], sel_w[MOE_MAX_TOP_K], gam;
  __shared__ __align__(16) uint32_t cand_key[64];
  __shared__ __align__(16) int32_t cand_idx[64];
  __shared__ float cand_val[64];
  __shared__ float red[4][kRowTile][2];
  __shared__ float dred[4][2][8];
  __shared__ float wsum[4];
  extern __shared__ float hs[];  // h chunks (CP floats each), then chunk sums

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int w = blockIdx.x, NWG = gridDim.x;
  const int E = p.E, k = p.k, I = p.I, Is = p.Is, L = p.L;
  const int hsh = p.has_shared;
  const uint32_t ep0 = p.ctr[0] + 1u;  // epoch of layer 0; layer l uses ep0 + l

  // phase B items: shared tiles first, then routed (j, tile)
  const int tiles_r = I / kRowTile, tiles_s = hsh ? Is / kRowTile : 0;
  const int NI = tiles_s + k * tiles_r;
  const int NH = k * I + (hsh ? Is : 0);      // h values per layer
  const int nchh = NH / CC;
  // phase C: half-tile w (8 output rows)
  const bool has_c = w < H / 8;
  const int ctile = w >> 1, chalf = w & 1;
  const int hw = wave * 2 + (lane >> 5), l32 = lane & 31;
  const int row8 = l32 >> 2, c4 = lane & 3;
  const int nkb_r = I / KBC, nkb_s = hsh ? Is / KBC : 0;
  const int n_units = k * nkb_r + nkb_s;
  const int dsb_off = kCodeBlockBytes + ((chalf * 8 + row8) * GPK + (c4 * CC) / kGroup) * 4;
  // gate/up lane geometry
  const int grow = lane >> 2;
  const int sbg_off = 2 * kCodeBlockBytes + (grow * GPK + (c4 * CC) / kGroup) * 4;
  const int sbu_off = sbg_off + kRowTile * GPK * 4;
  // router row of this wave
  const int my_row = w + NWG * wave;
  const bool has_row = my_row < E + hsh;

  uint4 qg[NKW], qu[NKW];
  uint32_t sg[NKW], su[NKW];
  uint4 dq[kMaxDownUnits];
  uint32_t dsb[kMaxDownUnits];
  float dw[kMaxDownUnits];

  auto issue_gu = [&](const uint8_t* blob, int tile, int64_t unit_b, int64_t tile_b) {
    const uint8_t* tb = blob + (int64_t)tile * tile_b;
#pragma unroll
    for (int i = 0; i < NKW; ++i) {
      const uint8_t* unit = tb + (int64_t)(wave + 4 * i) * unit_b;
      qg[i] = *reinterpret_cast<const uint4*>(unit + lane * 16);
      qu[i] = *reinterpret_cast<const uint4*>(unit + kCodeBlockBytes + lane * 16);
      sg[i] = *reinterpret_cast<const uint32_t*>(unit + sbg_off);
      su[i] = *reinterpret_cast<const uint32_t*>(unit + sbu_off);
    }
  };
  // gate/up of one 16-row tile from registers + staged x; h published
  // h exchange: one epoch-tagged word per h value
  auto compute_gu = [&](int64_t hoff, int item, uint32_t ep) {
    float g = 0.f, u = 0.f;
#pragma unroll
    for (int i = 0; i < NKW; ++i) {
      const int kb = wave + 4 * i;
      const int gc = kb * 4 + c4;
      const float2 c = cs[gc];
      float pg = 0.f, pu = 0.f;
      const uint32_t dg[4] = {qg[i].x, qg[i].y, qg[i].z, qg[i].w};
      const uint32_t du[4] = {qu[i].x, qu[i].y, qu[i].z, qu[i].w};
      if constexpr (BITS == 4) {
        const uint4* xq = reinterpret_cast<const uint4*>(xp + gc * XS);
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
        const uint4* xq = reinterpret_cast<const uint4*>(xp + gc * XS);
        const uint4 X0 = xq[0], X1 = xq[1];
        const uint32_t xv[8] = {X0.x, X0.y, X0.z, X0.w, X1.x, X1.y, X1.z, X1.w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          pg = dot2(__builtin_amdgcn_perm(0x64646464u, dg[m], 0x04010400u), xv[2 * m], pg);
          pg = dot2(__builtin_amdgcn_perm(0x64646464u, dg[m], 0x04030402u), xv[2 * m + 1], pg);
          pu = dot2(__builtin_amdgcn_perm(0x64646464u, du[m], 0x04010400u), xv[2 * m], pu);
          pu = dot2(__builtin_amdgcn_perm(0x64646464u, du[m], 0x04030402u), xv[2 * m + 1], pu);
        }
      }
      g += bf16_bits_to_f32(sg[i] & 0xFFFFu) * (pg - c.x) + bf16_bits_to_f32(sg[i] >> 16) * c.y;
      u += bf16_bits_to_f32(su[i] & 0xFFFFu) * (pu - c.x) + bf16_bits_to_f32(su[i] >> 16) * c.y;
    }
    g += __shfl_xor(g, 1, 64);
    g += __shfl_xor(g, 2, 64);
    u += __shfl_xor(u, 1, 64);
    u += __shfl_xor(u, 2, 64);
    if (c4 == 0) {
      red[wave][grow][0] = g;
      red[wave][grow][1] = u;
    }
    __syncthreads();
    if (tid < kRowTile) {
      const float gs = (red[0][tid][0] + red[1][tid][0]) + (red[2][tid][0] + red[3][tid][0]);
      const float us = (red[0][tid][1] + red[1][tid][1]) + (red[2][tid][1] + red[3][tid][1]);
      st_word(p.hw + hoff + tid, ep, __float_as_uint(silu_f32(gs) * us));
    }
    (void)item;
    __syncthreads();
  };

  for (int l = 0; l < L; ++l) {
    const uint32_t ep = ep0 + (uint32_t)l;
    const int32_t* st = p.slot_tables + (int64_t)l * E;
    const float* Wr = p.router_w + (int64_t)l * E * H;
    const uint8_t* sblob = p.shared_blobs + (int64_t)l * p.shared_stride;
    uint64_t* lwl = p.lw;

    // ---------------- prefetch (independent of x_l) ----------------
    float4 wr[NIT];
    float rbias = 0.f;
    if (has_row) {
      const float* rowp = my_row < E ? Wr + (int64_t)my_row * H
                                     : reinterpret_cast<const float*>(sblob + p.sg_off);
#pragma unroll
      for (int it = 0; it < NIT; ++it)
        wr[it] = *reinterpret_cast<const float4*>(rowp + it * 256 + lane * 4);
      if (my_row < E && p.router_bias != nullptr) rbias = p.router_bias[(int64_t)l * E + my_row];
    }
    int32_t slot_r[kChainMaxExperts / 256];
#pragma unroll
    for (int m = 0; m < kChainMaxExperts / 256; ++m)
      if (tid + 256 * m < E) slot_r[m] = st[tid + 256 * m];
    const int item0 = w, item1 = w + NWG;
    if (item0 < tiles_s) issue_gu(sblob, item0, p.gu_unit_s, p.gu_tile_s);
    if (has_c) {  // shared-expert down units of this half-tile
#pragma unroll
      for (int i = 0; i < kMaxDownUnits; ++i) {
        const int uidx = hw + 8 * i;
        if (uidx >= k * nkb_r && uidx < n_units) {
          const int kb = uidx - k * nkb_r;
          const uint8_t* unit = sblob + p.d_off_s + (int64_t)ctile * p.d_tile_s +
                                (int64_t)kb * p.d_unit_s;
          dq[i] = *reinterpret_cast<const uint4*>(unit + chalf * 512 + l32 * 16);
          dsb[i] = *reinterpret_cast<const uint32_t*>(unit + dsb_off);
        }
      }
    }

    // ---------------- A: input, RMSNorm, router ----------------
    {
      // thread tid owns words tid + 256 m (bf16 pairs 2i, 2i+1); its sum of
      // squares runs over them in a fixed order, so every workgroup gets
      // the same bits whatever order the words arrive in
      uint32_t xw4[H / 512];
      if (l == 0) {
#pragma unroll
        for (int m = 0; m < H / 512; ++m)
          xw4[m] = *reinterpret_cast<const uint32_t*>(p.x + 2 * (tid + 256 * m));
      } else {
        poll_words<H / 512>(p.xw, H / 2, tid, 256, ep - 1u, p.err,
                            [&](int i, uint32_t v) { xw4[(i - tid) >> 8] = v; });
      }
      float ss = 0.f;
#pragma unroll
      for (int m = 0; m < H / 512; ++m) {
        const int i = tid + 256 * m;
        const float a = bf16_bits_to_f32(xw4[m] & 0xFFFFu), b = bf16_bits_to_f32(xw4[m] >> 16);
        xs[2 * i] = a;
        xs[2 * i + 1] = b;
        ss += a * a + b * b;
      }
      ss = wave_sum_dpp(ss);
      if (lane == 0) wsum[wave] = ss;
    }
#pragma unroll
    for (int m = 0; m < kChainMaxExperts / 256; ++m)
      if (tid + 256 * m < E) slot_l[tid + 256 * m] = slot_r[m];
    __syncthreads();
    const float inv = 1.0f / sqrtf(((wsum[0] + wsum[1]) + (wsum[2] + wsum[3])) / (float)H + p.eps);
    // x_hat: stage for the gate/up dot products (4 threads per chunk, each
    // 8 columns for int4 / 4 for int8); block 0 stores it
    {
      constexpr int SUB = CC / 4;  // columns per thread
      for (int t = tid; t < NCH * 4; t += 256) {
        const int ch = t >> 2, jj = t & 3;
        const int c0 = ch * CC + jj * SUB;
        float xv[SUB];
#pragma unroll
        for (int q = 0; q < SUB; ++q) xv[q] = bf16r(xs[c0 + q] * inv);
        if (w == 0) {
#pragma unroll
          for (int q = 0; q < SUB; q += 2)
            *reinterpret_cast<uint32_t*>(p.x_hat + c0 + q) =
                (uint32_t)f32_to_bf16_bits(xv[q]) | ((uint32_t)f32_to_bf16_bits(xv[q + 1]) << 16);
        }
        float c, sx;
        if constexpr (BITS == 4) {
          const uint32_t pa = pack_f16x2(xv[0], xv[4]);
          const uint32_t pb = pack_f16x2(xv[1] * 0.0625f, xv[5] * 0.0625f);
          const uint32_t pc = pack_f16x2(xv[2], xv[6]);
          const uint32_t pf = pack_f16x2(xv[3] * 0.0625f, xv[7] * 0.0625f);
          *reinterpret_cast<uint4*>(xp + ch * XS + jj * 4) = make_uint4(pa, pb, pc, pf);
          c = f16lo(pa) + f16hi(pa) + f16lo(pb) + f16hi(pb) + f16lo(pc) + f16hi(pc) + f16lo(pf) +
              f16hi(pf);
          sx = f16lo(pa) + f16hi(pa) + f16lo(pc) + f16hi(pc) +
               16.0f * (f16lo(pb) + f16hi(pb) + f16lo(pf) + f16hi(pf));
        } else {
          const uint32_t p0 = pack_f16x2(xv[0], xv[1]), p1 = pack_f16x2(xv[2], xv[3]);
          *reinterpret_cast<uint2*>(xp + ch * XS + jj * 2) = make_uint2(p0, p1);
          c = f16lo(p0) + f16hi(p0) + f16lo(p1) + f16hi(p1);
          sx = c;
        }
        // combine the 4 threads of the chunk (adjacent lanes), fixed order
        c += __shfl_xor(c, 1, 64);
        c += __shfl_xor(c, 2, 64);
        sx += __shfl_xor(sx, 1, 64);
        sx += __shfl_xor(sx, 2, 64);
        if (jj == 0) cs[ch] = make_float2(1024.0f * c, sx);
      }
    }
    if (has_row) {
      float acc = 0.f;
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const float4 xv = *reinterpret_cast<const float4*>(xs + it * 256 + lane * 4);
        acc += wr[it].x * bf16r(xv.x * inv) + wr[it].y * bf16r(xv.y * inv) +
               wr[it].z * bf16r(xv.z * inv) + wr[it].w * bf16r(xv.w * inv);
      }
      acc = wave_sum_dpp(acc);
      if (lane == 0) st_word(lwl + my_row, ep, __float_as_uint(acc + rbias));
    }
    __syncthreads();

    // ---------------- B: shared tiles, top-k, routed tiles ----------------
    if (item0 < tiles_s) compute_gu((int64_t)k * I + item0 * kRowTile, item0, ep);
    if (wave == 0) {
      poll_words<(kChainMaxExperts + 64) / 64>(lwl, E + hsh, lane, 64, ep, p.err,
                                             [&](int i, uint32_t v) { lg[i] = __uint_as_float(v); });
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_s_waitcnt(0);
      wave_topk<kChainMaxExperts / 64>(lg, E, k, hsh != 0, sel_idx, sel_val, sel_w, &gam, cand_key,
                                       cand_idx, cand_val);
      if (w == 0) {
        if (lane < k) {
          p.r_idx[lane] = sel_idx[lane];
          p.r_w[lane] = sel_w[lane];
        }
        if (lane == 0 && hsh) *p.r_gamma = gam;
      }
    }
    __syncthreads();
    // routed gate/up tiles: loads of the first one go out before the down
    // units of phase C (needed later)
    int rj[2] = {-1, -1}, rt[2] = {0, 0};
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int item = s2 == 0 ? item0 : item1;
      if (item >= tiles_s && item < NI) {
        const int ii = item - tiles_s;
        rj[s2] = ii / tiles_r;
        rt[s2] = ii - rj[s2] * tiles_r;
      }
    }
    if (rj[0] >= 0)
      issue_gu(p.slab + (int64_t)slot_l[sel_idx[rj[0]]] * p.stride, rt[0], p.gu_unit_r,
               p.gu_tile_r);
    if (has_c) {  // routed down units of phase C
#pragma unroll
      for (int i = 0; i < kMaxDownUnits; ++i) {
        const int uidx = hw + 8 * i;
        if (uidx < k * nkb_r) {
          const int jj = uidx / nkb_r, kb = uidx - jj * nkb_r;
          const uint8_t* unit = p.slab + (int64_t)slot_l[sel_idx[jj]] * p.stride + p.d_off_r +
                                (int64_t)ctile * p.d_tile_r + (int64_t)kb * p.d_unit_r;
          dq[i] = *reinterpret_cast<const uint4*>(unit + chalf * 512 + l32 * 16);
          dsb[i] = *reinterpret_cast<const uint32_t*>(unit + dsb_off);
          dw[i] = sel_w[jj];
        } else if (uidx < n_units) {
          dw[i] = gam;
        }
      }
    }
    if (rj[0] >= 0) compute_gu((int64_t)rj[0] * I + rt[0] * kRowTile, item0, ep);
    if (rj[1] >= 0) {
      issue_gu(p.slab + (int64_t)slot_l[sel_idx[rj[1]]] * p.stride, rt[1], p.gu_unit_r,
               p.gu_tile_r);
      compute_gu((int64_t)rj[1] * I + rt[1] * kRowTile, item1, ep);
    } else if (item1 < tiles_s) {
      issue_gu(sblob, item1, p.gu_unit_s, p.gu_tile_s);
      compute_gu((int64_t)k * I + item1 * kRowTile, item1, ep);
    }

    // ---------------- C: down + combine + residual ----------------
    poll_words<24>(p.hw, NH, tid, 256, ep, p.err, [&](int i, uint32_t v) {
      const int ch = i / CC;
      hs[ch * CP + (i - ch * CC)] = __uint_as_float(v);
    });
    __syncthreads();
    if (has_c) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < kMaxDownUnits; ++i) {
        const int uidx = hw + 8 * i;
        if (uidx < n_units) {
          int hb, kb;
          if (uidx < k * nkb_r) {
            const int jj = uidx / nkb_r;
            kb = uidx - jj * nkb_r;
            hb = jj * I;
          } else {
            kb = uidx - k * nkb_r;
            hb = k * I;
          }
          const int ch = (hb + kb * KBC) / CC + c4;
          const float* hv = hs + ch * CP;
          const uint32_t d[4] = {dq[i].x, dq[i].y, dq[i].z, dq[i].w};
          float pp = 0.f, hsm = 0.f;
          if constexpr (BITS == 4) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
              const float4 a = *reinterpret_cast<const float4*>(hv + 8 * m);
              const float4 b = *reinterpret_cast<const float4*>(hv + 8 * m + 4);
              const uint32_t lo = d[m] & 0x0F0F0F0Fu, hi = (d[m] >> 4) & 0x0F0F0F0Fu;
              pp += (float)(lo & 0xFF) * a.x + (float)(hi & 0xFF) * a.y +
                    (float)((lo >> 8) & 0xFF) * a.z + (float)((hi >> 8) & 0xFF) * a.w +
                    (float)((lo >> 16) & 0xFF) * b.x + (float)((hi >> 16) & 0xFF) * b.y +
                    (float)(lo >> 24) * b.z + (float)(hi >> 24) * b.w;
              hsm += ((a.x + a.y) + (a.z + a.w)) + ((b.x + b.y) + (b.z + b.w));
            }
          } else {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
              const float4 a = *reinterpret_cast<const float4*>(hv + 4 * m);
              pp += (float)(d[m] & 0xFF) * a.x + (float)((d[m] >> 8) & 0xFF) * a.y +
                    (float)((d[m] >> 16) & 0xFF) * a.z + (float)(d[m] >> 24) * a.w;
              hsm += (a.x + a.y) + (a.z + a.w);
            }
          }
          const float sc = bf16_bits_to_f32(dsb[i] & 0xFFFFu), bi = bf16_bits_to_f32(dsb[i] >> 16);
          acc += dw[i] * (sc * pp + bi * hsm);
        }
      }
      acc += __shfl_xor(acc, 1, 64);
      acc += __shfl_xor(acc, 2, 64);
      if (c4 == 0) dred[wave][lane >> 5][row8] = acc;
    }
    __syncthreads();
    if (has_c && tid < 4) {
      uint32_t xb[2], ob[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int r = 2 * tid + q;
        float v = 0.f;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) v += dred[ww][0][r] + dred[ww][1][r];
        const int orow = ctile * kRowTile + chalf * 8 + r;
        ob[q] = f32_to_bf16_bits(v);
        xb[q] = f32_to_bf16_bits(xs[orow] + bf16_bits_to_f32(ob[q]));
      }
      const int orow0 = ctile * kRowTile + chalf * 8 + 2 * tid;
      if (l + 1 < L) {
        st_word(p.xw + orow0 / 2, ep, xb[0] | (xb[1] << 16));
      } else {
        *reinterpret_cast<uint32_t*>(p.x + orow0) = xb[0] | (xb[1] << 16);
        *reinterpret_cast<uint32_t*>(p.out + orow0) = ob[0] | (ob[1] << 16);
      }
    }
    __syncthreads();
  }
  if (w == 0 && tid == 0) p.ctr[0] = ep0 + (uint32_t)(L - 1);
}

int g_num_cus[16];

}  // namespace

int chain_grid(int device) {
  if (device < 0 || device >= 16) return 0;
  if (g_num_cus[device] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) return 0;
    g_num_cus[device] = prop.multiProcessorCount;
  }
  return g_num_cus[device];
}

bool chain_supported(int nwg, int T, int act, int H, int E, int k, int bits, int I, int Is,
                     bool has_shared) {
  if (T != 1 || act != MOE_ACT_BF16 || H != 2048 || bits != 4 || nwg < 1) return false;
  if (E > kChainMaxExperts) return false;
  const int kbc = kRowBytes * (8 / bits);
  if (E + (has_shared ? 1 : 0) > 4 * nwg) return false;
  const int NI = (has_shared ? Is / kRowTile : 0) + k * (I / kRowTile);
  if (NI > 2 * nwg || NI > 1024) return false;
  if (H / 8 > nwg) return false;
  const int n_units = k * (I / kbc) + (has_shared ? Is / kbc : 0);
  if (n_units > 8 * (bits == 4 ? max_down_units<4>() : max_down_units<8>())) return false;
  const int NH = k * I + (has_shared ? Is : 0);
  const int cc = bits == 4 ? 32 : 16;
  if ((size_t)(NH / cc * (cc + 4) + NH / cc) * sizeof(float) > 64 * 1024) return false;
  if (NH > 24 * 256 * 4) return false;
  return true;
}

size_t chain_lds_bytes(int bits, int NH) {
  const int cc = bits == 4 ? 32 : 16;
  return sizeof(float) * (size_t)(NH / cc * (cc + 4) + NH / cc);
}

hipError_t launch_chain(const ChainParams& prm, int nwg, hipStream_t s) {
  const int NH = prm.k * prm.I + (prm.has_shared ? prm.Is : 0);
  const size_t lds = chain_lds_bytes(prm.bits_, NH);
  void* args[] = {const_cast<ChainParams*>(&prm)};
  if (prm.bits_ != 4 || prm.H != 2048) return hipErrorInvalidValue;
  const void* fn = reinterpret_cast<const void*>(&chain_kernel<4, 8>);
  return hipLaunchCooperativeKernel(fn, dim3(nwg), dim3(256), args, (unsigned)lds, s);
}

}  // namespace moe
