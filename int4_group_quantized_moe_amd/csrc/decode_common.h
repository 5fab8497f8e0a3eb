// Device helpers shared by the decode kernels (three-kernel path and the
// persistent chain kernel): fp16 packing and dot products, DPP wave
// reductions, exact wave top-k, and the blob tiling constants.
#pragma once

#include "moe_internal.h"

namespace moe {
namespace dec {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c,
                                false);
}

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const _Float16 l = (_Float16)lo, h = (_Float16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, l) |
         ((uint32_t)__builtin_bit_cast(uint16_t, h) << 16);
}
__device__ __forceinline__ float f16lo(uint32_t p) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(p & 0xFFFFu));
}
__device__ __forceinline__ float f16hi(uint32_t p) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(p >> 16));
}

// DPP controls (gfx9): row_shr:n = 0x110+n, row_bcast:15 = 0x142, row_bcast:31 = 0x143.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f(float old, float src) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                               __builtin_bit_cast(int, src), CTRL,
                                                               ROW_MASK, 0xF, false));
}

// Sum over the 64 lanes, result returned in every lane.
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_f<0x111, 0xF>(0.0f, v);
  v += dpp_f<0x112, 0xF>(0.0f, v);
  v += dpp_f<0x114, 0xF>(0.0f, v);
  v += dpp_f<0x118, 0xF>(0.0f, v);
  v += dpp_f<0x142, 0xA>(0.0f, v);
  v += dpp_f<0x143, 0xC>(0.0f, v);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_u(uint32_t old, uint32_t src) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)src, CTRL, ROW_MASK, 0xF, false);
}

// Max over the 64 lanes (idempotent, so lanes without a DPP source keep
// their own value), result in every lane.
__device__ __forceinline__ uint32_t wave_max_dpp(uint32_t v) {
  v = max(v, dpp_u<0x111, 0xF>(v, v));
  v = max(v, dpp_u<0x112, 0xF>(v, v));
  v = max(v, dpp_u<0x114, 0xF>(v, v));
  v = max(v, dpp_u<0x118, 0xF>(v, v));
  v = max(v, dpp_u<0x142, 0xA>(v, v));
  v = max(v, dpp_u<0x143, 0xC>(v, v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Min over the 64 lanes, result in every lane.
__device__ __forceinline__ uint32_t wave_min_dpp(uint32_t v) {
  v = min(v, dpp_u<0x111, 0xF>(v, v));
  v = min(v, dpp_u<0x112, 0xF>(v, v));
  v = min(v, dpp_u<0x114, 0xF>(v, v));
  v = min(v, dpp_u<0x118, 0xF>(v, v));
  v = min(v, dpp_u<0x142, 0xA>(v, v));
  v = min(v, dpp_u<0x143, 0xC>(v, v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Waits for this wave's LDS operations only (vmcnt and expcnt left open).
__device__ __forceinline__ void lds_wave_sync() {
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ uint32_t mbcnt(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Monotonic map fp32 -> uint32 (larger value -> larger key); -0 maps as +0.
__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t b = __float_as_uint(v + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

constexpr int kMaxPerLane = MOE_MAX_EXPERTS / 64;

// Exact top-k of one token's E logits by one wave, ties to the lower index,
// ordered by logit descending; renormalised softmax weights over the k.
//   1. every lane keeps the max key of its logits; k rounds of a wave max
//      (removing the winning lanes) give tau <= the k-th largest lane
//      maximum, so at least k logits are >= tau and every top-k logit is;
//   2. the logits >= tau are compacted into LDS (usually about k of them);
//   3. each candidate's rank is counted against all candidates.
// More than 64 candidates (massive ties) take k rounds of wave argmax.
// Writes sel_idx[0..k), sel_w[0..k) and *gamma (if has_gate) in LDS.
template <int MPL = kMaxPerLane>
__device__ __forceinline__ void wave_topk(const float* __restrict__ logits, int E, int k, bool has_gate,
                          int32_t* sel_idx, float* sel_val, float* sel_w, float* gamma,
                          uint32_t* cand_key, int32_t* cand_idx, float* cand_val) {
  const int lane = threadIdx.x & 63;
  const int per = (E + 63) >> 6;
  float v[MPL];
  uint32_t u[MPL];
  uint32_t M = 0;
#pragma unroll
  for (int i = 0; i < MPL; ++i) {
    const int e = i * 64 + lane;
    const bool ok = i < per && e < E;
    v[i] = ok ? logits[e] : -INFINITY;
    u[i] = ok ? order_key(v[i]) : 0u;
    M = max(M, u[i]);
  }
  float gate_logit = 0.f;
  if (has_gate) gate_logit = logits[E];
  // 1. threshold on the lane maxima
  uint32_t tau = 0;
  {
    uint32_t Mr = M;
    for (int r = 0; r < k; ++r) {
      tau = wave_max_dpp(Mr);
      if (Mr == tau) Mr = 0u;
    }
  }
  // 2. compact the candidates
  uint32_t base = 0;
#pragma unroll
  for (int i = 0; i < MPL; ++i) {
    if (i < per) {
      const bool c = u[i] >= tau && (i * 64 + lane) < E;
      const uint64_t m = ballot(c);
      if (c) {
        const uint32_t pos = base + mbcnt(m);
        if (pos < 64) {
          cand_key[pos] = u[i];
          cand_idx[pos] = i * 64 + lane;
          cand_val[pos] = v[i];
        }
      }
      base += (uint32_t)__popcll(m);
    }
  }
  lds_wave_sync();
  const int ncand = (int)base;
  if (ncand <= 64) {
    // 3. rank among candidates (key descending, index ascending)
    if (lane < ncand) {
      const uint32_t K = cand_key[lane];
      const int I = cand_idx[lane];
      int rank = 0;
      for (int j0 = 0; j0 < ncand; j0 += 4) {
        const uint4 kk = *reinterpret_cast<const uint4*>(cand_key + j0);
        const int4 ii = *reinterpret_cast<const int4*>(cand_idx + j0);
        const uint32_t ks[4] = {kk.x, kk.y, kk.z, kk.w};
        const int is[4] = {ii.x, ii.y, ii.z, ii.w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
          rank += (j0 + q < ncand && (ks[q] > K || (ks[q] == K && is[q] < I))) ? 1 : 0;
      }
      if (rank < k) {
        sel_idx[rank] = I;
        sel_val[rank] = cand_val[lane];
      }
    }
  } else {
    // k rounds of (max key, lowest index) over the whole wave
    uint32_t taken = 0u;
    for (int r = 0; r < k; ++r) {
      uint32_t bk = 0;
      int bi = 0x7FFFFFFF;
#pragma unroll
      for (int i = 0; i < MPL; ++i) {
        const int e = i * 64 + lane;
        if (i < per && e < E && !((taken >> i) & 1u)) {
          if (u[i] > bk || (u[i] == bk && e < bi)) {
            bk = u[i];
            bi = e;
          }
        }
      }
      // wave max of bk, then min index among lanes holding it
      uint32_t mk = bk;
      for (int off = 32; off >= 1; off >>= 1) mk = max(mk, (uint32_t)__shfl_xor((int)mk, off, 64));
      int mi = (bk == mk) ? bi : 0x7FFFFFFF;
      for (int off = 32; off >= 1; off >>= 1) mi = min(mi, __shfl_xor(mi, off, 64));
      if ((mi & 63) == lane) {
        taken |= 1u << (mi >> 6);
        float sv = 0.f;
#pragma unroll
        for (int i = 0; i < MPL; ++i)
          if (i == (mi >> 6)) sv = v[i];
        sel_idx[r] = mi;
        sel_val[r] = sv;
      }
    }
  }
  lds_wave_sync();
  // renormalised softmax over the selected logits (fixed-order DPP sum)
  {
    const float l0 = sel_val[0];
    const float e = lane < k ? expf(sel_val[lane] - l0) : 0.0f;
    const float den = wave_sum_dpp(e);
    if (lane < k) sel_w[lane] = e / den;
  }
  if (lane == 0 && has_gate) *gamma = 1.0f / (1.0f + expf(-gate_logit));
  lds_wave_sync();
}


// The top-k SET of one token's E logits by one wave: the k experts with the
// largest logits, ties to the lower index, listed by ascending expert index
// (the order the decode chain lays out h in).  The weights are not needed to
// start loading the selected experts, so they come later (set_softmax).
//   1. every lane keeps the max key of its logits; tau = the k-th largest
//      of the 16 maxima of 4 adjacent lanes (k <= 16): the 16 maxima are
//      read into scalar registers, every lane counts those above its own,
//      and tau is the least group maximum with fewer than k above it (a
//      scalar minimum over the ballot of those groups).  At least k logits
//      are >= tau, and a logit below tau has k larger ones, so every top-k
//      logit is >= tau;
//   2. the logits >= tau are compacted into LDS in ascending index as
//      64-bit ranking words (order key << 32 | ~index: a larger word is a
//      larger logit, or an equal one with a lower index);
//   3. with exactly k candidates they are the set; otherwise each candidate
//      counts the words above its own, read 16 at a time as broadcast LDS
//      loads (unused slots hold 0, below every word), and those with fewer
//      than k above are the set, kept in ascending index.
// More than 64 candidates (massive ties) take k rounds of wave argmax.
// Writes set_idx[0..k), set_val[0..k) in LDS; cand[0..65) is LDS scratch
// (16-byte aligned).  on_sel(pos, idx) runs in the lane that writes
// set_idx[pos] = idx.
struct NoSel {
  __device__ void operator()(int, int) const {}
};
__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}
template <int MPL = kMaxPerLane, class OnSel = NoSel>
__device__ __forceinline__ void wave_topk_set(const float* __restrict__ logits, int E, int k,
                                              int32_t* set_idx, float* set_val, uint64_t* cand,
                                              OnSel on_sel = OnSel()) {
  static_assert(MOE_MAX_TOP_K <= 16, "the threshold takes the k-th of 16 group maxima");
  const int lane = threadIdx.x & 63;
  const int per = (E + 63) >> 6;
  uint32_t u[MPL];
  uint32_t M = 0;
#pragma unroll
  for (int i = 0; i < MPL; ++i) {
    const int e = i * 64 + lane;
    const bool ok = i < per && e < E;
    u[i] = ok ? order_key(logits[e]) : 0u;
    M = max(M, u[i]);
  }
  cand[lane] = 0ull;  // every slot below any ranking word
  // 1. tau = the k-th largest group maximum
  uint32_t g = max(M, dpp_u<0xB1, 0xF>(M, M));  // lane ^ 1
  g = max(g, dpp_u<0x4E, 0xF>(g, g));           // lane ^ 2
  uint32_t G[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) G[j] = (uint32_t)__builtin_amdgcn_readlane((int)g, 4 * j);
  uint32_t a[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < 16; ++j) a[j & 3] += G[j] > g ? 1u : 0u;
  const uint64_t below_k = ballot((a[0] + a[1]) + (a[2] + a[3]) < (uint32_t)k);
  uint32_t tau = 0xFFFFFFFFu;
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if ((below_k >> (4 * j)) & 1ull) tau = min(tau, G[j]);
  // 2. compact the candidates, ascending index; a lane that is not one
  //    writes to the spare slot 64
  uint64_t m[MPL];
  uint32_t base[MPL + 1];
  base[0] = 0u;
#pragma unroll
  for (int i = 0; i < MPL; ++i) {
    m[i] = ballot(i < per && u[i] >= tau && (i * 64 + lane) < E);
    base[i + 1] = base[i] + (i < per ? (uint32_t)__popcll(m[i]) : 0u);
  }
  const int ncand = (int)base[MPL];
  if (ncand <= 64) {
#pragma unroll
    for (int i = 0; i < MPL; ++i) {
      if (i < per) {
        const bool c = (m[i] >> lane) & 1ull;
        const uint32_t pos = c ? base[i] + mbcnt(m[i]) : 64u;
        cand[pos] = ((uint64_t)u[i] << 32) | (uint32_t)~(uint32_t)(i * 64 + lane);
      }
    }
    lds_wave_sync();
    // 3. the set: candidates ranked below k
    const uint64_t me = cand[lane];
    bool sel = lane < ncand;
    if (ncand > k) {
      uint32_t r[4] = {0u, 0u, 0u, 0u};
      for (int j0 = 0; j0 < ncand; j0 += 16) {
        const uint4* q = reinterpret_cast<const uint4*>(cand + j0);
        uint4 w[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) w[t] = q[t];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const uint64_t c0 = ((uint64_t)w[t].y << 32) | w[t].x;
          const uint64_t c1 = ((uint64_t)w[t].w << 32) | w[t].z;
          r[t & 3] += (c0 > me ? 1u : 0u) + (c1 > me ? 1u : 0u);
        }
      }
      sel = sel && (r[0] + r[1]) + (r[2] + r[3]) < (uint32_t)k;
    }
    const uint64_t ms = ballot(sel);
    if (sel) {
      const uint32_t pos = mbcnt(ms);
      const int I = (int)~(uint32_t)me;
      set_idx[pos] = I;
      set_val[pos] = key_value((uint32_t)(me >> 32));
      on_sel((int)pos, I);
    }
  } else {
    // k rounds of (max key, lowest index) over the whole wave; the winners
    // go to cand[0..k) in rank order as (key << 32 | index), then to set_*
    // by ascending index
    uint32_t taken = 0u;
    for (int r = 0; r < k; ++r) {
      uint32_t bk = 0;
      int bi = 0x7FFFFFFF;
#pragma unroll
      for (int i = 0; i < MPL; ++i) {
        const int e = i * 64 + lane;
        if (i < per && e < E && !((taken >> i) & 1u)) {
          if (u[i] > bk || (u[i] == bk && e < bi)) {
            bk = u[i];
            bi = e;
          }
        }
      }
      uint32_t mk = bk;
      for (int off = 32; off >= 1; off >>= 1) mk = max(mk, (uint32_t)__shfl_xor((int)mk, off, 64));
      int mi = (bk == mk) ? bi : 0x7FFFFFFF;
      for (int off = 32; off >= 1; off >>= 1) mi = min(mi, __shfl_xor(mi, off, 64));
      if ((mi & 63) == lane) {
        taken |= 1u << (mi >> 6);
        cand[r] = ((uint64_t)mk << 32) | (uint32_t)mi;
      }
    }
    lds_wave_sync();
    if (lane < k) {
      const uint64_t me = cand[lane];
      const int I = (int)(uint32_t)me;
      int pos = 0;
      for (int j = 0; j < k; ++j) pos += (int)(uint32_t)cand[j] < I ? 1 : 0;
      set_idx[pos] = I;
      set_val[pos] = key_value((uint32_t)(me >> 32));
      on_sel(pos, I);
    }
  }
  lds_wave_sync();
}

// Renormalised softmax over the k selected logits set_val[0..k) (max
// subtracted, fixed-order DPP sum); weights in the same order.
__device__ __forceinline__ void set_softmax(const float* set_val, int k, float* set_w) {
  const int lane = threadIdx.x & 63;
  const float x = lane < k ? set_val[lane] : -INFINITY;
  const uint32_t mk = wave_max_dpp(lane < k ? order_key(x) : 0u);
  const float xmax = __uint_as_float((mk & 0x80000000u) ? (mk & 0x7FFFFFFFu) : ~mk);
  const float e = lane < k ? expf(x - xmax) : 0.0f;
  const float den = wave_sum_dpp(e);
  if (lane < k) set_w[lane] = e / den;
  lds_wave_sync();
}

// Writes the set in routing order (logit descending, ties to the lower
// index): idx_out[r], w_out[r] for r < k.
__device__ __forceinline__ void set_rank_out(const int32_t* set_idx, const float* set_val,
                                             const float* set_w, int k, int32_t* idx_out,
                                             float* w_out) {
  const int lane = threadIdx.x & 63;
  if (lane < k) {
    const uint32_t K = order_key(set_val[lane]);
    const int I = set_idx[lane];
    int rank = 0;
    for (int j = 0; j < k; ++j) {
      const uint32_t Kj = order_key(set_val[j]);
      rank += (Kj > K || (Kj == K && set_idx[j] < I)) ? 1 : 0;
    }
    idx_out[rank] = I;
    w_out[rank] = set_w[lane];
  }
}

template <int BITS>
struct GuCfg {
  static constexpr int CC = BITS == 4 ? 32 : 16;  // columns per lane chunk
  static constexpr int GPK = BITS == 4 ? 2 : 1;
  static constexpr int KBC = kRowBytes * (8 / BITS);
  // staged activation dwords per chunk, padded so the 4 chunks a wave reads
  // at once fall in distinct LDS banks
  static constexpr int XS = BITS == 4 ? 20 : 8;
};

constexpr int kMaxKbPerWave = 8;

}  // namespace dec
}  // namespace moe
