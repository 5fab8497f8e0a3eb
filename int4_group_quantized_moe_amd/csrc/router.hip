// Router GEMV, shared-gate logit, and wavefront softmax / top-k / renormalise.
//
// Routing of every token to the top-k of E experts by a resident router
// (page "Paquets Swiftlet 80B Qwen ..." on xix.ai, 4th paragraph: 10 of 512
// or 8 of 256 experts per layer and token; the routers stay resident).
// Renormalised top-k weights equal the softmax over the k selected logits,
// so the E-way softmax sum is never formed.
#include "decode_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRouterWaves = 4;     // rows per workgroup (one per wave)
constexpr int kRouterMaxTT = 8;     // tokens per LDS chunk
constexpr int kRouterMaxRegIt = 8;  // row cached in registers when H <= 64*4*8
constexpr int kRouterMaxPlanes = 16;      // K split of the router GEMM (logit planes)
constexpr int kRouterFoldMaxBlocks = 256;  // router GEMM grid that still runs in one round

template <int ACT>
__device__ __forceinline__ float4 load_act4(const void* p, int64_t i) {
  if constexpr (ACT == MOE_ACT_F32) {
    return *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p) + i);
  } else {
    const uint2 v = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(p) + i);
    return make_float4(bf16_bits_to_f32(v.x & 0xFFFFu), bf16_bits_to_f32(v.x >> 16),
                       bf16_bits_to_f32(v.y & 0xFFFFu), bf16_bits_to_f32(v.y >> 16));
  }
}

// logits[t][r] = sum_c W[r][c] * x[t][c] (+ bias[r]) for rows r < E, and the
// shared-gate logit w_sg . x[t] as row E when w_sg is given.
template <int ACT, int NIT>
__global__ __launch_bounds__(256) void router_gemv_kernel(const void* __restrict__ x,
                                                          const float* __restrict__ W,
                                                          const float* __restrict__ bias,
                                                          const float* __restrict__ wsg,
                                                          float* __restrict__ logits, int T, int H,
                                                          int E, int TT) {
  extern __shared__ float xs[];  // [TT][H]
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = blockIdx.x * kRouterWaves + wave;
  const int R = E + (wsg != nullptr ? 1 : 0);
  const bool active = r < R;
  const float* wrow = nullptr;
  if (active) wrow = (r < E) ? W + (int64_t)r * H : wsg;
  const int nit = (H + 255) / 256;

  float4 wreg[NIT > 0 ? NIT : 1];
  if constexpr (NIT > 0) {
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int c = it * 256 + lane * 4;
      wreg[it] = (active && c < H) ? *reinterpret_cast<const float4*>(wrow + c)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  const float b = (active && r < E && bias != nullptr) ? bias[r] : 0.0f;

  // token chunks of TT are spread over blockIdx.y (strided when there are
  // more chunks than workgroup rows)
  for (int t0 = blockIdx.y * TT; t0 < T; t0 += gridDim.y * TT) {
    const int tt_n = min(TT, T - t0);
    __syncthreads();
    // stage the chunk's rows (contiguous in x): 4 values per thread and
    // iteration, all loads of a thread issued before its LDS stores
    {
      const int n4 = tt_n * H / 4;
      constexpr int kU = 8;
      for (int i0 = 0; i0 < n4; i0 += kU * 256) {
        float4 v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int i = i0 + u * 256 + threadIdx.x;
          if (i < n4) v[u] = load_act4<ACT>(x, (int64_t)t0 * H + 4 * (int64_t)i);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int i = i0 + u * 256 + threadIdx.x;
          if (i < n4) reinterpret_cast<float4*>(xs)[i] = v[u];
        }
      }
    }
    __syncthreads();
    if (!active) continue;
    float acc[kRouterMaxTT];
#pragma unroll
    for (int tt = 0; tt < kRouterMaxTT; ++tt) acc[tt] = 0.0f;
    if constexpr (NIT > 0) {
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int c = it * 256 + lane * 4;
        if (c < H) {
#pragma unroll
          for (int tt = 0; tt < kRouterMaxTT; ++tt) {
            if (tt < tt_n) {
              const float4 xv = *reinterpret_cast<const float4*>(xs + tt * H + c);
              acc[tt] += wreg[it].x * xv.x + wreg[it].y * xv.y + wreg[it].z * xv.z +
                         wreg[it].w * xv.w;
            }
          }
        }
      }
    } else {
      for (int it = 0; it < nit; ++it) {
        const int c = it * 256 + lane * 4;
        if (c < H) {
          const float4 wv = *reinterpret_cast<const float4*>(wrow + c);
#pragma unroll
          for (int tt = 0; tt < kRouterMaxTT; ++tt) {
            if (tt < tt_n) {
              const float4 xv = *reinterpret_cast<const float4*>(xs + tt * H + c);
              acc[tt] += wv.x * xv.x + wv.y * xv.y + wv.z * xv.z + wv.w * xv.w;
            }
          }
        }
      }
    }
#pragma unroll
    for (int tt = 0; tt < kRouterMaxTT; ++tt) {
      if (tt < tt_n) {
        const float s = warp_sum(acc[tt]);
        if (lane == 0) logits[(int64_t)(t0 + tt) * (E + 1) + r] = s + b;
      }
    }
  }
}

// Top-k of token t by one wave: the exact wavefront top-k (threshold from
// DPP wave maxima, ballot compaction, rank; k rounds of argmax when more than
// 64 logits tie at the threshold), then the softmax over the k selected
// logits.  The LDS arrays are the wave's own.  With x16, the wave also writes
// the token's activation row in fp16 (x16_row).
template <int MPL, int NP>
__device__ __forceinline__ void topk_token(const float* __restrict__ logits, int32_t* __restrict__ topk_idx,
                                           float* __restrict__ topk_w, float* __restrict__ gamma,
                                           int T, int E, int k, int has_gate, int nplanes, int t,
                                           int32_t* sel_idx, float* sel_val, float* sel_w,
                                           float* gam, uint32_t* cand_key, int32_t* cand_idx,
                                           float* cand_val, float* lsum,
                                           const uint16_t* __restrict__ xsrc,
                                           uint16_t* __restrict__ x16, int32_t* __restrict__ xe,
                                           int H, int x16_bits,
                                           const float* __restrict__ gate_w) {
  const int lane = threadIdx.x & 63;
  const float* lt = logits + (int64_t)t * (E + 1);
  // with gate_w (bf16 activations, logits in planes): the shared-gate logit
  // w_sg . x[t] here, 8 consecutive columns per lane and step, instead of
  // row E of the planes
  float gacc = 0.f;
  if (gate_w != nullptr) {
    const uint16_t* xr = xsrc + (int64_t)t * H;
#pragma unroll 4
    for (int c = 8 * lane; c < H; c += 512) {
      const uint4 xv = *reinterpret_cast<const uint4*>(xr + c);
      const float4 w0 = *reinterpret_cast<const float4*>(gate_w + c);
      const float4 w1 = *reinterpret_cast<const float4*>(gate_w + c + 4);
      gacc += bf16_bits_to_f32(xv.x & 0xFFFFu) * w0.x + bf16_bits_to_f32(xv.x >> 16) * w0.y +
              bf16_bits_to_f32(xv.y & 0xFFFFu) * w0.z + bf16_bits_to_f32(xv.y >> 16) * w0.w +
              bf16_bits_to_f32(xv.z & 0xFFFFu) * w1.x + bf16_bits_to_f32(xv.z >> 16) * w1.y +
              bf16_bits_to_f32(xv.w & 0xFFFFu) * w1.z + bf16_bits_to_f32(xv.w >> 16) * w1.w;
    }
  }
  if (nplanes > 1) {
    // logits split over K planes: add them in plane order (row E, the
    // shared-gate logit, too: a partial per plane, or the whole logit in
    // plane 0 and zeros in the others)
    // (every load of the token's E + 1 logits over the planes in flight
    // together: MPL * 64 + 1 >= E + 1 entries per lane group; the loads are
    // unconditional, past the last plane or logit at a clamped index and not
    // used, so that none waits for the one before it)
    const int64_t ps = (int64_t)T * (E + 1);
    float p[NP][MPL + 1];
#pragma unroll
    for (int z = 0; z < NP; ++z)
#pragma unroll
      for (int m = 0; m <= MPL; ++m)
        p[z][m] = lt[min(z, nplanes - 1) * ps + min(lane + 64 * m, E)];
    float v[MPL + 1];
#pragma unroll
    for (int m = 0; m <= MPL; ++m) {
      const bool ok = lane + 64 * m <= E;
      v[m] = ok ? p[0][m] : 0.f;
#pragma unroll
      for (int z = 1; z < NP; ++z)
        if (z < nplanes && ok) v[m] = v[m] + p[z][m];
    }
#pragma unroll
    for (int m = 0; m <= MPL; ++m) {
      const int e = lane + 64 * m;
      if (e <= E) lsum[e] = v[m];
    }
    if (gate_w != nullptr) {
      gacc = warp_sum(gacc);
      if (lane == 0) lsum[E] = gacc;  // (after the planes' row E above)
    }
    dec::lds_wave_sync();
    lt = lsum;
  }
  dec::wave_topk<MPL>(lt, E, k, has_gate != 0, sel_idx, sel_val, sel_w, gam, cand_key, cand_idx,
                      cand_val);
  if (lane < k) {
    topk_idx[(int64_t)t * k + lane] = sel_idx[lane];
    topk_w[(int64_t)t * k + lane] = sel_w[lane];
  }
  if (lane == 0 && has_gate && gamma != nullptr) gamma[t] = *gam;
  // the token's activation row in fp16 for the one-token-block grouped GEMMs
  if (x16 != nullptr)
    x16_row(xsrc + (int64_t)t * H, x16 + (int64_t)t * H, xe + t, H, x16_bits);
  dec::lds_wave_sync();  // the wave's LDS may be reused for its next token
}

// One wave per token.
// NP: the most logit planes of a call (nplanes <= NP).
template <int MPL, int NP>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits,
                                                   int32_t* __restrict__ topk_idx,
                                                   float* __restrict__ topk_w,
                                                   float* __restrict__ gamma, int T, int E,
                                                   int k, int has_gate, int nplanes,
                                                   const uint16_t* __restrict__ xsrc,
                                                   uint16_t* __restrict__ x16,
                                                   int32_t* __restrict__ xe, int H, int x16_bits,
                                                   const float* __restrict__ gate_w) {
  __shared__ int32_t sel_idx[4][MOE_MAX_TOP_K];
  __shared__ float sel_val[4][MOE_MAX_TOP_K], sel_w[4][MOE_MAX_TOP_K], gam[4];
  __shared__ __align__(16) uint32_t cand_key[4][64];
  __shared__ __align__(16) int32_t cand_idx[4][64];
  __shared__ float cand_val[4][64];
  __shared__ float lsum[4][MPL * 64 + 1];
  const int wave = threadIdx.x >> 6;
  const int t = blockIdx.x * (int)(blockDim.x >> 6) + wave;
  if (t >= T) return;
  topk_token<MPL, NP>(logits, topk_idx, topk_w, gamma, T, E, k, has_gate, nplanes, t, sel_idx[wave],
                  sel_val[wave], sel_w[wave], &gam[wave], cand_key[wave], cand_idx[wave],
                  cand_val[wave], lsum[wave], xsrc, x16, xe, H, x16_bits, gate_w);
}

hipError_t launch_topk(const RouterArgs& a, hipStream_t s, int nplanes, const float* gate_w) {
  // one wave per token; small batches one wave per workgroup, so that the
  // tokens' logit loads spread over more compute units
  const int wpb = a.T <= 1024 ? 1 : 4;
  const dim3 grid((a.T + wpb - 1) / wpb), block(64 * wpb);
  const int hg = a.shared_gate_w ? 1 : 0;
  const uint16_t* xs = reinterpret_cast<const uint16_t*>(a.x);
  if (nplanes > kRouterMaxPlanes) return hipErrorInvalidValue;
  // every plane load of a token is issued, so the bound follows the call's planes
  const int np = nplanes <= 2 ? 2 : (nplanes <= 8 ? 8 : kRouterMaxPlanes);
#define MOE_TOPK(MPL, NP)                                                                      \
  hipLaunchKernelGGL((topk_kernel<MPL, NP>), grid, block, 0, s, a.logits, a.topk_idx, a.topk_w, \
                     a.gamma, a.T, a.E, a.k, hg, nplanes, xs, a.x16, a.xe, a.H, a.x16_bits, gate_w)
#define MOE_TOPK_NP(MPL)      \
  if (np == 2)                \
    MOE_TOPK(MPL, 2);         \
  else if (np == 8)           \
    MOE_TOPK(MPL, 8);         \
  else                        \
    MOE_TOPK(MPL, kRouterMaxPlanes)
  if (a.E <= 256) {
    MOE_TOPK_NP(4);
  } else if (a.E <= 512) {
    MOE_TOPK_NP(8);
  } else {
    MOE_TOPK_NP(16);
  }
#undef MOE_TOPK_NP
#undef MOE_TOPK
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Large batches: the router as a GEMM on the matrix cores.  logits[t][e] for
// e < E, and the shared-gate logit w_sg . x[t] as row E when wsg is given,
// over 64-token x 64-row tiles (4 waves, one 32x32 block each),
// K staged 64 at a time.  Each fp32 router weight is split exactly into three
// bf16 parts (8 significant bits each: w = w1 + w2 + w3, by truncation), so
// that with bf16 activations every product is exact and only the fp32
// accumulation rounds, as in the fp32 GEMV.

typedef __bf16 rbf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t ru32x4 __attribute__((ext_vector_type(4)));
typedef float rf32x16 __attribute__((ext_vector_type(16)));

constexpr int kRouterTile = 64;
constexpr int kRouterLdsRow = 72;  // 64 K columns + 8 bf16 padding
constexpr int kRouterDepth = 4;    // K stages in flight per thread

__device__ __forceinline__ void split3_pair(float a, float b, uint32_t& p1, uint32_t& p2,
                                            uint32_t& p3) {
  const uint32_t ua = __float_as_uint(a) & 0xFFFF0000u, ub = __float_as_uint(b) & 0xFFFF0000u;
  const float ra = a - __uint_as_float(ua), rb = b - __uint_as_float(ub);
  const uint32_t va = __float_as_uint(ra) & 0xFFFF0000u, vb = __float_as_uint(rb) & 0xFFFF0000u;
  const float sa = ra - __uint_as_float(va), sb = rb - __uint_as_float(vb);
  p1 = (ua >> 16) | ub;
  p2 = (va >> 16) | vb;
  p3 = (__float_as_uint(sa) >> 16) | (__float_as_uint(sb) & 0xFFFF0000u);
}

// blockIdx.z splits K: split z sums columns [z*kseg, (z+1)*kseg) into its
// own logit plane (logits + z*T*(E+1)); the top-k kernel adds the planes.
// Both operands pass through LDS: the token rows as bf16, the weight rows
// as their three bf16 parts, split once per workgroup while staging (each
// row read by coalesced 16-byte loads, 16 lanes per 256-byte row piece).
// D: K stages in flight (a divisor of kseg / 64, at most kRouterDepth).
template <int D>
__global__ __launch_bounds__(256) void router_mfma_kernel(const uint16_t* __restrict__ x,
                                                          const float* __restrict__ W,
                                                          const float* __restrict__ bias,
                                                          const float* __restrict__ wsg,
                                                          float* __restrict__ logits,
                                                          int T, int H,
                                                          int E, int kseg) {
  constexpr int kTileElems = kRouterTile * kRouterLdsRow;
  __shared__ __align__(16) uint16_t A[2 * kTileElems];      // token rows, two stages
  __shared__ __align__(16) uint16_t Bp[2 * 3 * kTileElems];  // weight parts, two stages
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31, half = lane >> 5;
  const int t0 = blockIdx.y * kRouterTile, e0 = blockIdx.x * kRouterTile;
  const int k0 = blockIdx.z * kseg;
  logits += (int64_t)blockIdx.z * T * (E + 1);
  // token staging: row sr, 16 columns (2 x 16 bytes) per thread
  const int sr = tid >> 2, sq = tid & 3;
  const bool srow_ok = t0 + sr < T;
  const uint16_t* xrow = x + (int64_t)(srow_ok ? t0 + sr : 0) * H + k0 + 16 * sq;
  // weight staging: rows 16 j + (tid >> 4) (j = 0..3), 4 columns at 4 (tid & 15);
  // row E is the shared-gate vector when it rides in the GEMM, rows past it zeros
  const int wc = 4 * (tid & 15);
  const float* wrow[4];
  bool w_ok[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = e0 + 16 * j + (tid >> 4);
    const bool gate_row = e == E && wsg != nullptr;
    w_ok[j] = e < E || gate_row;
    wrow[j] = (gate_row ? wsg : W + (int64_t)(e < E ? e : 0) * H) + k0 + wc;
  }
  const int S = kseg / 64;

  // every load unconditional (rows past the tile read row 0 and are zeroed)
  auto load_stage = [&](int st, uint4 (&ra)[2], float4 (&rb)[4]) {
#pragma unroll
    for (int q = 0; q < 2; ++q) ra[q] = reinterpret_cast<const uint4*>(xrow + st * 64)[q];
#pragma unroll
    for (int j = 0; j < 4; ++j) rb[j] = *reinterpret_cast<const float4*>(wrow[j] + st * 64);
  };
  auto store_stage = [&](int buf, const uint4 (&ra)[2], const float4 (&rb)[4]) {
    uint16_t* dst = A + buf * kTileElems + sr * kRouterLdsRow + 16 * sq;
#pragma unroll
    for (int q = 0; q < 2; ++q)
      *reinterpret_cast<uint4*>(dst + 8 * q) = srow_ok ? ra[q] : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 v = w_ok[j] ? rb[j] : make_float4(0.f, 0.f, 0.f, 0.f);
      uint32_t p1[2], p2[2], p3[2];
      split3_pair(v.x, v.y, p1[0], p2[0], p3[0]);
      split3_pair(v.z, v.w, p1[1], p2[1], p3[1]);
      const int o = buf * 3 * kTileElems + (16 * j + (tid >> 4)) * kRouterLdsRow + wc;
      *reinterpret_cast<uint2*>(Bp + o) = make_uint2(p1[0], p1[1]);
      *reinterpret_cast<uint2*>(Bp + o + kTileElems) = make_uint2(p2[0], p2[1]);
      *reinterpret_cast<uint2*>(Bp + o + 2 * kTileElems) = make_uint2(p3[0], p3[1]);
    }
  };
  // one stage of products, the weights' three bf16 parts smallest first
  rf32x16 acc = {};
  auto multiply = [&](int buf) {
    const uint16_t* As = A + buf * kTileElems + (32 * wm + l32) * kRouterLdsRow + 32 * half;
    const uint16_t* Bs = Bp + buf * 3 * kTileElems + (32 * wn + l32) * kRouterLdsRow + 32 * half;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const rbf16x8 av = __builtin_bit_cast(rbf16x8, *reinterpret_cast<const ru32x4*>(As + 8 * ks));
      const rbf16x8 b1 =
          __builtin_bit_cast(rbf16x8, *reinterpret_cast<const ru32x4*>(Bs + 8 * ks));
      const rbf16x8 b2 =
          __builtin_bit_cast(rbf16x8, *reinterpret_cast<const ru32x4*>(Bs + kTileElems + 8 * ks));
      const rbf16x8 b3 = __builtin_bit_cast(
          rbf16x8, *reinterpret_cast<const ru32x4*>(Bs + 2 * kTileElems + 8 * ks));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b3, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b2, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b1, acc, 0, 0, 0);
    }
  };

  // a ring of D stages in registers: stage st is multiplied from LDS while
  // stages st + 1 .. st + D are in flight (its registers were written to LDS
  // one step earlier, so they take stage st + D at once), and stage st + 1 is
  // split into the other LDS buffer.  No load or store sits under a branch, so
  // each step waits only for the stage it stores: past the last stage the
  // indices are clamped and the extra copies go unused.
  {
    uint4 ra[D][2];
    float4 rb[D][4];
#pragma unroll
    for (int j = 0; j < D; ++j) load_stage(j, ra[j], rb[j]);
    store_stage(0, ra[0], rb[0]);
    __syncthreads();
    for (int st0 = 0; st0 < S; st0 += D) {
#pragma unroll
      for (int j = 0; j < D; ++j) {
        const int st = st0 + j;
        load_stage(min(st + D, S - 1), ra[j], rb[j]);
        multiply(st & 1);
        store_stage((st + 1) & 1, ra[(j + 1) % D], rb[(j + 1) % D]);
        __syncthreads();
      }
    }
  }
  const int e = e0 + 32 * wn + l32;
  if (!(e < E || (e == E && wsg != nullptr))) return;
  const float b = (bias != nullptr && blockIdx.z == 0 && e < E) ? bias[e] : 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int t = t0 + 32 * wm + 8 * (r / 4) + 4 * half + (r % 4);
    if (t < T) logits[(int64_t)t * (E + 1) + e] = acc[r] + b;
  }
}

// Shared-gate logit w_sg . x[t] (row E of plane 0 of the logits; row E of
// the other planes is zeroed, as the top-k adds the planes), one wave per
// token.  Used where folding w_sg into the router GEMM as row E would cost
// the GEMM another round of workgroups.
template <int ACT>
__global__ __launch_bounds__(256) void gate_logit_kernel(const void* __restrict__ x,
                                                         const float* __restrict__ wsg,
                                                         float* __restrict__ logits, int T, int H,
                                                         int E, int nplanes) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  // 4 consecutive columns per lane and step, loads of a few steps in flight
  float acc = 0.f;
  constexpr int kU = 4;
  for (int c0 = 4 * lane; c0 < H; c0 += 256 * kU) {
    float4 xv[kU], wv[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int c = c0 + 256 * u;
      const bool ok = c < H;
      xv[u] = ok ? load_act4<ACT>(x, (int64_t)t * H + c) : make_float4(0.f, 0.f, 0.f, 0.f);
      wv[u] = ok ? *reinterpret_cast<const float4*>(wsg + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
      acc += wv[u].x * xv[u].x + wv[u].y * xv[u].y + wv[u].z * xv[u].z + wv[u].w * xv[u].w;
  }
  acc = warp_sum(acc);
  if (lane == 0) logits[(int64_t)t * (E + 1) + E] = acc;
  if (lane > 0 && lane < nplanes) logits[((int64_t)lane * T + t) * (E + 1) + E] = 0.f;
}

template <int ACT>
hipError_t launch_router_gemv(const RouterArgs& a, hipStream_t s);

template <int ACT>
hipError_t launch_router_act(const RouterArgs& a, hipStream_t s) {
  int nplanes = 1;
  const float* gate_in_topk = nullptr;  // the shared-gate logit taken by the top-k kernel
  if (router_uses_mfma(a.act, a.T, a.H)) {
    // split K so that the grid fills the chip at two workgroups per CU (a
    // workgroup's split-weight work then overlaps the other's MFMAs; at most
    // the planes the workspace holds)
    const int tiles = ((a.E + kRouterTile - 1) / kRouterTile) * ((a.T + kRouterTile - 1) / kRouterTile);
    const int maxp = router_planes(a.T);
    while (nplanes < maxp && tiles * nplanes < 512 && (a.H / 64) % (2 * nplanes) == 0) nplanes *= 2;
    // the shared-gate vector rides as row E of the GEMM when that costs no
    // extra round of workgroups (a free row in the last tile, or the grid
    // still within one workgroup per CU); else its own small kernel
    const int etiles = (a.E + kRouterTile - 1) / kRouterTile;
    const int gtiles = (a.E + 1 + kRouterTile - 1) / kRouterTile;
    const int ytiles = (a.T + kRouterTile - 1) / kRouterTile;
    const bool fold = a.shared_gate_w != nullptr &&
                      (gtiles == etiles || gtiles * ytiles * nplanes <= kRouterFoldMaxBlocks);
    const dim3 grid(fold ? gtiles : etiles, ytiles, nplanes);
    const uint16_t* xb = reinterpret_cast<const uint16_t*>(a.x);
    const float* wg = fold ? a.shared_gate_w : nullptr;
    // K stages of each split; the stage ring is the largest of 4, 2, 1 dividing it
    const int S = a.H / nplanes / 64;
    static_assert(kRouterDepth == 4, "stage rings of 4, 2 and 1");
#define MOE_ROUTER_GEMM(D)                                                                   \
  hipLaunchKernelGGL(router_mfma_kernel<D>, grid, dim3(256), 0, s, xb, a.router_w,            \
                     a.router_bias, wg, a.logits, a.T, a.H, a.E, a.H / nplanes)
    if (S % 4 == 0)
      MOE_ROUTER_GEMM(4);
    else if (S % 2 == 0)
      MOE_ROUTER_GEMM(2);
    else
      MOE_ROUTER_GEMM(1);
#undef MOE_ROUTER_GEMM
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.shared_gate_w != nullptr && !fold) {
      // bf16 rows over several planes: the top-k kernel reads each token's
      // row anyway and writes the logit where it ranks; else its own kernel
      if (ACT == MOE_ACT_BF16 && nplanes > 1) {
        gate_in_topk = a.shared_gate_w;
      } else {
        hipLaunchKernelGGL((gate_logit_kernel<ACT>), dim3((a.T + 3) / 4), dim3(256), 0, s, a.x,
                           a.shared_gate_w, a.logits, a.T, a.H, a.E, nplanes);
        if ((e = hipGetLastError()) != hipSuccess) return e;
      }
    }
  } else {
    hipError_t e = launch_router_gemv<ACT>(a, s);
    if (e != hipSuccess) return e;
  }
  return launch_topk(a, s, nplanes, gate_in_topk);
}

template <int ACT>
hipError_t launch_router_gemv(const RouterArgs& a, hipStream_t s) {
  const int R = a.E + (a.shared_gate_w ? 1 : 0);
  const int TT = max(1, min(min(a.T, kRouterMaxTT), 16384 / a.H));
  const size_t lds = sizeof(float) * (size_t)TT * a.H;
  const int nchunk = (a.T + TT - 1) / TT;
  const int rblk = (R + kRouterWaves - 1) / kRouterWaves;
  const dim3 grid(rblk, max(1, min(nchunk, 4096 / rblk)));
  const int nit = (a.H + 255) / 256;
#define MOE_ROUTER_CASE(N)                                                                 \
  case N:                                                                                  \
    hipLaunchKernelGGL((router_gemv_kernel<ACT, N>), grid, dim3(256), lds, s, a.x,          \
                       a.router_w, a.router_bias, a.shared_gate_w, a.logits, a.T, a.H, a.E, \
                       TT);                                                                \
    break;
  switch (nit <= kRouterMaxRegIt ? nit : 0) {
    MOE_ROUTER_CASE(1)
    MOE_ROUTER_CASE(2)
    MOE_ROUTER_CASE(3)
    MOE_ROUTER_CASE(4)
    MOE_ROUTER_CASE(5)
    MOE_ROUTER_CASE(6)
    MOE_ROUTER_CASE(7)
    MOE_ROUTER_CASE(8)
    default:
      hipLaunchKernelGGL((router_gemv_kernel<ACT, 0>), grid, dim3(256), lds, s, a.x, a.router_w,
                         a.router_bias, a.shared_gate_w, a.logits, a.T, a.H, a.E, TT);
  }
#undef MOE_ROUTER_CASE
  return hipGetLastError();
}

}  // namespace

// ---------------------------------------------------------------------------
// Dense rows in 4 bits (MOE_FLAG_DENSE_Q4) for the GEMV / GEMM routers:
// w[r][c] = s q + b per group of 64 into fp32 rows, one block per row, each
// thread 8 consecutive values (one code word) per step.

__global__ __launch_bounds__(256) void dense_dequant_kernel(const uint8_t* __restrict__ blob,
                                                            float* __restrict__ out, int H,
                                                            int64_t words_off) {
  const int r = blockIdx.x;
  const uint8_t* codes = blob + (int64_t)r * (H / 2);
  const uint32_t* words = reinterpret_cast<const uint32_t*>(blob + words_off) + (int64_t)r * (H / kGroup);
  for (int c0 = 8 * threadIdx.x; c0 < H; c0 += 8 * 256) {
    const uint32_t q = *reinterpret_cast<const uint32_t*>(codes + c0 / 2);
    const uint32_t sb = words[c0 / kGroup];
    const float sc = bf16_bits_to_f32(sb & 0xFFFFu), bi = bf16_bits_to_f32(sb >> 16);
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = fmaf(sc, (float)((q >> (4 * i)) & 15u), bi);
    float4* o = reinterpret_cast<float4*>(out + (int64_t)r * H + c0);
    o[0] = make_float4(v[0], v[1], v[2], v[3]);
    o[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

hipError_t launch_dense_dequant(const uint8_t* blob, int rows, int H, int64_t words_off, float* out,
                                hipStream_t s) {
  hipLaunchKernelGGL(dense_dequant_kernel, dim3((unsigned)rows), dim3(256), 0, s, blob, out, H,
                     words_off);
  return hipGetLastError();
}

hipError_t launch_router_topk(const RouterArgs& a, hipStream_t s) {
  return a.act == MOE_ACT_F32 ? launch_router_act<MOE_ACT_F32>(a, s)
                              : launch_router_act<MOE_ACT_BF16>(a, s);
}

}  // namespace moe
