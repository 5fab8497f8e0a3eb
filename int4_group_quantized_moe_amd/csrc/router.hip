// Router GEMV, shared-gate logit, and wavefront softmax / top-k / renormalise.
//
// Routing of every token to the top-k of E experts by a resident router
// (page "Paquets Swiftlet 80B Qwen ..." on xix.ai, 4th paragraph: 10 of 512
// or 8 of 256 experts per layer and token; the routers stay resident).
// Renormalised top-k weights equal the softmax over the k selected logits,
// so the E-way softmax sum is never formed.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRouterWaves = 4;     // rows per workgroup (one per wave)
constexpr int kRouterMaxTT = 8;     // tokens per LDS chunk
constexpr int kRouterMaxRegIt = 8;  // row cached in registers when H <= 64*4*8

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

  for (int t0 = 0; t0 < T; t0 += TT) {
    const int tt_n = min(TT, T - t0);
    __syncthreads();
    for (int i = threadIdx.x; i < tt_n * H; i += blockDim.x) {
      const int tt = i / H, c = i - tt * H;
      xs[i] = load_act<ACT>(x, (int64_t)(t0 + tt) * H + c);
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

// One wave per token: k rounds of a wave-wide (max logit, lowest index)
// reduction, then the softmax over the k selected logits.
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits,
                                                   int32_t* __restrict__ topk_idx,
                                                   float* __restrict__ topk_w,
                                                   float* __restrict__ gamma, int T, int E,
                                                   int k, int has_gate) {
  constexpr int kMaxPerLane = MOE_MAX_EXPERTS / 64;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* l = logits + (int64_t)t * (E + 1);
  float v[kMaxPerLane];
  const int per_lane = (E + 63) / 64;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = i * 64 + lane;
    v[i] = (i < per_lane && e < E) ? l[e] : -INFINITY;
  }
  unsigned taken = 0u;  // bit i: v[i] already selected
  float sel_v[MOE_MAX_TOP_K];
  int sel_i[MOE_MAX_TOP_K];
  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int e = i * 64 + lane;
      if (i < per_lane && e < E && !((taken >> i) & 1u)) {
        if (v[i] > bv || (v[i] == bv && e < bi)) {
          bv = v[i];
          bi = e;
        }
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    sel_v[r] = bv;
    sel_i[r] = bi;
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
  }
  if (lane == 0) {
    float den = 0.0f;
    for (int r = 0; r < k; ++r) den += __expf(sel_v[r] - sel_v[0]);
    const float inv = 1.0f / den;
    for (int r = 0; r < k; ++r) {
      topk_idx[(int64_t)t * k + r] = sel_i[r];
      topk_w[(int64_t)t * k + r] = __expf(sel_v[r] - sel_v[0]) * inv;
    }
    if (has_gate && gamma != nullptr) gamma[t] = 1.0f / (1.0f + __expf(-l[E]));
  }
}

template <int ACT>
hipError_t launch_router_act(const RouterArgs& a, hipStream_t s) {
  const int R = a.E + (a.shared_gate_w ? 1 : 0);
  const int TT = max(1, min(min(a.T, kRouterMaxTT), 16384 / a.H));
  const size_t lds = sizeof(float) * (size_t)TT * a.H;
  const dim3 grid((R + kRouterWaves - 1) / kRouterWaves);
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
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_kernel, dim3((a.T + 3) / 4), dim3(256), 0, s, a.logits, a.topk_idx,
                     a.topk_w, a.gamma, a.T, a.E, a.k, a.shared_gate_w ? 1 : 0);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router_topk(const RouterArgs& a, hipStream_t s) {
  return a.act == MOE_ACT_F32 ? launch_router_act<MOE_ACT_F32>(a, s)
                              : launch_router_act<MOE_ACT_BF16>(a, s);
}

}  // namespace moe
