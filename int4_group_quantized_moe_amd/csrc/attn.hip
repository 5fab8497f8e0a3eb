// Gated GQA attention decode: one query token per sequence against its KV
// cache, for the layers of the hybrid models that use gated GQA attention
// (page "Paquets Swiftlet 80B Qwen ..." on xix.ai, last paragraph).
//
// Per sequence b, kv head c and its G = Hq / Hkv query heads h:
//   s_j = scale q_h . K_j (j < n),  p = softmax(s),  out_h = sigmoid(gate_h) * sum_j p_j V_j.
// The cache is read once (2 x n x D bf16 per kv head), so the call is
// HBM-bound; the G query heads of a kv head share every K and V row.
//
// attn_chunk_kernel: workgroup (chunk of 128 positions, kv head, sequence).
//   Scores on the matrix cores: v_mfma_f32_32x32x16_bf16 with A = 32 cache
//   rows K_j (each lane loads 16 contiguous bytes of its row straight from
//   memory) and B = the G query vectors (zero past G).  Then per head the
//   chunk's max m, the weights e^(s_j - m) and their sum l; then sum_j e_j V_j
//   on the vector units (each lane owns D / 64 columns, V rows read
//   coalesced), the 4 waves' position ranges added through LDS in a fixed
//   order.  Written: (m, l) and the unnormalised output per (head, chunk).
// attn_merge_kernel: per (sequence, head) the chunks in a fixed order:
//   M = max m_c, L = sum l_c e^(m_c - M), out = gate * sum O_c e^(m_c - M) / L.
#include <math.h>

#include "host.h"
#include "moe_internal.h"
#include "moe_mixers.h"

namespace moe {
namespace {

constexpr int kAttnChunk = 128;  // positions per workgroup (32 per wave)
constexpr int kAttnMaxGroup = 16;  // query heads per kv head held in registers

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16_t mfma_bf16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ float wave_add(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Workspace: per (sequence, query head, chunk) an (m, l) pair, then the D
// unnormalised output values.
struct AttnWs {
  size_t ml, o, total;
};
inline AttnWs attn_ws(int B, int Hq, int D, int nch) {
  AttnWs w{};
  const size_t n = (size_t)B * Hq * nch;
  w.ml = 0;
  w.o = (size_t)align_up((int64_t)(n * 2 * sizeof(float)), 256);
  w.total = w.o + (size_t)align_up((int64_t)(n * D * sizeof(float)), 256);
  return w;
}

// D: head size; GM: query heads per kv head in registers (>= G).
template <int D, int GM>
__global__ __launch_bounds__(256) void attn_chunk_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ lengths,
    float2* __restrict__ part_ml, float* __restrict__ part_o, int Hq, int Hkv, int max_len,
    int nch, float scale) {
  constexpr int kSteps = D / 16;    // K steps of the score MFMAs
  constexpr int kCols = D / 64;     // output columns per lane
  __shared__ float sc[GM][kAttnChunk];               // scores
  __shared__ __align__(16) float pt[kAttnChunk][GM];  // weights, position-major
  __shared__ float red[4][GM][D];                    // the waves' partial outputs
  __shared__ float hm[GM], hl[GM];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int chunk = blockIdx.x, c = blockIdx.y, b = blockIdx.z;
  const int G = Hq / Hkv;
  const int n = min(max(lengths[b], 0), max_len);  // a length past the cache reads no further
  const int j0 = chunk * kAttnChunk;
  const size_t head0 = (size_t)b * Hq + (size_t)c * G;  // first query head of the group
  if (j0 >= n) {  // past the sequence: an empty chunk
    if (tid < G) part_ml[(head0 + tid) * nch + chunk] = make_float2(-INFINITY, 0.0f);
    return;
  }
  const int nj = min(kAttnChunk, n - j0);
  const size_t row0 = ((size_t)b * Hkv + c) * max_len;  // first cache row of (b, c)
  const int l32 = lane & 31, half = lane >> 5;

  // B operand: query head l32 (< G), d = 16 s + 8 half .. + 7 for step s
  u32x4_t qb[kSteps];
  {
    const bool real = l32 < G;
    const uint16_t* qp = q + (head0 + (real ? l32 : 0)) * D + 8 * half;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const uint4 t = *reinterpret_cast<const uint4*>(qp + 16 * s);
      qb[s] = real ? u32x4_t{t.x, t.y, t.z, t.w} : u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  // this wave's 32 V rows (positions 32 wave ..; rows past the chunk's valid
  // ones clamped in-bounds, weight 0) are requested first, so that they
  // arrive while the scores and weights are computed
  constexpr int kVB = kAttnChunk / 4;
  const int jb = wave * kVB, je = min(jb + kVB, nj);
  uint32_t vr[kVB][(kCols + 1) / 2];
#pragma unroll
  for (int u = 0; u < kVB; ++u) {
    const uint16_t* vp = vc + (row0 + j0 + min(jb + u, nj - 1)) * D + kCols * lane;
    if constexpr (kCols == 4) {
      const uint2 t = *reinterpret_cast<const uint2*>(vp);
      vr[u][0] = t.x;
      vr[u][1] = t.y;
    } else if constexpr (kCols == 2) {
      vr[u][0] = *reinterpret_cast<const uint32_t*>(vp);
    } else {
      vr[u][0] = *vp;
    }
  }
  // scores: wave w takes row block w (32 positions); its K fragments are
  // all requested before the multiplies
  constexpr int kBlocks = kAttnChunk / 32 / 4;
  u32x4_t ka[kBlocks][kSteps];
#pragma unroll
  for (int rb = 0; rb < kBlocks; ++rb) {
    const int jl = (wave + 4 * rb) * 32 + l32;        // position in the chunk
    const int jr = j0 + min(jl, nj - 1);              // clamped row (past n: discarded)
    const uint16_t* kp = kc + (row0 + jr) * D + 8 * half;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const uint4 t = *reinterpret_cast<const uint4*>(kp + 16 * s);
      ka[rb][s] = u32x4_t{t.x, t.y, t.z, t.w};
    }
  }
#pragma unroll
  for (int rb = 0; rb < kBlocks; ++rb) {
    const int blk = wave + 4 * rb;
    f32x16_t acc = {};
#pragma unroll
    for (int s = 0; s < kSteps; ++s) acc = mfma_bf16(ka[rb][s], qb[s], acc);
    // lane holds rows (positions) 8 (r / 4) + 4 half + r % 4 of column l32 (head)
    if (l32 < G) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int p = blk * 32 + 8 * (r / 4) + 4 * half + (r % 4);
        sc[l32][p] = p < nj ? acc[r] * scale : -INFINITY;
      }
    }
  }
  __syncthreads();
  // per head: max, weights, sum (wave w takes heads w, w + 4, ...)
  for (int hh = wave; hh < G; hh += 4) {
    float v[kAttnChunk / 64];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < kAttnChunk / 64; ++i) {
      v[i] = sc[hh][lane + 64 * i];
      m = fmaxf(m, v[i]);
    }
    m = wave_max(m);
    float l = 0.0f;
#pragma unroll
    for (int i = 0; i < kAttnChunk / 64; ++i) {
      const float e = expf(v[i] - m);  // -inf -> 0
      pt[lane + 64 * i][hh] = e;
      l += e;
    }
    l = wave_add(l);
    if (lane == 0) {
      hm[hh] = m;
      hl[hh] = l;
    }
  }
  __syncthreads();
  // sum_j e_j V_j: wave w takes positions w * 64 .. w * 64 + 63; lane owns
  // columns kCols lane .. kCols lane + kCols - 1
  float acc[GM][kCols];
#pragma unroll
  for (int hh = 0; hh < GM; ++hh)
#pragma unroll
    for (int e = 0; e < kCols; ++e) acc[hh][e] = 0.0f;
  {
    const int j = jb;
#pragma unroll
    for (int u = 0; u < kVB; ++u) {
      float vv[kCols];
#pragma unroll
      for (int e = 0; e < kCols; ++e)
        vv[e] = bf16_bits_to_f32((e & 1) ? (vr[u][e >> 1] >> 16) : (vr[u][e >> 1] & 0xFFFFu));
      const bool ok = j + u < je;
      float p[GM];
#pragma unroll
      for (int h4 = 0; h4 < GM; h4 += 4) {
        const float4 t = *reinterpret_cast<const float4*>(&pt[min(j + u, kAttnChunk - 1)][h4]);
        p[h4] = t.x;
        p[h4 + 1] = t.y;
        p[h4 + 2] = t.z;
        p[h4 + 3] = t.w;
      }
#pragma unroll
      for (int hh = 0; hh < GM; ++hh) {
        const float w = (ok && hh < G) ? p[hh] : 0.0f;
#pragma unroll
        for (int e = 0; e < kCols; ++e) acc[hh][e] += w * vv[e];
      }
    }
  }
#pragma unroll
  for (int hh = 0; hh < GM; ++hh)
#pragma unroll
    for (int e = 0; e < kCols; ++e) red[wave][hh][kCols * lane + e] = acc[hh][e];
  __syncthreads();
  // the 4 waves' partial sums in wave order; one (head, column) per thread
  for (int idx = tid; idx < G * D; idx += 256) {
    const int hh = idx / D, d = idx - hh * D;
    const float o = (red[0][hh][d] + red[1][hh][d]) + (red[2][hh][d] + red[3][hh][d]);
    part_o[((head0 + hh) * nch + chunk) * D + d] = o;
  }
  if (tid < G) part_ml[(head0 + tid) * nch + chunk] = make_float2(hm[tid], hl[tid]);
}

// Merge of one (sequence, query head, 64-column slice)'s chunk partials:
// NG chunk groups x 64 columns (NG = 16 for long caches, fewer for short
// ones).  Thread (group cg, column d) folds the chunks cg, cg + NG, ... into a
// running (m, l, o) (8 chunk loads in flight at a time), then the NG groups'
// triples are folded in group order:
//   (m1, l1, o1) + (m2, l2, o2) = (M, l1 e^(m1-M) + l2 e^(m2-M), o1 e^(m1-M) + o2 e^(m2-M)).
constexpr int kMergeCols = 64;

__device__ __forceinline__ void fold(float& m, float& l, float& o, float m2, float l2, float o2) {
  if (l2 <= 0.0f) return;          // an empty part
  if (l <= 0.0f) {
    m = m2;
    l = l2;
    o = o2;
    return;
  }
  const float M = fmaxf(m, m2);
  const float a = expf(m - M), b = expf(m2 - M);
  l = l * a + l2 * b;
  o = o * a + o2 * b;
  m = M;
}

template <int D, int NG>
__global__ __launch_bounds__(NG * 64) void attn_merge_kernel(const float2* __restrict__ part_ml,
                                                          const float* __restrict__ part_o,
                                                          const uint16_t* __restrict__ gate,
                                                          uint16_t* __restrict__ out, int Hq,
                                                          int nch) {
  constexpr int kMB = 8;
  __shared__ float3 tri[NG][kMergeCols];
  const int tid = threadIdx.x, dl = tid % kMergeCols, cg = tid / kMergeCols;
  const int d = blockIdx.x * kMergeCols + dl;
  const size_t head = (size_t)blockIdx.z * Hq + blockIdx.y;
  const float2* ml = part_ml + head * nch;
  float m = 0.0f, l = 0.0f, o = 0.0f;
  for (int c0 = cg; c0 < nch; c0 += kMB * NG) {
    float2 t[kMB];
    float v[kMB];
#pragma unroll
    for (int u = 0; u < kMB; ++u) {
      const int c = c0 + u * NG;
      t[u] = c < nch ? ml[c] : make_float2(0.0f, 0.0f);
      v[u] = (c < nch && t[u].y > 0.0f) ? part_o[(head * nch + c) * D + d] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kMB; ++u) fold(m, l, o, t[u].x, t[u].y, v[u]);
  }
  tri[cg][dl] = make_float3(m, l, o);
  __syncthreads();
  if (cg == 0) {
#pragma unroll
    for (int g2 = 1; g2 < NG; ++g2) {
      const float3 t = tri[g2][dl];
      fold(m, l, o, t.x, t.y, t.z);
    }
    const float gv = bf16_bits_to_f32(gate[head * D + d]);
    const float r = l > 0.0f ? o / l : 0.0f;
    out[head * D + d] = f32_to_bf16_bits(r / (1.0f + expf(-gv)));
  }
}

int attn_check(const moe_attn_desc* d) {
  if (d == nullptr) return MOE_ERR_INVALID_ARG;
  if (d->n_seqs < 0 || d->n_seqs > 65535 || d->n_kv_heads < 1 || d->n_q_heads < 1 ||
      d->n_q_heads % d->n_kv_heads || d->n_kv_heads > 65535 || d->max_len < 1 ||
      !(d->scale >= 0.0f))
    return MOE_ERR_INVALID_ARG;
  if (d->head_dim != 64 && d->head_dim != 128 && d->head_dim != 256) return MOE_ERR_UNSUPPORTED;
  if (d->n_q_heads / d->n_kv_heads > kAttnMaxGroup) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)d->max_len > (1LL << 24)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

template <int D, int GM>
void launch_attn_t(const moe_attn_desc* d, const uint16_t* q, const uint16_t* gate,
                   const uint16_t* kc, const uint16_t* vc, const int32_t* lengths, uint16_t* out,
                   uint8_t* ws, float scale, hipStream_t s) {
  const int nch = (d->max_len + kAttnChunk - 1) / kAttnChunk;
  const AttnWs w = attn_ws(d->n_seqs, d->n_q_heads, D, nch);
  float2* ml = reinterpret_cast<float2*>(ws + w.ml);
  float* po = reinterpret_cast<float*>(ws + w.o);
  hipLaunchKernelGGL((attn_chunk_kernel<D, GM>), dim3(nch, d->n_kv_heads, d->n_seqs), dim3(256),
                     0, s, q, kc, vc, lengths, ml, po, d->n_q_heads, d->n_kv_heads, d->max_len,
                     nch, scale);
  const dim3 mg(D / kMergeCols, d->n_q_heads, d->n_seqs);
  if (nch >= 64)
    hipLaunchKernelGGL((attn_merge_kernel<D, 16>), mg, dim3(16 * 64), 0, s, ml, po, gate, out,
                       d->n_q_heads, nch);
  else if (nch >= 8)
    hipLaunchKernelGGL((attn_merge_kernel<D, 4>), mg, dim3(4 * 64), 0, s, ml, po, gate, out,
                       d->n_q_heads, nch);
  else
    hipLaunchKernelGGL((attn_merge_kernel<D, 1>), mg, dim3(64), 0, s, ml, po, gate, out,
                       d->n_q_heads, nch);
}

template <int D>
void launch_attn_d(const moe_attn_desc* d, const uint16_t* q, const uint16_t* gate,
                   const uint16_t* kc, const uint16_t* vc, const int32_t* lengths, uint16_t* out,
                   uint8_t* ws, float scale, hipStream_t s) {
  const int G = d->n_q_heads / d->n_kv_heads;
  if (G <= 4)
    launch_attn_t<D, 4>(d, q, gate, kc, vc, lengths, out, ws, scale, s);
  else if (G <= 8)
    launch_attn_t<D, 8>(d, q, gate, kc, vc, lengths, out, ws, scale, s);
  else
    launch_attn_t<D, 16>(d, q, gate, kc, vc, lengths, out, ws, scale, s);
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_attn_workspace_bytes(const moe_attn_desc* d) {
  if (attn_check(d) != MOE_OK) return 0;
  const int nch = (d->max_len + kAttnChunk - 1) / kAttnChunk;
  return attn_ws(d->n_seqs, d->n_q_heads, d->head_dim, nch).total;
}

extern "C" int moe_attn_decode(const moe_attn_desc* d, const void* q, const void* gate,
                               const void* k_cache, const void* v_cache, const int32_t* lengths,
                               void* out, void* ws, hipStream_t stream) {
  MOE_TRY(attn_check(d));
  if (d->n_seqs == 0) return MOE_OK;
  MOE_TRY(check_ptr(q));
  MOE_TRY(check_ptr(gate));
  MOE_TRY(check_ptr(k_cache));
  MOE_TRY(check_ptr(v_cache));
  MOE_TRY(check_ptr(lengths, 4));
  MOE_TRY(check_ptr(out));
  MOE_TRY(check_ptr(ws, 256));
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n < 1) return MOE_ERR_NO_DEVICE;
  const float scale = d->scale > 0.0f ? d->scale : 1.0f / sqrtf((float)d->head_dim);
  const auto* qq = reinterpret_cast<const uint16_t*>(q);
  const auto* gg = reinterpret_cast<const uint16_t*>(gate);
  const auto* kk = reinterpret_cast<const uint16_t*>(k_cache);
  const auto* vv = reinterpret_cast<const uint16_t*>(v_cache);
  auto* oo = reinterpret_cast<uint16_t*>(out);
  auto* w8 = reinterpret_cast<uint8_t*>(ws);
  switch (d->head_dim) {
    case 64: launch_attn_d<64>(d, qq, gg, kk, vv, lengths, oo, w8, scale, stream); break;
    case 128: launch_attn_d<128>(d, qq, gg, kk, vv, lengths, oo, w8, scale, stream); break;
    default: launch_attn_d<256>(d, qq, gg, kk, vv, lengths, oo, w8, scale, stream); break;
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}
