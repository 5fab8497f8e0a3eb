// Gated DeltaNet decode step: one new token per sequence through the
// recurrent state of every value head.
//
// 75% of the layers of the hybrid models use Gated DeltaNet linear attention
// with a fixed-size recurrent state (page "Paquets Swiftlet 80B Qwen ..." on
// xix.ai, 5th paragraph).  With the gated delta rule (Yang, Kautz and
// Hatamizadeh, 2024) one step of value head h is, for the normalised key k^
// and query q^ of its query/key head and alpha = exp(g):
//   u = v - alpha S k^,   S <- alpha S + beta u k^T,   o = S q^.
// Row i of S (d_k values) needs only v_i and the two head vectors, so every
// row is independent: the step is one pass over the state, read once and
// written once, HBM-bound at 8 bytes per state element.
//
// Layout: state [B][Hv][d_v][d_k] fp32 row-major.  A workgroup of 4 waves
// updates 16 rows of one head; d_k / 4 lanes hold one row as float4s (a row
// of 128 is one 512-byte coalesced access per half-wave), and the two dot
// products per row are butterflies over those lanes in a fixed order.
#include "host.h"
#include "moe_internal.h"
#include "moe_mixers.h"

namespace moe {
namespace {

constexpr int kGdnRows = 16;  // state rows per workgroup

// Sum over the LPR consecutive lanes of a row group (LPR a power of two),
// every lane of the group getting the same bits.
template <int LPR>
__device__ __forceinline__ float row_sum(float v) {
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <int DK>
__global__ __launch_bounds__(256) void gdn_decode_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ g, const float* __restrict__ beta,
    float* __restrict__ state, uint16_t* __restrict__ out, int Hk, int Hv, int dv, float eps,
    float scale) {
  constexpr int LPR = DK / 4;              // lanes per state row
  constexpr int RPW = 64 / LPR;            // rows per wave per pass
  constexpr int kPasses = kGdnRows / (4 * RPW);
  static_assert(kPasses >= 1 && kGdnRows % (4 * RPW) == 0, "rows per workgroup");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane / LPR, li = lane % LPR;
  const int h = blockIdx.y, b = blockIdx.z;
  const int kh = h / (Hv / Hk);
  // this lane's 4 columns of the head's key and query, L2-normalised
  const size_t qk_off = ((size_t)b * Hk + kh) * DK + 4 * li;
  const uint2 kr = *reinterpret_cast<const uint2*>(k + qk_off);
  const uint2 qr = *reinterpret_cast<const uint2*>(q + qk_off);
  float kv[4] = {bf16_bits_to_f32(kr.x & 0xFFFFu), bf16_bits_to_f32(kr.x >> 16),
                 bf16_bits_to_f32(kr.y & 0xFFFFu), bf16_bits_to_f32(kr.y >> 16)};
  float qv[4] = {bf16_bits_to_f32(qr.x & 0xFFFFu), bf16_bits_to_f32(qr.x >> 16),
                 bf16_bits_to_f32(qr.y & 0xFFFFu), bf16_bits_to_f32(qr.y >> 16)};
  const float ssk = row_sum<LPR>((kv[0] * kv[0] + kv[1] * kv[1]) + (kv[2] * kv[2] + kv[3] * kv[3]));
  const float ssq = row_sum<LPR>((qv[0] * qv[0] + qv[1] * qv[1]) + (qv[2] * qv[2] + qv[3] * qv[3]));
  const float rk = 1.0f / sqrtf(ssk + eps), rq = scale / sqrtf(ssq + eps);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    kv[i] *= rk;
    qv[i] *= rq;
  }
  const size_t head = (size_t)b * Hv + h;
  const float alpha = expf(g[head]), bt = beta[head];
  float* S = state + head * (size_t)dv * DK;
  const uint16_t* vp = v + head * dv;
  uint16_t* op = out + head * dv;
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int row = blockIdx.x * kGdnRows + pass * 4 * RPW + wave * RPW + sub;
    float4* sp = reinterpret_cast<float4*>(S + (size_t)row * DK + 4 * li);
    float4 s = *sp;
    const float a = row_sum<LPR>((s.x * kv[0] + s.y * kv[1]) + (s.z * kv[2] + s.w * kv[3]));
    const float c = bt * (bf16_bits_to_f32(vp[row]) - alpha * a);
    s.x = alpha * s.x + c * kv[0];
    s.y = alpha * s.y + c * kv[1];
    s.z = alpha * s.z + c * kv[2];
    s.w = alpha * s.w + c * kv[3];
    const float o = row_sum<LPR>((s.x * qv[0] + s.y * qv[1]) + (s.z * qv[2] + s.w * qv[3]));
    *sp = s;
    if (li == 0) op[row] = f32_to_bf16_bits(o);
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_gdn_decode(const moe_gdn_desc* d, const void* q, const void* k, const void* v,
                              const float* g, const float* beta, float* state, void* out,
                              hipStream_t stream) {
  if (d == nullptr) return MOE_ERR_INVALID_ARG;
  if (d->n_seqs < 0 || d->n_k_heads < 1 || d->n_v_heads < 1 || d->n_v_heads % d->n_k_heads)
    return MOE_ERR_INVALID_ARG;
  if (d->n_seqs > 65535 || d->n_v_heads > 65535) return MOE_ERR_INVALID_ARG;
  if (!(d->eps >= 0.0f) || !(d->scale >= 0.0f)) return MOE_ERR_INVALID_ARG;
  if (d->d_k != 64 && d->d_k != 128 && d->d_k != 256) return MOE_ERR_UNSUPPORTED;
  if (d->d_v < kGdnRows || d->d_v % kGdnRows || d->d_v > 4096) return MOE_ERR_UNSUPPORTED;
  if (d->n_seqs == 0) return MOE_OK;
  MOE_TRY(check_ptr(q));
  MOE_TRY(check_ptr(k));
  MOE_TRY(check_ptr(v));
  MOE_TRY(check_ptr(g, 4));
  MOE_TRY(check_ptr(beta, 4));
  MOE_TRY(check_ptr(state));
  MOE_TRY(check_ptr(out));
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n < 1) return MOE_ERR_NO_DEVICE;
  const float scale = d->scale > 0.0f ? d->scale : 1.0f / sqrtf((float)d->d_k);
  const dim3 grid(d->d_v / kGdnRows, d->n_v_heads, d->n_seqs);
  const auto* qq = reinterpret_cast<const uint16_t*>(q);
  const auto* kk = reinterpret_cast<const uint16_t*>(k);
  const auto* vv = reinterpret_cast<const uint16_t*>(v);
  auto* oo = reinterpret_cast<uint16_t*>(out);
  switch (d->d_k) {
    case 64:
      hipLaunchKernelGGL(gdn_decode_kernel<64>, grid, dim3(256), 0, stream, qq, kk, vv, g, beta,
                         state, oo, d->n_k_heads, d->n_v_heads, d->d_v, d->eps, scale);
      break;
    case 128:
      hipLaunchKernelGGL(gdn_decode_kernel<128>, grid, dim3(256), 0, stream, qq, kk, vv, g, beta,
                         state, oo, d->n_k_heads, d->n_v_heads, d->d_v, d->eps, scale);
      break;
    default:
      hipLaunchKernelGGL(gdn_decode_kernel<256>, grid, dim3(256), 0, stream, qq, kk, vv, g, beta,
                         state, oo, d->n_k_heads, d->n_v_heads, d->d_v, d->eps, scale);
      break;
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}
