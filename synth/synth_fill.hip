// Device fill of the seeded synthetic expert weights.
//
// Same generator as synth/__init__.py (host): SplitMix64 output finaliser
// (Steele, Lea & Flood 2014) over a counter, stream key from
// (seed, tensor, layer, expert).  Integer codes take the top bits of a draw;
// bf16 uniforms are a + (b - a) * u in fp32 with separate roundings, then
// rounded to bf16 (nearest even).  Built with -ffp-contract=off so no
// multiply-add is fused, which keeps host and device bit-equal.
//
// Writes *logical* arrays only (one code per byte; scale plane then bias
// plane of bf16 bits), the input format of the library's blob packer.  No
// arithmetic of the MoE layer lives here.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__host__ __device__ inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;

__host__ __device__ inline uint64_t stream_key(uint64_t seed, uint64_t tensor, uint64_t layer,
                                               uint64_t expert) {
  return mix64((seed << 48) | (tensor << 40) | (layer << 24) | expert);
}

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// codes of n_exp consecutive experts, elements [0, n) each
__global__ void fill_codes_kernel(uint64_t seed, int tensor, int layer, int expert0, int64_t n,
                                  int bits, uint8_t* __restrict__ out) {
  const int e = blockIdx.y;
  const uint64_t key = stream_key(seed, tensor, layer, (uint64_t)(expert0 + e));
  uint8_t* o = out + (int64_t)e * n;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const uint64_t d = mix64(key + (uint64_t)(i + 1) * kGolden);
    o[i] = (uint8_t)(d >> (64 - bits));
  }
}

__global__ void fill_uniform_bf16_kernel(uint64_t seed, int tensor, int layer, int expert0,
                                         int64_t n, float lo, float hi, int64_t out_stride,
                                         uint16_t* __restrict__ out) {
  const int e = blockIdx.y;
  const uint64_t key = stream_key(seed, tensor, layer, (uint64_t)(expert0 + e));
  uint16_t* o = out + (int64_t)e * out_stride;
  const float width = hi - lo;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const uint64_t d = mix64(key + (uint64_t)(i + 1) * kGolden);
    const float u = (float)(uint32_t)(d >> 40) * 5.9604644775390625e-08f;  // 2^-24
    const float t = width * u;
    const float v = lo + t;
    o[i] = f32_to_bf16_rne(v);
  }
}

dim3 grid_for(int64_t n, int n_exp) {
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  return dim3((unsigned)blocks, (unsigned)n_exp);
}

}  // namespace

extern "C" {

// Stream tensor ids (same numbering as the host generator).
enum { T_QGATE = 1, T_QUP, T_QDOWN, T_SGATE, T_BGATE, T_SUP, T_BUP, T_SDOWN, T_BDOWN };

// Fills the logical arrays of experts expert0 .. expert0 + n_exp - 1 of one
// layer (expert ids are the 24-bit stream field; the shared expert is
// 0xFFFFFF with n_exp = 1):
//   qg, qu [n_exp][inter][hidden], qd [n_exp][hidden][inter]  (uint8 codes)
//   sbg, sbu [n_exp][2][inter][hidden/64]                      (bf16 bits)
//   sbd [n_exp][2][hidden][inter/64]
// All device pointers.  Returns 0 or the HIP error code.
int synth_fill_experts(uint64_t seed, int bits, int hidden, int inter, int layer, int expert0,
                       int n_exp, float scale_lo, float scale_hi, float bias_lo, float bias_hi,
                       uint8_t* qg, uint8_t* qu, uint8_t* qd, uint16_t* sbg, uint16_t* sbu,
                       uint16_t* sbd, hipStream_t stream) {
  if (n_exp <= 0) return 0;
  const int64_t nq = (int64_t)hidden * inter;
  const int64_t ngu = (int64_t)inter * (hidden / 64);
  const int64_t nd = (int64_t)hidden * (inter / 64);
  hipLaunchKernelGGL(fill_codes_kernel, grid_for(nq, n_exp), dim3(256), 0, stream, seed, T_QGATE,
                     layer, expert0, nq, bits, qg);
  hipLaunchKernelGGL(fill_codes_kernel, grid_for(nq, n_exp), dim3(256), 0, stream, seed, T_QUP,
                     layer, expert0, nq, bits, qu);
  hipLaunchKernelGGL(fill_codes_kernel, grid_for(nq, n_exp), dim3(256), 0, stream, seed, T_QDOWN,
                     layer, expert0, nq, bits, qd);
  struct {
    int tensor;
    uint16_t* base;
    int64_t n;
    int plane;
    float lo, hi;
  } sb[6] = {{T_SGATE, sbg, ngu, 0, scale_lo, scale_hi}, {T_BGATE, sbg, ngu, 1, bias_lo, bias_hi},
             {T_SUP, sbu, ngu, 0, scale_lo, scale_hi},   {T_BUP, sbu, ngu, 1, bias_lo, bias_hi},
             {T_SDOWN, sbd, nd, 0, scale_lo, scale_hi},  {T_BDOWN, sbd, nd, 1, bias_lo, bias_hi}};
  for (int i = 0; i < 6; ++i) {
    hipLaunchKernelGGL(fill_uniform_bf16_kernel, grid_for(sb[i].n, n_exp), dim3(256), 0, stream,
                       seed, sb[i].tensor, layer, expert0, sb[i].n, sb[i].lo, sb[i].hi,
                       2 * sb[i].n, sb[i].base + sb[i].plane * sb[i].n);
  }
  return (int)hipGetLastError();
}

// Elements [0, n) of one stream of bf16 uniforms U(lo, hi) (the definition of
// the scale and bias planes above) into a device array of n bf16 bits.
// Returns 0 or the HIP error code.
int synth_fill_uniform_bf16(uint64_t seed, int tensor, int layer, int expert, int64_t n,
                            float lo, float hi, uint16_t* out, hipStream_t stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(fill_uniform_bf16_kernel, grid_for(n, 1), dim3(256), 0, stream, seed, tensor,
                     layer, expert, n, lo, hi, n, out);
  return (int)hipGetLastError();
}

}  // extern "C"
