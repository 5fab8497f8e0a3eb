/* Host C implementation of the seeded generator (same definition as the numpy
 * reference in synth/__init__.py and the device fill in synth_fill.hip).
 * Built with -ffp-contract=off so the fp32 uniform is a + fl(fl(b - a) * u)
 * with separate roundings.  Inputs only: no arithmetic of the MoE layer. */
#include <stdint.h>

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static const uint64_t kGolden = 0x9E3779B97F4A7C15ull;

void synth_host_codes(uint64_t key, int64_t n, int bits, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)(mix64(key + (uint64_t)(i + 1) * kGolden) >> (64 - bits));
}

void synth_host_uniform_bf16(uint64_t key, int64_t n, float lo, float hi, uint16_t* out) {
  const float width = hi - lo;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const uint64_t d = mix64(key + (uint64_t)(i + 1) * kGolden);
    const float u = (float)(uint32_t)(d >> 40) * 5.9604644775390625e-08f;
    const float t = width * u;
    const float v = lo + t;
    union { float f; uint32_t u; } c;
    c.f = v;
    uint32_t b = c.u + 0x7FFFu + ((c.u >> 16) & 1u);
    out[i] = (uint16_t)(b >> 16);
  }
}
