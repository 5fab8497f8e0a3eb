// Prefill / large-batch path: grouped GEMMs on the MFMA matrix cores.
//
// When many tokens share an expert (a prefill chunk routes ~T*k/E tokens to
// each expert) the expert FFN is a dense contraction: per expert e with its
// bucket of n_e tokens,
//   G|U = X_e [n_e x H] . [Wg_e | Wu_e]^T,  h = silu(G) * U,
//   Y_e = h [n_e x I] . Wd_e^T,  out[t] += w_{t,j} Y_e[t]
// and the shared expert is the same with all T tokens.  The pages call prefill
// the bottleneck for long contexts (page "Swiftlet: 在 Mac 和 iPhone 上執行 ..."
// on agentlenshq.com, section "社群觀點"); the weights are MLX-style
// group-quantised int4/int8 (page "Paquets Swiftlet 80B Qwen ..." on xix.ai,
// last paragraph).
//
// Both GEMMs run on v_mfma_f32_32x32x16_bf16 with fp32 accumulation, and no
// operand is rounded on its way into the matrix cores:
//  * weights enter as their integer codes, which bf16 holds exactly (int4 as
//    1 + q/16, int8 as q); the group's bf16 scale is applied in fp32 to the
//    group's code sums, and the group's bias multiplies the group sum of the
//    activations (w = s q + b factors as s * sum(q x) + b * sum(x));
//  * the gate/up input x_hat is bf16 already; the down GEMM runs on
//    v_mfma_f32_32x32x16_f16: h is stored in fp16 (11 significant bits)
//    after a power-of-two scale per (row tile, group) that puts the tile's
//    largest |h| in [2^13, 2^14), and the codes enter as fp16 (int4 as
//    1 + q/16, int8 as q), in a K order permuted within each 8-value chunk
//    so that a code word expands with masks and shifts (the h chunks are
//    written in the same order).
// Dequantising to bf16 instead (s*q + b rounded, and h rounded to bf16)
// would add ~2^-9 relative error per weight and per h value; h in bf16
// alone measured 0.01 rms of the output on the batched 80B layer.
#include "mfma_common.h"

namespace moe {
namespace {

// ---------------------------------------------------------------------------
// tile list: every expert bucket of at least min_rows tokens (and the shared
// expert's T tokens as bucket E) cut into tiles of kMT rows.  One workgroup.

__global__ __launch_bounds__(1024) void tile_list_kernel(const int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ tiles,
                                                         int32_t* __restrict__ ntiles, int E,
                                                         int has_shared, int max_tiles,
                                                         int min_rows) {
  __shared__ int wsum[16];
  __shared__ int carry_s;
  __shared__ int tbase[MOE_MAX_EXPERTS + 2];
  const int n_b = E + has_shared;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int carry = 0;
  // exclusive scan of the per-bucket tile counts, 1024 buckets per pass
  for (int b0 = 0; b0 < n_b; b0 += 1024) {
    const int b = b0 + threadIdx.x;
    const int nb = b < n_b ? counts[b] : 0;
    const int c = nb >= min_rows ? (nb + kMT - 1) / kMT : 0;
    int v = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(v, off, 64);
      if (lane >= off) v += o;
    }
    if (lane == 63) wsum[wave] = v;
    __syncthreads();
    int wb = carry;
    for (int w = 0; w < wave; ++w) wb += wsum[w];
    if (b < n_b) tbase[b] = wb + v - c;
    if (threadIdx.x == 1023) carry_s = wb + v;
    __syncthreads();
    carry = carry_s;
    __syncthreads();
  }
  const int total = min(carry, max_tiles);
  if (threadIdx.x == 0) *ntiles = total;
  for (int b = threadIdx.x; b < n_b; b += 1024) {
    const int c = counts[b] >= min_rows ? (counts[b] + kMT - 1) / kMT : 0;
    for (int i = 0; i < c; ++i) {
      const int t = tbase[b] + i;
      if (t < max_tiles) {
        tiles[2 * t] = b;
        tiles[2 * t + 1] = i * kMT;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// per-group sums of the activations: xsum[t][g] = sum of x[t][64g .. 64g+63]

__global__ __launch_bounds__(256) void group_sum_kernel(const uint16_t* __restrict__ x,
                                                        float* __restrict__ xsum, int T, int H) {
  const int G = H / kGroup;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)T * G) return;
  const uint4* p = reinterpret_cast<const uint4*>(x + (i / G) * H + (i % G) * kGroup);
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kGroup / 8; ++c) {
    const uint4 v = p[c];
    s += (bf16_bits_to_f32(v.x & 0xFFFFu) + bf16_bits_to_f32(v.x >> 16)) +
         (bf16_bits_to_f32(v.y & 0xFFFFu) + bf16_bits_to_f32(v.y >> 16)) +
         (bf16_bits_to_f32(v.z & 0xFFFFu) + bf16_bits_to_f32(v.z >> 16)) +
         (bf16_bits_to_f32(v.w & 0xFFFFu) + bf16_bits_to_f32(v.w >> 16));
  }
  xsum[i] = s;
}

// ---------------------------------------------------------------------------
// Shared tile structure of both GEMMs.  A workgroup computes a 128-row x
// 128-column tile; wave (wm, wn) = (wave / 2, wave % 2) owns rows
// 64 wm .. 64 wm + 63 (two 32-row blocks mb) and two 32-column blocks nb.
// K runs one quantisation group (64) per stage: the activation rows of the
// group are staged in LDS (double-buffered, next stage's loads in flight
// during the MFMAs); each lane reads its weight row's 32 codes of the group
// straight from memory into registers (lane half 0: codes 0..31, half 1:
// 32..63) and expands them to exact bf16 operands.  Per group the code sums
// go into a fresh accumulator that is then scaled into the tile:
//   C += scale_g[n] * acc_g,
// and the bias terms are added at the end by bias_mfma.

// gate/up: grid (max(I, Is)/64, tiles).  Tile columns: 64 gate rows and the
// 64 up rows of the same h columns; wave wn holds h columns n0 + 32 wn ..
// n0 + 32 wn + 31 as block 0 (gate) and block 1 (up).  Writes per row the
// 64 h values in fp16 after the tile's power-of-two scale, in the K order the
// down GEMM stages, the row's group sum of the stored values (unscaled), and
// the scale's inverse.  An h row keeps the byte stride of the fp32 h rows of
// the GEMV kernels (4 x inter bytes), so buckets of either path index the
// one h buffer alike; the fp16 row fills the first half, and the second
// half holds, per group g, the inverse scale as a float at element 2 g.

#define MOE_PGU_PARAMS                                                                       \
  const uint16_t* __restrict__ x, const float* __restrict__ xsum,                              \
      const int32_t* __restrict__ pairs, const int32_t* __restrict__ counts,                  \
      const int32_t* __restrict__ offsets, const int32_t* __restrict__ tiles,                 \
      const int32_t* __restrict__ ntiles, const uint8_t* __restrict__ slab,                   \
      const int32_t* __restrict__ slot_table, int64_t stride,                                 \
      const uint8_t* __restrict__ shared_blob, uint16_t* __restrict__ h,                      \
      float* __restrict__ hsum, int T, int H, int E, int k, int I, int Is, int64_t gu_unit_r,   \
      int64_t gu_tile_r, int64_t gu_unit_s, int64_t gu_tile_s, int nbg
#define MOE_PGU_ARGS                                                                       \
  x, xsum, pairs, counts, offsets, tiles, ntiles, slab, slot_table, stride, shared_blob, h, \
      hsum, T, H, E, k, I, Is, gu_unit_r, gu_tile_r, gu_unit_s, gu_tile_s, nbg

// Gate/up K pipeline.  Everything a K stage (one quantisation group) needs
// arrives by asynchronous global->LDS loads (global_load_lds): the 128
// activation rows (16 KiB), the 128 weight rows' codes (4 or 8 KiB) and
// their (scale, bias) words.  Each stage has its own __shared__ object, so
// the compiler's wait accounting for these loads is per stage and a read of
// stage s never waits for the loads of the stages behind it; kStages - 1
// stages are in flight while one is multiplied.  Chunk c of activation row r
// sits at r*8 + (c ^ ((r >> 1) & 7)): the 16 consecutive rows of a 16-lane
// group of an MFMA operand read, all at the same chunk, then land on 16
// distinct 16-byte slots of every 256-byte window of LDS banks.
constexpr int kStages = 3;
constexpr int kStageChunks = kMT * kGroup / 8;  // 1024 chunks of 16 bytes
typedef uint4 StageBuf[kStageChunks];

template <int BITS>
struct GuStage {
  uint4 A[kStageChunks];               // activations
  // codes: 128 rows x 32 (int4) / 64 (int8) bytes of the stage's group, then
  // of the second-half group when the wave rows split K (else a copy)
  uint4 B[2 * 128 * (kGroup * BITS / 8) / 16];
  uint32_t S[256];                     // (scale, bias) of rows 0..127, then of the second-half group
};

__device__ __forceinline__ int swz(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }

// Code chunks (16 bytes) of weight row r in a stage: int4 rows hold two, and
// rows 8..15 of every 16 swap them, so that the 16 rows a 16-lane group reads
// (all at the same chunk) cover 16 distinct slots of a 256-byte bank window;
// int8 rows (four chunks, read as pairs) keep the natural order.
template <int BITS>
__device__ __forceinline__ int code_chunk(int r, int c) {
  return BITS == 4 ? c ^ ((r >> 3) & 1) : c;
}

// Workgroup barrier for the K pipeline: waits for this wave's LDS reads
// and writes (lgkmcnt) but not for its global->LDS loads in flight, which a
// release fence would also wait for.  The asm "memory" clobber keeps the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt vmcnt(N): at most N of this wave's vector memory loads
// (including global->LDS loads) still outstanding; they complete in order.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

#define MOE_G1(p) ((const void __attribute__((address_space(1)))*)(p))
#define MOE_L3(p) ((void __attribute__((address_space(3)))*)(p))

// Loads a thread issues per stage: 4 activation chunks, 2 x BITS/4 code
// chunks (both K halves), one (scale, bias) word.
template <int BITS>
constexpr int gu_stage_loads() { return 4 + 2 * (BITS / 4) + 1; }

// Load sources of a stage: a uniform base (scalar registers) plus a 32-bit
// per-lane byte offset, so that the loads use scalar-base addressing and the
// per-stage advance is scalar arithmetic.
template <int BITS>
struct GuSrc {
  const uint8_t* x;            // activations (uniform)
  const uint8_t* sec;          // blob gate/up section (uniform)
  int64_t unit_b;
  uint32_t a[4];               // activation chunk offsets (stage 0)
  uint32_t b[BITS / 4];        // code chunk offsets (k-block 0, group 0)
  uint32_t sb;                 // (scale, bias) word offset (k-block 0, group 0)
  int g2off;                   // second-half group of a stage: g + g2off (uniform)
};

template <int BITS>
__device__ __forceinline__ void gu_issue(const GuSrc<BITS>& P, GuStage<BITS>& st, int g,
                                         int wave) {
  constexpr int GPK = kRowBytes * (8 / BITS) / kGroup;
  constexpr int GBYTES = kGroup * BITS / 8;
  const uint8_t* xa = P.x + (int64_t)g * kGroup * 2;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    __builtin_amdgcn_global_load_lds(MOE_G1(xa + P.a[j]), MOE_L3(&st.A[j * 256 + wave * 64]), 16,
                                     0, 0);
  const uint8_t* wb = P.sec + (int64_t)(g / GPK) * P.unit_b + (g % GPK) * GBYTES;
#pragma unroll
  for (int j = 0; j < BITS / 4; ++j)
    __builtin_amdgcn_global_load_lds(MOE_G1(wb + P.b[j]), MOE_L3(&st.B[j * 256 + wave * 64]), 16,
                                     0, 0);
  const int g2 = g + P.g2off;
  const uint8_t* wb2 = P.sec + (int64_t)(g2 / GPK) * P.unit_b + (g2 % GPK) * GBYTES;
#pragma unroll
  for (int j = 0; j < BITS / 4; ++j)
    __builtin_amdgcn_global_load_lds(MOE_G1(wb2 + P.b[j]),
                                     MOE_L3(&st.B[(BITS / 4 + j) * 256 + wave * 64]), 16, 0, 0);
  const uint8_t* sbb = P.sec + (int64_t)(g / GPK) * P.unit_b + (g % GPK) * 4;
  __builtin_amdgcn_global_load_lds(MOE_G1(sbb + P.sb), MOE_L3(&st.S[wave * 64]), 4, 0, 0);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)p;
}

// All LDS reads of one K stage for this lane, in one asm block that ends
// with its own lgkmcnt wait: the A operands of both row blocks for the 4 K
// steps, the lane's codes of both weight rows, and their (scale, bias)
// words.  (The compiler's wait accounting for global->LDS loads does not
// survive the pipeline's loop back-edge and would drain every load in
// flight before the first read; the explicit vmcnt wait before the stage
// barrier is what orders these reads after their loads.)  The outputs are
// early-clobber: each is written while later reads still need addresses.
template <int BITS>
struct GuFrags {
  u32x4 a[2][2];               // A operands of two K steps, both row blocks
  u32x4 q[2][BITS / 4];        // the lane's codes of both weight rows
  uint32_t sb[2];
};

// Every LDS read of one K stage in one asm block with one wait: the A
// operands of the 4 K steps (both row blocks; a2 holds steps 2-3), the
// lane's codes of both weight rows and their (scale, bias) words.
template <int BITS>
__device__ __forceinline__ void gu_read_all(const GuStage<BITS>& st, int wm, int wn, int l32,
                                            int half, int khalf, GuFrags<BITS>& f,
                                            u32x4 (&a2)[2][2]) {
  const uint32_t a00 = lds_addr(&st.A[swz(64 * wm + l32, 4 * half + 0)]);
  const uint32_t a01 = lds_addr(&st.A[swz(64 * wm + l32, 4 * half + 1)]);
  const uint32_t a10 = lds_addr(&st.A[swz(64 * wm + 32 + l32, 4 * half + 0)]);
  const uint32_t a11 = lds_addr(&st.A[swz(64 * wm + 32 + l32, 4 * half + 1)]);
  const uint32_t c00 = lds_addr(&st.A[swz(64 * wm + l32, 4 * half + 2)]);
  const uint32_t c01 = lds_addr(&st.A[swz(64 * wm + l32, 4 * half + 3)]);
  const uint32_t c10 = lds_addr(&st.A[swz(64 * wm + 32 + l32, 4 * half + 2)]);
  const uint32_t c11 = lds_addr(&st.A[swz(64 * wm + 32 + l32, 4 * half + 3)]);
  const int r0 = 32 * wn + l32, r1 = 64 + 32 * wn + l32;
  constexpr int CPR = kGroup * BITS / 8 / 16;  // code chunks per row
  const int kb = khalf * 128 * CPR, ks = khalf * 128;  // second-half codes and words
  const uint32_t b0 = lds_addr(&st.B[kb + r0 * CPR + code_chunk<BITS>(r0, half * (CPR / 2))]);
  const uint32_t b1 = lds_addr(&st.B[kb + r1 * CPR + code_chunk<BITS>(r1, half * (CPR / 2))]);
  const uint32_t s0 = lds_addr(&st.S[ks + r0]), s1 = lds_addr(&st.S[ks + r1]);
  if constexpr (BITS == 4) {
    asm volatile(
        "ds_read_b128 %0, %12\n\t"
        "ds_read_b128 %1, %13\n\t"
        "ds_read_b128 %2, %14\n\t"
        "ds_read_b128 %3, %15\n\t"
        "ds_read_b128 %4, %16\n\t"
        "ds_read_b128 %5, %17\n\t"
        "ds_read_b128 %6, %18\n\t"
        "ds_read_b128 %7, %19\n\t"
        "ds_read_b128 %8, %20\n\t"
        "ds_read_b128 %9, %21\n\t"
        "ds_read_b32 %10, %22\n\t"
        "ds_read_b32 %11, %23\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(f.a[0][0]), "=&v"(f.a[0][1]), "=&v"(f.a[1][0]), "=&v"(f.a[1][1]),
          "=&v"(a2[0][0]), "=&v"(a2[0][1]), "=&v"(a2[1][0]), "=&v"(a2[1][1]),
          "=&v"(f.q[0][0]), "=&v"(f.q[1][0]), "=&v"(f.sb[0]), "=&v"(f.sb[1])
        : "v"(a00), "v"(a01), "v"(a10), "v"(a11), "v"(c00), "v"(c01), "v"(c10), "v"(c11),
          "v"(b0), "v"(b1), "v"(s0), "v"(s1)
        : "memory");
  } else {
    asm volatile(
        "ds_read_b128 %0, %14\n\t"
        "ds_read_b128 %1, %15\n\t"
        "ds_read_b128 %2, %16\n\t"
        "ds_read_b128 %3, %17\n\t"
        "ds_read_b128 %4, %18\n\t"
        "ds_read_b128 %5, %19\n\t"
        "ds_read_b128 %6, %20\n\t"
        "ds_read_b128 %7, %21\n\t"
        "ds_read_b128 %8, %22\n\t"
        "ds_read_b128 %9, %22 offset:16\n\t"
        "ds_read_b128 %10, %23\n\t"
        "ds_read_b128 %11, %23 offset:16\n\t"
        "ds_read_b32 %12, %24\n\t"
        "ds_read_b32 %13, %25\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(f.a[0][0]), "=&v"(f.a[0][1]), "=&v"(f.a[1][0]), "=&v"(f.a[1][1]),
          "=&v"(a2[0][0]), "=&v"(a2[0][1]), "=&v"(a2[1][0]), "=&v"(a2[1][1]),
          "=&v"(f.q[0][0]), "=&v"(f.q[0][1]), "=&v"(f.q[1][0]), "=&v"(f.q[1][1]),
          "=&v"(f.sb[0]), "=&v"(f.sb[1])
        : "v"(a00), "v"(a01), "v"(a10), "v"(a11), "v"(c00), "v"(c01), "v"(c10), "v"(c11),
          "v"(b0), "v"(b1), "v"(s0), "v"(s1)
        : "memory");
  }
}

// MFMA operand of K step ks from the lane's codes of one weight row.
template <int BITS>
__device__ __forceinline__ u32x4 gu_bfrag(const u32x4 (&q)[BITS / 4], int ks) {
  if constexpr (BITS == 4) {
    const uint32_t d = ks == 0 ? q[0].x : ks == 1 ? q[0].y : ks == 2 ? q[0].z : q[0].w;
    return code_frag4(d);
  } else {
    const u32x4 v = q[ks >> 1];
    return (ks & 1) ? code_frag8(v.z, v.w) : code_frag8(v.x, v.y);
  }
}

// One K stage: wait for this stage's loads (the later stages' stay in
// flight); read K steps 0-1 with the codes, multiply; read K steps 2-3,
// barrier (after which the stage may be refilled: `refill` runs there),
// multiply; scale the group's sums into C.
template <int BITS, typename F>
__device__ __forceinline__ void gu_stage(const GuStage<BITS>& st, int later, int wm, int wn,
                                         int l32, int half, int khalf, f32x16 (&C)[2][2],
                                         F&& refill) {
  constexpr int L = gu_stage_loads<BITS>();
  static_assert(kStages == 3, "wait ladder below covers kStages - 1 = 2 later stages");
  if (later >= 2) wait_vm<2 * L>();
  else if (later == 1) wait_vm<L>();
  else wait_vm<0>();
  lds_barrier();
  GuFrags<BITS> f;
  const f32x16 zero = {};
  f32x16 acc[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = zero;
  // all of the stage's operands in one read, then the stage may be refilled
  // before its MFMAs
  u32x4 a2[2][2];
  gu_read_all<BITS>(st, wm, wn, l32, half, khalf, f, a2);
  lds_barrier();
  refill();
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    u32x4 b[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) b[nb] = gu_bfrag<BITS>(f.q[nb], kk);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        acc[mb][nb] = mfma(kk < 2 ? f.a[mb][kk & 1] : a2[mb][kk & 1], b[nb], acc[mb][nb]);
  }
  const float scl[2] = {code_scale<BITS>(f.sb[0]), code_scale<BITS>(f.sb[1])};
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) C[mb][nb][r] += scl[nb] * acc[mb][nb][r];
}

// fp32 h tile halves in a stage's activation buffer: 64 rows x 64 floats,
// 4-float chunks XOR-swizzled by the row.
__device__ __forceinline__ void ht_store(StageBuf& buf, const f32x16 (&C)[2][2], int wn, int l32,
                                         int half) {
  float* ht = reinterpret_cast<float*>(&buf[0]);
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 32 * mb + 8 * (r / 4) + 4 * half + (r % 4);  // row inside the half
      const float gv = C[mb][0][r], uv = C[mb][1][r];
      const int col = 32 * wn + l32;
      ht[m * 64 + (((col >> 2) ^ (m & 15)) << 2) + (col & 3)] = gv / (1.0f + __expf(-gv)) * uv;
    }
}
__device__ __forceinline__ void ht_load(const StageBuf& buf, int lr, int sc, float (&v)[32]) {
  const float* hr = reinterpret_cast<const float*>(&buf[0]);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const float4 t =
        *reinterpret_cast<const float4*>(hr + lr * 64 + (((8 * sc + q) ^ (lr & 15)) << 2));
    v[4 * q] = t.x;
    v[4 * q + 1] = t.y;
    v[4 * q + 2] = t.z;
    v[4 * q + 3] = t.w;
  }
}

// One gate/up tile: 128 bucket rows x (64 gate + 64 up weight rows = 64 h
// columns).  Waves (wm, wn) = (wave / 2, wave % 2) own rows 64 wm .. +63 and
// h columns 32 wn .. +31 (block 0 gate, block 1 up).
template <int BITS>
__device__ __forceinline__ void prefill_gateup_item(MOE_PGU_PARAMS, GuStage<BITS>& s0,
                                                    GuStage<BITS>& s1, GuStage<BITS>& s2,
                                                    int32_t* rowsrc, XcdItem it) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31, half = lane >> 5;
  const TileInfo ti = get_tile(tiles, counts, offsets, it.tile, E);
  const bool shared = ti.e == E;
  const int inter = shared ? Is : I;
  const int n0 = it.nb * kGroup;
  if (n0 >= inter) return;
  const uint8_t* sec = shared ? shared_blob : slab + (int64_t)slot_table[ti.e] * stride;
  const int64_t unit_b = shared ? gu_unit_s : gu_unit_r, tile_b = shared ? gu_tile_s : gu_tile_r;
  if (tid < kMT) {
    int src = -1;
    if (tid < ti.rows) src = shared ? ti.base + tid : pairs[ti.base + tid] / k;
    rowsrc[tid] = src;
  }
  __syncthreads();
  const int G = H / kGroup;
  // A tile of at most 64 rows splits K between the wave rows: waves 0-1
  // (wm = 0) take groups 0 .. G/2-1 of rows 0..63, waves 2-3 (wm = 1) groups
  // G/2 .. G-1 of the same rows, held as LDS rows 64..127 of each stage; the
  // halves are added before the epilogue.  (G/2 a multiple of the groups per
  // k-block, so a stage's two groups sit at one k-block distance apart.)
  constexpr int GPK = kRowBytes * (8 / BITS) / kGroup;
  const bool split = ti.rows <= 64 && G % (2 * GPK) == 0;
  const int Gs = split ? G / 2 : G;
  const int khalf = split ? wm : 0;

  // load roles (fixed for the tile)
  GuSrc<BITS> P;
  P.x = reinterpret_cast<const uint8_t*>(x);
  P.sec = sec;
  P.unit_b = unit_b;
  P.g2off = split ? G / 2 : 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // activation chunk j*256 + tid: LDS row ch / 8, slot ch % 8 holds column
    // chunk (slot ^ ((row >> 1) & 7)); rows past the tile read row 0's token
    // (their results are discarded).  Split: LDS row r >= 64 holds token row
    // r - 64 at the second-half group.
    const int ch = j * 256 + tid, r = ch >> 3, c = (ch & 7) ^ ((r >> 1) & 7);
    const bool hi = split && r >= 64;
    const int tr = hi ? r - 64 : r;
    const int src = tr < ti.rows ? rowsrc[tr] : rowsrc[0];
    P.a[j] = (uint32_t)(((int64_t)src * H + c * 8) * 2 + (hi ? (G / 2) * kGroup * 2 : 0));
  }
  {
    constexpr int CPR = kGroup * BITS / 8 / 16;  // 16-byte code chunks per row and group
#pragma unroll
    for (int j = 0; j < BITS / 4; ++j) {
      const int ch = j * 256 + tid, rr = ch / CPR, c = code_chunk<BITS>(rr, ch % CPR);
      const RowAddr<BITS> ra(sec, unit_b, tile_b, 2, rr >> 6, n0 + (rr & 63), 0);
      P.b[j] = (uint32_t)(ra.codes - sec) + c * 16;
    }
    // (scale, bias) words: lane `tid` of rows 0..127; rows 128..255 repeat
    // them, or with the split hold the second-half group's (G/2 groups on)
    const int rr = tid & 127;
    const RowAddr<BITS> ra(sec, unit_b, tile_b, 2, rr >> 6, n0 + (rr & 63), 0);
    P.sb = (uint32_t)(ra.sb - sec) +
           ((split && tid >= 128) ? (uint32_t)((G / 2 / GPK) * unit_b) : 0u);
  }
  const int wv = __builtin_amdgcn_readfirstlane(wave);

  f32x16 C[2][2];
  const f32x16 zero = {};
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) C[mb][nb] = zero;

  // Stage t lives in s[t % kStages]: it is multiplied at step t and its
  // buffer is refilled with stage t + kStages right after.  The first pass
  // (g < 0) only issues stages 0 .. kStages-1, from the same instructions as
  // the steady state, so that the compiler sees one set of loads in flight.
  for (int g = -kStages; g < Gs; g += kStages) {
#define MOE_GU_STEP(I, BUF)                                                              \
  if (g + I >= Gs) break;                                                                \
  {                                                                                      \
    auto refill = [&]() {                                                                \
      if (g + I + kStages < Gs) gu_issue<BITS>(P, BUF, g + I + kStages, wv);             \
    };                                                                                   \
    if (g >= 0) gu_stage<BITS>(BUF, min(kStages - 1, Gs - 1 - g - I), wm, wn, l32, half,  \
                               khalf, C, refill);                                        \
    else refill();                                                                       \
  }
    MOE_GU_STEP(0, s0)
    MOE_GU_STEP(1, s1)
    MOE_GU_STEP(2, s2)
#undef MOE_GU_STEP
  }

  // split K: the wm = 1 waves' sums (second half of K for rows 0..63) are
  // added to the wm = 0 waves' through LDS (stage 0's activations for wn = 0,
  // stage 1's for wn = 1; separate branches so that every LDS access names
  // its object)
  if (split) {
    __syncthreads();  // every wave is done with the stage buffers
    if (wm == 1) {
      if (wn == 0) {
        float* rd = reinterpret_cast<float*>(&s0.A[0]);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) rd[((mb * 2 + nb) * 16 + r) * 64 + lane] = C[mb][nb][r];
      } else {
        float* rd = reinterpret_cast<float*>(&s1.A[0]);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) rd[((mb * 2 + nb) * 16 + r) * 64 + lane] = C[mb][nb][r];
      }
    }
    __syncthreads();
    if (wm == 0) {
      if (wn == 0) {
        const float* rd = reinterpret_cast<const float*>(&s0.A[0]);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) C[mb][nb][r] += rd[((mb * 2 + nb) * 16 + r) * 64 + lane];
      } else {
        const float* rd = reinterpret_cast<const float*>(&s1.A[0]);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) C[mb][nb][r] += rd[((mb * 2 + nb) * 16 + r) * 64 + lane];
      }
    }
    __syncthreads();  // before the epilogue reuses the stage buffers
  }

  // bias terms from the group sums of the activation rows
  {
    const RowAddr<BITS> wr[2] = {RowAddr<BITS>(sec, unit_b, tile_b, 2, 0, n0 + 32 * wn + l32, half),
                                 RowAddr<BITS>(sec, unit_b, tile_b, 2, 1, n0 + 32 * wn + l32, half)};
    const float* srow[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int src = rowsrc[64 * wm + 32 * mb + l32];
      srow[mb] = src >= 0 ? xsum + (int64_t)src * G : nullptr;
    }
    bias_mfma<BITS>(srow, wr, G, half, C);
  }

  // epilogue: h = silu(g) * u into fp32 LDS tiles (rows 0..63 in stage 0's
  // activation buffer, 64..127 in stage 1's; separate branches so that every
  // LDS access names its object)
  if (wm == 0) ht_store(s0.A, C, wn, l32, half);
  else ht_store(s1.A, C, wn, l32, half);
  __syncthreads();
  // row sr, columns 32 sc .. 32 sc + 31: the tile's scale (largest |h| of
  // its rows to [2^13, 2^14)), the scaled values in fp16, their group sum
  const int sr = tid >> 1, sc = tid & 1;
  float v[32];
  if (sr < 64) ht_load(s0.A, sr, sc, v);
  else ht_load(s1.A, sr & 63, sc, v);
  uint32_t amax = 0u;
  if (sr < ti.rows) {
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = max(amax, __float_as_uint(v[i]) & 0x7FFFFFFFu);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, off, 64));
  __shared__ uint32_t wmax[4];
  if (lane == 0) wmax[wave] = amax;
  __syncthreads();
  amax = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  const int ex = max((int)(amax >> 23), 14);
  const float down = __uint_as_float((uint32_t)(267 - ex) << 23);  // 2^(140 - ex)
  const float up = __uint_as_float((uint32_t)(ex - 13) << 23);     // 2^(ex - 140)
  _Float16 hv[32];
  float part = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    hv[i] = (_Float16)(v[i] * down);
    part += (float)hv[i];
  }
  part *= up;
  const float other = __shfl_xor(part, 1, 64);
  const float total = sc == 0 ? part + other : other + part;
  if (sr < ti.rows) {
    const int gi = n0 / kGroup;
    int64_t hrow, srow_i;
    if (shared) {
      hrow = (int64_t)T * k * 2 * I + (int64_t)(ti.base + sr) * 2 * Is;
      srow_i = (int64_t)T * k * (I / kGroup) + (int64_t)(ti.base + sr) * (Is / kGroup) + gi;
    } else {
      hrow = (int64_t)(ti.base + sr) * 2 * I;
      srow_i = (int64_t)(ti.base + sr) * (I / kGroup) + gi;
    }
    if (sc == 0) {
      hsum[srow_i] = total;
      *reinterpret_cast<float*>(h + hrow + inter + 2 * gi) = up;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t w4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w4[j] = (uint32_t)__builtin_bit_cast(uint16_t, hv[8 * q + dn_perm<BITS>(2 * j)]) |
                ((uint32_t)__builtin_bit_cast(uint16_t, hv[8 * q + dn_perm<BITS>(2 * j + 1)]) << 16);
      *reinterpret_cast<u32x4*>(h + hrow + n0 + 32 * sc + 8 * q) = u32x4{w4[0], w4[1], w4[2], w4[3]};
    }
  }
}

// ---------------------------------------------------------------------------
// down: grid (H/128 column blocks, tiles).  A = h in scaled fp16, B = the
// codes in fp16, one MFMA per K step and output block.  Writes the weighted expert output of every bucket entry
// to partial[(t*(k+1) + j) * H + col] (fp32; the shared expert is j = k).

#define MOE_PDN_PARAMS                                                                       \
  const uint16_t* __restrict__ h, const float* __restrict__ hsum,                              \
      const int32_t* __restrict__ pairs, const float* __restrict__ topk_w,                    \
      const float* __restrict__ gamma, const int32_t* __restrict__ counts,                    \
      const int32_t* __restrict__ offsets, const int32_t* __restrict__ tiles,                 \
      const int32_t* __restrict__ ntiles, const uint8_t* __restrict__ slab,                   \
      const int32_t* __restrict__ slot_table, int64_t stride,                                 \
      const uint8_t* __restrict__ shared_blob, float* __restrict__ partial, int T, int H, int E, \
      int k, int I, int Is, int64_t d_off_r, int64_t d_unit_r, int64_t d_tile_r,                \
      int64_t d_off_s, int64_t d_unit_s, int64_t d_tile_s, int nbg
#define MOE_PDN_ARGS                                                                           \
  h, hsum, pairs, topk_w, gamma, counts, offsets, tiles, ntiles, slab, slot_table, stride,      \
      shared_blob, partial, T, H, E, k, I, Is, d_off_r, d_unit_r, d_tile_r, d_off_s, d_unit_s, \
      d_tile_s, nbg

// Down K pipeline: the same scheme as gate/up with 512 threads and a
// 128-row x 256-column tile; a stage holds the 128 h rows (fp16) and the
// 256 output rows' codes and (scale, bias) words.
constexpr int kDnThreads = 512;
constexpr int kDnCols = 256;

template <int BITS>
struct DnStage {
  uint4 Ah[kStageChunks];
  // codes of the stage's group, then of the second-half group when the wave
  // rows split K (else a copy)
  uint4 B[2 * kDnCols * (kGroup * BITS / 8) / 16];
  uint32_t S[kDnThreads];  // (scale, bias) of rows 0..255, then of the second-half group
};

template <int BITS>
constexpr int dn_stage_loads() { return 2 + 2 * (BITS / 4) + 1; }

template <int BITS>
struct DnSrc {
  const uint8_t* h;    // h rows of the tile (uniform base)
  const uint8_t* sec;  // blob down section (uniform)
  int64_t unit_b;
  uint32_t a[2];       // h chunk offsets (stage 0, hi part)
  uint32_t b[BITS / 4];  // code chunk offsets (k-block 0, group 0)
  uint32_t sb;         // (scale, bias) word offset
  int g2off;           // second-half group of a stage: g + g2off (uniform)
};

template <int BITS>
__device__ __forceinline__ void dn_issue(const DnSrc<BITS>& P, DnStage<BITS>& st, int g,
                                         int wave) {
  constexpr int GPK = kRowBytes * (8 / BITS) / kGroup;
  constexpr int GBYTES = kGroup * BITS / 8;
  const uint8_t* ha = P.h + (int64_t)g * kGroup * 2;
#pragma unroll
  for (int j = 0; j < 2; ++j)
    __builtin_amdgcn_global_load_lds(MOE_G1(ha + P.a[j]), MOE_L3(&st.Ah[j * 512 + wave * 64]), 16,
                                     0, 0);
  const uint8_t* wb = P.sec + (int64_t)(g / GPK) * P.unit_b + (g % GPK) * GBYTES;
#pragma unroll
  for (int j = 0; j < BITS / 4; ++j)
    __builtin_amdgcn_global_load_lds(MOE_G1(wb + P.b[j]), MOE_L3(&st.B[j * 512 + wave * 64]), 16,
                                     0, 0);
  const int g2 = g + P.g2off;
  const uint8_t* wb2 = P.sec + (int64_t)(g2 / GPK) * P.unit_b + (g2 % GPK) * GBYTES;
#pragma unroll
  for (int j = 0; j < BITS / 4; ++j)
    __builtin_amdgcn_global_load_lds(MOE_G1(wb2 + P.b[j]),
                                     MOE_L3(&st.B[(BITS / 4 + j) * 512 + wave * 64]), 16, 0, 0);
  const uint8_t* sbb = P.sec + (int64_t)(g / GPK) * P.unit_b + (g % GPK) * 4;
  __builtin_amdgcn_global_load_lds(MOE_G1(sbb + P.sb), MOE_L3(&st.S[wave * 64]), 4, 0, 0);
}

template <int BITS>
struct DnFrags {
  u32x4 ah[2][2];  // A operands of two K steps, both row blocks
  u32x4 q[2][BITS / 4];
  uint32_t sb[2];
};

// A operands of K steps k0, k0+1 (both row blocks); with CODES
// also the lane's codes and (scale, bias) words of both output rows.
template <int BITS, bool CODES>
__device__ __forceinline__ void dn_read(const DnStage<BITS>& st, int k0, int wm, int wn, int l32,
                                        int half, int khalf, DnFrags<BITS>& f) {
  const int i00 = swz(64 * wm + l32, 4 * half + k0), i01 = swz(64 * wm + l32, 4 * half + k0 + 1);
  const int i10 = swz(64 * wm + 32 + l32, 4 * half + k0);
  const int i11 = swz(64 * wm + 32 + l32, 4 * half + k0 + 1);
  const uint32_t h00 = lds_addr(&st.Ah[i00]), h01 = lds_addr(&st.Ah[i01]);
  const uint32_t h10 = lds_addr(&st.Ah[i10]), h11 = lds_addr(&st.Ah[i11]);
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(f.ah[0][0]), "=&v"(f.ah[0][1]), "=&v"(f.ah[1][0]), "=&v"(f.ah[1][1])
      : "v"(h00), "v"(h01), "v"(h10), "v"(h11)
      : "memory");
  if constexpr (CODES) {
    const int r0 = 64 * wn + l32, r1 = 64 * wn + 32 + l32;
    constexpr int CPR = kGroup * BITS / 8 / 16;
    const int kb = khalf * kDnCols * CPR, ks = khalf * kDnCols;  // second-half codes, words
    const uint32_t b0 = lds_addr(&st.B[kb + r0 * CPR + code_chunk<BITS>(r0, half * (CPR / 2))]);
    const uint32_t b1 = lds_addr(&st.B[kb + r1 * CPR + code_chunk<BITS>(r1, half * (CPR / 2))]);
    const uint32_t s0 = lds_addr(&st.S[ks + r0]), s1 = lds_addr(&st.S[ks + r1]);
    if constexpr (BITS == 4) {
      asm volatile(
          "ds_read_b128 %0, %4\n\t"
          "ds_read_b128 %1, %5\n\t"
          "ds_read_b32 %2, %6\n\t"
          "ds_read_b32 %3, %7\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(f.q[0][0]), "=&v"(f.q[1][0]), "=&v"(f.sb[0]), "=&v"(f.sb[1])
          : "v"(b0), "v"(b1), "v"(s0), "v"(s1)
          : "memory");
    } else {
      asm volatile(
          "ds_read_b128 %0, %6\n\t"
          "ds_read_b128 %1, %6 offset:16\n\t"
          "ds_read_b128 %2, %7\n\t"
          "ds_read_b128 %3, %7 offset:16\n\t"
          "ds_read_b32 %4, %8\n\t"
          "ds_read_b32 %5, %9\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(f.q[0][0]), "=&v"(f.q[0][1]), "=&v"(f.q[1][0]), "=&v"(f.q[1][1]),
            "=&v"(f.sb[0]), "=&v"(f.sb[1])
          : "v"(b0), "v"(b1), "v"(s0), "v"(s1)
          : "memory");
    }
  }
}

// MFMA operand of K step ks from the lane's codes of one output row, in
// the down GEMM's fp16 K order.
template <int BITS>
__device__ __forceinline__ u32x4 dn_bfrag(const u32x4 (&q)[BITS / 4], int ks) {
  if constexpr (BITS == 4) {
    const uint32_t d = ks == 0 ? q[0].x : ks == 1 ? q[0].y : ks == 2 ? q[0].z : q[0].w;
    return code_frag4_f16(d);
  } else {
    const u32x4 v = q[ks >> 1];
    return (ks & 1) ? code_frag8_f16(v.z, v.w) : code_frag8_f16(v.x, v.y);
  }
}

// hs: the inverse of the h scale of this stage's group (in LDS, read after
// the stage barrier).
template <int BITS, typename F>
__device__ __forceinline__ void dn_stage(const DnStage<BITS>& st, int later, int wm, int wn,
                                         int l32, int half, int khalf, f32x16 (&C)[2][2],
                                         F&& refill, const float* hs) {
  constexpr int L = dn_stage_loads<BITS>();
  static_assert(kStages == 3, "wait ladder below covers kStages - 1 = 2 later stages");
  if (later >= 2) wait_vm<2 * L>();
  else if (later == 1) wait_vm<L>();
  else wait_vm<0>();
  lds_barrier();
  DnFrags<BITS> f;
  const f32x16 zero = {};
  f32x16 acc[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = zero;
  dn_read<BITS, true>(st, 0, wm, wn, l32, half, khalf, f);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    if (kk == 2) {
      dn_read<BITS, false>(st, 2, wm, wn, l32, half, khalf, f);
      lds_barrier();
      refill();
    }
    u32x4 b[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) b[nb] = dn_bfrag<BITS>(f.q[nb], kk);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma_f16(f.ah[mb][kk & 1], b[nb], acc[mb][nb]);
  }
  const float hsc = *hs;
  const float scl[2] = {code_scale<BITS>(f.sb[0]) * hsc, code_scale<BITS>(f.sb[1]) * hsc};
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) C[mb][nb][r] += scl[nb] * acc[mb][nb][r];
}

// One down tile: 128 bucket rows x 256 output columns (down weight rows
// n0 .. n0+255).  Wave (wm, wn) = (wave / 4, wave % 4) owns rows
// 64 wm .. +63 and columns 64 wn .. +63 (two blocks of 32).  Writes
// roww * (h . Wd^T) of every row to its partial row.
template <int BITS>
__device__ __forceinline__ void prefill_down_item(MOE_PDN_PARAMS, DnStage<BITS>& s0,
                                                  DnStage<BITS>& s1, DnStage<BITS>& s2,
                                                  int32_t* rowdst, float* roww, float* hsl,
                                                  XcdItem it) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3, l32 = lane & 31, half = lane >> 5;
  const TileInfo ti = get_tile(tiles, counts, offsets, it.tile, E);
  const bool shared = ti.e == E;
  const int inter = shared ? Is : I;
  const int n0 = it.nb * kDnCols;
  const uint8_t* sec = shared ? shared_blob + d_off_s
                              : slab + (int64_t)slot_table[ti.e] * stride + d_off_r;
  const int64_t unit_b = shared ? d_unit_s : d_unit_r, tile_b = shared ? d_tile_s : d_tile_r;
  if (tid < kMT) {
    int dst = -1;
    float wv = 0.f;
    if (tid < ti.rows) {
      if (shared) {
        const int t = ti.base + tid;
        dst = t * (k + 1) + k;
        wv = gamma[t];
      } else {
        const int p = pairs[ti.base + tid];
        dst = (p / k) * (k + 1) + (p % k);
        wv = topk_w[p];
      }
    }
    rowdst[tid] = dst;
    roww[tid] = wv;
  }
  const int G = inter / kGroup;
  // h rows and group-sum rows of the tile
  const int64_t hbase = shared ? (int64_t)T * k * 2 * I + (int64_t)ti.base * 2 * Is
                               : (int64_t)ti.base * 2 * I;
  // the inverse h scale of each group of the tile (stored with its first row)
  if (tid < G) hsl[tid] = *reinterpret_cast<const float*>(h + hbase + inter + 2 * tid);
  const int64_t sbase = shared ? (int64_t)T * k * (I / kGroup) + (int64_t)ti.base * G
                               : (int64_t)ti.base * G;

  // A tile of at most 64 rows splits K between the wave rows, as in the
  // gate/up GEMM: waves 0-3 take groups 0 .. G/2-1 of rows 0..63, waves 4-7
  // groups G/2 .. G-1 of the same rows (LDS rows 64..127); the halves are
  // added before the bias term.
  constexpr int GPK = kRowBytes * (8 / BITS) / kGroup;
  const bool split = ti.rows <= 64 && G % (2 * GPK) == 0;
  const int Gs = split ? G / 2 : G;
  const int khalf = split ? wm : 0;
  DnSrc<BITS> P;
  P.h = reinterpret_cast<const uint8_t*>(h + hbase);
  P.sec = sec;
  P.unit_b = unit_b;
  P.g2off = split ? G / 2 : 0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int ch = j * 512 + tid, r = ch >> 3, c = (ch & 7) ^ ((r >> 1) & 7);
    const bool hi = split && r >= 64;
    const int tr = hi ? r - 64 : r;
    const int rr = tr < ti.rows ? tr : 0;  // rows past the tile read row 0 (discarded)
    P.a[j] = (uint32_t)(((int64_t)rr * 2 * inter + c * 8) * 2 + (hi ? (G / 2) * kGroup * 2 : 0));
  }
  {
    constexpr int CPR = kGroup * BITS / 8 / 16;
#pragma unroll
    for (int j = 0; j < BITS / 4; ++j) {
      const int ch = j * 512 + tid, rr = ch / CPR, c = code_chunk<BITS>(rr, ch % CPR);
      const RowAddr<BITS> ra(sec, unit_b, tile_b, 1, 0, n0 + rr, 0);
      P.b[j] = (uint32_t)(ra.codes - sec) + c * 16;
    }
    // (scale, bias) words of rows 0..255; threads 256..511 repeat them, or
    // with the split load the second-half group's
    const RowAddr<BITS> ra(sec, unit_b, tile_b, 1, 0, n0 + (tid & (kDnCols - 1)), 0);
    P.sb = (uint32_t)(ra.sb - sec) +
           ((split && tid >= kDnCols) ? (uint32_t)((G / 2 / GPK) * unit_b) : 0u);
  }
  const int wv = __builtin_amdgcn_readfirstlane(wave);

  f32x16 C[2][2];
  const f32x16 zero = {};
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) C[mb][nb] = zero;

  const int hofs = khalf * (G / 2);  // this wave's groups of the per-group h scales
  for (int g = -kStages; g < Gs; g += kStages) {
#define MOE_DN_STEP(I, BUF)                                                              \
  if (g + I >= Gs) break;                                                                \
  {                                                                                      \
    auto refill = [&]() {                                                                \
      if (g + I + kStages < Gs) dn_issue<BITS>(P, BUF, g + I + kStages, wv);             \
    };                                                                                   \
    if (g >= 0) dn_stage<BITS>(BUF, min(kStages - 1, Gs - 1 - g - I), wm, wn, l32, half,  \
                               khalf, C, refill, hsl + g + I + hofs);                    \
    else refill();                                                                       \
  }
    MOE_DN_STEP(0, s0)
    MOE_DN_STEP(1, s1)
    MOE_DN_STEP(2, s2)
#undef MOE_DN_STEP
  }
  __syncthreads();

  // split K: the wm = 1 waves' sums (second half of K for rows 0..63) are
  // added to the wm = 0 waves' through LDS, one 16 KiB buffer per column
  // wave: stage 0, 1 and 2's activation buffers and stage 0's codes
  // (separate branches so that every LDS access names its object)
  if (split) {
#define MOE_DN_RED(BUFEXPR, OP)                                                          \
  {                                                                                      \
    float* rd = reinterpret_cast<float*>(BUFEXPR);                                       \
    _Pragma("unroll") for (int mb = 0; mb < 2; ++mb)                                     \
    _Pragma("unroll") for (int nb = 0; nb < 2; ++nb)                                     \
    _Pragma("unroll") for (int r = 0; r < 16; ++r) OP;                                   \
  }
#define MOE_DN_IDX (((mb * 2 + nb) * 16 + r) * 64 + lane)
    if (wm == 1) {
      if (wn == 0) MOE_DN_RED(&s0.Ah[0], rd[MOE_DN_IDX] = C[mb][nb][r])
      else if (wn == 1) MOE_DN_RED(&s1.Ah[0], rd[MOE_DN_IDX] = C[mb][nb][r])
      else if (wn == 2) MOE_DN_RED(&s2.Ah[0], rd[MOE_DN_IDX] = C[mb][nb][r])
      else MOE_DN_RED(&s0.B[0], rd[MOE_DN_IDX] = C[mb][nb][r])
    }
    __syncthreads();
    if (wm == 0) {
      if (wn == 0) MOE_DN_RED(&s0.Ah[0], C[mb][nb][r] += rd[MOE_DN_IDX])
      else if (wn == 1) MOE_DN_RED(&s1.Ah[0], C[mb][nb][r] += rd[MOE_DN_IDX])
      else if (wn == 2) MOE_DN_RED(&s2.Ah[0], C[mb][nb][r] += rd[MOE_DN_IDX])
      else MOE_DN_RED(&s0.B[0], C[mb][nb][r] += rd[MOE_DN_IDX])
    }
#undef MOE_DN_IDX
#undef MOE_DN_RED
  }

  // bias terms from the group sums of the h rows
  {
    const RowAddr<BITS> wr[2] = {
        RowAddr<BITS>(sec, unit_b, tile_b, 1, 0, n0 + 64 * wn + l32, half),
        RowAddr<BITS>(sec, unit_b, tile_b, 1, 0, n0 + 64 * wn + 32 + l32, half)};
    const float* srow[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int m = 64 * wm + 32 * mb + l32;
      srow[mb] = m < ti.rows ? hsum + sbase + (int64_t)m * G : nullptr;
    }
    bias_mfma<BITS>(srow, wr, G, half, C);
  }

#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = 64 * wm + 32 * mb + 8 * (r / 4) + 4 * half + (r % 4);
        const int dst = rowdst[m];
        if (dst >= 0)
          partial[(int64_t)dst * H + n0 + 64 * wn + 32 * nb + l32] = roww[m] * C[mb][nb][r];
      }
}

// Persistent grids: workgroup w serves XCD w % 8 and walks that XCD's item
// range (see xcd_item) with a stride of gridDim.x / 8.
template <int BITS>
__global__ __launch_bounds__(256, BITS == 4 ? 2 : 1) void prefill_gateup_kernel(MOE_PGU_PARAMS) {
  __shared__ __align__(16) GuStage<BITS> s0;
  __shared__ __align__(16) GuStage<BITS> s1;
  __shared__ __align__(16) GuStage<BITS> s2;
  __shared__ int32_t rowsrc[kMT];
  const int total = *ntiles * nbg;
  const int per = (total + 7) / 8, c = blockIdx.x & 7;
  for (int i = blockIdx.x >> 3; i < per; i += gridDim.x >> 3) {
    const int q = c * per + i;
    if (q >= total) break;
    prefill_gateup_item<BITS>(MOE_PGU_ARGS, s0, s1, s2, rowsrc,
                              XcdItem{q / nbg, q % nbg, true});
    __syncthreads();
  }
}

template <int BITS>
__global__ __launch_bounds__(kDnThreads) void prefill_down_kernel(MOE_PDN_PARAMS) {
  __shared__ __align__(16) DnStage<BITS> s0;
  __shared__ __align__(16) DnStage<BITS> s1;
  __shared__ __align__(16) DnStage<BITS> s2;
  __shared__ int32_t rowdst[kMT];
  __shared__ float roww[kMT];
  __shared__ float hsl[MOE_MAX_INTER / kGroup];
  const int total = *ntiles * nbg;
  const int per = (total + 7) / 8, c = blockIdx.x & 7;
  for (int i = blockIdx.x >> 3; i < per; i += gridDim.x >> 3) {
    const int q = c * per + i;
    if (q >= total) break;
    prefill_down_item<BITS>(MOE_PDN_ARGS, s0, s1, s2, rowdst, roww, hsl,
                            XcdItem{q / nbg, q % nbg, true});
    __syncthreads();
  }
}

template <int BITS>
hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t s) {
  const int hs = a.has_shared ? 1 : 0;
  hipError_t e;
  if (!a.tiles_ready) {
    hipLaunchKernelGGL(tile_list_kernel, dim3(1), dim3(1024), 0, s, a.counts, a.tiles, a.ntiles,
                       a.E, hs, a.max_tiles, a.min_rows);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (!a.xsum_ready && (e = launch_group_sum(a.x, a.xsum, a.T, a.H, s)) != hipSuccess) return e;
  const int nbg = (max(a.I, a.Is) + kGroup - 1) / kGroup;
  const unsigned slots_gu = (unsigned)min((a.max_tiles * nbg + 7) / 8 * 8, kPersistSlots);
  hipLaunchKernelGGL((prefill_gateup_kernel<BITS>), dim3(slots_gu), dim3(256), 0, s, a.x,
                     a.xsum, a.pairs, a.counts, a.offsets, a.tiles, a.ntiles, a.slab, a.slot_table,
                     a.stride, a.shared_blob, a.h, a.hsum, a.T, a.H, a.E, a.k, a.I, a.Is,
                     a.L.gu_unit, a.L.gu_tile, a.Ls.gu_unit, a.Ls.gu_tile, nbg);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int nbd = a.H / kDnCols;
  const unsigned slots_d = (unsigned)min((a.max_tiles * nbd + 7) / 8 * 8, kPersistSlots);
  hipLaunchKernelGGL((prefill_down_kernel<BITS>), dim3(slots_d), dim3(kDnThreads), 0, s,
                     a.h, a.hsum, a.pairs, a.topk_w, a.gamma, a.counts, a.offsets, a.tiles,
                     a.ntiles, a.slab, a.slot_table, a.stride, a.shared_blob, a.partial, a.T, a.H,
                     a.E, a.k, a.I, a.Is, a.L.d_off, a.L.d_unit, a.L.d_tile, a.Ls.d_off,
                     a.Ls.d_unit, a.Ls.d_tile, nbd);
  if ((e = hipGetLastError()) != hipSuccess) return e;
return hipSuccess;
}

}  // namespace

hipError_t launch_group_sum(const uint16_t* x, float* xsum, int T, int H, hipStream_t s) {
  const int64_t nsum = (int64_t)T * (H / kGroup);
  hipLaunchKernelGGL(group_sum_kernel, dim3((unsigned)((nsum + 255) / 256)), dim3(256), 0, s, x,
                     xsum, T, H);
  return hipGetLastError();
}

int prefill_max_tiles(int T, int E, int k, bool has_shared) {
  // sum over buckets of ceil(n_b / kMT) <= sum(n_b) / kMT + number of buckets
  const int64_t rows = (int64_t)T * k + (has_shared ? T : 0);
  return (int)(rows / kMT + E + (has_shared ? 1 : 0) + 1);
}

bool prefill_supported(int act, int H, int I, int Is, bool has_shared) {
  if (act != MOE_ACT_BF16) return false;
  if (H % kDnCols != 0 || I % kGroup != 0 || (has_shared && Is % kGroup != 0)) return false;
  return true;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
  return a.bits == 4 ? launch_prefill_t<4>(a, s) : launch_prefill_t<8>(a, s);
}

}  // namespace moe
