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
// Both GEMMs run on v_mfma_f32_32x32x16_f16 with fp32 accumulation, one
// accumulator chain per 32 x 32 block over the whole K:
//  * each lane dequantises the codes of its own weight rows into fp16 MFMA
//    operands in registers: the code as an exact fp16 value c (int4:
//    1 + q/16; int8: q), then w = S c + B with one packed FMA per two codes,
//    where (S, B) = (16 s, b - 16 s) for int4 and (s, b) for int8 are rounded
//    to fp16 once per group; the group bias is thus folded into the weights;
//  * the gate/up GEMM reads the activations in fp16 after a power-of-two
//    scale per token row (written by the router's top-k kernel), undone on
//    the fp32 results;
//  * the gate/up epilogue writes h in fp16 after a power-of-two scale per
//    (row tile, 128-column block) that puts the block's largest |h| in
//    [2^13, 2^14); the down GEMM brings each group to the largest of its
//    tile's scales by multiplying the group's (S, B) by the ratio (a power of
//    two of at most 1) before rounding, and multiplies the results by that
//    largest scale once.
// The fp16 values of a code word come out of the expansion in a K order
// permuted within each 8-value chunk ((0,4), (1,5), (2,6), (3,7) for int4;
// (0,2), (1,3) per word for int8); the activations and h are stored in the
// same order, so the products pair up.
#include "decode_common.h"
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
// Both GEMMs share one tile shape and K pipeline.  A workgroup of 4 waves
// computes 128 bucket rows x 256 weight rows; wave w owns all 128 rows and
// two 32-row blocks of weight rows (gate/up: gate rows 32 w .. + 31 and the
// up rows of the same h columns; down: output rows 64 w .. + 63), i.e. 4 x 2
// MFMA blocks of 32 x 32 with fp32 accumulators.  K runs one quantisation
// group (64) per stage.  Everything a stage needs arrives by asynchronous
// global->LDS loads (global_load_lds) into a ring of kStages slots: the 128
// activation (or h) rows in fp16, the 256 weight rows' codes and their
// (scale, bias) words; kStages - 1 stages are in flight while one is
// multiplied.  Each lane expands the codes of its own weight rows into fp16
// MFMA operands in registers (every weight row belongs to exactly one wave,
// so each code is expanded once per workgroup).
// Per stage: wait for its loads, barrier; read codes, scales and the first
// half of the activation operands, expand and multiply; read the second
// half, barrier (the slot is then free: it is refilled with the stage
// kStages ahead), expand and multiply.
// LDS layouts (16-byte chunks; verified free of bank conflicts for the reads
// below, at 8 lanes per 128 bytes and at 16 lanes per 256 bytes):
//  * activation row r, K chunk c (8 values) at r*8 + (c ^ f(r)), f(r) =
//    ((r >> 1) & 7) ^ ((r & 1) << 2);
//  * code chunk c of weight row r at r*CPR + (c ^ x(r)) (CPR = 2 for int4,
//    4 for int8; x(r) = ((r >> 2) ^ (r >> 3)) & 1, resp. a 2-bit map of
//    bits 1..3).
// Every LDS access of the K loop is inline asm with its own lgkmcnt wait
// (the compiler's wait accounting for global->LDS loads would otherwise
// drain every load in flight before the first read).
constexpr int kStages = 3;
constexpr int kTileN = 256;    // weight rows per tile
constexpr int kGemmThreads = 256;
constexpr int kHCols = kTileN / 2;  // h columns per gate/up tile

// 16-byte code chunks of one weight row per group: 2 (int4), 4 (int8)
template <int BITS>
constexpr int cpr() { return kGroup * BITS / 8 / 16; }

__device__ __forceinline__ int a_slot(int r, int c) {
  return r * 8 + (c ^ (((r >> 1) & 7) ^ ((r & 1) << 2)));
}
template <int BITS>
__device__ __forceinline__ int b_xor(int r) {
  if constexpr (BITS == 4) return ((r >> 2) ^ (r >> 3)) & 1;
  return ((r >> 2) & 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 1);
}
template <int BITS>
__device__ __forceinline__ int b_slot(int r, int c) {
  return r * cpr<BITS>() + (c ^ b_xor<BITS>(r));
}

template <int BITS>
struct Stage {
  uint4 A[kMT * 8];              // 128 rows x 64 K in fp16
  uint4 B[kTileN * cpr<BITS>()];  // codes of the 256 weight rows
  uint32_t S[kTileN];            // their (scale, bias) words
};
// global->LDS loads per wave and stage with MB live row blocks of 32
template <int BITS, int MB>
constexpr int stage_loads() { return MB + cpr<BITS>() + 1; }

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

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }

// Per-thread load roles of a tile (fixed for its K loop): byte offsets of
// this thread's activation chunks (from the uniform row-block base), code
// chunks and (scale, bias) word (from the weight section's k-block 0).
template <int BITS>
struct LoadRoles {
  uint32_t a[4], b[cpr<BITS>()], s;
};

// Issue one stage: activation chunks from `abase` (+ group offset) of the MB
// live row blocks (load j covers rows 32 j .. 32 j + 31 in every wave), codes
// and words of group g of the weight section.
// Buffer views of a tile's two sources: the activation (or h) rows and the
// weight section.  A stage's loads add the lane's fixed 32-bit offset (its
// load role) to a scalar offset that advances with the group, so they take
// no per-lane address arithmetic; an offset past the view reads zeros.
struct TileSrc {
  __amdgpu_buffer_rsrc_t a, w;
};
__device__ __forceinline__ __amdgpu_buffer_rsrc_t src_view(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// One buffer load of 16 (4) bytes per lane into LDS at `lds` + 16 (4) bytes
// per lane.  (Only the device pass compiles the builtin; the host pass never
// runs it.)
__device__ __forceinline__ void buf_lds16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff,
                                          int soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, MOE_L3(lds), 16, voff, soff, 0, 0);
#endif
}
__device__ __forceinline__ void buf_lds4(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff,
                                         int soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, MOE_L3(lds), 4, voff, soff, 0, 0);
#endif
}

template <int BITS, int MB>
__device__ __forceinline__ void issue_stage(Stage<BITS>& st, const LoadRoles<BITS>& lr,
                                            const TileSrc& src, int64_t unit_b, int g, int wv) {
  constexpr int GPK = kRowBytes * (8 / BITS) / kGroup;
  constexpr int GBYTES = kGroup * BITS / 8;
  const int ao = g * kGroup * 2;
#pragma unroll
  for (int j = 0; j < MB; ++j) buf_lds16(src.a, &st.A[j * 256 + wv * 64], lr.a[j], ao);
  const int ko = (int)((g / GPK) * unit_b);
#pragma unroll
  for (int j = 0; j < cpr<BITS>(); ++j)
    buf_lds16(src.w, &st.B[j * 256 + wv * 64], lr.b[j], ko + (g % GPK) * GBYTES);
  buf_lds4(src.w, &st.S[wv * 64], lr.s, ko + (g % GPK) * 4);
}

// Operand roles of a lane: LDS byte offsets (within a stage) of its A chunks
// for K steps 0..3 (row block 0; block mb adds mb * 4096), of its code
// chunk(s) and (scale, bias) words of weight block 0 (block 1 adds db / ds
// bytes).
struct FragRoles {
  uint32_t a[4], b, s;
};

// (scale, bias) word -> fp16 pairs of w = S c + B (sb_f16), both multiplied
// by `ratio` (a power of two; 1 outside the down GEMM) before rounding.
template <int BITS>
__device__ __forceinline__ void sb_f16_scaled(uint32_t sb, float ratio, f16x2& S2, f16x2& B2) {
  const float sc = bf16_bits_to_f32(sb & 0xFFFFu), bi = bf16_bits_to_f32(sb >> 16);
  const _Float16 S = (_Float16)((BITS == 4 ? 16.0f * sc : sc) * ratio);
  const _Float16 B = (_Float16)((BITS == 4 ? bi - 16.0f * sc : bi) * ratio);
  S2 = f16x2{S, S};
  B2 = f16x2{B, B};
}

__device__ __forceinline__ uint32_t fma_pair(uint32_t c, f16x2 S2, f16x2 B2) {
  return __builtin_bit_cast(uint32_t,
                            __builtin_elementwise_fma(__builtin_bit_cast(f16x2, c), S2, B2));
}

// A 32-bit constant in a VGPR the compiler cannot see through: with both
// operands of a mask-and-merge in VGPRs, the expansions below compile to one
// v_and_or_b32 per output (VOP3 takes no literal operand on this target).
__device__ __forceinline__ uint32_t vgpr_const(uint32_t v) {
  uint32_t r;
  asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(v));
  return r;
}
struct ExpandConsts {
  uint32_t m, o;  // int4: nibble mask at mantissa bits 6..9, 1.0; int8: byte mask, 1024.0
};
template <int BITS>
__device__ __forceinline__ ExpandConsts expand_consts() {
  return BITS == 4 ? ExpandConsts{vgpr_const(0x03C003C0u), vgpr_const(0x3C003C00u)}
                   : ExpandConsts{vgpr_const(0x00FF00FFu), vgpr_const(0x64006400u)};
}

// fp16 weights of K step kk from one lane's codes of a block (int4: the 16
// bytes of its 32 codes; int8: 32 bytes), in the K order of code_frag4_f16 /
// code_frag8_f16 (the same values, computed with the masks in registers)
template <int BITS>
__device__ __forceinline__ u32x4 expand(const u32x4 (&q)[BITS / 4], int kk, f16x2 S2, f16x2 B2,
                                        const ExpandConsts& ec) {
  uint32_t c[4];
  if constexpr (BITS == 4) {
    const uint32_t d = q[0][kk];
    c[0] = ((d << 6) & ec.m) | ec.o;
    c[1] = ((d << 2) & ec.m) | ec.o;
    c[2] = ((d >> 2) & ec.m) | ec.o;
    c[3] = ((d >> 6) & ec.m) | ec.o;
  } else {
    const uint32_t d0 = q[kk >> 1][2 * (kk & 1)], d1 = q[kk >> 1][2 * (kk & 1) + 1];
    const uint32_t w[4] = {d0, d0 >> 8, d1, d1 >> 8};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f16x2 v = __builtin_bit_cast(f16x2, (w[i] & ec.m) | ec.o) - (f16x2){1024, 1024};
      c[i] = __builtin_bit_cast(uint32_t, v);
    }
  }
  return u32x4{fma_pair(c[0], S2, B2), fma_pair(c[1], S2, B2), fma_pair(c[2], S2, B2),
               fma_pair(c[3], S2, B2)};
}

// A operands of K steps k0, k0 + 1 for the MB live row blocks: lane LDS
// addresses p (step k0) and q (k0 + 1) of row block 0 in the stage at byte
// offset SO past them (block mb adds mb * 4096)
template <int MB, uint32_t SO>
__device__ __forceinline__ void read_a_at(uint32_t p, uint32_t q, u32x4 (&a)[2][MB]) {
  static_assert(SO + 4096 * (MB - 1) < 65536, "ds_read offset field");
  if constexpr (MB == 4) {
    asm volatile(
        "ds_read_b128 %0, %8 offset:%10\n\t"
        "ds_read_b128 %1, %8 offset:%11\n\t"
        "ds_read_b128 %2, %8 offset:%12\n\t"
        "ds_read_b128 %3, %8 offset:%13\n\t"
        "ds_read_b128 %4, %9 offset:%10\n\t"
        "ds_read_b128 %5, %9 offset:%11\n\t"
        "ds_read_b128 %6, %9 offset:%12\n\t"
        "ds_read_b128 %7, %9 offset:%13\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a[0][0]), "=&v"(a[0][1]), "=&v"(a[0][2]), "=&v"(a[0][3]), "=&v"(a[1][0]),
          "=&v"(a[1][1]), "=&v"(a[1][2]), "=&v"(a[1][3])
        : "v"(p), "v"(q), "i"(SO + 0), "i"(SO + 4096), "i"(SO + 8192), "i"(SO + 12288)
        : "memory");
  } else if constexpr (MB == 3) {
    asm volatile(
        "ds_read_b128 %0, %6 offset:%8\n\t"
        "ds_read_b128 %1, %6 offset:%9\n\t"
        "ds_read_b128 %2, %6 offset:%10\n\t"
        "ds_read_b128 %3, %7 offset:%8\n\t"
        "ds_read_b128 %4, %7 offset:%9\n\t"
        "ds_read_b128 %5, %7 offset:%10\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a[0][0]), "=&v"(a[0][1]), "=&v"(a[0][2]), "=&v"(a[1][0]), "=&v"(a[1][1]),
          "=&v"(a[1][2])
        : "v"(p), "v"(q), "i"(SO + 0), "i"(SO + 4096), "i"(SO + 8192)
        : "memory");
  } else if constexpr (MB == 2) {
    asm volatile(
        "ds_read_b128 %0, %4 offset:%6\n\t"
        "ds_read_b128 %1, %4 offset:%7\n\t"
        "ds_read_b128 %2, %5 offset:%6\n\t"
        "ds_read_b128 %3, %5 offset:%7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a[0][0]), "=&v"(a[0][1]), "=&v"(a[1][0]), "=&v"(a[1][1])
        : "v"(p), "v"(q), "i"(SO + 0), "i"(SO + 4096)
        : "memory");
  } else {
    static_assert(MB == 1, "1..4 row blocks");
    asm volatile(
        "ds_read_b128 %0, %2 offset:%4\n\t"
        "ds_read_b128 %1, %3 offset:%4\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a[0][0]), "=&v"(a[1][0])
        : "v"(p), "v"(q), "i"(SO + 0)
        : "memory");
  }
}
template <int MB>
__device__ __forceinline__ void read_a(uint32_t base, const FragRoles& fr, int k0,
                                       u32x4 (&a)[2][MB]) {
  read_a_at<MB, 0>(base + fr.a[k0], base + fr.a[k0 + 1], a);
}

// codes and (scale, bias) words of the lane's two weight blocks: lane LDS
// addresses pb (codes) and ps (words) in the stage at byte offset SO past them
template <int BITS, int DB, int DS, uint32_t SO>
__device__ __forceinline__ void read_b_at(uint32_t pb, uint32_t ps, u32x4 (&q)[2][BITS / 4],
                                          uint32_t (&sb)[2]) {
  static_assert(SO + (DB > DS ? DB : DS) < 65536, "ds_read offset field");
  if constexpr (BITS == 4) {
    asm volatile(
        "ds_read_b128 %0, %4 offset:%6\n\t"
        "ds_read_b128 %1, %4 offset:%7\n\t"
        "ds_read_b32 %2, %5 offset:%6\n\t"
        "ds_read_b32 %3, %5 offset:%8\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(q[0][0]), "=&v"(q[1][0]), "=&v"(sb[0]), "=&v"(sb[1])
        : "v"(pb), "v"(ps), "i"(SO), "i"(SO + DB), "i"(SO + DS)
        : "memory");
  } else {
    // the lane's second chunk (2h + 1) sits in the slot whose index differs
    // from its first chunk's (2h) in bit 0 only: byte address ^ 16
    const uint32_t pb2 = pb ^ 16u;
    asm volatile(
        "ds_read_b128 %0, %6 offset:%9\n\t"
        "ds_read_b128 %1, %7 offset:%9\n\t"
        "ds_read_b128 %2, %6 offset:%10\n\t"
        "ds_read_b128 %3, %7 offset:%10\n\t"
        "ds_read_b32 %4, %8 offset:%9\n\t"
        "ds_read_b32 %5, %8 offset:%11\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(q[0][0]), "=&v"(q[0][1]), "=&v"(q[1][0]), "=&v"(q[1][1]), "=&v"(sb[0]),
          "=&v"(sb[1])
        : "v"(pb), "v"(pb2), "v"(ps), "i"(SO), "i"(SO + DB), "i"(SO + DS)
        : "memory");
  }
}
template <int BITS, int DB, int DS>
__device__ __forceinline__ void read_b(uint32_t base, const FragRoles& fr,
                                       u32x4 (&q)[2][BITS / 4], uint32_t (&sb)[2]) {
  read_b_at<BITS, DB, DS, 0>(base + fr.b, base + fr.s, q, sb);
}

// 2 x 2 x MB products of K steps k0, k0 + 1
template <int BITS, int MB>
__device__ __forceinline__ void multiply(const u32x4 (&a)[2][MB], const u32x4 (&q)[2][BITS / 4],
                                         const f16x2 (&S2)[2], const f16x2 (&B2)[2], int k0,
                                         const ExpandConsts& ec, f32x16 (&C)[MB][2]) {
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const u32x4 b = expand<BITS>(q[nb], k0 + t, S2[nb], B2[nb], ec);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) C[mb][nb] = mfma_f16(a[t][mb], b, C[mb][nb]);
    }
}

// The K loop of one tile over G groups.  `ratio(g)` is the factor of the
// group's (scale, bias) pair (the down GEMM's h scale alignment).
// One K stage of ring slot SLOT with the lane's LDS addresses of slot 0 in fa
// (the slot's offset goes into the reads' offset fields).
template <int BITS, int MB, int DB, int DS, int SLOT, typename R>
__device__ __forceinline__ void k_stage(Stage<BITS>* st, const LoadRoles<BITS>& lr,
                                        const FragRoles& fa, const TileSrc& src, int64_t unit_b,
                                        int G, int g, int wv, const ExpandConsts& ec,
                                        f32x16 (&C)[MB][2], R&& ratio) {
  constexpr int L = stage_loads<BITS, MB>();
  constexpr uint32_t SO = SLOT * (uint32_t)sizeof(Stage<BITS>);
  const int later = min(kStages - 1, G - 1 - g);
  if (later >= 2) wait_vm<2 * L>();
  else if (later == 1) wait_vm<L>();
  else wait_vm<0>();
  lds_barrier();
  u32x4 q[2][BITS / 4];
  uint32_t sb[2];
  read_b_at<BITS, DB, DS, SO>(fa.b, fa.s, q, sb);
  f16x2 S2[2], B2[2];
  const float rg = ratio(g);
  sb_f16_scaled<BITS>(sb[0], rg, S2[0], B2[0]);
  sb_f16_scaled<BITS>(sb[1], rg, S2[1], B2[1]);
  u32x4 a[2][MB];
  read_a_at<MB, SO>(fa.a[0], fa.a[1], a);
  multiply<BITS, MB>(a, q, S2, B2, 0, ec, C);
  read_a_at<MB, SO>(fa.a[2], fa.a[3], a);
  lds_barrier();
  if (g + kStages < G) issue_stage<BITS, MB>(st[SLOT], lr, src, unit_b, g + kStages, wv);
  multiply<BITS, MB>(a, q, S2, B2, 2, ec, C);
}

template <int BITS, int MB, int DB, int DS, typename R>
__device__ __forceinline__ void k_loop(Stage<BITS>* st, const LoadRoles<BITS>& lr,
                                       const FragRoles& fr, const TileSrc& src, int64_t unit_b,
                                       int G, int wv, f32x16 (&C)[MB][2], R&& ratio) {
  constexpr int L = stage_loads<BITS, MB>();
  static_assert(kStages == 3, "wait ladder below covers kStages - 1 = 2 later stages");
  const ExpandConsts ec = expand_consts<BITS>();
  for (int g = 0; g < min(kStages, G); ++g) issue_stage<BITS, MB>(st[g], lr, src, unit_b, g, wv);
  constexpr uint32_t kLastSlot = (kStages - 1) * (uint32_t)sizeof(Stage<BITS>);
  if constexpr (kLastSlot + 4096 * (MB - 1) < 65536 && kLastSlot + (DB > DS ? DB : DS) < 65536) {
    // the ring unrolled by its slots: every LDS read adds only an immediate
    // offset to the lane's address in slot 0
    const uint32_t b0 = lds_addr(st);
    FragRoles fa = fr;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) fa.a[kk] += b0;
    fa.b += b0;
    fa.s += b0;
    for (int g = 0; g < G; g += kStages) {
      k_stage<BITS, MB, DB, DS, 0>(st, lr, fa, src, unit_b, G, g, wv, ec, C, ratio);
      if (g + 1 < G)
        k_stage<BITS, MB, DB, DS, 1>(st, lr, fa, src, unit_b, G, g + 1, wv, ec, C, ratio);
      if (g + 2 < G)
        k_stage<BITS, MB, DB, DS, 2>(st, lr, fa, src, unit_b, G, g + 2, wv, ec, C, ratio);
    }
    return;
  }
  for (int g = 0, slot = 0; g < G; ++g, slot = slot == kStages - 1 ? 0 : slot + 1) {
    const int later = min(kStages - 1, G - 1 - g);
    if (later >= 2) wait_vm<2 * L>();
    else if (later == 1) wait_vm<L>();
    else wait_vm<0>();
    lds_barrier();
    const uint32_t base = lds_addr(&st[slot]);
    u32x4 q[2][BITS / 4];
    uint32_t sb[2];
    read_b<BITS, DB, DS>(base, fr, q, sb);
    f16x2 S2[2], B2[2];
    const float rg = ratio(g);
    sb_f16_scaled<BITS>(sb[0], rg, S2[0], B2[0]);
    sb_f16_scaled<BITS>(sb[1], rg, S2[1], B2[1]);
    u32x4 a[2][MB];
    read_a<MB>(base, fr, 0, a);
    multiply<BITS, MB>(a, q, S2, B2, 0, ec, C);
    read_a<MB>(base, fr, 2, a);
    lds_barrier();
    if (g + kStages < G) issue_stage<BITS, MB>(st[slot], lr, src, unit_b, g + kStages, wv);
    multiply<BITS, MB>(a, q, S2, B2, 2, ec, C);
  }
}

// Roles of a tile.  Tile row r of the weights (0..255) maps to the weight
// section row `wrow(r)` of matrix `wmat(r)`.  `arow_off(r)` is the byte
// offset of activation row r from the row-block base.
template <int BITS, typename WR, typename AR>
__device__ __forceinline__ void make_roles(LoadRoles<BITS>& lr, FragRoles& fr, int tid, int l32,
                                           int half, int rb0, const uint8_t* sec, int64_t unit_b,
                                           int64_t tile_b, int nmat, WR&& wrow, AR&& arow_off) {
  constexpr int CPR = cpr<BITS>();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int ch = j * 256 + tid, r = ch >> 3;
    const int c = (ch & 7) ^ (((r >> 1) & 7) ^ ((r & 1) << 2));
    lr.a[j] = arow_off(r) + c * 16;
  }
#pragma unroll
  for (int j = 0; j < CPR; ++j) {
    const int ch = j * 256 + tid, r = ch / CPR;
    const int c = (ch % CPR) ^ b_xor<BITS>(r);
    int mat, row;
    wrow(r, mat, row);
    const RowAddr<BITS> ra(sec, unit_b, tile_b, nmat, mat, row, 0);
    lr.b[j] = (uint32_t)(ra.codes - sec) + c * 16;
  }
  {
    int mat, row;
    wrow(tid, mat, row);
    const RowAddr<BITS> ra(sec, unit_b, tile_b, nmat, mat, row, 0);
    lr.s = (uint32_t)(ra.sb - sec);
  }
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) fr.a[kk] = a_slot(l32, 4 * half + kk) * 16;
  fr.b = b_slot<BITS>(rb0, BITS == 4 ? half : 2 * half) * 16 +
         (uint32_t)offsetof(Stage<BITS>, B);
  fr.s = rb0 * 4 + (uint32_t)offsetof(Stage<BITS>, S);
}

// ---------------------------------------------------------------------------
// gate/up: tile = 128 bucket rows x 128 h columns (gate rows n0 .. n0+127 and
// the same up rows).  Writes per row the tile's 128 h values in fp16 after a
// power-of-two scale that puts the tile's largest |h| in [2^13, 2^14), in the
// K order the down GEMM's weights expand to, and the scale's inverse.  An h
// row keeps the byte stride of the fp32 h rows of the GEMV kernels (4 x inter
// bytes), so buckets of either path index the one h buffer alike; the fp16
// row fills the first half, and the second half holds, per group g, the
// inverse scale as a float at element 2 g.

#define MOE_PGU_PARAMS                                                                       \
  const uint16_t* __restrict__ x16, const int32_t* __restrict__ xe,                            \
      const int32_t* __restrict__ pairs, const int32_t* __restrict__ counts,                  \
      const int32_t* __restrict__ offsets, const int32_t* __restrict__ tiles,                 \
      const int32_t* __restrict__ ntiles, const uint8_t* __restrict__ slab,                   \
      const int32_t* __restrict__ slot_table, int64_t stride,                                 \
      const uint8_t* __restrict__ shared_blob, uint16_t* __restrict__ h, int T, int H, int E,  \
      int k, int I, int Is, int64_t gu_unit_r, int64_t gu_tile_r, int64_t gu_unit_s,          \
      int64_t gu_tile_s, int nbg
#define MOE_PGU_ARGS                                                                        \
  x16, xe, pairs, counts, offsets, tiles, ntiles, slab, slot_table, stride, shared_blob, h, T, \
      H, E, k, I, Is, gu_unit_r, gu_tile_r, gu_unit_s, gu_tile_s, nbg

// slot, within an 8-value chunk of the down GEMM's K order, of natural
// position p (the inverse of dn_perm)
template <int BITS>
__device__ __forceinline__ constexpr int dn_slot(int p) {
  return BITS == 4 ? 2 * (p & 3) + (p >> 2) : dn_perm<8>(p);
}

// Rows of the fp16 h staging tile in LDS: 128 values plus 16 bytes of
// padding (272 bytes), so that a lane's 64 values of one column sit at one
// base address plus immediate offsets and the row reads are conflict free.
constexpr int kHStageRow = 272;
// down epilogue: a wave's 32 x 64 fp32 block staged with rows of 72 floats
// (16-byte aligned rows; a column write's two half-waves, 4 rows apart, fall
// 32 banks apart); the offset given to rows past a tile (the partial buffer
// is kept below 2 GiB), and their row marker
constexpr int kEpRow = 72;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
constexpr uint32_t kDropOffset = 0x80000000u;

// silu(g) * u with a hardware reciprocal (the result is rounded to fp16)
__device__ __forceinline__ float swiglu(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

template <int BITS, int MB>
__device__ __forceinline__ void prefill_gateup_item(MOE_PGU_PARAMS, Stage<BITS>* st,
                                                    int32_t* rowsrc, int32_t* te, uint32_t* wmax,
                                                    const TileInfo& ti, int nb) {
  // (the thread index passes through an empty asm so that nothing derived
  // from it is hoisted out of the persistent loop into spilled registers)
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63, wave = tid >> 6, l32 = lane & 31, half = lane >> 5;
  const bool shared = ti.e == E;
  const int inter = shared ? Is : I;
  const int n0 = nb * kHCols;
  if (n0 >= inter) return;
  const uint8_t* sec = shared ? shared_blob : slab + (int64_t)slot_table[ti.e] * stride;
  const int64_t unit_b = shared ? gu_unit_s : gu_unit_r, tile_b = shared ? gu_tile_s : gu_tile_r;
  if (tid < kMT) {
    int src = -1;
    if (tid < ti.rows) src = shared ? ti.base + tid : pairs[ti.base + tid] / k;
    rowsrc[tid] = src;
  }
  __syncthreads();
  // the rows' activation exponents (needed in the epilogue; the load runs
  // under the K loop)
  const int my_e = tid < kMT ? xe[rowsrc[tid] >= 0 ? rowsrc[tid] : rowsrc[0]] : 0;
  LoadRoles<BITS> lr;
  FragRoles fr;
  // rows past the tile read row 0's token (their results are discarded)
  make_roles<BITS>(
      lr, fr, tid, l32, half, 32 * wave + l32, sec, unit_b, tile_b, 2,
      [&](int r, int& mat, int& row) {
        mat = r >> 7;
        row = n0 + (r & 127);
      },
      [&](int r) {
        const int src = r < ti.rows ? rowsrc[r] : rowsrc[0];
        return (uint32_t)src * (uint32_t)H * 2u;
      });
  f32x16 C[MB][2];
  const f32x16 zero = {};
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) C[mb][0] = C[mb][1] = zero;
  // (views: the fp16 activation rows of all tokens; the section's row tiles
  // of gate and up rows)
  const TileSrc src{src_view(x16, (uint32_t)T * (uint32_t)H * 2u),
                    src_view(sec, (uint32_t)((inter / kRowTile) * tile_b))};
  k_loop<BITS, MB, 128 * cpr<BITS>() * 16, 128 * 4>(
      st, lr, fr, src, unit_b, H / kGroup, __builtin_amdgcn_readfirstlane(wave), C,
      [](int) { return 1.0f; });

  // epilogue: undo the rows' activation scales, h = silu(g) * u
  if (tid < kMT) te[tid] = my_e;
  __syncthreads();  // (every wave is also past the K loop: the ring is free)
  uint32_t amax = 0u;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m0 = 32 * mb + 8 * q + 4 * half;
      const int4 e4 = *reinterpret_cast<const int4*>(&te[m0]);
      const int ev[4] = {e4.x, e4.y, e4.z, e4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float f = exp2i(ev[i]);
        const float hh = swiglu(C[mb][0][4 * q + i] * f, C[mb][1][4 * q + i] * f);
        C[mb][0][4 * q + i] = hh;
        // (rows past the tile computed row 0's token: the same values)
        amax = max(amax, __float_as_uint(hh) & 0x7FFFFFFFu);
      }
    }
  amax = dec::wave_max_dpp(amax);
  if (lane == 0) wmax[wave] = amax;
  __syncthreads();
  amax = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  const int ex = max((int)(amax >> 23), 14);
  const float down = __uint_as_float((uint32_t)(267 - ex) << 23);  // 2^(140 - ex)
  const float up = __uint_as_float((uint32_t)(ex - 13) << 23);     // 2^(ex - 140)
  // stage the tile's fp16 rows in the ring: row m at m * kHStageRow bytes,
  // 16-byte chunk ch at ch * 16, the value of column p of a chunk at slot
  // dn_slot(p)
  uint8_t* hs = reinterpret_cast<uint8_t*>(st);
  {
    const int col = 32 * wave + l32;
    uint16_t* base = reinterpret_cast<uint16_t*>(hs + 4 * half * kHStageRow + (col >> 3) * 16) +
                     dn_slot<BITS>(col & 7);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = 32 * mb + 8 * (r >> 2) + (r & 3);  // minus 4 * half
        base[m * (kHStageRow / 2)] = __builtin_bit_cast(uint16_t, (_Float16)(C[mb][0][r] * down));
      }
  }
  __syncthreads();
  const int64_t hrow0 = shared ? (int64_t)T * k * 2 * I + (int64_t)ti.base * 2 * Is
                               : (int64_t)ti.base * 2 * I;
#pragma unroll
  for (int j = 0; j < 2 * MB; ++j) {
    const int idx = j * 256 + tid, m = idx >> 4, c = idx & 15;
    if (m < ti.rows) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(hs + m * kHStageRow + c * 16);
      *reinterpret_cast<u32x4*>(h + hrow0 + (int64_t)m * 2 * inter + n0 + 8 * c) = v;
    }
  }
  if (tid < ti.rows) {
    float* sl = reinterpret_cast<float*>(h + hrow0 + (int64_t)tid * 2 * inter + inter);
    sl[n0 / kGroup] = up;
    sl[n0 / kGroup + 1] = up;
  }
}

// ---------------------------------------------------------------------------
// down: tile = 128 bucket rows x 256 output columns (down weight rows
// n0 .. n0+255).  Each staged group of h is brought to the tile's largest h
// scale through the group's (scale, bias) pair (a power-of-two factor of at
// most 1); the results are multiplied by that scale once.  Writes
// roww * (h . Wd^T) of every row to its partial row (the shared expert's row
// is j = k) in fp16 after a power-of-two scale per 32-row x 64-column block
// of a wave: the bound max|value| x max|row factor| is brought to
// [2^14, 2^15), so every value at or above 2^-29 of it keeps 11 significant
// bits (relative error at most 2^-11); the scale's exponent is stored as a
// byte per (row, 64-column block) behind the fp16 rows.

#define MOE_PDN_PARAMS                                                                       \
  const uint16_t* __restrict__ h, const int32_t* __restrict__ pairs,                           \
      const float* __restrict__ topk_w, const float* __restrict__ gamma,                       \
      const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,                 \
      const int32_t* __restrict__ tiles, const int32_t* __restrict__ ntiles,                   \
      const uint8_t* __restrict__ slab, const int32_t* __restrict__ slot_table, int64_t stride, \
      const uint8_t* __restrict__ shared_blob, float* __restrict__ partial, int T, int H, int E, \
      int k, int I, int Is, int64_t d_off_r, int64_t d_unit_r, int64_t d_tile_r,                \
      int64_t d_off_s, int64_t d_unit_s, int64_t d_tile_s, int nbg
#define MOE_PDN_ARGS                                                                           \
  h, pairs, topk_w, gamma, counts, offsets, tiles, ntiles, slab, slot_table, stride, shared_blob, \
      partial, T, H, E, k, I, Is, d_off_r, d_unit_r, d_tile_r, d_off_s, d_unit_s, d_tile_s, nbg

template <int BITS, int MB>
__device__ __forceinline__ void prefill_down_item(MOE_PDN_PARAMS, Stage<BITS>* st,
                                                  uint32_t* rowdst, float* roww, float* hsl,
                                                  const TileInfo& ti, int nb) {
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));  // (as in the gate/up item)
  const int lane = tid & 63, wave = tid >> 6, l32 = lane & 31, half = lane >> 5;
  const bool shared = ti.e == E;
  const int inter = shared ? Is : I;
  const int n0 = nb * kTileN;
  const uint8_t* sec = shared ? shared_blob + d_off_s
                              : slab + (int64_t)slot_table[ti.e] * stride + d_off_r;
  const int64_t unit_b = shared ? d_unit_s : d_unit_r, tile_b = shared ? d_tile_s : d_tile_r;
  if (tid < kMT) {
    // byte offset of the row's fp16 partial row (rows past the tile: an
    // offset past the buffer, whose stores the hardware drops)
    uint32_t off = kDropOffset;
    float wv = 0.f;
    if (tid < ti.rows) {
      int dst;
      if (shared) {
        const int t = ti.base + tid;
        dst = t * (k + 1) + k;
        wv = gamma[t];
      } else {
        const int p = pairs[ti.base + tid];
        dst = (p / k) * (k + 1) + (p % k);
        wv = topk_w[p];
      }
      off = (uint32_t)dst * (uint32_t)H * 2u;
    }
    rowdst[tid] = off;
    roww[tid] = wv;
  }
  const int G = inter / kGroup;
  const int64_t hbase = shared ? (int64_t)T * k * 2 * I + (int64_t)ti.base * 2 * Is
                               : (int64_t)ti.base * 2 * I;
  // the inverse h scale of each group of the tile (stored with every row)
  if (tid < G) hsl[tid] = *reinterpret_cast<const float*>(h + hbase + inter + 2 * tid);
  __syncthreads();
  float hmax = 0.f;
  for (int g = 0; g < G; ++g) hmax = fmaxf(hmax, hsl[g]);
  const float inv_hmax = 1.0f / hmax;  // powers of two: exact
  LoadRoles<BITS> lr;
  FragRoles fr;
  // rows past the tile read row 0 (their results are discarded)
  make_roles<BITS>(
      lr, fr, tid, l32, half, 64 * wave + l32, sec, unit_b, tile_b, 1,
      [&](int r, int& mat, int& row) {
        mat = 0;
        row = n0 + r;
      },
      [&](int r) { return (uint32_t)(r < ti.rows ? r : 0) * (uint32_t)inter * 4u; });
  f32x16 C[MB][2];
  const f32x16 zero = {};
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) C[mb][0] = C[mb][1] = zero;
  // (views: the tile's h rows; the section's row tiles of down rows)
  const TileSrc src{src_view(h + hbase, (uint32_t)ti.rows * (uint32_t)inter * 4u),
                    src_view(sec, (uint32_t)((H / kRowTile) * tile_b))};
  k_loop<BITS, MB, 32 * cpr<BITS>() * 16, 32 * 4>(
      st, lr, fr, src, unit_b, G, __builtin_amdgcn_readfirstlane(wave), C, [&](int g) {
        float hs;
        asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                     : "=v"(hs)
                     : "v"(lds_addr(&hsl[g]))
                     : "memory");
        return hs * inv_hmax;
      });

  // Epilogue.  The ring is free (every wave is past the last stage's
  // barrier).  Each wave turns its 32 x 64 blocks into rows through its own
  // LDS region and stores each row as 8-byte fp16 pieces of 4 columns: lane
  // (c4, r4) takes columns 4 c4 .. 4 c4 + 3 of rows r4, r4 + 4, ...  The
  // row factor roww * hmax and the block's scale 2^-e are powers of two
  // times roww, so (value x factor) x scale is one product.  The exponent
  // byte of (row, block) sits at the row's fp16 byte offset / 128 (H fp16
  // values, H / 64 bytes) behind the fp16 rows.
  float* ep = reinterpret_cast<float*>(st) + wave * (32 * kEpRow);
  const uint32_t nrows = (uint32_t)T * (uint32_t)(k + 1);
  const auto rp = __builtin_amdgcn_make_buffer_rsrc(partial, (short)0,
                                                    (int)(nrows * (uint32_t)H * 2u), 0x00020000);
  const auto re = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<uint8_t*>(partial) + (size_t)nrows * (size_t)H * 2u, (short)0,
      (int)(nrows * (uint32_t)(H / 64)), 0x00020000);
  const int c4 = lane & 15, r4 = lane >> 4;
  const uint32_t col_b = (uint32_t)(n0 + 64 * wave + 4 * c4) * 2u;
  const uint32_t blk = (uint32_t)(n0 + 64 * wave) / 64u;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        ep[(8 * (r >> 2) + 4 * half + (r & 3)) * kEpRow + 32 * nb + l32] = C[mb][nb][r];
    asm volatile("" ::: "memory");  // the wave's LDS accesses stay in order
    float4 v[8];
    float f[8];
    float bnd = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = r4 + 4 * j, m = 32 * mb + row;
      v[j] = *reinterpret_cast<const float4*>(&ep[row * kEpRow + 4 * c4]);
      f[j] = roww[m] * hmax;
      const float a = fmaxf(fmaxf(fabsf(v[j].x), fabsf(v[j].y)), fmaxf(fabsf(v[j].z), fabsf(v[j].w)));
      bnd = fmaxf(bnd, a * fabsf(f[j]));
    }
    const uint32_t mx = dec::wave_max_dpp(__float_as_uint(bnd) & 0x7FFFFFFFu);
    int e = mx == 0 ? 0 : (int)(mx >> 23) - 127 - 14;
    e = e < -100 ? -100 : (e > 100 ? 100 : e);
    const float sc = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int m = 32 * mb + r4 + 4 * j;
      const float g = f[j] * sc;
      const uint32_t h0 = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(v[j].x * g)) |
                          ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(v[j].y * g)) << 16);
      const uint32_t h1 = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(v[j].z * g)) |
                          ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(v[j].w * g)) << 16);
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{h0, h1}, rp, rowdst[m] + col_b, 0, 0);
    }
    // the block's exponent byte for each of its rows: lane (c4 < 8, r4) writes
    // row r4 + 4 c4's (the other lanes' go past the buffer)
    const uint32_t eoff = c4 < 8 ? (rowdst[32 * mb + r4 + 4 * (c4 & 7)] >> 7) + blk : kDropOffset;
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(int8_t)e, re, eoff, 0, 0);
    asm volatile("" ::: "memory");
  }
}

// Persistent grids: workgroup w serves XCD w % 8 and walks that XCD's item
// range with a stride of gridDim.x / 8, column block fastest (the column
// blocks of one row tile share its activation rows, the row tiles of one
// expert its weights, on the same L2).  Each item runs with as many 32-row
// blocks as its tile has rows.
template <int BITS>
__global__ __launch_bounds__(kGemmThreads, BITS == 4 ? 2 : 1) void prefill_gateup_kernel(
    MOE_PGU_PARAMS) {
  __shared__ __align__(256) Stage<BITS> st[kStages];
  __shared__ __align__(16) int32_t rowsrc[kMT];
  __shared__ __align__(16) int32_t te[kMT];
  __shared__ uint32_t wmax[4];
  const int total = *ntiles * nbg;
  const int per = (total + 7) / 8, c = blockIdx.x & 7;
  for (int i = blockIdx.x >> 3; i < per; i += gridDim.x >> 3) {
    const int q = c * per + i;
    if (q >= total) break;
    const TileInfo ti = get_tile(tiles, counts, offsets, q / nbg, E);
    const int nb = q % nbg;
    if (ti.rows > 96)
      prefill_gateup_item<BITS, 4>(MOE_PGU_ARGS, st, rowsrc, te, wmax, ti, nb);
    else if (ti.rows > 64)
      prefill_gateup_item<BITS, 3>(MOE_PGU_ARGS, st, rowsrc, te, wmax, ti, nb);
    else if (ti.rows > 32)
      prefill_gateup_item<BITS, 2>(MOE_PGU_ARGS, st, rowsrc, te, wmax, ti, nb);
    else
      prefill_gateup_item<BITS, 1>(MOE_PGU_ARGS, st, rowsrc, te, wmax, ti, nb);
    __syncthreads();
  }
}

template <int BITS>
__global__ __launch_bounds__(kGemmThreads, BITS == 4 ? 2 : 1) void prefill_down_kernel(
    MOE_PDN_PARAMS) {
  __shared__ __align__(256) Stage<BITS> st[kStages];
  __shared__ __align__(16) uint32_t rowdst[kMT];
  __shared__ __align__(16) float roww[kMT];
  __shared__ float hsl[MOE_MAX_INTER / kGroup];
  const int total = *ntiles * nbg;
  const int per = (total + 7) / 8, c = blockIdx.x & 7;
  for (int i = blockIdx.x >> 3; i < per; i += gridDim.x >> 3) {
    const int q = c * per + i;
    if (q >= total) break;
    const TileInfo ti = get_tile(tiles, counts, offsets, q / nbg, E);
    const int nb = q % nbg;
    if (ti.rows > 96)
      prefill_down_item<BITS, 4>(MOE_PDN_ARGS, st, rowdst, roww, hsl, ti, nb);
    else if (ti.rows > 64)
      prefill_down_item<BITS, 3>(MOE_PDN_ARGS, st, rowdst, roww, hsl, ti, nb);
    else if (ti.rows > 32)
      prefill_down_item<BITS, 2>(MOE_PDN_ARGS, st, rowdst, roww, hsl, ti, nb);
    else
      prefill_down_item<BITS, 1>(MOE_PDN_ARGS, st, rowdst, roww, hsl, ti, nb);
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
  if (!a.x16_ready && (e = launch_x16(a.x, a.x16, a.xe, a.T, a.H, a.bits, s)) != hipSuccess)
    return e;
  const int nbg = (max(a.I, a.Is) + kHCols - 1) / kHCols;
  const unsigned slots_gu = (unsigned)min((a.max_tiles * nbg + 7) / 8 * 8, kPersistSlots);
  hipLaunchKernelGGL((prefill_gateup_kernel<BITS>), dim3(slots_gu), dim3(kGemmThreads), 0, s,
                     a.x16, a.xe, a.pairs, a.counts, a.offsets, a.tiles, a.ntiles, a.slab,
                     a.slot_table, a.stride, a.shared_blob, a.h, a.T, a.H, a.E, a.k, a.I, a.Is,
                     a.L.gu_unit, a.L.gu_tile, a.Ls.gu_unit, a.Ls.gu_tile, nbg);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int nbd = a.H / kTileN;
  const unsigned slots_d = (unsigned)min((a.max_tiles * nbd + 7) / 8 * 8, kPersistSlots);
  hipLaunchKernelGGL((prefill_down_kernel<BITS>), dim3(slots_d), dim3(kGemmThreads), 0, s, a.h,
                     a.pairs, a.topk_w, a.gamma, a.counts, a.offsets, a.tiles, a.ntiles, a.slab,
                     a.slot_table, a.stride, a.shared_blob, a.partial, a.T, a.H, a.E, a.k, a.I,
                     a.Is, a.L.d_off, a.L.d_unit, a.L.d_tile, a.Ls.d_off, a.Ls.d_unit, a.Ls.d_tile,
                     nbd);
  return hipGetLastError();
}

}  // namespace

int prefill_max_tiles(int T, int E, int k, bool has_shared) {
  // sum over buckets of ceil(n_b / kMT) <= sum(n_b) / kMT + number of buckets
  const int64_t rows = (int64_t)T * k + (has_shared ? T : 0);
  return (int)(rows / kMT + E + (has_shared ? 1 : 0) + 1);
}

bool prefill_supported(int act, int64_t T, int H, int k, int I, int Is, bool has_shared) {
  if (act != MOE_ACT_BF16) return false;
  if (H % kTileN != 0 || I % kHCols != 0 || (has_shared && Is % kHCols != 0)) return false;
  // the gate/up kernel addresses the fp16 activation rows with 32-bit byte offsets
  if (T * H * 2 >= (int64_t)1 << 32) return false;
  // the down kernel's partial rows (fp16, then the exponent bytes): 32-bit
  // offsets below kDropOffset
  if (T * (k + 1) * H * 4 > (int64_t)kDropOffset - (int64_t)H * 4) return false;
  return true;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
  return a.bits == 4 ? launch_prefill_t<4>(a, s) : launch_prefill_t<8>(a, s);
}

}  // namespace moe
