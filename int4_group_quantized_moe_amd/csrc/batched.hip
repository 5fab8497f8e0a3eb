// Grouped GEMMs of one token block: batched decode of at most 64 tokens, so
// that every expert bucket (and the shared expert's T rows) has at most 64
// rows.  Per expert e with its bucket of n_e tokens,
//   G|U = X_e . [Wg_e | Wu_e]^T,  h = silu(G) * U,  Y_e = h . Wd_e^T,
// on v_mfma_f32_32x32x16_f16 with fp32 accumulation (the SwiGLU experts of
// the pages' MoE layer: page "Paquets Swiftlet 80B Qwen ..." on xix.ai, 4th
// paragraph; the int4 / int8 group-affine weights: same page, last
// paragraph).
//
// At this size the work per expert is small and the time is the latency of
// getting each expert's weights on chip, so both kernels request every
// weight byte of a workgroup before its first product:
//  * gate/up: a workgroup owns (bucket, 64 h columns) = 128 weight rows; its
//    4 waves split them (waves 0-1 the gate rows, 2-3 the up rows of the same
//    h columns) and each lane loads its weight row's codes of the whole K
//    into registers at the start.  The bucket's activation rows are shared by
//    the 4 waves: they are staged in LDS 256 columns at a time by coalesced
//    asynchronous global->LDS loads, three chunks in flight.  The up waves
//    hand their tile to the gate waves through LDS, which write
//    h = silu(g) * u in fp32.
//  * down: a workgroup owns (bucket, 256 output columns); each of its 8
//    waves holds its 32 output rows' codes of the whole K in registers, and
//    the bucket's h rows are staged once in LDS.
// Operands: the weights are dequantised in registers to fp16, w = s q + b
// with one packed FMA per two codes (one rounding, relative error at most
// 2^-11; the scale and bias are bf16, so fp16 holds them exactly in its
// normal range), which also folds the group bias into the product.  The
// activations enter as fp16 after a power-of-two scale per token row (the
// router's top-k kernel writes that copy, see x16_row); the h rows likewise,
// after a power-of-two scale per row chosen here.  Both scales are undone
// exactly on the fp32 results.  With one MFMA chain per 32-row block over the
// whole K there is no per-group rescaling of partial sums.
#include "mfma_common.h"

namespace moe {
namespace {

constexpr int kBgCols = 64;                // h columns per gate/up item
constexpr int kBgSlots = 256;              // persistent gate/up workgroups (1 per CU)
constexpr int kBdCols = 256;               // output columns per down item
constexpr int kBdThreads = 512;            // 8 waves x 32 output columns
constexpr int kBdSlots = 256;              // persistent down workgroups (1 per CU)
constexpr int kBdMaxGroups = 8;            // groups of K of the down GEMM (inter <= 512)
constexpr int kBdLdsRow = kBdMaxGroups * kGroup + 8;  // staged h row (fp16), padded
constexpr int kBatchRows = kOneBlockTokens;  // rows of every bucket (tokens of the block)

#define MOE_G1(p) ((const void __attribute__((address_space(1)))*)(p))
#define MOE_L3(p) ((void __attribute__((address_space(3)))*)(p))

template <int N>
__device__ __forceinline__ void bt_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// s_waitcnt vmcnt(n): at most n of this wave's vector memory loads (global->
// LDS loads included) outstanding; they complete in order.  n is a constant
// wherever this is inlined into unrolled code, so one branch remains.
__device__ __forceinline__ void bt_wait_vm_n(int n) {
#define MOE_W(N) \
  if (n == N) {  \
    bt_wait_vm<N>(); \
    return;      \
  }
  MOE_W(0) MOE_W(1) MOE_W(2) MOE_W(3) MOE_W(4) MOE_W(5) MOE_W(6) MOE_W(7) MOE_W(8)
  MOE_W(9) MOE_W(10) MOE_W(11) MOE_W(12) MOE_W(13) MOE_W(14) MOE_W(15) MOE_W(16)
  MOE_W(17) MOE_W(18) MOE_W(19) MOE_W(20) MOE_W(21) MOE_W(22) MOE_W(23) MOE_W(24)
#undef MOE_W
  bt_wait_vm<0>();
}
// Workgroup barrier that waits for this wave's LDS accesses (lgkmcnt) but not
// for its global loads in flight (a release fence would drain those too).
__device__ __forceinline__ void bt_lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

constexpr int kBgChunk = 4;   // quantisation groups (256 columns) per staged activation chunk
constexpr int kBgStages = 3;  // activation chunks in LDS (two in flight while one is used)

// LDS of a gate/up workgroup for K = 64 G.
template <int G>
struct BgLds {
  uint4 a[kBgStages][kBatchRows * 32];  // activation chunks: 64 rows x 32 units of 16 bytes
  uint32_t sb[4][G][64];                // (scale, bias) word of each wave's lane rows, per group
  int32_t tok[kBatchRows];              // token of each bucket row
  int32_t te[kBatchRows];               // its activation row's exponent
};

#define MOE_BG_PARAMS                                                                        \
  const uint16_t* __restrict__ x16, const int32_t* __restrict__ xe,                            \
      const int32_t* __restrict__ pairs, const int32_t* __restrict__ counts,                  \
      const int32_t* __restrict__ offsets, const int32_t* __restrict__ tiles,                 \
      const int32_t* __restrict__ ntiles, const uint8_t* __restrict__ slab,                   \
      const int32_t* __restrict__ slot_table, int64_t stride,                                 \
      const uint8_t* __restrict__ shared_blob, float* __restrict__ h, int T, int H, int E,     \
      int k, int I, int Is, int64_t gu_unit_r, int64_t gu_tile_r, int64_t gu_unit_s,          \
      int64_t gu_tile_s
#define MOE_BG_ARGS                                                                            \
  x16, xe, pairs, counts, offsets, tiles, ntiles, slab, slot_table, stride, shared_blob, h, T, \
      H, E, k, I, Is, gu_unit_r, gu_tile_r, gu_unit_s, gu_tile_s

// Unit (16 bytes) c16 of bucket row r of a chunk sits at r * 32 + (c16 ^ (r & 15)): the 32
// rows an MFMA operand read touches, all at one c16, land on 16 distinct 16-byte slots of
// each 256-byte window of LDS banks.
__device__ __forceinline__ int bg_unit(int r, int c16) { return r * 32 + (c16 ^ (r & 15)); }

// One gate/up item: bucket rows 0 .. 32 MB - 1 (rows past ti.rows compute row 0's token and
// are discarded) x h columns n0 .. n0 + 63.  Wave w holds the weight row of h column
// n0 + 32 (w & 1) + (lane & 31) of the gate (w < 2) or up (w >= 2) matrix.
template <int BITS, int G, int MB>
__device__ __forceinline__ void bg_gateup_item(MOE_BG_PARAMS, BgLds<G>& sm, const TileInfo& ti,
                                               int nb) {
  constexpr int NCH = G / kBgChunk;                      // activation chunks along K
  constexpr int CH = BITS / 4;                           // 16-byte code chunks per group
  constexpr int RD = BITS == 4 ? G : (G < 16 ? G : 16);  // groups of codes held in registers
  constexpr int AL = 4 * MB;                             // chunk loads per wave (64 units each)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, half = lane >> 5;
  const bool shared = ti.e == E;
  const int inter = shared ? Is : I;
  const int n0 = nb * kBgCols;
  if (n0 >= inter) return;
  // the bucket rows' tokens first (the oldest load: waiting for it waits for nothing else)
  int my_tok = 0;
  if (tid < 32 * MB) {
    const int r = tid < ti.rows ? tid : 0;
    my_tok = shared ? ti.base + r : pairs[ti.base + r] / k;
  }
  asm volatile("" ::: "memory");  // issued before the code loads below
  const uint8_t* sec = shared ? shared_blob : slab + (int64_t)slot_table[ti.e] * stride;
  const int64_t unit_b = shared ? gu_unit_s : gu_unit_r, tile_b = shared ? gu_tile_s : gu_tile_r;
  const int col = n0 + 32 * (wave & 1) + l32;
  const RowAddr<BITS> ra(sec, unit_b, tile_b, 2, wave >> 1, col, half);
  // the lane's codes of the whole K (int8: the first RD groups; the rest are loaded as
  // groups are consumed), then the (scale, bias) words of every group into LDS
  LaneCodes<BITS> q[RD];
#pragma unroll
  for (int g = 0; g < RD; ++g) q[g].load(ra.group_codes(g));
#pragma unroll
  for (int g = 0; g < G; ++g)
    __builtin_amdgcn_global_load_lds(MOE_G1(ra.group_sb_ptr(g)), MOE_L3(&sm.sb[wave][g][0]), 4, 0,
                                     0);
  if (tid < 32 * MB) sm.tok[tid] = my_tok;
  bt_lds_barrier();
  // the row exponents (needed at the end) and the first activation chunks
  const int my_e = tid < 32 * MB ? xe[sm.tok[tid]] : 0;
  uint32_t aoff[AL];
#pragma unroll
  for (int j = 0; j < AL; ++j) {
    const int u = (wave * AL + j) * 64 + lane, r = u >> 5, c16 = (u & 31) ^ (r & 15);
    aoff[j] = (uint32_t)sm.tok[r] * (uint32_t)(2 * H) + 16u * (uint32_t)c16;
  }
  const uint8_t* xb = reinterpret_cast<const uint8_t*>(x16);
  auto issue_chunk = [&](int c) {
#pragma unroll
    for (int j = 0; j < AL; ++j)
      __builtin_amdgcn_global_load_lds(MOE_G1(xb + aoff[j] + 512u * (uint32_t)c),
                                       MOE_L3(&sm.a[c % kBgStages][(wave * AL + j) * 64]), 16, 0,
                                       0);
  };
#pragma unroll
  for (int c = 0; c < kBgStages - 1; ++c)
    if (c < NCH) issue_chunk(c);

  f32x16 acc[MB];
  const f32x16 zero = {};
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = zero;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    // chunk c is in once the loads issued after it are at most: chunk c + 1, and (int8)
    // the code loads issued while chunk c - 1 was multiplied
    int later = c + 1 < NCH ? AL : 0;
    if (c >= 1)
#pragma unroll
      for (int gi = 0; gi < kBgChunk; ++gi)
        later += (kBgChunk * (c - 1) + gi + RD < G) ? CH : 0;
    bt_wait_vm_n(later);
    bt_lds_barrier();
    if (c + kBgStages - 1 < NCH) issue_chunk(c + kBgStages - 1);
    const uint4* ab = sm.a[c % kBgStages];
#pragma unroll
    for (int gi = 0; gi < kBgChunk; ++gi) {
      const int g = kBgChunk * c + gi;
      f16x2 S2, B2;
      sb_f16<BITS>(sm.sb[wave][g][lane], S2, B2);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const u32x4 b = w_frag_f16<BITS>(q[g % RD], kk, S2, B2);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const uint4 av = ab[bg_unit(32 * mb + l32, gi * 8 + 4 * half + kk)];
          acc[mb] = mfma_f16(u32x4{av.x, av.y, av.z, av.w}, b, acc[mb]);
        }
      }
      if (g + RD < G) q[g % RD].load(ra.group_codes(g + RD));
    }
  }

  // undo the rows' activation scales; the up waves hand their tile to the gate waves
  // (through chunk buffer 0, free after the barrier)
  if (tid < 32 * MB) sm.te[tid] = my_e;
  bt_lds_barrier();
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      acc[mb][r] *= exp2i(sm.te[32 * mb + 8 * (r >> 2) + 4 * half + (r & 3)]);
  float* red = reinterpret_cast<float*>(&sm.a[0][0]);
  if (wave >= 2) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) red[(((wave & 1) * MB + mb) * 16 + r) * 64 + lane] = acc[mb][r];
  }
  bt_lds_barrier();
  if (wave < 2) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float gv = acc[mb][r], uv = red[((wave * MB + mb) * 16 + r) * 64 + lane];
        const int row = 32 * mb + 8 * (r >> 2) + 4 * half + (r & 3);
        if (row < ti.rows) {
          const int64_t hrow = shared ? (int64_t)T * k * I + (int64_t)(ti.base + row) * Is
                                      : (int64_t)(ti.base + row) * I;
          h[hrow + col] = __fdividef(gv, 1.0f + __expf(-gv)) * uv;
        }
      }
  }
}

// Persistent grid: workgroup w serves XCD w % 8 and walks that XCD's contiguous range of
// (tile, column block) items, column block fastest, so the column blocks of one bucket
// (which stage the same activation rows) share an L2.
template <int BITS, int G>
__global__ __launch_bounds__(256) void bg_gateup_kernel(MOE_BG_PARAMS) {
  __shared__ __align__(16) BgLds<G> sm;
  const int nbg = (I > Is ? I : Is) / kBgCols;
  const int total = *ntiles * nbg;
  const int per = (total + 7) / 8, c = blockIdx.x & 7;
  for (int i = blockIdx.x >> 3; i < per; i += gridDim.x >> 3) {
    const int q = c * per + i;
    if (q >= total) break;
    const TileInfo ti = get_tile(tiles, counts, offsets, q / nbg, E);
    if (ti.rows > 32) bg_gateup_item<BITS, G, 2>(MOE_BG_ARGS, sm, ti, q % nbg);
    else bg_gateup_item<BITS, G, 1>(MOE_BG_ARGS, sm, ti, q % nbg);
    bt_lds_barrier();
  }
}

#define MOE_BD_PARAMS                                                                        \
  const float* __restrict__ h, const int32_t* __restrict__ pairs,                              \
      const float* __restrict__ topk_w, const float* __restrict__ gamma,                       \
      const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,                 \
      const int32_t* __restrict__ tiles, const int32_t* __restrict__ ntiles,                   \
      const uint8_t* __restrict__ slab, const int32_t* __restrict__ slot_table, int64_t stride, \
      const uint8_t* __restrict__ shared_blob, float* __restrict__ partial, int T, int H,        \
      int E, int k, int I, int Is, int64_t d_off_r, int64_t d_unit_r, int64_t d_tile_r,         \
      int64_t d_off_s, int64_t d_unit_s, int64_t d_tile_s
#define MOE_BD_ARGS                                                                            \
  h, pairs, topk_w, gamma, counts, offsets, tiles, ntiles, slab, slot_table, stride, shared_blob, \
      partial, T, H, E, k, I, Is, d_off_r, d_unit_r, d_tile_r, d_off_s, d_unit_s, d_tile_s

struct BdLds {
  uint16_t h16[kBatchRows * kBdLdsRow];  // staged h rows in fp16, scaled per row
  int32_t he[kBatchRows];                // the rows' exponents
  int32_t rowdst[kBatchRows];            // partial row of each bucket row, or -1
  float roww[kBatchRows];                // its routing weight (gamma for the shared expert)
};

// One down item: bucket rows 0 .. 32 MB - 1 x output columns n0 .. n0 + 255;
// wave w owns columns n0 + 32 w .. + 31.  Writes roww * (h . Wd^T) of every
// row to its partial row.
template <int BITS, int MB>
__device__ __forceinline__ void bd_down_item(MOE_BD_PARAMS, BdLds& sm, const TileInfo& ti,
                                             int cb) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const bool shared = ti.e == E;
  const int inter = shared ? Is : I;
  const int GD = inter / kGroup;
  const int col = cb * kBdCols + 32 * wave + l32;
  const uint8_t* sec = shared ? shared_blob + d_off_s
                              : slab + (int64_t)slot_table[ti.e] * stride + d_off_r;
  const int64_t unit_b = shared ? d_unit_s : d_unit_r, tile_b = shared ? d_tile_s : d_tile_r;
  const RowAddr<BITS> ra(sec, unit_b, tile_b, 1, 0, col, half);
  // every code and (scale, bias) word of the lane's output row first
  LaneCodes<BITS> q[kBdMaxGroups];
  uint32_t sbw[kBdMaxGroups];
#pragma unroll
  for (int g = 0; g < kBdMaxGroups; ++g)
    if (g < GD) {
      q[g].load(ra.group_codes(g));
      sbw[g] = ra.group_sb(g);
    }
  if (tid < kBatchRows) {
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
    sm.rowdst[tid] = dst;
    sm.roww[tid] = wv;
  }
  // stage h: thread (row, group) holds the row's 64 fp32 values of the group;
  // the 8 threads of a row (consecutive lanes) agree on the row's scale 2^-e
  // (its largest magnitude to [2^14, 2^15)) and store the scaled values in
  // fp16, in the weights' fp16 K order.  Group g's 16-byte chunk c sits at
  // chunk c ^ (g & 6) of the group: with 1040-byte rows the groups g, g + 2,
  // g + 4, g + 6 of a row would otherwise start on the same banks, so that
  // the staging stores of a wave hit each bank four times.
  {
    const int row = tid >> 3, g = tid & 7;
    const bool ok = row < 32 * MB && row < ti.rows && g < GD;
    const int64_t hrow = shared ? (int64_t)T * k * I + (int64_t)(ti.base + (ok ? row : 0)) * Is
                                : (int64_t)(ti.base + (ok ? row : 0)) * I;
    const float4* src = reinterpret_cast<const float4*>(h + hrow + (ok ? g : 0) * kGroup);
    float v[64];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float4 t4 = ok ? src[j] : make_float4(0.f, 0.f, 0.f, 0.f);
      v[4 * j] = t4.x;
      v[4 * j + 1] = t4.y;
      v[4 * j + 2] = t4.z;
      v[4 * j + 3] = t4.w;
    }
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 64; ++j) m = max(m, __float_as_uint(v[j]) & 0x7FFFFFFFu);
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
    int e = m == 0 ? 0 : (int)(m >> 23) - 127 - 14;
    e = e < -100 ? -100 : (e > 100 ? 100 : e);
    const float sc = exp2i(-e);
    if (row < 32 * MB && g < GD) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float lo = v[8 * c + dn_perm<BITS>(2 * i)] * sc;
          const float hi = v[8 * c + dn_perm<BITS>(2 * i + 1)] * sc;
          o[i] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
        }
        *reinterpret_cast<u32x4*>(&sm.h16[row * kBdLdsRow + g * kGroup + 8 * (c ^ (g & 6))]) =
            u32x4{o[0], o[1], o[2], o[3]};
      }
      if (g == 0) sm.he[row] = e;
    }
  }
  __syncthreads();

  f32x16 acc[MB];
  const f32x16 zero = {};
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = zero;
#pragma unroll
  for (int g = 0; g < kBdMaxGroups; ++g) {
    if (g < GD) {
      f16x2 S2, B2;
      sb_f16<BITS>(sbw[g], S2, B2);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const u32x4 b = w_frag_f16<BITS>(q[g], kk, S2, B2);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int o =
              (32 * mb + l32) * kBdLdsRow + g * kGroup + 8 * ((4 * half + kk) ^ (g & 6));
          acc[mb] = mfma_f16(*reinterpret_cast<const u32x4*>(&sm.h16[o]), b, acc[mb]);
        }
      }
    }
  }
  // the weighted partial rows, the rows' h scales undone
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 32 * mb + 8 * (r >> 2) + 4 * half + (r & 3);
      const int dst = sm.rowdst[row];
      if (dst >= 0)
        partial[(int64_t)dst * H + col] = sm.roww[row] * (exp2i(sm.he[row]) * acc[mb][r]);
    }
}

template <int BITS>
__global__ __launch_bounds__(kBdThreads) void bd_down_kernel(MOE_BD_PARAMS) {
  __shared__ __align__(16) BdLds sm;
  const int nbd = H / kBdCols;
  const int total = *ntiles * nbd;
  const int per = (total + 7) / 8, c = blockIdx.x & 7;
  for (int i = blockIdx.x >> 3; i < per; i += gridDim.x >> 3) {
    const int q = c * per + i;
    if (q >= total) break;
    const TileInfo ti = get_tile(tiles, counts, offsets, q / nbd, E);
    if (ti.rows > 32) bd_down_item<BITS, 2>(MOE_BD_ARGS, sm, ti, q % nbd);
    else bd_down_item<BITS, 1>(MOE_BD_ARGS, sm, ti, q % nbd);
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void x16_kernel(const uint16_t* __restrict__ x,
                                                  uint16_t* __restrict__ x16,
                                                  int32_t* __restrict__ xe, int T, int H,
                                                  int bits) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  x16_row(x + (int64_t)t * H, x16 + (int64_t)t * H, xe + t, H, bits);
}

template <int BITS, int G>
hipError_t launch_bg(const PrefillArgs& a, hipStream_t s) {
  float* h = reinterpret_cast<float*>(a.h);
  const int nbg = (a.I > a.Is ? a.I : a.Is) / kBgCols;
  const unsigned slots_gu = (unsigned)min((a.max_tiles * nbg + 7) / 8 * 8, kBgSlots);
  hipLaunchKernelGGL((bg_gateup_kernel<BITS, G>), dim3(slots_gu), dim3(256), 0, s, a.x16, a.xe,
                     a.pairs, a.counts, a.offsets, a.tiles, a.ntiles, a.slab, a.slot_table,
                     a.stride, a.shared_blob, h, a.T, a.H, a.E, a.k, a.I, a.Is, a.L.gu_unit,
                     a.L.gu_tile, a.Ls.gu_unit, a.Ls.gu_tile);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nbd = a.H / kBdCols;
  const unsigned slots_d = (unsigned)min((a.max_tiles * nbd + 7) / 8 * 8, kBdSlots);
  hipLaunchKernelGGL((bd_down_kernel<BITS>), dim3(slots_d), dim3(kBdThreads), 0, s, h, a.pairs,
                     a.topk_w, a.gamma, a.counts, a.offsets, a.tiles, a.ntiles, a.slab,
                     a.slot_table, a.stride, a.shared_blob, a.partial, a.T, a.H, a.E, a.k, a.I,
                     a.Is, a.L.d_off, a.L.d_unit, a.L.d_tile, a.Ls.d_off, a.Ls.d_unit,
                     a.Ls.d_tile);
  return hipGetLastError();
}

}  // namespace

bool batched_supported(int act, int T, int H, int I, int Is, bool has_shared) {
  if (act != MOE_ACT_BF16 || T < 1 || T > kBatchRows) return false;
  if (H != 1024 && H != 2048) return false;
  if (I % kBgCols != 0 || I > kBdMaxGroups * kGroup) return false;
  if (has_shared && (Is % kBgCols != 0 || Is > kBdMaxGroups * kGroup)) return false;
  return true;
}

hipError_t launch_x16(const uint16_t* x, uint16_t* x16, int32_t* xe, int T, int H, int bits,
                      hipStream_t s) {
  hipLaunchKernelGGL(x16_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, x, x16, xe, T, H,
                     bits);
  return hipGetLastError();
}

hipError_t launch_batched(const PrefillArgs& a, hipStream_t s) {
  if (!a.x16_ready) {
    hipError_t e = launch_x16(a.x, a.x16, a.xe, a.T, a.H, a.bits, s);
    if (e != hipSuccess) return e;
  }
  if (a.H == 2048) return a.bits == 4 ? launch_bg<4, 32>(a, s) : launch_bg<8, 32>(a, s);
  return a.bits == 4 ? launch_bg<4, 16>(a, s) : launch_bg<8, 16>(a, s);
}

}  // namespace moe
