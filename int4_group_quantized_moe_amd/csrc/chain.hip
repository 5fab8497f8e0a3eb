// Persistent batch-1 decode chain: every layer of the chain in ONE launch,
// one workgroup per compute unit.  The launch is an ordinary one after a
// check that the device holds the whole grid at once (a cooperative launch
// makes the same check, and costs about 10 us of idle GPU on each side of it
// inside a graph replay); should other work hold compute units at the same
// time, a bounded wait below expires and says so in the status word.
//
// A layer needs three all-to-all exchanges (the full input before the
// router, the full logits before the top-k, every selected expert's full h
// before the down projection).  Kernel boundaries cost about as much as an
// in-kernel exchange plus a cold first load, so here the exchanges stay
// inside the kernel: each producer stores 64-bit words (epoch << 32 | payload)
// with device-coherent stores, each consumer polls them with device-coherent
// loads, two words per 16-byte access.  A word is its own ready flag (no
// fences, no counters, no contention).  The epoch is read from the workspace at start
// and advanced by workgroup 0 at the end, so graph replays never see stale
// words.  Every poll is bounded: on expiry an error bit is set and the
// workgroup carries on, so the grid always drains.
//
// Per layer l, workgroup w of NWG:
//   A   x_l (layer 0: input buffer; else polled), RMSNorm, router logit(s)
//       published, then x_hat staged for the gate/up dot products
//   B   wave 0 polls the logits and finds the top-k set while waves 1-3
//       take their share of the shared expert's (prefetched) tile; the
//       routed gate/up tiles are loaded; while they load, wave 0 computes
//       the routing weights and its share of the shared tile, whose h is
//       published; then the routed tiles; h published; then the down units
//       of phase C are issued
//   C   all h polled; the next layer's router row and slot table are
//       prefetched; down GEMV of 8 output rows over all selected experts in
//       a fixed order; the next layer's shared tile is requested; residual
//       add; x_{l+1} published
//
// Routing: top-k of E experts per token plus an always-active shared expert
// (page "Paquets Swiftlet 80B Qwen ..." on xix.ai, 4th paragraph); weights
// are MLX-style group-quantised int4/int8 (same page, last paragraph).
#include <atomic>

#include "decode_common.h"

namespace moe {
namespace {

using namespace dec;

constexpr uint32_t kSpinLimit = 1u << 18;
constexpr int kChainMaxExperts = 512;  // top-k over at most 8 logits per lane
template <int BITS>
constexpr int max_down_units() { return BITS == 4 ? 6 : 12; }  // per half-wave
constexpr int kHPairs = 8;     // h word pairs per thread per poll batch (run-time k)
constexpr int kHqStride = 20;  // LDS words per staged 32-column chunk of h
constexpr int kHTilePairs = 6; // exchange word pairs per 16-row tile of h

typedef int i32x4 __attribute__((ext_vector_type(4)));
// Cache policy of every exchange access: sc1 (device scope), so loads are
// served past the XCD-local L2 and see what other XCDs stored.
constexpr int kCoherent = 16;

// Buffer view of an exchange region of n 64-bit words, rounded up to a whole
// pair (the workspace pads every region to 256 bytes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t word_rsrc(const uint64_t* base, int n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint64_t*>(base), (short)0,
                                           ((n + 1) & ~1) * 8, 0x00020000);
}

__device__ __forceinline__ void st_word(uint64_t* p, uint32_t ep, uint32_t payload) {
  __hip_atomic_store(p, ((uint64_t)ep << 32) | payload, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// Publishes words 2q and 2q+1 with one 16-byte store; each aligned 8-byte
// half is a whole word (payload low, epoch high).
__device__ __forceinline__ void st_pair(__amdgpu_buffer_rsrc_t r, int q, uint32_t ep, uint32_t a,
                                        uint32_t b) {
  const i32x4 v = {(int)a, (int)ep, (int)b, (int)ep};
  __builtin_amdgcn_raw_buffer_store_b128(v, r, q * 16, 0, kCoherent);
}

// Polls words [0, n) of an exchange region two at a time until each carries
// epoch `ep`: thread `tid` of a group of `gsize` threads handles the pairs
// tid, tid + gsize, ...  All of a thread's loads of one batch are in flight
// together and share one offset register.  f(q, w0, w1) is called once per
// pair with the payloads of words 2q and 2q+1 (w1 means nothing when
// 2q + 1 == n).
template <int NB, class F>
__device__ __forceinline__ void poll_pairs(__amdgpu_buffer_rsrc_t r, int n, int tid, int gsize,
                                           uint32_t ep, uint32_t* err, F&& f) {
  const int np = (n + 1) >> 1;
  for (int b0 = 0; b0 < np; b0 += NB * gsize) {
    uint32_t pending = 0;
#pragma unroll
    for (int m = 0; m < NB; ++m)
      if (b0 + m * gsize + tid < np) pending |= 1u << m;
    i32x4 v[NB];
    uint32_t spins = 0;
    while (pending) {
      __asm__ volatile("" ::: "memory");  // every round reloads
#pragma unroll
      for (int m = 0; m < NB; ++m)
        if ((pending >> m) & 1u)
          v[m] = __builtin_amdgcn_raw_buffer_load_b128(r, tid * 16, (b0 + m * gsize) * 16,
                                                       kCoherent);
#pragma unroll
      for (int m = 0; m < NB; ++m) {
        const int q = b0 + m * gsize + tid;
        if (((pending >> m) & 1u) && (uint32_t)v[m].y == ep &&
            (2 * q + 1 >= n || (uint32_t)v[m].w == ep)) {
          f(q, (uint32_t)v[m].x, (uint32_t)v[m].z);
          pending &= ~(1u << m);
        }
      }
      if (pending) {
        if (++spins > kSpinLimit) {
          atomicOr(err, 1u);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
  }
}

__device__ __forceinline__ float bf16r(float v) { return bf16_bits_to_f32(f32_to_bf16_bits(v)); }

// Workgroup barrier for LDS traffic: this wave's LDS (and scalar) accesses
// are complete before it arrives; its global loads and stores may still be
// in flight.  (__syncthreads also waits for those: for the routed tiles just
// requested, the next layer's prefetch, and the acknowledgement of every
// exchange store.)  Every workgroup exchange in this kernel goes through LDS.
__device__ __forceinline__ void wg_barrier() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Weight addresses as global-memory pointers (an address read back from LDS
// would otherwise be accessed with flat instructions, which also hold the
// LDS counter).
typedef const __attribute__((address_space(1))) uint8_t gbyte;
__device__ __forceinline__ gbyte* gptr(const uint8_t* a) { return (gbyte*)a; }
__device__ __forceinline__ gbyte* gptr(uint64_t a) { return (gbyte*)a; }
#define CH_G1(p) ((const void __attribute__((address_space(1)))*)(p))
#define CH_L3(p) ((void __attribute__((address_space(3)))*)(p))
// A value the whole wave holds, moved to scalar registers (both halves
// zero-extended).
__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
  return ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32)) << 32) |
         (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
}
typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 gload16(gbyte* a) {
  const u32x4v v = *(const __attribute__((address_space(1))) u32x4v*)a;
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t gload4(gbyte* a) {
  return *(const __attribute__((address_space(1))) uint32_t*)a;
}

// IR, IS: intermediate size of the routed and of the shared experts; the
// blob geometry is compile-time.
// EPL: logits per lane of the top-k wave (E <= 64 EPL).  EC, KC: the
// number of experts and top-k when fixed at compile time (0: from p).  DQ4:
// the router rows and shared gate come as 4-bit dense rows (p.dense).
template <int BITS, int NIT, bool SHARED, int IR, int IS, int EPL, int EC, int KC, bool DQ4>
__global__ __launch_bounds__(256, 1) void chain_kernel(ChainParams p) {
  static_assert(BITS == 4, "the chain runs int4 weights");
  using C = GuCfg<BITS>;
  constexpr BlobLayout LR = make_layout(BITS, NIT * 256, IR);
  constexpr BlobLayout LS = make_layout(BITS, NIT * 256, SHARED ? IS : 64);
  constexpr int CC = C::CC, GPK = C::GPK, KBC = C::KBC, XS = C::XS;
  constexpr int H = NIT * 256;
  constexpr int NKB = H / KBC;       // gate/up k-blocks
  constexpr int NKW = NKB / 4;       // k-blocks per wave
  constexpr int NCH = H / CC;        // staged activation chunks
  constexpr int NXP = H / 1024;      // x word pairs per thread
  static_assert(NXP == 2 && CC == 32, "thread tid owns x elements 8 tid .. 8 tid + 7");
  constexpr int hsh = SHARED ? 1 : 0;
  // down units per half-wave: enough for the 8 half-waves to cover every
  // unit (all k * I / KBC + Is / KBC of them) when k is compile-time
  constexpr int kMaxDownUnits =
      KC ? (KC * (IR / C::KBC) + (SHARED ? IS / C::KBC : 0) + 7) / 8 : max_down_units<BITS>();
  static_assert(kMaxDownUnits <= max_down_units<BITS>(), "down units per half-wave");
  // h word pairs per thread of the h poll: with a compile-time k, all of a
  // thread's pairs in one batch (a second batch would start only once the
  // first has arrived: one more poll round trip); else kHPairs per batch
  constexpr int kHPoll =
      KC ? ((KC * IR + (SHARED ? IS : 0)) / kRowTile * kHTilePairs + 255) / 256 : kHPairs;
  __shared__ __align__(16) float xs[H];
  __shared__ __align__(16) uint32_t xp[NCH * XS];
  __shared__ float2 cs[NCH];
  constexpr int EMAX = 64 * EPL;
  __shared__ float lg[EMAX + 2];
  __shared__ int32_t slot_l[EMAX];
  __shared__ int32_t sel_idx[MOE_MAX_TOP_K];
  __shared__ float sel_val[MOE_MAX_TOP_K], sel_w[MOE_MAX_TOP_K], gam;
  __shared__ uint64_t sel_base[MOE_MAX_TOP_K];
  __shared__ __align__(16) uint64_t cand[66];  // top-k ranking words (+ a spare slot)
  __shared__ float red[4][kRowTile][2], red_s[4][kRowTile][2];
  __shared__ float dred[4][2][8];
  __shared__ float wsum[4];
  // router rows of this workgroup: w + NWG r.  The grid has at least H / 8
  // = 256 workgroups, so at most this many rows fall to one workgroup
  constexpr int kRR = ((EC ? EC : kChainMaxExperts) + hsh + 255) / 256;
  __shared__ float rred[kRR][4];
  __shared__ uint32_t tt[kRowTile];
  // the shared expert's gate/up tile of this workgroup (when it has one)
  constexpr int kShChunks = SHARED ? (int)(LS.gu_tile / 1024) : 4;
  static_assert(!SHARED || LS.gu_tile % 4096 == 0, "shared tile: whole 1 KiB chunks per wave");
  __shared__ __align__(16) uint8_t sh_tile[SHARED ? LS.gu_tile : 16];
  __shared__ uint32_t shcnt;  // waves 2-3: shared-tile partial sums written (count)
  // staged h of the down projection, per 32-column chunk (two 16-row
  // tiles): 16 words of fp16 pairs (padded to 20 so that the 4 chunks a
  // half-wave reads at once fall in distinct banks), then per tile (C, up)
  extern __shared__ __align__(16) uint32_t hq[];
  float* const hcst = reinterpret_cast<float*>(hq + (size_t)((p.k * IR + (SHARED ? IS : 0)) / CC) * kHqStride);
  float* const hsm = hcst + (size_t)((p.k * IR + (SHARED ? IS : 0)) / CC) * 4;  // sum of h per tile

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int w = blockIdx.x, NWG = gridDim.x;
  constexpr int I = IR, Is = SHARED ? IS : 0;
  const int E = EC ? EC : p.E, k = KC ? KC : p.k, L = p.L;
  const uint32_t ep0 = p.ctr[0] + 1u;  // epoch of layer 0; layer l uses ep0 + l

  // phase B items: shared tiles first, then routed (j, tile)
  constexpr int tiles_r = I / kRowTile, tiles_s = Is / kRowTile;
  const int NI = tiles_s + k * tiles_r;
  const int NH = k * I + Is;  // h values per layer
  const int nchh = NH / CC;
  // phase C: half-tile w (8 output rows)
  const bool has_c = w < H / 8;
  const int ctile = w >> 1, chalf = w & 1;
  const int hw = wave * 2 + (lane >> 5), l32 = lane & 31;
  const int row8 = l32 >> 2, c4 = lane & 3;
  constexpr int nkb_r = I / KBC, nkb_s = Is / KBC;
  const int n_units = k * nkb_r + nkb_s;
  const int dsb_off = kCodeBlockBytes + ((chalf * 8 + row8) * GPK + (c4 * CC) / kGroup) * 4;
  // gate/up lane geometry
  const int grow = lane >> 2;
  const int sbg_off = 2 * kCodeBlockBytes + (grow * GPK + (c4 * CC) / kGroup) * 4;
  const int sbu_off = sbg_off + kRowTile * GPK * 4;
  int nrows = 0;
#pragma unroll
  for (int r = 0; r < kRR; ++r)
    if (w + NWG * r < E + hsh) nrows = r + 1;
  const int item0 = w, item1 = w + NWG;
  const auto rx = word_rsrc(p.xw, H / 2);
  const auto rl = word_rsrc(p.lw, E + hsh);
  const auto rh = word_rsrc(p.hw, NH);

  struct GuRegs {
    uint4 g[NKW], u[NKW];
    uint32_t sg[NKW], su[NKW];
  };
  GuRegs ra, rb;  // routed tiles
  uint4 dq[kMaxDownUnits];
  uint32_t dsb[kMaxDownUnits];
  float4 wr[kRR][NXP];  // router rows: the weights of the owned x elements
  uint32_t wq[DQ4 ? kRR : 1], wsb[DQ4 ? kRR : 1];  // 4-bit dense rows: the owned elements' codes,
                                                   // their group's word
  float rbias = 0.0f;   // lane r: bias of router row r (when that row has one)
  int32_t slot_r[(EMAX + 255) / 256];

  auto issue_gu = [&](GuRegs& R, gbyte* blob, int tile, int64_t unit_b, int64_t tile_b) {
    gbyte* tb = gptr(uniform_u64(reinterpret_cast<uint64_t>(blob + (int64_t)tile * tile_b)));
#pragma unroll
    for (int i = 0; i < NKW; ++i) {
      gbyte* unit = tb + (int64_t)(wave + 4 * i) * unit_b;
      R.g[i] = gload16(unit + lane * 16);
      R.u[i] = gload16(unit + kCodeBlockBytes + lane * 16);
      R.sg[i] = gload4(unit + sbg_off);
      R.su[i] = gload4(unit + sbu_off);
    }
  };
  // one k-block (128 columns) of a 16-row gate/up tile against the staged
  // x, accumulated into this lane's partial g, u (4 lanes per row)
  auto gu_block = [&](int kb, const uint4 cg, const uint4 cu, uint32_t sgw, uint32_t suw, float& g,
                      float& u) {
    uint32_t mlo = 0x000F000Fu, mhi = 0x00F000F0u, magic = 0x64006400u;
    asm volatile("" : "+v"(mlo), "+v"(mhi), "+v"(magic));  // keep in VGPRs: v_and_or_b32
    const int gc = kb * 4 + c4;
    const float2 c = cs[gc];
    float pg = 0.f, pu = 0.f;
    const uint32_t dg[4] = {cg.x, cg.y, cg.z, cg.w};
    const uint32_t du[4] = {cu.x, cu.y, cu.z, cu.w};
    const uint4* xq = reinterpret_cast<const uint4*>(xp + gc * XS);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint4 X = xq[m];
      const uint32_t eg = dg[m] >> 8, eu = du[m] >> 8;
      pg = dot2((dg[m] & mlo) | magic, X.x, pg);
      pu = dot2((du[m] & mlo) | magic, X.x, pu);
      pg = dot2((dg[m] & mhi) | magic, X.y, pg);
      pu = dot2((du[m] & mhi) | magic, X.y, pu);
      pg = dot2((eg & mlo) | magic, X.z, pg);
      pu = dot2((eu & mlo) | magic, X.z, pu);
      pg = dot2((eg & mhi) | magic, X.w, pg);
      pu = dot2((eu & mhi) | magic, X.w, pu);
    }
    g += bf16_bits_to_f32(sgw & 0xFFFFu) * (pg - c.x) + bf16_bits_to_f32(sgw >> 16) * c.y;
    u += bf16_bits_to_f32(suw & 0xFFFFu) * (pu - c.x) + bf16_bits_to_f32(suw >> 16) * c.y;
  };
  auto gu_store = [&](float g, float u, float (*rd)[kRowTile][2]) {
    g = quad_sum(g);
    u = quad_sum(u);
    if (c4 == 0) {
      rd[wave][grow][0] = g;
      rd[wave][grow][1] = u;
    }
  };
  // dot products of one 16-row tile over this wave's k-blocks (wave + 4 i),
  // from registers; the per-row partial sums go to rd[wave]
  auto gu_dots = [&](const GuRegs& R, float (*rd)[kRowTile][2]) {
    float g = 0.f, u = 0.f;
#pragma unroll
    for (int i = 0; i < NKW; ++i) gu_block(wave + 4 * i, R.g[i], R.u[i], R.sg[i], R.su[i], g, u);
    gu_store(g, u, rd);
  };
  // waves 1-3: the shared tile from LDS, k-blocks (wave - 1) + 3 i
  auto gu_dots_shared = [&](float (*rd)[kRowTile][2], const uint8_t* sh_tile) {
    float g = 0.f, u = 0.f;
#pragma unroll
    for (int i = 0; i < (NKB + 2) / 3; ++i) {
      const int kb = (wave - 1) + 3 * i;
      if (kb < NKB) {
        const uint8_t* unit = sh_tile + kb * LS.gu_unit;
        gu_block(kb, *reinterpret_cast<const uint4*>(unit + lane * 16),
                 *reinterpret_cast<const uint4*>(unit + kCodeBlockBytes + lane * 16),
                 *reinterpret_cast<const uint32_t*>(unit + sbg_off),
                 *reinterpret_cast<const uint32_t*>(unit + sbu_off), g, u);
      }
    }
    gu_store(g, u, rd);
  };
  // one wave, once all 4 waves' partial sums are in rd: the tile's h,
  // staged and published as word pairs
  auto gu_finish = [&](float (*rd)[kRowTile][2], int64_t hoff, uint32_t ep) {
    {
      // h of the tile's 16 rows, staged for the down dot products: scaled by
      // a power of two so that the largest |h| lands in [2^13, 2^14), rounded
      // to fp16, and paired (row s, row s + 4) within each group of 8 rows,
      // the order in which the int4 code masks pick two nibbles of a code
      // word.  Published as 6 word pairs: 4 of fp16 pairs, (1024 x the sum
      // of the 16 staged values, the scale to undo), (the sum of h, 0).
      float hv = 0.0f;
      if (lane < kRowTile) {
        const float gs = (rd[0][lane][0] + rd[1][lane][0]) + (rd[2][lane][0] + rd[3][lane][0]);
        const float us = (rd[0][lane][1] + rd[1][lane][1]) + (rd[2][lane][1] + rd[3][lane][1]);
        hv = silu_f32(gs) * us;
      }
      const uint32_t amax = wave_max_dpp(__float_as_uint(hv) & 0x7FFFFFFFu);
      const int ex = max((int)(amax >> 23), 14);
      const float down = __uint_as_float((uint32_t)(267 - ex) << 23);  // 2^(140 - ex)
      const float up = __uint_as_float((uint32_t)(ex - 13) << 23);     // 2^(ex - 140)
      // odd rows (picked by the code mask 0x00F000F0, i.e. as 16 q) are
      // staged divided by 16
      const _Float16 t = (_Float16)(hv * down * ((lane & 1) ? 0.0625f : 1.0f));
      const float tsum = wave_sum_dpp(lane < kRowTile ? (float)t : 0.0f);
      const float hsum = wave_sum_dpp(hv);
      if (lane < kRowTile) tt[lane] = (uint32_t)__builtin_bit_cast(uint16_t, t);
      lds_wave_sync();
      const int tile = (int)(hoff >> 4);
      if (lane < 4) {
        uint32_t w2[2];
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2) {
          const int wd = 2 * lane + e2, g8 = (wd >> 2) * 8, sl = wd & 3;
          w2[e2] = tt[g8 + sl] | (tt[g8 + sl + 4] << 16);
        }
        st_pair(rh, tile * kHTilePairs + lane, ep, w2[0], w2[1]);
      } else if (lane == 4) {
        st_pair(rh, tile * kHTilePairs + 4, ep, __float_as_uint(1024.0f * tsum), __float_as_uint(up));
      } else if (lane == 5) {
        st_pair(rh, tile * kHTilePairs + 5, ep, __float_as_uint(hsum), 0u);
      }
    }
  };
  auto compute_gu = [&](const GuRegs& R, int64_t hoff, uint32_t ep) {
    gu_dots(R, red);
    wg_barrier();
    if (wave == 0) gu_finish(red, hoff, ep);
    wg_barrier();
  };
  // loads of layer l that do not depend on its input: the router row and
  // the slot table.  Issued after the previous layer's h poll (whose wait
  // retires every earlier load), so that the down projection never waits
  // for them.  (The shared tile: load_shared_tile.)
  auto prefetch = [&](int l) {
    const uint8_t* sblob = p.shared_blobs + (int64_t)l * p.shared_stride;
    if constexpr (DQ4) {
      // dense blob: the 8 codes of the owned elements (one word) and the
      // (scale, bias) word of their group; the shared gate is row E
      const uint8_t* db = p.dense + (int64_t)l * p.dense_stride;
#pragma unroll
      for (int r = 0; r < kRR; ++r) {
        const int row = w + NWG * r;
        if (r < nrows) {
          wq[r] = *reinterpret_cast<const uint32_t*>(db + (int64_t)row * (H / 2) + 4 * tid);
          wsb[r] = *reinterpret_cast<const uint32_t*>(db + p.dense_words +
                                                     ((int64_t)row * (H / kGroup) + tid / 8) * 4);
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < kRR; ++r) {
        const int row = w + NWG * r;
        if (r < nrows) {
          const float* rowp = row < E ? p.router_w + ((int64_t)l * E + row) * H
                                      : reinterpret_cast<const float*>(sblob + LS.sg_off);
#pragma unroll
          for (int m = 0; m < NXP; ++m) wr[r][m] = *reinterpret_cast<const float4*>(rowp + 8 * tid + 4 * m);
        }
      }
    }
    // every lane loads (a clamped row): a load under a lane mask followed by
    // a read under the complement would wait for the whole prefetch
    if (p.router_bias != nullptr)
      rbias = p.router_bias[(int64_t)l * E + min(w + NWG * min(lane, kRR - 1), E - 1)];
    const int32_t* st = p.slot_tables + (int64_t)l * E;
#pragma unroll
    for (int m = 0; m < (EMAX + 255) / 256; ++m)
      if (tid + 256 * m < E) slot_r[m] = st[tid + 256 * m];
  };



  // the shared tile of layer l: by all 4 waves, straight into LDS (1 KiB
  // per wave instruction, each lane 16 bytes)
  auto load_shared_tile = [&](int l) {
    if (SHARED && item0 < tiles_s) {
      const uint8_t* tb = p.shared_blobs + (int64_t)l * p.shared_stride + (int64_t)item0 * LS.gu_tile;
#pragma unroll
      for (int j = 0; j < kShChunks / 4; ++j) {
        const int c = wave + 4 * j;
        __builtin_amdgcn_global_load_lds(CH_G1(tb + c * 1024 + lane * 16), CH_L3(sh_tile + c * 1024),
                                         16, 0, 0);
      }
    }
  };
  if (tid == 0) shcnt = 0u;
  if (tid < 2 * kRowTile) red_s[0][tid >> 1][tid & 1] = 0.0f;  // wave 0 takes no share
  prefetch(0);
  load_shared_tile(0);
  for (int l = 0; l < L; ++l) {
    const uint32_t ep = ep0 + (uint32_t)l;
    const uint8_t* sblob = p.shared_blobs + (int64_t)l * p.shared_stride;

    // ---------------- A: input, RMSNorm, router ----------------
    {
      // thread tid polls the word pairs tid + 256 m (x elements 4q .. 4q+3);
      // its sum of squares runs over them in a fixed order, so every
      // workgroup gets the same bits whatever order the words arrive in
      uint32_t xw[2 * NXP];
      if (l == 0) {
#pragma unroll
        for (int m = 0; m < NXP; ++m) {
          const uint2 t = *reinterpret_cast<const uint2*>(p.x + 4 * (tid + 256 * m));
          xw[2 * m] = t.x;
          xw[2 * m + 1] = t.y;
        }
      } else {
        poll_pairs<NXP>(rx, H / 2, tid, 256, ep - 1u, p.err, [&](int q, uint32_t a, uint32_t b) {
          const int m = (q - tid) >> 8;
          xw[2 * m] = a;
          xw[2 * m + 1] = b;
        });
      }
      float ss = 0.f;
#pragma unroll
      for (int m = 0; m < NXP; ++m) {
        const float a0 = bf16_bits_to_f32(xw[2 * m] & 0xFFFFu);
        const float a1 = bf16_bits_to_f32(xw[2 * m] >> 16);
        const float a2 = bf16_bits_to_f32(xw[2 * m + 1] & 0xFFFFu);
        const float a3 = bf16_bits_to_f32(xw[2 * m + 1] >> 16);
        *reinterpret_cast<float4*>(xs + 4 * (tid + 256 * m)) = make_float4(a0, a1, a2, a3);
        ss += (a0 * a0 + a1 * a1) + (a2 * a2 + a3 * a3);
      }
      ss = wave_sum_dpp(ss);
      if (lane == 0) wsum[wave] = ss;
    }
#pragma unroll
    for (int m = 0; m < (EMAX + 255) / 256; ++m)
      if (tid + 256 * m < E) slot_l[tid + 256 * m] = slot_r[m];
    wg_barrier();
    // v_rsq_f32 (within 1 ulp; every workgroup computes the same bits)
    const float inv =
        __builtin_amdgcn_rsqf(((wsum[0] + wsum[1]) + (wsum[2] + wsum[3])) / (float)H + p.eps);
    // x_hat of the elements 8 tid .. 8 tid + 7 (quarter tid % 4 of staged
    // chunk tid / 4), rounded to bf16: the router's and the experts' input
    float xv[8];
    {
      const float4 u0 = *reinterpret_cast<const float4*>(xs + 8 * tid);
      const float4 u1 = *reinterpret_cast<const float4*>(xs + 8 * tid + 4);
      xv[0] = bf16r(u0.x * inv);
      xv[1] = bf16r(u0.y * inv);
      xv[2] = bf16r(u0.z * inv);
      xv[3] = bf16r(u0.w * inv);
      xv[4] = bf16r(u1.x * inv);
      xv[5] = bf16r(u1.y * inv);
      xv[6] = bf16r(u1.z * inv);
      xv[7] = bf16r(u1.w * inv);
    }
    // the router logits first (their exchange gates the top-k): each
    // thread's partial dot product over its elements, summed per wave, then
    // over the 4 waves in a fixed order
    // (4-bit dense rows: sum_i (s q_i + b) x_i = s sum_i q_i x_i + b sum_i x_i)
#pragma unroll
    for (int r = 0; r < kRR; ++r) {
      if (r < nrows) {
        float acc = 0.f;
        if constexpr (DQ4) {
          const float xsum8 =
              ((xv[0] + xv[1]) + (xv[2] + xv[3])) + ((xv[4] + xv[5]) + (xv[6] + xv[7]));
          float qx = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) qx += (float)((wq[r] >> (4 * i)) & 15u) * xv[i];
          acc = bf16_bits_to_f32(wsb[r] & 0xFFFFu) * qx + bf16_bits_to_f32(wsb[r] >> 16) * xsum8;
        } else {
#pragma unroll
          for (int m = 0; m < NXP; ++m)
            acc += (wr[r][m].x * xv[4 * m] + wr[r][m].y * xv[4 * m + 1]) +
                   (wr[r][m].z * xv[4 * m + 2] + wr[r][m].w * xv[4 * m + 3]);
        }
        acc = wave_sum_dpp(acc);
        if (lane == 0) rred[r][wave] = acc;
      }
    }
    wg_barrier();
    if (wave == 0 && lane < nrows) {
      const float b = (p.router_bias != nullptr && w + NWG * lane < E) ? rbias : 0.0f;
      st_word(p.lw + w + NWG * lane, ep,
              __float_as_uint(((rred[lane][0] + rred[lane][1]) + (rred[lane][2] + rred[lane][3])) + b));
    }
    // x_hat staged for the gate/up dot products: thread tid takes quarter
    // tid % 4 of chunk tid / 4 (its own 8 elements); block 0 stores it
    {
      const int ch = tid >> 2, jj = tid & 3;
      if (w == 0) {
#pragma unroll
        for (int q = 0; q < 8; q += 2)
          *reinterpret_cast<uint32_t*>(p.x_hat + 8 * tid + q) =
              (uint32_t)f32_to_bf16_bits(xv[q]) | ((uint32_t)f32_to_bf16_bits(xv[q + 1]) << 16);
      }
      const uint32_t pa = pack_f16x2(xv[0], xv[4]);
      const uint32_t pb = pack_f16x2(xv[1] * 0.0625f, xv[5] * 0.0625f);
      const uint32_t pc = pack_f16x2(xv[2], xv[6]);
      const uint32_t pf = pack_f16x2(xv[3] * 0.0625f, xv[7] * 0.0625f);
      *reinterpret_cast<uint4*>(xp + ch * XS + jj * 4) = make_uint4(pa, pb, pc, pf);
      float c = f16lo(pa) + f16hi(pa) + f16lo(pb) + f16hi(pb) + f16lo(pc) + f16hi(pc) + f16lo(pf) +
                f16hi(pf);
      float sx = f16lo(pa) + f16hi(pa) + f16lo(pc) + f16hi(pc) +
                 16.0f * (f16lo(pb) + f16hi(pb) + f16lo(pf) + f16hi(pf));
      // combine the 4 threads of the chunk (adjacent lanes), fixed order
      c = quad_sum(c);
      sx = quad_sum(sx);
      if (jj == 0) cs[ch] = make_float2(1024.0f * c, sx);
    }
    wg_barrier();

    // ---------------- B: top-k, routed tiles, shared tile ----------------
    // a workgroup with a shared tile: waves 1-3 take their share of its dot
    // products while wave 0 polls the logits and finds the top-k; wave 0
    // takes its share while the routed tiles load
    const bool sh0 = SHARED && item0 < tiles_s;
    if (sh0 && wave != 0) {
      // waves 1-3: the whole shared tile, while wave 0 polls and ranks; wave
      // 1 finishes it once waves 2-3 have written their partial sums
      gu_dots_shared(red_s, sh_tile);
      if (wave != 1) {
        lds_wave_sync();
        if (lane == 0) __hip_atomic_fetch_add(&shcnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      } else {
        const uint32_t target = 2u * (uint32_t)(l + 1);
        uint32_t spins = 0;
        while (__hip_atomic_load(&shcnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target) {
          if (++spins > kSpinLimit) {
            atomicOr(p.err, 1u);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        gu_finish(red_s, (int64_t)k * I + item0 * kRowTile, ep);
      }
    }
    if (wave == 0) {
      poll_pairs<(EMAX + 128) / 128>(rl, E + hsh, lane, 64, ep, p.err,
                                                 [&](int q, uint32_t a, uint32_t b) {
                                                   lg[2 * q] = __uint_as_float(a);
                                                   if (2 * q + 1 < E + hsh)
                                                     lg[2 * q + 1] = __uint_as_float(b);
                                                 });
      lds_wave_sync();
      wave_topk_set<EPL>(lg, E, k, sel_idx, sel_val, cand,
                         [&](int pos, int idx) {
                           sel_base[pos] = reinterpret_cast<uint64_t>(p.slab + (int64_t)slot_l[idx] * p.stride);
                         });
    }
    wg_barrier();
    // routed gate/up tiles of this workgroup (both issued before either is
    // computed)
    int rj[2] = {-1, -1}, rt[2] = {0, 0};
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int item = s2 == 0 ? item0 : item1;
      if (item >= tiles_s && item < NI) {
        const int ii = item - tiles_s;
        rj[s2] = ii / tiles_r;
        rt[s2] = ii - rj[s2] * tiles_r;
      }
    }
    if (rj[0] >= 0) issue_gu(ra, gptr(sel_base[rj[0]]), rt[0], LR.gu_unit, LR.gu_tile);
    if (rj[1] >= 0)
      issue_gu(rb, gptr(sel_base[rj[1]]), rt[1], LR.gu_unit, LR.gu_tile);
    else if (SHARED && item1 < tiles_s)
      issue_gu(rb, gptr(sblob), item1, LS.gu_unit, LS.gu_tile);
    // routing weights (needed from phase C on), off the load path
    if (wave == 0) {
      set_softmax(sel_val, k, sel_w);
      if (lane == 0) gam = SHARED ? 1.0f / (1.0f + expf(-lg[E])) : 0.0f;
    }
    if (rj[0] >= 0) compute_gu(ra, (int64_t)rj[0] * I + rt[0] * kRowTile, ep);
    if (rj[1] >= 0)
      compute_gu(rb, (int64_t)rj[1] * I + rt[1] * kRowTile, ep);
    else if (SHARED && item1 < tiles_s)
      compute_gu(rb, (int64_t)k * I + item1 * kRowTile, ep);
    // down units of phase C, routed then shared: issued once this
    // workgroup's gate/up tiles have arrived, so that they do not compete
    // with the gate/up loads every workgroup is still waiting for
    if (has_c) {
      // unit slot i of this wave: units u0 = 8 i + 2 wave (half-wave 0) and
      // u0 + 1 (half-wave 1).  nkb_r and nkb_s are even, so both are of the
      // same expert and kind: the blob base is wave-uniform, the rest a
      // 32-bit per-lane offset
      static_assert(nkb_r % 2 == 0 && (nkb_s % 2 == 0), "down units pair up per wave");
      const uint32_t kbo = (uint32_t)(hw & (nkb_r - 1));  // k-block of this half-wave's unit
      const uint32_t oc_r = (uint32_t)(LR.d_off + ctile * LR.d_tile + kbo * LR.d_unit) + chalf * 512 + l32 * 16;
      const uint32_t os_r = (uint32_t)(LR.d_off + ctile * LR.d_tile + kbo * LR.d_unit) + dsb_off;
      const uint32_t oc_s = (uint32_t)(LS.d_off + ctile * LS.d_tile + kbo * LS.d_unit) + chalf * 512 + l32 * 16;
      const uint32_t os_s = (uint32_t)(LS.d_off + ctile * LS.d_tile + kbo * LS.d_unit) + dsb_off;
#pragma unroll
      for (int i = 0; i < kMaxDownUnits; ++i) {
        const int u0 = 8 * i + 2 * wave;
        if (u0 < n_units) {
          const bool routed = u0 < k * nkb_r;
          gbyte* base = gptr(uniform_u64(routed ? sel_base[u0 / nkb_r] : reinterpret_cast<uint64_t>(sblob)));
          dq[i] = gload16(base + (routed ? oc_r : oc_s));
          dsb[i] = gload4(base + (routed ? os_r : os_s));
        }
      }
    }

    // ---------------- C: down + combine + residual ----------------
    // h arrives staged: 6 word pairs per 16-row tile (4 of fp16 pairs, then
    // (1024 x sum of the staged values, scale), (sum of h, 0))
    poll_pairs<kHPoll>(rh, (NH >> 4) * 2 * kHTilePairs, tid, 256, ep, p.err,
                        [&](int q, uint32_t a, uint32_t b) {
      const int tile = q / kHTilePairs, slot = q - tile * kHTilePairs;
      if (slot < 4)
        *reinterpret_cast<uint2*>(hq + (tile >> 1) * kHqStride + (tile & 1) * 8 + 2 * slot) =
            make_uint2(a, b);
      else if (slot == 4)
        *reinterpret_cast<float2*>(hcst + 4 * (tile >> 1) + 2 * (tile & 1)) =
            make_float2(__uint_as_float(a), __uint_as_float(b));
      else
        hsm[tile] = __uint_as_float(a);
    });
    // every load issued so far has returned (the poll waited for them); say
    // so, so that the down projection below does not wait for the prefetch
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    prefetch(min(l + 1, L - 1));
    wg_barrier();
    if (has_c) {
      // units hw, hw + 8, ... of this half-wave (a unit past the last is
      // computed on unit 0's data and dropped)
      uint32_t mlo = 0x000F000Fu, mhi = 0x00F000F0u, magic = 0x64006400u;
      asm volatile("" : "+v"(mlo), "+v"(mhi), "+v"(magic));  // keep in VGPRs: v_and_or_b32
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < kMaxDownUnits; ++i) {
        const int uidx = hw + 8 * i;
        const bool valid = uidx < n_units;
        const int u = valid ? uidx : 0;
        int hb, kb;
        float dwi;
        if (u < k * nkb_r) {
          const int jj = u / nkb_r;
          kb = u - jj * nkb_r;
          hb = jj * I;
          dwi = sel_w[jj];
        } else {
          kb = u - k * nkb_r;
          hb = k * I;
          dwi = gam;
        }
        const int ch = (hb + kb * KBC) / CC + c4;
        const uint4* X = reinterpret_cast<const uint4*>(hq + ch * kHqStride);
        const float4 K = *reinterpret_cast<const float4*>(hcst + 4 * ch);
        const float2 S = *reinterpret_cast<const float2*>(hsm + 2 * ch);
        // word m of the codes: nibbles (n, n + 4) pair up as the staging
        // paired rows (s, s + 4); words 0-1 are the chunk's first tile
        float pt[2];
#pragma unroll
        for (int tl = 0; tl < 2; ++tl) {
          float pa = 0.f, pb = 0.f;
#pragma unroll
          for (int mm = 0; mm < 2; ++mm) {
            const int m = 2 * tl + mm;
            const uint32_t d = m == 0 ? dq[i].x : m == 1 ? dq[i].y : m == 2 ? dq[i].z : dq[i].w;
            const uint32_t e = d >> 8;
            const uint4 Xm = X[m];
            pa = dot2((d & mlo) | magic, Xm.x, pa);
            pb = dot2((d & mhi) | magic, Xm.y, pb);
            pa = dot2((e & mlo) | magic, Xm.z, pa);
            pb = dot2((e & mhi) | magic, Xm.w, pb);
          }
          pt[tl] = pa + pb;
        }
        const float sq = K.y * (pt[0] - K.x) + K.w * (pt[1] - K.z);  // sum of q h
        const float sc = bf16_bits_to_f32(dsb[i] & 0xFFFFu), bi = bf16_bits_to_f32(dsb[i] >> 16);
        const float term = dwi * (sc * sq + bi * (S.x + S.y));
        acc += valid ? term : 0.0f;
      }
      acc = quad_sum(acc);
      if (c4 == 0) dred[wave][lane >> 5][row8] = acc;
    }
    wg_barrier();
    // the next layer's shared tile (this layer's was consumed in phase B),
    // over the x exchange
    if (l + 1 < L) load_shared_tile(l + 1);
    if (has_c && tid < 8) {
      // lane r: row r of the half-tile; lanes 4 q .. 4 q + 3 gather their
      // four rows into lane 4 q (DPP within the quad), which publishes them
      const int r = tid;
      float v = 0.f;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) v += dred[ww][0][r] + dred[ww][1][r];
      const int orow = ctile * kRowTile + chalf * 8 + r;
      const uint32_t ov = f32_to_bf16_bits(v);
      const uint32_t xv = f32_to_bf16_bits(xs[orow] + bf16_bits_to_f32(ov));
      // quad_perm [1,1,3,3]: lanes 0, 2 take lanes 1, 3; [2,3,2,3]: lane 0 takes lane 2
      const uint32_t x01 = xv | (dpp_u<0xF5, 0xF>(0u, xv) << 16);
      const uint32_t o01 = ov | (dpp_u<0xF5, 0xF>(0u, ov) << 16);
      const uint32_t x23 = dpp_u<0xEE, 0xF>(0u, x01);
      const uint32_t o23 = dpp_u<0xEE, 0xF>(0u, o01);
      if ((tid & 3) == 0) {
        const int orow0 = ctile * kRowTile + chalf * 8 + tid;
        if (l + 1 < L) {
          st_pair(rx, orow0 / 4, ep, x01, x23);
        } else {
          *reinterpret_cast<uint2*>(p.x + orow0) = make_uint2(x01, x23);
          *reinterpret_cast<uint2*>(p.out + orow0) = make_uint2(o01, o23);
        }
      }
    }
    wg_barrier();
  }
  // the last layer's routing, in routing order
  if (w == 0 && wave == 0) {
    set_rank_out(sel_idx, sel_val, sel_w, k, p.r_idx, p.r_w);
    if (lane == 0 && SHARED) *p.r_gamma = gam;
  }
  if (w == 0 && tid == 0) p.ctr[0] = ep0 + (uint32_t)(L - 1);
}

// Compute units of each device, read once.  Concurrent first calls may both
// query the device; they store the same value, and the atomic makes the
// store and the loads race-free.
std::atomic<int> g_num_cus[16];

}  // namespace

int chain_grid(int device) {
  if (device < 0 || device >= 16) return 0;
  int n = g_num_cus[device].load(std::memory_order_relaxed);
  if (n == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) return 0;
    n = prop.multiProcessorCount;
    g_num_cus[device].store(n, std::memory_order_relaxed);
  }
  return n;
}

size_t chain_lds_bytes(int bits, int NH) {
  (void)bits;
  const int nch = NH / 32;  // 32-column chunks (int4)
  return (size_t)nch * (kHqStride * sizeof(uint32_t) + 6 * sizeof(float));
}

bool chain_supported(int nwg, int T, int act, int H, int E, int k, int bits, int I, int Is,
                     bool has_shared) {
  if (T != 1 || act != MOE_ACT_BF16 || H != 2048 || bits != 4 || nwg < 1) return false;
  // the kernel is compiled for expert (and shared) intermediate size 512
  if (I != 512 || (has_shared && Is != 512)) return false;
  if (E > kChainMaxExperts) return false;
  const int kbc = kRowBytes * (8 / bits);
  if (E + (has_shared ? 1 : 0) > 4 * nwg) return false;
  const int NI = (has_shared ? Is / kRowTile : 0) + k * (I / kRowTile);
  if (NI > 2 * nwg || NI > 1024) return false;
  if (H / 8 > nwg) return false;
  const int n_units = k * (I / kbc) + (has_shared ? Is / kbc : 0);
  if (n_units > 8 * (bits == 4 ? max_down_units<4>() : max_down_units<8>())) return false;
  const int NH = k * I + (has_shared ? Is : 0);
  if (chain_lds_bytes(bits, NH) > 64 * 1024) return false;
  if (NH > 24 * 256 * 4) return false;
  return true;
}


hipError_t launch_chain(const ChainParams& prm, int nwg, hipStream_t s) {
  const int NH = prm.k * prm.I + (prm.has_shared ? prm.Is : 0);
  const size_t lds = chain_lds_bytes(prm.bits_, NH);
  void* args[] = {const_cast<ChainParams*>(&prm)};
  if (prm.bits_ != 4 || prm.H != 2048 || prm.I != 512) return hipErrorInvalidValue;
  if (prm.has_shared && prm.Is != 512) return hipErrorInvalidValue;
  const bool small = prm.E <= 256, dq = prm.dense != nullptr;
#define MOE_CHAIN_FN(SH, EPL, EC, KC)                                                         \
  (dq ? reinterpret_cast<const void*>(&chain_kernel<4, 8, SH, 512, 512, EPL, EC, KC, true>) \
      : reinterpret_cast<const void*>(&chain_kernel<4, 8, SH, 512, 512, EPL, EC, KC, false>))
  const void* fn;
  if (prm.has_shared && prm.E == 256 && prm.k == 8)
    fn = MOE_CHAIN_FN(true, 4, 256, 8);
  else if (prm.has_shared && prm.E == 512 && prm.k == 10)
    fn = MOE_CHAIN_FN(true, 8, 512, 10);
  else if (prm.has_shared)
    fn = small ? MOE_CHAIN_FN(true, 4, 0, 0) : MOE_CHAIN_FN(true, 8, 0, 0);
  else
    fn = small ? MOE_CHAIN_FN(false, 4, 0, 0) : MOE_CHAIN_FN(false, 8, 0, 0);
#undef MOE_CHAIN_FN
  // every workgroup must be resident together: the exchanges wait on each other
  int per_cu = 0, dev = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, lds);
  if (e != hipSuccess) return e;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((int64_t)per_cu * chain_grid(dev) < nwg) return hipErrorCooperativeLaunchTooLarge;
  return hipLaunchKernel(fn, dim3(nwg), dim3(256), args, lds, s);
}

}  // namespace moe
