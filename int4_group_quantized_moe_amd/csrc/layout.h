// Blob layout arithmetic and workspace plan of the MoE layer library: plain
// host C++ (no HIP), shared by the host entry points and the kernels' host
// launch code.  Not installed.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kRowTile = 16;         // rows per tile in both blob sections
constexpr int kRowBytes = 64;        // code bytes per row per k-block
constexpr int kCodeBlockBytes = kRowTile * kRowBytes;  // 1 KiB
constexpr int kGroup = 64;
constexpr int kDecodeMaxTokens = 8;    // up to this many tokens: per-pair GEMV path
// bf16 buckets of this many tokens run on the MFMA grouped GEMMs: every
// bucket (1), since a tile of at most 64 rows halves its K loop between the
// wave rows and the grouped GEMMs' time is per-tile latency, not work
constexpr int kMfmaMinRows = 1;
constexpr int kMfmaTileRows = 128;  // rows (bucket entries) per grouped-GEMM tile
constexpr int kOneBlockTokens = 64;  // batches up to this size: every bucket fits one 64-row tile

constexpr int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

// Byte layout of one blob.  Everything is a multiple of 64 bytes; blob sizes
// are multiples of 256.
struct BlobLayout {
  int bits, hidden, inter;
  int kb_cols;        // columns per k-block (64 bytes of codes per row)
  int gpk;            // quantisation groups per k-block
  int n_kb_gu;        // k-blocks along H (gate/up)
  int n_tiles_gu;     // row tiles along I (gate/up)
  int n_kb_d;         // k-blocks along I (down)
  int n_tiles_d;      // row tiles along H (down)
  int64_t gu_unit, gu_tile, gu_off;
  int64_t d_unit, d_tile, d_off;
  int64_t blob, sg_off, shared_bytes;
};

constexpr BlobLayout make_layout(int bits, int hidden, int inter) {
  BlobLayout L{};
  L.bits = bits;
  L.hidden = hidden;
  L.inter = inter;
  L.kb_cols = kRowBytes * (8 / bits);
  L.gpk = L.kb_cols / kGroup;
  L.n_kb_gu = hidden / L.kb_cols;
  L.n_tiles_gu = inter / kRowTile;
  L.n_kb_d = inter / L.kb_cols;
  L.n_tiles_d = hidden / kRowTile;
  const int64_t sb_block = (int64_t)kRowTile * L.gpk * 4;
  L.gu_unit = 2 * kCodeBlockBytes + 2 * sb_block;
  L.gu_tile = L.gu_unit * L.n_kb_gu;
  L.gu_off = 0;
  L.d_unit = kCodeBlockBytes + sb_block;
  L.d_tile = L.d_unit * L.n_kb_d;
  L.d_off = L.gu_off + L.gu_tile * L.n_tiles_gu;
  L.blob = align_up(L.d_off + L.d_tile * L.n_tiles_d, 256);
  L.sg_off = L.blob;
  L.shared_bytes = align_up(L.sg_off + (int64_t)hidden * 4, 256);
  return L;
}

// Dense blob of a layer (MOE_FLAG_DENSE_Q4): rows x hidden/2 code bytes, then
// rows x hidden/64 (scale, bias) words.
struct DenseLayout {
  int64_t rows, words_off, bytes;
};
inline DenseLayout make_dense_layout(const moe_layer_desc& d) {
  DenseLayout L;
  L.rows = (int64_t)d.n_experts + ((d.flags & MOE_FLAG_SHARED) ? 1 : 0);
  L.words_off = align_up(L.rows * d.hidden / 2, 256);
  L.bytes = align_up(L.words_off + L.rows * (d.hidden / kGroup) * 4, 256);
  return L;
}

// Workspace plan (byte offsets into the caller's workspace).
struct WsPlan {
  size_t logits, idx, w, gamma, h, partial, counts, offsets, pairs, slots, masks, blkoff, xprep;
  size_t small, nsmall;  // buckets left to the GEMV kernels, and their count
  size_t xw, lw, hw;  // persistent-chain exchange words (batch 1)
  size_t ctr;         // persistent-chain epoch, then status word
  size_t tiles, ntiles;    // grouped-GEMM tile list (large batches)
  size_t x16, xe;          // grouped GEMMs: activations in fp16 and their row exponents
  size_t dense;            // MOE_FLAG_DENSE_Q4: the dense rows dequantised to fp32
  int max_tiles;
  size_t total;
  bool bucketed;
};

// Logit planes of the router GEMM's K split (up to 16 for one token block,
// 8 for other small batches, 2 for large ones: two workgroups per CU).
inline int router_planes(int64_t T) { return T <= kOneBlockTokens ? 16 : (T < 1024 ? 8 : 2); }

inline WsPlan make_ws_plan(const moe_layer_desc& d) {
  WsPlan p{};
  const int64_t T = d.n_tokens, E = d.n_experts, k = d.top_k, H = d.hidden;
  const int64_t I = d.inter;
  const int64_t Is = (d.flags & MOE_FLAG_SHARED) ? d.shared_inter : 0;
  const int64_t nblk = (T + 63) / 64;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = (size_t)align_up((int64_t)(o + bytes), 256);
    return at;
  };
  p.bucketed = T > kDecodeMaxTokens;
  p.logits = take(sizeof(float) * T * (E + 1) * router_planes(T));
  p.idx = take(sizeof(int32_t) * T * k);
  p.w = take(sizeof(float) * T * k);
  p.gamma = take(sizeof(float) * T);
  p.h = take(sizeof(float) * (T * k * I + T * Is));
  p.partial = take(p.bucketed ? sizeof(float) * T * (k + 1) * H : 0);
  p.counts = take(sizeof(int32_t) * (E + 1));
  p.offsets = take(sizeof(int32_t) * (E + 2));
  p.pairs = take(sizeof(int32_t) * T * k);
  p.slots = take(sizeof(int32_t) * MOE_MAX_TOP_K);
  p.masks = take(p.bucketed ? sizeof(uint64_t) * nblk * E : 0);
  p.blkoff = take(p.bucketed ? sizeof(int32_t) * nblk * E : 0);
  p.xprep = take(0);
  p.small = take(p.bucketed ? sizeof(int32_t) * (E + 1) : 0);
  p.nsmall = take(p.bucketed ? sizeof(int32_t) : 0);
  p.max_tiles = (int)((T * k + T) / 128 + E + 2);
  p.tiles = take(p.bucketed ? sizeof(int32_t) * 2 * p.max_tiles : 0);
  p.ntiles = take(p.bucketed ? sizeof(int32_t) : 0);
  const bool gemm = p.bucketed && d.act_dtype == MOE_ACT_BF16;
  p.x16 = take(gemm ? sizeof(uint16_t) * T * H : 0);
  p.xe = take(gemm ? sizeof(int32_t) * T : 0);
  p.dense = take((d.flags & MOE_FLAG_DENSE_Q4) ? sizeof(float) * (E + 1) * H : 0);
  if (T == 1) {
    p.xw = take(sizeof(uint64_t) * (H / 2));
    p.lw = take(sizeof(uint64_t) * (E + 1));
    p.hw = take(sizeof(uint64_t) * (k * I + Is));
  }
  // two 32-bit words: the persistent chain's last epoch, then its status word
  // (bit 0: a bounded wait expired); present for every shape, written only
  // by the persistent chain
  p.ctr = take(sizeof(uint32_t) * 2);
  p.total = o;
  return p;
}

}  // namespace moe
