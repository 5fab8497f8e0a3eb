// C ABI of the MoE layer library: the pure host entry points (version,
// status strings, blob layout, host packer, workspace plan and the device
// addresses inside a workspace) and the argument validation that every entry
// point shares.  Plain C++ with no HIP calls, so it also builds with g++
// under the address and undefined-behaviour sanitizers for a CPU test.
#include <string.h>

#include "host.h"
#include "layout.h"

namespace moe {

namespace {
bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }
}  // namespace

int check_shape(const moe_layer_desc* d) {
  if (d == nullptr) return MOE_ERR_INVALID_ARG;
  if (d->bits != 4 && d->bits != 8) return MOE_ERR_UNSUPPORTED;
  if (d->group != kGroup) return MOE_ERR_UNSUPPORTED;
  if (d->act_dtype != MOE_ACT_F32 && d->act_dtype != MOE_ACT_BF16) return MOE_ERR_UNSUPPORTED;
  if (d->n_tokens < 0) return MOE_ERR_INVALID_ARG;
  if (d->n_experts < 1 || d->n_experts > MOE_MAX_EXPERTS) return MOE_ERR_INVALID_ARG;
  if (d->top_k < 1 || d->top_k > d->n_experts || d->top_k > MOE_MAX_TOP_K)
    return MOE_ERR_INVALID_ARG;
  const int kbc = kRowBytes * (8 / d->bits);
  if (d->hidden < kbc || d->hidden > MOE_MAX_HIDDEN || d->hidden % kbc) return MOE_ERR_UNSUPPORTED;
  if (d->inter < kbc || d->inter > MOE_MAX_INTER || d->inter % kbc) return MOE_ERR_UNSUPPORTED;
  if (d->flags & MOE_FLAG_SHARED) {
    if (d->shared_inter < kbc || d->shared_inter > MOE_MAX_INTER || d->shared_inter % kbc)
      return MOE_ERR_UNSUPPORTED;
  }
  if (d->flags & ~(uint32_t)(MOE_FLAG_ROUTER_BIAS | MOE_FLAG_SHARED | MOE_FLAG_DENSE_Q4))
    return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

int check_stride(const moe_layer_desc* d) {
  const BlobLayout L = make_layout(d->bits, d->hidden, d->inter);
  if (d->expert_stride < L.blob || d->expert_stride % 256) return MOE_ERR_MISALIGNED;
  return MOE_OK;
}

int check_ptr(const void* p, uintptr_t align) {
  if (p == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned(p, align)) return MOE_ERR_MISALIGNED;
  return MOE_OK;
}

int check_opt_ptr(const void* p, uintptr_t align) {
  return p == nullptr ? MOE_OK : check_ptr(p, align);
}

}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_version(void) { return "moe-gfx950 0.1.0"; }

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape, format or dtype";
    case MOE_ERR_MISALIGNED: return "misaligned pointer or stride";
    case MOE_ERR_NO_DEVICE: return "no HIP device";
    case MOE_ERR_LAUNCH: return "kernel launch failed";
    case MOE_ERR_TOO_LARGE: return "problem exceeds a fixed-size buffer (the no-allocation scratch)";
    default: return "unknown status";
  }
}

int moe_blob_layout(const moe_layer_desc* desc, int32_t inter, moe_blob_layout_t* out) {
  if (desc == nullptr || out == nullptr) return MOE_ERR_INVALID_ARG;
  if (desc->bits != 4 && desc->bits != 8) return MOE_ERR_UNSUPPORTED;
  if (desc->group != kGroup) return MOE_ERR_UNSUPPORTED;
  const int kbc = kRowBytes * (8 / desc->bits);
  if (desc->hidden < kbc || desc->hidden > MOE_MAX_HIDDEN || desc->hidden % kbc)
    return MOE_ERR_UNSUPPORTED;
  if (inter < kbc || inter > MOE_MAX_INTER || inter % kbc) return MOE_ERR_UNSUPPORTED;
  const BlobLayout L = make_layout(desc->bits, desc->hidden, inter);
  memset(out, 0, sizeof(*out));
  out->gu_offset = L.gu_off;
  out->gu_unit_bytes = L.gu_unit;
  out->gu_tile_bytes = L.gu_tile;
  out->down_offset = L.d_off;
  out->down_unit_bytes = L.d_unit;
  out->down_tile_bytes = L.d_tile;
  out->blob_bytes = L.blob;
  out->shared_gate_offset = L.sg_off;
  out->shared_bytes = L.shared_bytes;
  out->row_tile = kRowTile;
  out->kblock_cols = L.kb_cols;
  out->groups_per_kblock = L.gpk;
  return MOE_OK;
}

int moe_pack_expert(const moe_layer_desc* desc, int32_t inter, const uint8_t* q_gate,
                    const uint8_t* q_up, const uint8_t* q_down, const uint16_t* sb_gate,
                    const uint16_t* sb_up, const uint16_t* sb_down, const float* shared_gate_w,
                    void* blob_out) {
  moe_blob_layout_t bl;
  MOE_TRY(moe_blob_layout(desc, inter, &bl));
  if (!q_gate || !q_up || !q_down || !sb_gate || !sb_up || !sb_down || !blob_out)
    return MOE_ERR_INVALID_ARG;
  const BlobLayout L = make_layout(desc->bits, desc->hidden, inter);
  const int64_t H = desc->hidden, I = inter;
  const int qmax = (1 << desc->bits) - 1;
  for (int64_t i = 0; i < I * H; ++i)
    if (q_gate[i] > qmax || q_up[i] > qmax || q_down[i] > qmax) return MOE_ERR_INVALID_ARG;
  uint8_t* blob = reinterpret_cast<uint8_t*>(blob_out);
  const int64_t total = shared_gate_w ? L.shared_bytes : L.blob;
  memset(blob, 0, (size_t)total);
  const int cc = 16 * (8 / desc->bits);  // columns per 16-byte lane chunk
  // one section: rows x cols matrices a (and b), tile/k-block units
  auto pack_section = [&](uint8_t* sec, const uint8_t* qa, const uint8_t* qb, const uint16_t* sba,
                          const uint16_t* sbb, int64_t rows, int64_t cols, int64_t unit_bytes,
                          int64_t tile_bytes) {
    const int nmat = qb ? 2 : 1;
    const int64_t G = cols / kGroup;
    const int64_t nkb = cols / L.kb_cols;
    for (int64_t tile = 0; tile < rows / kRowTile; ++tile) {
      for (int64_t kb = 0; kb < nkb; ++kb) {
        uint8_t* unit = sec + tile * tile_bytes + kb * unit_bytes;
        for (int m = 0; m < nmat; ++m) {
          const uint8_t* q = m ? qb : qa;
          const uint16_t* sb = m ? sbb : sba;
          for (int rl = 0; rl < kRowTile; ++rl) {
            const int64_t r = tile * kRowTile + rl;
            uint8_t* dst = unit + m * kCodeBlockBytes + rl * kRowBytes;
            for (int c = 0; c < L.kb_cols; ++c) {
              const uint8_t code = q[r * cols + kb * L.kb_cols + c];
              if (desc->bits == 4) dst[c / 2] |= (uint8_t)(code << (4 * (c & 1)));
              else dst[c] = code;
            }
            for (int gi = 0; gi < L.gpk; ++gi) {
              const int64_t g = kb * L.gpk + gi;
              const uint16_t sc = sb[r * G + g], bi = sb[rows * G + r * G + g];
              uint8_t* p = unit + nmat * kCodeBlockBytes + m * kRowTile * L.gpk * 4 +
                           (rl * L.gpk + gi) * 4;
              memcpy(p, &sc, 2);
              memcpy(p + 2, &bi, 2);
            }
          }
        }
      }
    }
    (void)cc;
  };
  pack_section(blob + L.gu_off, q_gate, q_up, sb_gate, sb_up, I, H, L.gu_unit, L.gu_tile);
  pack_section(blob + L.d_off, q_down, nullptr, sb_down, nullptr, H, I, L.d_unit, L.d_tile);
  if (shared_gate_w) memcpy(blob + L.sg_off, shared_gate_w, sizeof(float) * H);
  return MOE_OK;
}

int moe_dense_layout(const moe_layer_desc* desc, moe_dense_layout_t* out) {
  if (desc == nullptr || out == nullptr) return MOE_ERR_INVALID_ARG;
  if (desc->group != kGroup) return MOE_ERR_UNSUPPORTED;
  if (desc->hidden < kGroup || desc->hidden > MOE_MAX_HIDDEN || desc->hidden % kGroup)
    return MOE_ERR_UNSUPPORTED;
  if (desc->n_experts < 1 || desc->n_experts > MOE_MAX_EXPERTS) return MOE_ERR_INVALID_ARG;
  const DenseLayout L = make_dense_layout(*desc);
  out->rows = L.rows;
  out->words_offset = L.words_off;
  out->bytes = L.bytes;
  return MOE_OK;
}

int moe_pack_dense(const moe_layer_desc* desc, const uint8_t* q, const uint16_t* sb,
                   void* blob_out) {
  moe_dense_layout_t dl;
  MOE_TRY(moe_dense_layout(desc, &dl));
  if (!q || !sb || !blob_out) return MOE_ERR_INVALID_ARG;
  const int64_t H = desc->hidden, R = dl.rows, G = H / kGroup;
  for (int64_t i = 0; i < R * H; ++i)
    if (q[i] > 15) return MOE_ERR_INVALID_ARG;
  uint8_t* blob = reinterpret_cast<uint8_t*>(blob_out);
  memset(blob, 0, (size_t)dl.bytes);
  for (int64_t r = 0; r < R; ++r) {
    for (int64_t c = 0; c < H; ++c)
      blob[r * (H / 2) + c / 2] |= (uint8_t)(q[r * H + c] << (4 * (c & 1)));
    for (int64_t g = 0; g < G; ++g) {
      const uint16_t sc = sb[r * G + g], bi = sb[R * G + r * G + g];
      uint8_t* p = blob + dl.words_offset + (r * G + g) * 4;
      memcpy(p, &sc, 2);
      memcpy(p + 2, &bi, 2);
    }
  }
  return MOE_OK;
}

size_t moe_workspace_bytes(const moe_layer_desc* desc) {
  if (check_shape(desc) != MOE_OK) return 0;
  return make_ws_plan(*desc).total;
}

int moe_workspace_routing(const moe_layer_desc* desc, void* ws, int32_t** topk_idx,
                          float** topk_w, float** shared_gate) {
  MOE_TRY(check_shape(desc));
  if (ws == nullptr) return MOE_ERR_INVALID_ARG;
  const WsPlan P = make_ws_plan(*desc);
  uint8_t* b = reinterpret_cast<uint8_t*>(ws);
  if (topk_idx) *topk_idx = reinterpret_cast<int32_t*>(b + P.idx);
  if (topk_w) *topk_w = reinterpret_cast<float*>(b + P.w);
  if (shared_gate) *shared_gate = reinterpret_cast<float*>(b + P.gamma);
  return MOE_OK;
}

int moe_chain_status(const moe_layer_desc* desc, void* ws, uint32_t** status_word) {
  MOE_TRY(check_shape(desc));
  if (ws == nullptr || status_word == nullptr) return MOE_ERR_INVALID_ARG;
  const WsPlan P = make_ws_plan(*desc);
  *status_word = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(ws) + P.ctr) + 1;
  return MOE_OK;
}

}  // extern "C"
