// C ABI of the MoE layer library: the device entry points (argument checks,
// then the stream-ordered dispatch of the kernels).  The pure host entry
// points and the shared validation are in host.cpp.
#include "host.h"
#include "moe_internal.h"

using namespace moe;

namespace {

int device_ok() {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n < 1) return MOE_ERR_NO_DEVICE;
  return MOE_OK;
}

int to_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH; }

// router_w: fp32 rows, or with MOE_FLAG_DENSE_Q4 a dense blob (256-byte aligned)
uintptr_t router_align(const moe_layer_desc* d) {
  return (d->flags & MOE_FLAG_DENSE_Q4) ? 256 : 16;
}

int enqueue_router(const moe_layer_desc* d, const void* x, const float* router_w,
                   const float* router_bias, const float* wsg, int32_t* idx, float* w,
                   float* gamma, uint8_t* ws, hipStream_t s) {
  const WsPlan P = make_ws_plan(*d);
  RouterArgs a{};
  a.x = x;
  a.router_w = router_w;
  a.router_bias = (d->flags & MOE_FLAG_ROUTER_BIAS) ? router_bias : nullptr;
  a.shared_gate_w = wsg;
  if (d->flags & MOE_FLAG_DENSE_Q4) {
    // router_w is the layer's dense blob: its rows (with the shared gate as
    // row E) dequantised to fp32 for the GEMV / GEMM routers
    const DenseLayout DL = make_dense_layout(*d);
    float* dense = reinterpret_cast<float*>(ws + P.dense);
    MOE_TRY(to_status(launch_dense_dequant(reinterpret_cast<const uint8_t*>(router_w),
                                           (int)DL.rows, d->hidden, DL.words_off, dense, s)));
    a.router_w = dense;
    a.shared_gate_w = (gamma != nullptr && (d->flags & MOE_FLAG_SHARED))
                          ? dense + (int64_t)d->n_experts * d->hidden
                          : nullptr;
  }
  a.logits = reinterpret_cast<float*>(ws + P.logits);
  a.topk_idx = idx;
  a.topk_w = w;
  a.gamma = gamma;
  a.T = d->n_tokens;
  a.H = d->hidden;
  a.E = d->n_experts;
  a.k = d->top_k;
  a.act = d->act_dtype;
  if (mfma_path(*d)) {
    a.x16 = reinterpret_cast<uint16_t*>(ws + P.x16);
    a.xe = reinterpret_cast<int32_t*>(ws + P.xe);
    a.x16_bits = d->bits;
  }
  return to_status(launch_router_topk(a, s));
}

bool fast_decode(const moe_layer_desc* d) {
  const bool sh = (d->flags & MOE_FLAG_SHARED) != 0;
  return decode_fast_supported(d->n_tokens, d->act_dtype, d->hidden, d->top_k, d->n_experts,
                               d->bits, d->inter, sh ? d->shared_inter : 0, sh);
}

int enqueue_decode(const moe_layer_desc* d, const void* x_in, void* x_hat, bool do_norm,
                   const float* router_w, const float* router_bias, const void* slab,
                   const int32_t* slot_table, const void* shared_blob, void* out, void* x_res,
                   uint8_t* ws, hipStream_t s) {
  const WsPlan P = make_ws_plan(*d);
  DecodeArgs a{};
  a.has_shared = (d->flags & MOE_FLAG_SHARED) != 0;
  a.L = make_layout(d->bits, d->hidden, d->inter);
  a.Ls = make_layout(d->bits, d->hidden, a.has_shared ? d->shared_inter : d->inter);
  a.x_in = reinterpret_cast<const uint16_t*>(x_in);
  a.x_hat = reinterpret_cast<uint16_t*>(x_hat);
  a.router_w = router_w;
  a.router_bias = (d->flags & MOE_FLAG_ROUTER_BIAS) ? router_bias : nullptr;
  a.shared_gate_w =
      a.has_shared ? reinterpret_cast<const float*>(
                         reinterpret_cast<const uint8_t*>(shared_blob) + a.Ls.sg_off)
                   : nullptr;
  if (d->flags & MOE_FLAG_DENSE_Q4) {  // router rows and shared gate from the dense blob
    a.dense = reinterpret_cast<const uint8_t*>(router_w);
    a.dense_words = make_dense_layout(*d).words_off;
    a.router_w = nullptr;
    a.shared_gate_w = nullptr;
  }
  a.logits = reinterpret_cast<float*>(ws + P.logits);
  a.idx = reinterpret_cast<int32_t*>(ws + P.idx);
  a.w = reinterpret_cast<float*>(ws + P.w);
  a.gamma = reinterpret_cast<float*>(ws + P.gamma);
  a.slots = reinterpret_cast<int32_t*>(ws + P.slots);
  a.h = reinterpret_cast<float*>(ws + P.h);
  a.slab = reinterpret_cast<const uint8_t*>(slab);
  a.slot_table = slot_table;
  a.stride = d->expert_stride;
  a.shared_blob = reinterpret_cast<const uint8_t*>(shared_blob);
  a.out = reinterpret_cast<uint16_t*>(out);
  a.x_res = reinterpret_cast<uint16_t*>(x_res);
  a.H = d->hidden;
  a.E = d->n_experts;
  a.k = d->top_k;
  a.bits = d->bits;
  a.eps = d->rms_eps;
  a.do_norm = do_norm;
  return to_status(launch_decode(a, s));
}

int enqueue_experts(const moe_layer_desc* d, const void* x, const int32_t* idx, const float* w,
                    const float* gamma, const void* slab, const int32_t* slot_table,
                    const void* shared_blob, void* out, uint8_t* ws, hipStream_t s,
                    int epi = 0, void* x_res = nullptr, void* x_hat_next = nullptr,
                    bool x16_ready = false) {
  ExpertArgs a{};
  a.x16_ready = x16_ready;
  a.epi = epi;
  a.x_res = x_res;
  a.x_hat_next = x_hat_next;
  a.eps = d->rms_eps;
  a.x = x;
  a.topk_idx = idx;
  a.topk_w = w;
  a.gamma = gamma;
  a.slab = reinterpret_cast<const uint8_t*>(slab);
  a.slot_table = slot_table;
  a.stride = d->expert_stride;
  a.has_shared = (d->flags & MOE_FLAG_SHARED) != 0;
  a.shared_blob = reinterpret_cast<const uint8_t*>(shared_blob);
  a.out = out;
  a.ws = ws;
  a.plan = make_ws_plan(*d);
  a.L = make_layout(d->bits, d->hidden, d->inter);
  a.Ls = make_layout(d->bits, d->hidden, a.has_shared ? d->shared_inter : d->inter);
  a.T = d->n_tokens;
  a.H = d->hidden;
  a.E = d->n_experts;
  a.k = d->top_k;
  a.act = d->act_dtype;
  a.bits = d->bits;
  a.mfma = a.plan.bucketed &&
           prefill_supported(a.act, a.T, a.H, a.k, d->inter, a.Ls.inter, a.has_shared);
  return to_status(launch_experts(a, s));
}

// One layer of a bucketed chain (T > kDecodeMaxTokens): router and experts on
// x_hat, with the residual add and, unless this is the last layer, the next
// layer's RMSNorm fused into the combine.
int chain_layer_bucketed(const moe_layer_desc* desc, void* x, void* x_hat, const float* router_w,
                         const float* router_bias, const void* expert_slab,
                         const int32_t* slot_table, const void* shared_blob, void* out,
                         uint8_t* w8, bool last, hipStream_t stream) {
  const bool shared = (desc->flags & MOE_FLAG_SHARED) != 0;
  const WsPlan P = make_ws_plan(*desc);
  int32_t* idx = reinterpret_cast<int32_t*>(w8 + P.idx);
  float* w = reinterpret_cast<float*>(w8 + P.w);
  float* gamma = reinterpret_cast<float*>(w8 + P.gamma);
  const float* wsg = nullptr;
  if (shared) {
    const BlobLayout Ls = make_layout(desc->bits, desc->hidden, desc->shared_inter);
    wsg = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(shared_blob) + Ls.sg_off);
  }
  MOE_TRY(enqueue_router(desc, x_hat, router_w, router_bias, wsg, idx, w,
                         shared ? gamma : nullptr, w8, stream));
  return enqueue_experts(desc, x_hat, idx, w, shared ? gamma : nullptr, expert_slab, slot_table,
                         shared_blob, out, w8, stream, last ? 1 : 2, x, x_hat, true);
}

}  // namespace

extern "C" {

int moe_pack_experts_device(const moe_layer_desc* desc, int32_t inter, int32_t n,
                            const uint8_t* q_gate, const uint8_t* q_up, const uint8_t* q_down,
                            const uint16_t* sb_gate, const uint16_t* sb_up,
                            const uint16_t* sb_down, void* slab, const int64_t* dst_slots,
                            hipStream_t stream) {
  moe_blob_layout_t bl;
  MOE_TRY(moe_blob_layout(desc, inter, &bl));
  if (n < 0 || !dst_slots) return MOE_ERR_INVALID_ARG;
  if (n == 0) return MOE_OK;
  MOE_TRY(check_ptr(q_gate, 16));
  MOE_TRY(check_ptr(q_up, 16));
  MOE_TRY(check_ptr(q_down, 16));
  MOE_TRY(check_ptr(sb_gate, 4));
  MOE_TRY(check_ptr(sb_up, 4));
  MOE_TRY(check_ptr(sb_down, 4));
  MOE_TRY(check_ptr(slab, 256));
  if (desc->expert_stride < bl.blob_bytes || desc->expert_stride % 256) return MOE_ERR_MISALIGNED;
  for (int i = 0; i < n; ++i)
    if (dst_slots[i] < 0) return MOE_ERR_INVALID_ARG;
  MOE_TRY(device_ok());
  const BlobLayout L = make_layout(desc->bits, desc->hidden, inter);
  return to_status(launch_pack_device(L, n, q_gate, q_up, q_down, sb_gate, sb_up, sb_down,
                                      reinterpret_cast<uint8_t*>(slab), desc->expert_stride,
                                      dst_slots, stream));
}

int moe_router_topk(const moe_layer_desc* desc, const void* x, const float* router_w,
                    const float* router_bias, const float* shared_gate_w, int32_t* topk_idx,
                    float* topk_w, float* shared_gate, void* ws, hipStream_t stream) {
  MOE_TRY(check_shape(desc));
  if (desc->n_tokens == 0) return MOE_OK;
  MOE_TRY(check_ptr(x));
  const bool q4 = (desc->flags & MOE_FLAG_DENSE_Q4) != 0;
  MOE_TRY(check_ptr(router_w, router_align(desc)));
  MOE_TRY(check_ptr(topk_idx, 4));
  MOE_TRY(check_ptr(topk_w, 4));
  MOE_TRY(check_ptr(ws, 256));
  if (desc->flags & MOE_FLAG_ROUTER_BIAS) MOE_TRY(check_ptr(router_bias, 4));
  MOE_TRY(check_opt_ptr(shared_gate_w));
  MOE_TRY(check_opt_ptr(shared_gate, 4));
  if (q4) {
    // the gate vector is row E of the dense blob
    if (shared_gate_w != nullptr) return MOE_ERR_INVALID_ARG;
    if (shared_gate != nullptr && !(desc->flags & MOE_FLAG_SHARED)) return MOE_ERR_INVALID_ARG;
  } else if (shared_gate != nullptr && shared_gate_w == nullptr) {
    return MOE_ERR_INVALID_ARG;
  }
  MOE_TRY(device_ok());
  return enqueue_router(desc, x, router_w, router_bias, shared_gate_w, topk_idx, topk_w,
                        shared_gate, reinterpret_cast<uint8_t*>(ws), stream);
}

int moe_experts_forward(const moe_layer_desc* desc, const void* x, const int32_t* topk_idx,
                        const float* topk_w, const float* shared_gate, const void* expert_slab,
                        const int32_t* slot_table, const void* shared_blob, void* out, void* ws,
                        hipStream_t stream) {
  MOE_TRY(check_shape(desc));
  MOE_TRY(check_stride(desc));
  if (desc->n_tokens == 0) return MOE_OK;
  MOE_TRY(check_ptr(x));
  MOE_TRY(check_ptr(topk_idx, 4));
  MOE_TRY(check_ptr(topk_w, 4));
  MOE_TRY(check_ptr(expert_slab, 256));
  MOE_TRY(check_ptr(slot_table, 4));
  MOE_TRY(check_ptr(out));
  MOE_TRY(check_ptr(ws, 256));
  if (desc->flags & MOE_FLAG_SHARED) {
    MOE_TRY(check_ptr(shared_gate, 4));
    MOE_TRY(check_ptr(shared_blob, 256));
  }
  MOE_TRY(device_ok());
  return enqueue_experts(desc, x, topk_idx, topk_w, shared_gate, expert_slab, slot_table,
                         shared_blob, out, reinterpret_cast<uint8_t*>(ws), stream);
}

int moe_layer_forward(const moe_layer_desc* desc, const void* x, const float* router_w,
                      const float* router_bias, const void* expert_slab,
                      const int32_t* slot_table, const void* shared_blob, void* out, void* ws,
                      hipStream_t stream) {
  MOE_TRY(check_shape(desc));
  MOE_TRY(check_stride(desc));
  if (desc->n_tokens == 0) return MOE_OK;
  MOE_TRY(check_ptr(x));
  MOE_TRY(check_ptr(router_w, router_align(desc)));
  if (desc->flags & MOE_FLAG_ROUTER_BIAS) MOE_TRY(check_ptr(router_bias, 4));
  MOE_TRY(check_ptr(expert_slab, 256));
  MOE_TRY(check_ptr(slot_table, 4));
  MOE_TRY(check_ptr(out));
  MOE_TRY(check_ptr(ws, 256));
  const bool shared = (desc->flags & MOE_FLAG_SHARED) != 0;
  if (shared) MOE_TRY(check_ptr(shared_blob, 256));
  MOE_TRY(device_ok());
  uint8_t* w8 = reinterpret_cast<uint8_t*>(ws);
  if (fast_decode(desc))
    return enqueue_decode(desc, x, const_cast<void*>(x), false, router_w, router_bias,
                          expert_slab, slot_table, shared_blob, out, nullptr, w8, stream);
  const WsPlan P = make_ws_plan(*desc);
  int32_t* idx = reinterpret_cast<int32_t*>(w8 + P.idx);
  float* w = reinterpret_cast<float*>(w8 + P.w);
  float* gamma = reinterpret_cast<float*>(w8 + P.gamma);
  const float* wsg = nullptr;
  if (shared) {
    const BlobLayout Ls = make_layout(desc->bits, desc->hidden, desc->shared_inter);
    wsg = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(shared_blob) + Ls.sg_off);
  }
  MOE_TRY(enqueue_router(desc, x, router_w, router_bias, wsg, idx, w, shared ? gamma : nullptr, w8,
                         stream));
  return enqueue_experts(desc, x, idx, w, shared ? gamma : nullptr, expert_slab, slot_table,
                         shared_blob, out, w8, stream, 0, nullptr, nullptr, true);
}

int moe_residual_rmsnorm(const moe_layer_desc* desc, void* x_res, const void* out,
                         void* x_next, hipStream_t stream) {
  MOE_TRY(check_shape(desc));
  if (desc->n_tokens == 0) return MOE_OK;
  MOE_TRY(check_ptr(x_res));
  MOE_TRY(check_opt_ptr(out));
  MOE_TRY(check_ptr(x_next));
  if (!(desc->rms_eps >= 0.0f)) return MOE_ERR_INVALID_ARG;
  MOE_TRY(device_ok());
  return to_status(launch_rmsnorm(x_res, out, x_next, desc->n_tokens, desc->hidden,
                                  desc->act_dtype, desc->rms_eps, true, stream));
}

int moe_rmsnorm(const moe_layer_desc* desc, void* x, const void* out, void* x_hat,
                hipStream_t stream) {
  return moe_residual_rmsnorm(desc, x, out, x_hat, stream);
}

int moe_chain_forward(const moe_layer_desc* desc, int32_t n_layers, void* x,
                      const float* router_w, const float* router_bias, const void* expert_slab,
                      const int32_t* slot_tables, const void* shared_blobs,
                      int64_t shared_stride, void* x_hat, void* out, void* ws,
                      hipStream_t stream) {
  MOE_TRY(check_shape(desc));
  MOE_TRY(check_stride(desc));
  if (n_layers < 1) return MOE_ERR_INVALID_ARG;
  if (desc->n_tokens == 0) return MOE_OK;
  MOE_TRY(check_ptr(x));
  MOE_TRY(check_ptr(router_w, router_align(desc)));
  if (desc->flags & MOE_FLAG_ROUTER_BIAS) MOE_TRY(check_ptr(router_bias, 4));
  MOE_TRY(check_ptr(expert_slab, 256));
  MOE_TRY(check_ptr(slot_tables, 4));
  MOE_TRY(check_ptr(x_hat));
  MOE_TRY(check_ptr(out));
  MOE_TRY(check_ptr(ws, 256));
  const bool shared = (desc->flags & MOE_FLAG_SHARED) != 0;
  if (shared) {
    MOE_TRY(check_ptr(shared_blobs, 256));
    const BlobLayout Ls = make_layout(desc->bits, desc->hidden, desc->shared_inter);
    if (shared_stride < Ls.shared_bytes || shared_stride % 256) return MOE_ERR_MISALIGNED;
  }
  if (!(desc->rms_eps >= 0.0f)) return MOE_ERR_INVALID_ARG;
  MOE_TRY(device_ok());
  const bool q4 = (desc->flags & MOE_FLAG_DENSE_Q4) != 0;
  // layer l's router rows: fp32 [E][H], or its dense blob
  const int64_t router_step = q4 ? make_dense_layout(*desc).bytes
                                 : (int64_t)desc->n_experts * desc->hidden * (int64_t)sizeof(float);
  auto layer_router = [&](int l) {
    return reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(router_w) +
                                          (int64_t)l * router_step);
  };
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_NO_DEVICE;
  const int nwg = chain_grid(dev);
  if (chain_supported(nwg, desc->n_tokens, desc->act_dtype, desc->hidden, desc->n_experts,
                      desc->top_k, desc->bits, desc->inter, shared ? desc->shared_inter : 0,
                      shared)) {
    const WsPlan P = make_ws_plan(*desc);
    uint8_t* w8 = reinterpret_cast<uint8_t*>(ws);
    const BlobLayout Lr = make_layout(desc->bits, desc->hidden, desc->inter);
    const BlobLayout Ls = make_layout(desc->bits, desc->hidden, shared ? desc->shared_inter : desc->inter);
    ChainParams c{};
    c.x = reinterpret_cast<uint16_t*>(x);
    c.x_hat = reinterpret_cast<uint16_t*>(x_hat);
    c.out = reinterpret_cast<uint16_t*>(out);
    c.router_w = router_w;
    c.router_bias = (desc->flags & MOE_FLAG_ROUTER_BIAS) ? router_bias : nullptr;
    if (q4) {
      c.dense = reinterpret_cast<const uint8_t*>(router_w);
      c.dense_stride = router_step;
      c.dense_words = make_dense_layout(*desc).words_off;
    }
    c.slab = reinterpret_cast<const uint8_t*>(expert_slab);
    c.stride = desc->expert_stride;
    c.slot_tables = slot_tables;
    c.shared_blobs = reinterpret_cast<const uint8_t*>(shared_blobs);
    c.shared_stride = shared_stride;
    c.L = n_layers;
    c.H = desc->hidden;
    c.E = desc->n_experts;
    c.k = desc->top_k;
    c.I = desc->inter;
    c.Is = shared ? desc->shared_inter : 0;
    c.has_shared = shared ? 1 : 0;
    c.bits_ = desc->bits;
    c.eps = desc->rms_eps;
    c.gu_unit_r = Lr.gu_unit;
    c.gu_tile_r = Lr.gu_tile;
    c.d_off_r = Lr.d_off;
    c.d_unit_r = Lr.d_unit;
    c.d_tile_r = Lr.d_tile;
    c.gu_unit_s = Ls.gu_unit;
    c.gu_tile_s = Ls.gu_tile;
    c.d_off_s = Ls.d_off;
    c.d_unit_s = Ls.d_unit;
    c.d_tile_s = Ls.d_tile;
    c.sg_off = Ls.sg_off;
    c.xw = reinterpret_cast<uint64_t*>(w8 + P.xw);
    c.lw = reinterpret_cast<uint64_t*>(w8 + P.lw);
    c.hw = reinterpret_cast<uint64_t*>(w8 + P.hw);
    c.ctr = reinterpret_cast<uint32_t*>(w8 + P.ctr);
    c.err = c.ctr + 1;
    c.r_idx = reinterpret_cast<int32_t*>(w8 + P.idx);
    c.r_w = reinterpret_cast<float*>(w8 + P.w);
    c.r_gamma = reinterpret_cast<float*>(w8 + P.gamma);
    return to_status(launch_chain(c, nwg, stream));
  }
  if (fast_decode(desc)) {
    for (int l = 0; l < n_layers; ++l) {
      const float* rb = (desc->flags & MOE_FLAG_ROUTER_BIAS)
                            ? router_bias + (int64_t)l * desc->n_experts
                            : nullptr;
      const void* sb = shared ? reinterpret_cast<const uint8_t*>(shared_blobs) + l * shared_stride
                              : nullptr;
      MOE_TRY(enqueue_decode(desc, x, x_hat, true, layer_router(l), rb, expert_slab,
                             slot_tables + (int64_t)l * desc->n_experts, sb, out, x,
                             reinterpret_cast<uint8_t*>(ws), stream));
    }
    return MOE_OK;
  }
  if (make_ws_plan(*desc).bucketed) {
    MOE_TRY(to_status(launch_rmsnorm(x, nullptr, x_hat, desc->n_tokens, desc->hidden,
                                     desc->act_dtype, desc->rms_eps, true, stream)));
    for (int l = 0; l < n_layers; ++l) {
      const float* rb = (desc->flags & MOE_FLAG_ROUTER_BIAS)
                            ? router_bias + (int64_t)l * desc->n_experts
                            : nullptr;
      const void* sb = shared ? reinterpret_cast<const uint8_t*>(shared_blobs) + l * shared_stride
                              : nullptr;
      MOE_TRY(chain_layer_bucketed(desc, x, x_hat, layer_router(l), rb, expert_slab,
                                   slot_tables + (int64_t)l * desc->n_experts, sb, out,
                                   reinterpret_cast<uint8_t*>(ws), l == n_layers - 1, stream));
    }
    return MOE_OK;
  }
  for (int l = 0; l < n_layers; ++l) {
    MOE_TRY(to_status(launch_rmsnorm(x, l == 0 ? nullptr : out, x_hat, desc->n_tokens,
                                     desc->hidden, desc->act_dtype, desc->rms_eps, true, stream)));
    const float* rb = (desc->flags & MOE_FLAG_ROUTER_BIAS) ? router_bias + (int64_t)l * desc->n_experts
                                                          : nullptr;
    const void* sb = shared ? reinterpret_cast<const uint8_t*>(shared_blobs) + l * shared_stride
                            : nullptr;
    MOE_TRY(moe_layer_forward(desc, x_hat, layer_router(l), rb, expert_slab,
                              slot_tables + (int64_t)l * desc->n_experts, sb, out, ws, stream));
  }
  return to_status(launch_rmsnorm(x, out, x_hat, desc->n_tokens, desc->hidden, desc->act_dtype,
                                  desc->rms_eps, false, stream));
}

}  // extern "C"
