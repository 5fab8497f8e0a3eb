/*
 * moe.h -- C ABI of the int4/int8 group-quantized sparse MoE layer for
 * AMD Instinct MI355X (gfx950).
 *
 * One call computes one sparse Mixture-of-Experts layer of the kind the
 * Swiftlet pages describe for the Qwen3-Next / Qwen3.5-3.6 hybrid models:
 * every token is routed to the top-k of E experts (10 of 512 for the
 * 80B-A3B family, 8 of 256 for the 35B-A3B family) by a resident router, an
 * always-active shared expert is added, and the routed experts' weights are
 * MLX-style int4/int8 group-quantized and held as fixed-stride blobs, one
 * contiguous blob per expert, addressed with 64-bit offsets
 * (page "Paquets Swiftlet 80B Qwen ..." on xix.ai, 4th and last paragraphs;
 * the untitled Swiftlet news item on news.bugfactory.tech, 3rd paragraph;
 * page "Swiftlet: 在 Mac 和 iPhone 上執行 80B 與 35B Qwen 模型"
 * on agentlenshq.com, section "記憶體管理與權重串流").  On one MI355X the whole
 * expert pack fits in HBM, so a per-layer slot table maps expert -> slot of a
 * device-resident slab instead of a host-side pool.
 *
 * What one layer computes, per token t with input x_hat[t] (stored values of
 * the activation dtype):
 *   l      = Wr x_hat (+ router bias)                       (router, fp32 Wr)
 *   S, w   = top-k of softmax(l), renormalised over the k selected
 *            (ordered by logit descending, ties to the lower expert index)
 *   gamma  = sigmoid(w_sg . x_hat)                           (shared gate)
 *   y_e    = Wd_e (silu(Wg_e x_hat) * (Wu_e x_hat))          (SwiGLU expert)
 *   out    = sum_j w_j y_{S_j} + gamma y_shared
 * with W[r,c] = scale[r, c/64] * q[r,c] + bias[r, c/64], q unsigned
 * (0..15 int4, 0..255 int8), scale and bias bf16, groups of 64 consecutive
 * input columns.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Return value: MOE_OK (0) or a negative moe_status.  Arguments are fully
 *   validated before anything is enqueued; on error nothing is enqueued.
 * - Memory: every tensor argument is a caller-owned *device* pointer unless
 *   the parameter documentation says "host".  The library never allocates,
 *   frees or synchronises; all work is enqueued on the given HIP stream and
 *   the pointers must stay valid until that work completes.  Device faults
 *   surface at the caller's next synchronisation.
 * - Layouts are row-major and dense.  Activations are [n_tokens x hidden] of
 *   act_dtype (fp32 or bf16).  Device pointers must be 16-byte aligned; the
 *   expert slab and every blob must be 256-byte aligned.
 * - Slab addressing is 64-bit: blob of expert e = slab + slot_table[e] *
 *   expert_stride.  slot_table entries are not range-checked on the device.
 * - Global state: a per-device cache of the compute-unit count, filled on
 *   first use with atomic stores, and the per-device scratch of
 *   moe_layer_forward_noalloc (with its address cache, filled under a lock).
 *   Calls are otherwise reentrant; concurrent calls must use distinct
 *   workspaces.
 * - Citations: each declaration names the passage of the pages that defines
 *   what it computes, by page title and paragraph or section.  Where the
 *   pages are silent (the affine group format, SwiGLU, the sigmoid gate,
 *   softmax -> top-k -> renormalise, the pre-RMSNorm chain) the declaration
 *   says so: these are the workload definition this library implements.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null pointer, size out of range, k > E ...   */
  MOE_ERR_UNSUPPORTED = -2, /* bits, group, dtype or shape not implemented  */
  MOE_ERR_MISALIGNED = -3,  /* pointer or stride alignment violated         */
  MOE_ERR_NO_DEVICE = -4,   /* no HIP device visible                        */
  MOE_ERR_LAUNCH = -5,      /* a kernel launch returned an error            */
  MOE_ERR_TOO_LARGE = -6    /* the call needs more than a fixed-size buffer */
};

/* activation dtypes */
enum moe_act_dtype { MOE_ACT_F32 = 0, MOE_ACT_BF16 = 1 };

/* desc.flags */
enum moe_flags {
  MOE_FLAG_ROUTER_BIAS = 1u, /* an additive fp32 router bias [E] is given */
  MOE_FLAG_SHARED = 2u,      /* the layer has a sigmoid-gated shared expert */
  MOE_FLAG_DENSE_Q4 = 4u     /* router rows and shared gate in 4 bits: `router_w`
                                points to the layer's dense blob (moe_dense_layout) */
};

/* Limits of this implementation (validated). */
#define MOE_MAX_TOP_K 16
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_HIDDEN 8192
#define MOE_MAX_INTER 4096
/* Device scratch of moe_layer_forward_noalloc, per GPU (32 MiB). */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * Shape and format of one MoE layer.  Host memory, read at call time only.
 *   n_tokens      tokens in the call (1 for batch-1 decode)
 *   hidden        H: multiple of 128 (int4) / 64 (int8), <= MOE_MAX_HIDDEN
 *   n_experts     E: 1 .. MOE_MAX_EXPERTS routed experts
 *   top_k         k: 1 .. min(E, MOE_MAX_TOP_K)
 *   inter         I: routed-expert intermediate size, multiple of 128 (int4)
 *                 / 64 (int8), 16 <= I <= MOE_MAX_INTER
 *   shared_inter  Is: shared-expert intermediate size, same rule (ignored
 *                 without MOE_FLAG_SHARED)
 *   group         quantisation group along the input axis; must be 64
 *   bits          4 or 8
 *   act_dtype     enum moe_act_dtype
 *   expert_stride bytes between consecutive slab slots; >= the blob size of
 *                 moe_blob_layout(), multiple of 256
 *   flags         enum moe_flags
 *   rms_eps       epsilon of the RMSNorm of moe_residual_rmsnorm / chains
 */
typedef struct moe_layer_desc {
  int32_t n_tokens;
  int32_t hidden;
  int32_t n_experts;
  int32_t top_k;
  int32_t inter;
  int32_t shared_inter;
  int32_t group;
  int32_t bits;
  int32_t act_dtype;
  int32_t reserved0;
  int64_t expert_stride;
  uint32_t flags;
  float rms_eps;
} moe_layer_desc;

/*
 * Physical layout of one expert blob (the fixed-stride unit the pages
 * describe; the format itself is this library's own).
 *
 * Both sections are made of row tiles of `row_tile` (16) consecutive output
 * rows.  A tile is split along the input axis into k-blocks of
 * `kblock_cols` columns (128 for int4, 64 for int8: 64 bytes of codes per
 * row).  Per (tile, k-block) the codes are stored row-major, 64 bytes per row
 * (16 x 64 B = 1 KiB), followed by the bf16 (scale, bias) pairs of the
 * block's groups, row-major [row][group][scale, bias].
 *   gate/up section: unit = gate codes 1 KiB | up codes 1 KiB |
 *                    gate (scale,bias) | up (scale,bias);
 *                    tiles over I rows, k-blocks over H columns.
 *   down section:    unit = down codes 1 KiB | down (scale,bias);
 *                    tiles over H rows, k-blocks over I columns.
 * Within a row's 64 bytes, byte i holds columns 2i (low nibble) and 2i+1
 * (high nibble) for int4, column i for int8 (columns relative to the
 * k-block).  Units are stored k-block-fastest, then tile.
 * The shared-expert blob uses the same layout with I = shared_inter and is
 * followed, at shared_gate_offset, by the shared gate weight w_sg: fp32[H].
 */
typedef struct moe_blob_layout_t {
  int64_t gu_offset;         /* start of the gate/up section            */
  int64_t gu_unit_bytes;     /* bytes of one (tile, k-block) unit       */
  int64_t gu_tile_bytes;     /* bytes of one row tile (all k-blocks)    */
  int64_t down_offset;       /* start of the down section               */
  int64_t down_unit_bytes;
  int64_t down_tile_bytes;
  int64_t blob_bytes;        /* bytes of the blob, multiple of 256      */
  int64_t shared_gate_offset;/* shared blob: byte offset of w_sg fp32[H]*/
  int64_t shared_bytes;      /* shared blob incl. w_sg, multiple of 256 */
  int32_t row_tile;          /* 16                                      */
  int32_t kblock_cols;       /* 128 (int4) / 64 (int8)                  */
  int32_t groups_per_kblock; /* 2 (int4) / 1 (int8)                     */
  int32_t reserved0;
} moe_blob_layout_t;

/* Library version string, e.g. "moe-gfx950 0.1.0".  Pure host function. */
const char* moe_version(void);

/* Human-readable name of a status code (never NULL).  Pure host function. */
const char* moe_status_string(int status);

/*
 * Byte layout of one expert blob with intermediate size `inter` (pass
 * desc->inter for routed experts, desc->shared_inter for the shared blob).
 * `out` is host memory.  Pure host function; needs no device.
 * Defined by: routed experts repacked into fixed-stride blocks, one read per
 * expert (xix.ai page "Paquets Swiftlet 80B Qwen dans Mac avec 4,3 Go de
 * mémoire ; iPhone 17 exécutera nativement 35B", 4th paragraph;
 * agentlenshq.com page "Swiftlet: 在 Mac 和 iPhone 上執行 80B 與 35B Qwen 模型",
 * section "記憶體管理與權重串流", item "固定步長 Blob"), with 64-bit offsets
 * (xix.ai page, last paragraph).  The byte format itself is this library's.
 * Errors: INVALID_ARG (null), UNSUPPORTED (bits, group, hidden or inter).
 */
int moe_blob_layout(const moe_layer_desc* desc, int32_t inter, moe_blob_layout_t* out);

/*
 * Host packer (the analogue of the pages' repack tool): writes one blob from
 * logical arrays, all in host memory.
 *   q_gate, q_up  [inter x hidden] codes, one code per byte (0..2^bits-1)
 *   q_down        [hidden x inter] codes, one code per byte
 *   sb_gate, sb_up  scale then bias planes: 2 x [inter x hidden/64] bf16 bits
 *                   (uint16), i.e. scale[inter][G] followed by bias[inter][G]
 *   sb_down         2 x [hidden x inter/64] bf16 bits, scale plane then bias
 *   shared_gate_w   fp32[hidden] or NULL; when given, written at
 *                   shared_gate_offset (shared blob)
 *   blob_out      host buffer of at least blob_bytes (shared_bytes when
 *                 shared_gate_w is given); padding bytes are zeroed
 * Codes out of range return MOE_ERR_INVALID_ARG.
 * Defined by: the repack tool that builds the fixed-stride containers from
 * MLX checkpoints (xix.ai page, 7th paragraph; agentlenshq.com page, section
 * "實作與工具"); MLX-style int4/int8 group quantisation (xix.ai page, last
 * paragraph).  Pure host function; needs no device.
 */
int moe_pack_expert(const moe_layer_desc* desc, int32_t inter, const uint8_t* q_gate,
                    const uint8_t* q_up, const uint8_t* q_down, const uint16_t* sb_gate,
                    const uint16_t* sb_up, const uint16_t* sb_down, const float* shared_gate_w,
                    void* blob_out);

/*
 * Device packer: packs n experts from device-resident logical arrays into the
 * slab.  Arrays are as for moe_pack_expert, stacked over the n experts
 * (expert i's q_gate at q_gate + i*inter*hidden, its sb_gate at
 * sb_gate + i*2*inter*(hidden/64), ...).  Expert i is written to
 * slab + dst_slots[i] * desc->expert_stride; dst_slots is a *host* int64
 * array of n slots.  Codes must already be in range (not checked).  The
 * shared gate vector of a shared blob is not written by this packer; copy it
 * to shared_gate_offset separately.
 * Defined by: as moe_pack_expert.  Errors: INVALID_ARG (null, n < 0, a
 * negative slot), UNSUPPORTED (shape), MISALIGNED (array alignment, stride),
 * NO_DEVICE, LAUNCH.
 */
int moe_pack_experts_device(const moe_layer_desc* desc, int32_t inter, int32_t n,
                            const uint8_t* q_gate, const uint8_t* q_up, const uint8_t* q_down,
                            const uint16_t* sb_gate, const uint16_t* sb_up,
                            const uint16_t* sb_down, void* slab, const int64_t* dst_slots,
                            hipStream_t stream);

/* Dense blob layout (moe_dense_layout): rows, byte offset of the words, size. */
typedef struct moe_dense_layout_t {
  int64_t rows;
  int64_t words_offset;
  int64_t bytes;
} moe_dense_layout_t;

/*
 * The layer's dense weights in 4 bits (MOE_FLAG_DENSE_Q4): the E router rows
 * and, with MOE_FLAG_SHARED, the shared expert's gate vector as row E, each
 * of `hidden` values quantised like the experts' (w = scale * q + bias per
 * group of 64 consecutive values, unsigned 4-bit codes, bf16 scale and
 * bias).  One dense blob per layer, `rows` = E (+1 with MOE_FLAG_SHARED):
 *   codes   rows x hidden/2 bytes from offset 0: value 2j of a row in the
 *           low nibble of byte j, value 2j+1 in the high nibble
 *   words   rows x hidden/64 uint32 from words_offset: scale bits in the
 *           low half, bias bits in the high half
 *   bytes   the blob size (a multiple of 256); consecutive layers of a
 *           chain sit `bytes` apart
 * With the flag, the `router_w` argument of every compute entry point points
 * to this blob (device memory, 256-byte aligned; for moe_chain_forward the
 * first of n_layers blobs), the shared gate comes from its row E (the shared
 * blob's fp32 gate vector is not read), and moe_router_topk takes
 * shared_gate_w = NULL.
 * Defined by: the dense weights, routers and shared experts among them, kept
 * resident in 4 bits (xix.ai page "Paquets Swiftlet 80B Qwen ...", 4th
 * paragraph; agentlenshq.com page, section "記憶體管理與權重串流", item
 * "常駐密集權重"; news.bugfactory.tech Swiftlet item, 3rd paragraph).  The
 * byte format is this library's.
 * Errors: INVALID_ARG (null), UNSUPPORTED (hidden, group).  Pure host
 * function; needs no device.
 */
int moe_dense_layout(const moe_layer_desc* desc, moe_dense_layout_t* out);

/*
 * Host packer of a dense blob from logical arrays in host memory:
 *   q         [rows x hidden] codes, one code per byte (0..15)
 *   sb        scale then bias planes: 2 x [rows x hidden/64] bf16 bits
 *   blob_out  host buffer of at least `bytes`; padding bytes are zeroed
 * Codes out of range return MOE_ERR_INVALID_ARG.
 * Defined by: as moe_dense_layout.  Pure host function; needs no device.
 */
int moe_pack_dense(const moe_layer_desc* desc, const uint8_t* q, const uint16_t* sb,
                   void* blob_out);

/*
 * Workspace bytes needed by the compute entry points for `desc` (host), or 0
 * for an invalid descriptor.  The caller allocates the workspace (device
 * memory); the library never allocates.  Not a passage of the pages: the
 * scratch of this implementation (logits, routing, h, buckets, partial rows,
 * exchange words).
 */
size_t moe_workspace_bytes(const moe_layer_desc* desc);

/*
 * Router, softmax, top-k and renormalisation, plus the shared gate.
 *   x             [T x H] act_dtype, the layer input x_hat
 *   router_w      [E x H] fp32, or the dense blob with MOE_FLAG_DENSE_Q4
 *   router_bias   [E] fp32 or NULL (required iff MOE_FLAG_ROUTER_BIAS)
 *   shared_gate_w [H] fp32 or NULL (NULL with MOE_FLAG_DENSE_Q4)
 *   topk_idx      out [T x k] int32, by logit descending (ties: lower index)
 *   topk_w        out [T x k] fp32, sums to 1 per token
 *   shared_gate   out [T] fp32 sigmoid(w_sg . x), or NULL (needs shared_gate_w,
 *                 or with MOE_FLAG_DENSE_Q4 MOE_FLAG_SHARED)
 *   ws            workspace of moe_workspace_bytes(desc) bytes
 * Defined by: every layer routes each token to 10 of 512 experts (80B) or 8
 * of 256 (35B), with the routers resident (xix.ai page, 4th paragraph;
 * news.bugfactory.tech Swiftlet item, 3rd paragraph); the shared expert is
 * resident beside them (same passages).  softmax -> top-k -> renormalise and
 * the sigmoid gate are the workload definition (the pages are silent).
 * Errors: INVALID_ARG (null, shared_gate without its gate vector,
 * shared_gate_w given with MOE_FLAG_DENSE_Q4, router_bias missing with
 * MOE_FLAG_ROUTER_BIAS), UNSUPPORTED, MISALIGNED, NO_DEVICE, LAUNCH.
 */
int moe_router_topk(const moe_layer_desc* desc, const void* x, const float* router_w,
                    const float* router_bias, const float* shared_gate_w, int32_t* topk_idx,
                    float* topk_w, float* shared_gate, void* ws, hipStream_t stream);

/*
 * The experts with a given routing ("forward with given routing"): steps
 * after the router.
 *   x            [T x H] act_dtype
 *   topk_idx     [T x k] int32 expert ids in [0, E)
 *   topk_w       [T x k] fp32 routing weights
 *   shared_gate  [T] fp32 gamma, required iff MOE_FLAG_SHARED
 *   expert_slab  base of the slab (256-byte aligned)
 *   slot_table   [E] int32 slab slot of each expert
 *   shared_blob  shared-expert blob (layout above) iff MOE_FLAG_SHARED
 *   out          out [T x H] act_dtype
 * Defined by: high-sparsity MoE with a shared expert and MLX-style int4/int8
 * group quantisation computed with byte-addressable kernels and 64-bit
 * offsets (xix.ai page, last paragraph; news.bugfactory.tech item, last
 * paragraph); one fixed-stride blob per expert (xix.ai page, 4th paragraph).
 * SwiGLU and w = scale * q + bias per group of 64 are the workload
 * definition.  Errors: INVALID_ARG, UNSUPPORTED, MISALIGNED (pointers,
 * expert_stride), NO_DEVICE, LAUNCH.
 */
int moe_experts_forward(const moe_layer_desc* desc, const void* x, const int32_t* topk_idx,
                        const float* topk_w, const float* shared_gate, const void* expert_slab,
                        const int32_t* slot_table, const void* shared_blob, void* out, void* ws,
                        hipStream_t stream);

/*
 * One whole MoE layer: router + top-k + shared gate + experts + combine.
 * The shared gate weight is read from the shared blob (with
 * MOE_FLAG_DENSE_Q4: row E of the dense blob that `router_w` points to).
 * The routing of the call stays in the workspace and can be read with
 * moe_workspace_routing().
 * Arguments as for moe_router_topk and moe_experts_forward.
 * Defined by: the sparse MoE block of each layer of the hybrid Qwen3-Next /
 * Qwen3.5-3.6 models (xix.ai page, 4th and last paragraphs;
 * news.bugfactory.tech item, 3rd paragraph).  Errors: as
 * moe_experts_forward.
 */
int moe_layer_forward(const moe_layer_desc* desc, const void* x, const float* router_w,
                      const float* router_bias, const void* expert_slab,
                      const int32_t* slot_table, const void* shared_blob, void* out, void* ws,
                      hipStream_t stream);

/*
 * Device pointers, inside `ws`, of the routing written by the last
 * moe_layer_forward / moe_chain_forward layer that used `ws`:
 * topk_idx [T x k] int32, topk_w [T x k] fp32, shared_gate [T] fp32.
 * Any output pointer may be NULL.  Pure host arithmetic on `ws`.
 * Not a passage of the pages: access to this implementation's workspace.
 */
int moe_workspace_routing(const moe_layer_desc* desc, void* ws, int32_t** topk_idx,
                          float** topk_w, float** shared_gate);

/*
 * Chain step around a layer: optional residual add, then RMSNorm.
 *   x_res    in/out [T x H] act_dtype residual stream.  If `out` is non-NULL,
 *            x_res <- act(x_res + out) first.
 *   out      [T x H] act_dtype layer output, or NULL
 *   x_next   out [T x H] act_dtype, the next layer's input:
 *            act(x_res / sqrt(mean(x_res^2) + rms_eps)) (unit weight)
 * Not a passage of the pages: the residual add and pre-RMSNorm around each
 * MoE layer are the workload definition of a chain of layers.
 * Errors: INVALID_ARG (null, negative or NaN rms_eps), UNSUPPORTED,
 * MISALIGNED, NO_DEVICE, LAUNCH.
 */
int moe_residual_rmsnorm(const moe_layer_desc* desc, void* x_res, const void* out,
                         void* x_next, hipStream_t stream);

/* The same call as moe_residual_rmsnorm, under its earlier name. */
int moe_rmsnorm(const moe_layer_desc* desc, void* x, const void* out, void* x_hat,
                hipStream_t stream);

/*
 * A chain of n_layers distinct layers over one batch:
 *   for l: x_hat = rmsnorm(x); out = layer_l(x_hat); x <- act(x + out).
 *   x             in/out [T x H] act_dtype
 *   router_w      layer l at router_w + l * E * H (fp32); with
 *                 MOE_FLAG_DENSE_Q4 layer l's dense blob at l * bytes
 *                 (moe_dense_layout) from router_w
 *   router_bias   layer l at router_bias + l * E, or NULL
 *   expert_slab   one slab for all layers
 *   slot_tables   layer l at slot_tables + l * E
 *   shared_blobs  layer l at shared_blobs + l * shared_stride bytes
 *   shared_stride bytes between shared blobs, multiple of 256
 *   x_hat, out    [T x H] act_dtype scratch tensors (hold the last layer's).
 *                 For T > 8 the residual add and the next layer's RMSNorm run
 *                 inside each layer's combine; its sum of squares is taken in
 *                 another order than moe_rmsnorm's, so x_hat may differ from
 *                 moe_rmsnorm's by one rounding of the act dtype.
 *   ws            workspace of moe_workspace_bytes(desc) bytes.  For T = 1 the
 *                 chain may run as one persistent kernel (one workgroup per
 *                 compute unit, all resident at once) that exchanges data
 *                 between workgroups through epoch-tagged words in ws: ws must
 *                 be zero-filled before its first chain call and then reused
 *                 only by chain calls of the same desc (it keeps the last
 *                 epoch; 2^32 layers before the counter wraps).  A bounded wait
 *                 that expires (for instance when other work holds compute
 *                 units at the same time, so that not every workgroup is
 *                 resident) sets bit 0 of the chain status word
 *                 (moe_chain_status); results of that call are then invalid.
 * Defined by: each token's decode step runs every layer's forward pass in
 * turn, the MoE block after the mixer (xix.ai page, 4th and 5th paragraphs;
 * agentlenshq.com page, section "效能與模型支援": decode tokens/s of the
 * whole model).  The residual add and pre-RMSNorm are the workload
 * definition.  Errors: INVALID_ARG (n_layers < 1, null, rms_eps), MISALIGNED
 * (pointers, strides), UNSUPPORTED, NO_DEVICE, LAUNCH.
 */
int moe_chain_forward(const moe_layer_desc* desc, int32_t n_layers, void* x,
                      const float* router_w, const float* router_bias, const void* expert_slab,
                      const int32_t* slot_tables, const void* shared_blobs,
                      int64_t shared_stride, void* x_hat, void* out, void* ws,
                      hipStream_t stream);

/*
 * moe_layer_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same kernels and results as
 * moe_layer_forward, with the workspace taken from a device array of the
 * library, MOE_NOALLOC_SCRATCH_BYTES per GPU, which each GPU the library runs
 * on holds until the process ends.  Its device address is looked up on the
 * first call on each device.  It allocates and frees nothing.
 * Limit: calls whose moe_workspace_bytes(desc) exceeds
 * MOE_NOALLOC_SCRATCH_BYTES return MOE_ERR_TOO_LARGE before anything is
 * enqueued (at hidden 2048, 512 experts, top-10, inter 512: up to 251
 * tokens).  Every call on a GPU shares that GPU's scratch, which keeps the
 * last call's contents: calls that overlap on one GPU (other streams, other
 * threads) race and must be serialised by the caller.  The routing stays in
 * the scratch and is not exposed.  Arguments and other errors as for
 * moe_layer_forward.
 */
int moe_layer_forward_noalloc(const moe_layer_desc* desc, const void* x, const float* router_w,
                              const float* router_bias, const void* expert_slab,
                              const int32_t* slot_table, const void* shared_blob, void* out,
                              hipStream_t stream);

/*
 * Device address, inside `ws`, of the persistent chain's status word
 * (uint32).  Bit 0 is set when a bounded wait between workgroups of a
 * moe_chain_forward call expired; the results of that call are then invalid.
 * The word is zero in a zero-filled workspace, is never cleared by the
 * library (it is sticky over calls), and is written only by the persistent
 * batch-1 chain; the caller reads it after synchronising the stream and may
 * reset it to 0 when no call using `ws` is in flight.  Pure host arithmetic
 * on `ws`.  Not a passage of the pages: error reporting of this
 * implementation.  Errors: INVALID_ARG (null), UNSUPPORTED (descriptor).
 */
int moe_chain_status(const moe_layer_desc* desc, void* ws, uint32_t** status_word);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
