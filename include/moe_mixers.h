/*
 * moe_mixers.h -- C ABI of the two token mixers of the hybrid layers, for
 * AMD Instinct MI355X (gfx950): the Gated DeltaNet decode step and gated GQA
 * attention decode.
 *
 * The hybrid Qwen3-Next / Qwen3.5 models the Swiftlet pages describe put a
 * token mixer before every sparse MoE block: in 75% of the layers Gated
 * DeltaNet linear attention with a fixed-size recurrent state, in the rest
 * gated GQA attention (page "Paquets Swiftlet 80B Qwen dans Mac avec 4,3 Go de
 * mémoire ; iPhone 17 exécutera nativement 35B" on xix.ai, 5th and last
 * paragraphs; the untitled Swiftlet news item on news.bugfactory.tech, 3rd and
 * 5th paragraphs).  The pages give no formula; the readings below are the
 * published definitions, stated in each declaration.
 *
 * Conventions are those of moe.h: MOE_OK or a negative moe_status; full
 * validation before anything is enqueued; caller-owned device pointers
 * (16-byte aligned) unless marked host; asynchronous on the given stream; the
 * library never allocates, frees or synchronises.
 */
#ifndef MOE_MIXERS_H_
#define MOE_MIXERS_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Shape of a Gated DeltaNet decode step.  Host memory, read at call time.
 *   n_seqs     B: sequences, one new token each (>= 0)
 *   n_k_heads  Hk: query/key heads
 *   n_v_heads  Hv: value heads, a multiple of Hk; value head h reads
 *              query/key head h / (Hv / Hk)
 *   d_k        key/query head size: 64, 128 or 256
 *   d_v        value head size: a multiple of 16
 *   eps        epsilon of the L2 normalisation of q and k
 *   scale      query scale; 0 means 1 / sqrt(d_k)
 */
typedef struct moe_gdn_desc {
  int32_t n_seqs;
  int32_t n_k_heads;
  int32_t n_v_heads;
  int32_t d_k;
  int32_t d_v;
  int32_t reserved0;
  float eps;
  float scale;
} moe_gdn_desc;

/*
 * Gated DeltaNet decode step: per sequence b and value head h, with
 * kh = h / (Hv / Hk), k^ = k[b][kh] / sqrt(|k|^2 + eps),
 * q^ = scale q[b][kh] / sqrt(|q|^2 + eps), alpha = exp(g[b][h]):
 *   u        = v[b][h] - alpha S k^
 *   S       <- alpha S + beta[b][h] u k^T
 *   out[b][h] = S q^              (after the update)
 * with S = state[b][h], a d_v x d_k row-major fp32 matrix, updated in place.
 *   q, k    [B][Hk][d_k] bf16
 *   v       [B][Hv][d_v] bf16
 *   g, beta [B][Hv] fp32 (log decay, write strength)
 *   state   [B][Hv][d_v][d_k] fp32, in/out
 *   out     [B][Hv][d_v] bf16 (round to nearest even)
 * Defined by: 75% of the layers use Gated DeltaNet linear attention with a
 * fixed-size recurrent state (xix.ai page, 5th paragraph; news.bugfactory.tech
 * item, 3rd paragraph).  The update is the gated delta rule as published
 * (Yang, Kautz, Hatamizadeh, "Gated Delta Networks", 2024); the pages print
 * no formula.  Errors: INVALID_ARG (null, Hv not a multiple of Hk, eps < 0),
 * UNSUPPORTED (d_k, d_v), MISALIGNED, NO_DEVICE, LAUNCH.
 */
int moe_gdn_decode(const moe_gdn_desc* desc, const void* q, const void* k, const void* v,
                   const float* g, const float* beta, float* state, void* out,
                   hipStream_t stream);

/*
 * Shape of a gated GQA attention decode call.  Host memory.
 *   n_seqs      B: sequences, one query token each (>= 0)
 *   n_q_heads   Hq: query heads, a multiple of n_kv_heads, Hq / Hkv <= 16
 *   n_kv_heads  Hkv: key/value heads; query head h reads kv head h / (Hq / Hkv)
 *   head_dim    D: 64, 128 or 256
 *   max_len     KV cache capacity per sequence (positions), >= 1
 *   scale       score scale; 0 means 1 / sqrt(D)
 */
typedef struct moe_attn_desc {
  int32_t n_seqs;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t max_len;
  int32_t reserved0;
  float scale;
  float reserved1;
} moe_attn_desc;

/*
 * Workspace bytes of moe_attn_decode for `desc`, or 0 when invalid.  Pure
 * host function.  Not a passage of the pages: the per-chunk partial sums of
 * this implementation (per sequence, query head and 128-position chunk: the
 * running max and sum, and D floats).
 */
size_t moe_attn_workspace_bytes(const moe_attn_desc* desc);

/*
 * Gated GQA attention decode: per sequence b and query head h, with
 * c = h / (Hq / Hkv) and n = lengths[b] valid cache positions,
 *   s_j        = scale * q[b][h] . K[b][c][j]      (j < n)
 *   p          = softmax(s)
 *   out[b][h]  = sigmoid(gate[b][h]) * sum_j p_j V[b][c][j]   (elementwise gate)
 *   q, gate        [B][Hq][D] bf16
 *   k_cache, v_cache [B][Hkv][max_len][D] bf16 (rows j >= lengths[b] unread)
 *   lengths        [B] int32, device, each in [1, max_len]; the device clamps
 *                  a length to [0, max_len], and a length of 0 gives zeros
 *   out            [B][Hq][D] bf16 (round to nearest even)
 *   ws             workspace of moe_attn_workspace_bytes(desc) bytes
 * Runs as chunks of 128 positions, whose partial softmax sums a second kernel
 * merges in a fixed order (deterministic).
 * Defined by: the remaining layers use gated GQA attention (xix.ai page, last
 * paragraph; news.bugfactory.tech item, 5th paragraph): grouped-query
 * attention with a sigmoid output gate; the pages print no formula.
 * Errors: INVALID_ARG (null, Hq not a multiple of Hkv, max_len < 1),
 * UNSUPPORTED (head_dim, group > 16), MISALIGNED, NO_DEVICE, LAUNCH.
 */
int moe_attn_decode(const moe_attn_desc* desc, const void* q, const void* gate,
                    const void* k_cache, const void* v_cache, const int32_t* lengths,
                    void* out, void* ws, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MIXERS_H_ */
