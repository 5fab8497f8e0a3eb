/*
 * moe_pool.h -- bounded expert slot pool over a host-memory tier, for
 * AMD Instinct MI355X (gfx950).
 *
 * The Swiftlet pages keep only the dense weights resident and stream routed
 * experts on demand into a bounded pool of slots, each expert one read of a
 * fixed-stride blob, evicting by LFU combined with recency; they quote hit
 * rates of 43-70% (page "Paquets Swiftlet 80B Qwen dans Mac avec 4,3 Go de
 * mémoire ; iPhone 17 exécutera nativement 35B" on xix.ai, 4th and 8th
 * paragraphs; page "Swiftlet: 在 Mac 和 iPhone 上執行 80B 與 35B Qwen 模型" on
 * agentlenshq.com, section "記憶體管理與權重串流").  Here the pool is a slab of
 * slots in HBM and the tier below it is the whole expert pack in pinned host
 * memory: a miss is one asynchronous host-to-device copy of the expert's
 * blob, and the layer's device slot table (the one moe_layer_forward /
 * moe_experts_forward index) is updated on the same stream.  One MI355X
 * holds every expert of both model families in HBM, so the pool is for packs
 * larger than HBM, or several models sharing one GPU.
 *
 * Replacement policy (the pages give no rule beyond "LFU with recency"):
 *   - a key is (layer, expert); one moe_pool_require call is one tick;
 *   - a hit adds 1 to the key's use count and sets its last use to the tick;
 *   - a miss takes the lowest free slot, else the slot of the resident key
 *     with the smallest (use count, last use, slot index) among the keys the
 *     current call has not used; the new key starts at count 1;
 *   - experts are processed in the order given; a repeat is a hit.
 *
 * The pool is a host object created by moe_pool_create (host allocation of
 * its bookkeeping only); every device buffer and the host pack belong to the
 * caller.  A pool is not thread-safe: one caller at a time.
 */
#ifndef MOE_POOL_H_
#define MOE_POOL_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moe_pool moe_pool;

/* Counters since creation (host memory). */
typedef struct moe_pool_stats_t {
  int64_t requests;      /* moe_pool_require calls                     */
  int64_t lookups;       /* experts named, repeats included            */
  int64_t hits;
  int64_t misses;        /* = loads = host-to-device blob copies       */
  int64_t evictions;     /* misses that replaced a resident expert     */
  int64_t bytes_copied;  /* host-to-device bytes enqueued              */
} moe_pool_stats_t;

/* moe_pool_create flags */
enum moe_pool_flags {
  /* bookkeeping only: no device pointer is used and moe_pool_require
   * enqueues nothing (tests of the replacement policy on a host) */
  MOE_POOL_HOST_ONLY = 1u
};

/*
 * Creates a pool of n_slots expert slots.
 *   desc            layer shape (n_experts, blob layout, expert_stride: the
 *                   stride of the device slab's slots)
 *   n_layers        layers whose experts the pack holds
 *   n_slots         slots of the device slab, >= 1
 *   host_pack       host memory, pinned (hipHostMalloc) so that copies are
 *                   asynchronous: the blob of (layer l, expert e) at
 *                   host_pack + (l * E + e) * host_stride
 *   host_stride     bytes, >= the blob size
 *   device_slab     n_slots * desc->expert_stride bytes of device memory
 *   slot_tables     device int32 [n_layers][E]: entry (l, e) is written with
 *                   the slot of (l, e) when it is loaded; entries of experts
 *                   not resident are stale (kernels read only the entries of
 *                   the experts a call routes to, which moe_pool_require
 *                   has made resident)
 *   flags           enum moe_pool_flags
 *   pool            out: the new pool (host)
 * Defined by: the bounded slot pool with LFU + recency eviction and
 * one-read fixed-stride experts (pages and sections above).  Errors:
 * INVALID_ARG (null, sizes), UNSUPPORTED / MISALIGNED (desc, stride),
 * NO_DEVICE.
 */
int moe_pool_create(const moe_layer_desc* desc, int32_t n_layers, int32_t n_slots,
                    const void* host_pack, int64_t host_stride, void* device_slab,
                    int32_t* slot_tables, uint32_t flags, moe_pool** pool);

/*
 * Makes experts[0..n) of `layer` resident (host array of expert ids), in
 * order: for each miss a blob copy host_pack -> device_slab is enqueued on
 * `stream`, then one small kernel writes the new slot-table entries, on the
 * same stream.  Work already enqueued on `stream` that reads a replaced slot
 * runs before its copy.  n_missed (host, may be NULL) receives the misses of
 * this call.  Defined by: the pool's replacement policy above.  Errors:
 * INVALID_ARG (null, layer or expert out of range, more distinct experts
 * than slots: nothing changes), LAUNCH.
 */
int moe_pool_require(moe_pool* pool, int32_t layer, const int32_t* experts, int32_t n,
                     int32_t* n_missed, hipStream_t stream);

/* Counters of the pool (host).  Not a passage of the pages: accounting. */
int moe_pool_stats(const moe_pool* pool, moe_pool_stats_t* out);

/*
 * Slot holding (layer, expert), or -1 when it is not resident (host query,
 * no device access).  Not a passage of the pages: inspection for tests.
 */
int32_t moe_pool_slot(const moe_pool* pool, int32_t layer, int32_t expert);

/* Frees the pool's bookkeeping (not the caller's buffers).  NULL is a no-op.
 * Not a passage of the pages: lifetime. */
void moe_pool_destroy(moe_pool* pool);

#ifdef __cplusplus
}
#endif

#endif /* MOE_POOL_H_ */
