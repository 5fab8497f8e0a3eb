// Bounded expert slot pool over a host-memory tier: the replacement policy
// (LFU with recency, see moe_pool.h), the host-to-device blob copies of the
// misses and the device slot-table updates.
//
// Policy state per slot: the key (layer * E + expert) it holds, its use
// count and its last use tick.  Occupied slots sit in an ordered set by
// (count, last use, slot), so the victim of a miss is the first entry whose
// last use is before the current tick (the keys of the current call, whose
// last use is the tick, are skipped: at most n of them).  Free slots are
// taken lowest first.
#include <new>
#include <set>
#include <tuple>
#include <vector>

#include "host.h"
#include "moe_internal.h"
#include "moe_pool.h"

namespace moe {
namespace {

constexpr int kTableUpdates = 64;  // slot-table entries per update launch

struct TableUpdate {
  int32_t n;
  int32_t expert[kTableUpdates];
  int32_t slot[kTableUpdates];
};

__global__ void pool_table_kernel(int32_t* __restrict__ row, TableUpdate u) {
  const int i = threadIdx.x;
  if (i < u.n) row[u.expert[i]] = u.slot[i];
}

}  // namespace
}  // namespace moe

struct moe_pool {
  int32_t E = 0, n_layers = 0, n_slots = 0;
  uint32_t flags = 0;
  int64_t blob_bytes = 0, host_stride = 0, slab_stride = 0;
  const uint8_t* host_pack = nullptr;
  uint8_t* slab = nullptr;
  int32_t* tables = nullptr;
  // policy state
  std::vector<int32_t> slot_of_key;   // [n_layers * E], -1 when not resident
  std::vector<int64_t> key_of_slot;   // -1 when free
  std::vector<int64_t> count, last;   // per slot
  std::set<std::tuple<int64_t, int64_t, int32_t>> order;  // occupied: (count, last, slot)
  std::set<int32_t> free_slots;
  int64_t tick = 0;
  moe_pool_stats_t st{};
};

using namespace moe;

extern "C" int moe_pool_create(const moe_layer_desc* desc, int32_t n_layers, int32_t n_slots,
                               const void* host_pack, int64_t host_stride, void* device_slab,
                               int32_t* slot_tables, uint32_t flags, moe_pool** pool) {
  if (pool == nullptr) return MOE_ERR_INVALID_ARG;
  *pool = nullptr;
  MOE_TRY(check_shape(desc));
  MOE_TRY(check_stride(desc));
  if (n_layers < 1 || n_slots < 1 || (flags & ~(uint32_t)MOE_POOL_HOST_ONLY))
    return MOE_ERR_INVALID_ARG;
  if ((int64_t)n_layers * desc->n_experts > (1LL << 30)) return MOE_ERR_INVALID_ARG;
  const BlobLayout L = make_layout(desc->bits, desc->hidden, desc->inter);
  const bool host_only = (flags & MOE_POOL_HOST_ONLY) != 0;
  if (!host_only) {
    if (host_pack == nullptr || host_stride < L.blob) return MOE_ERR_INVALID_ARG;
    MOE_TRY(check_ptr(device_slab, 256));
    MOE_TRY(check_ptr(slot_tables, 4));
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n < 1) return MOE_ERR_NO_DEVICE;
  }
  moe_pool* p = new (std::nothrow) moe_pool();
  if (p == nullptr) return MOE_ERR_INVALID_ARG;
  p->E = desc->n_experts;
  p->n_layers = n_layers;
  p->n_slots = n_slots;
  p->flags = flags;
  p->blob_bytes = L.blob;
  p->host_stride = host_stride;
  p->slab_stride = desc->expert_stride;
  p->host_pack = reinterpret_cast<const uint8_t*>(host_pack);
  p->slab = reinterpret_cast<uint8_t*>(device_slab);
  p->tables = slot_tables;
  p->slot_of_key.assign((size_t)n_layers * desc->n_experts, -1);
  p->key_of_slot.assign(n_slots, -1);
  p->count.assign(n_slots, 0);
  p->last.assign(n_slots, 0);
  for (int32_t s = 0; s < n_slots; ++s) p->free_slots.insert(s);
  *pool = p;
  return MOE_OK;
}

extern "C" int moe_pool_require(moe_pool* p, int32_t layer, const int32_t* experts, int32_t n,
                                int32_t* n_missed, hipStream_t stream) {
  if (p == nullptr || n < 0 || (n > 0 && experts == nullptr)) return MOE_ERR_INVALID_ARG;
  if (layer < 0 || layer >= p->n_layers) return MOE_ERR_INVALID_ARG;
  // validate everything before any state changes
  int32_t distinct = 0;
  {
    std::set<int32_t> seen;
    for (int32_t i = 0; i < n; ++i) {
      if (experts[i] < 0 || experts[i] >= p->E) return MOE_ERR_INVALID_ARG;
      seen.insert(experts[i]);
    }
    distinct = (int32_t)seen.size();
  }
  if (distinct > p->n_slots) return MOE_ERR_INVALID_ARG;
  p->tick += 1;
  p->st.requests += 1;
  std::vector<std::pair<int32_t, int32_t>> loads;  // (expert, slot)
  for (int32_t i = 0; i < n; ++i) {
    const int64_t key = (int64_t)layer * p->E + experts[i];
    p->st.lookups += 1;
    const int32_t s0 = p->slot_of_key[key];
    if (s0 >= 0) {  // hit
      p->order.erase(std::make_tuple(p->count[s0], p->last[s0], s0));
      p->count[s0] += 1;
      p->last[s0] = p->tick;
      p->order.insert(std::make_tuple(p->count[s0], p->last[s0], s0));
      p->st.hits += 1;
      continue;
    }
    int32_t slot;
    if (!p->free_slots.empty()) {
      slot = *p->free_slots.begin();
      p->free_slots.erase(p->free_slots.begin());
    } else {
      auto it = p->order.begin();
      while (it != p->order.end() && std::get<1>(*it) >= p->tick) ++it;
      // the distinct-count check guarantees a victim outside this call
      slot = std::get<2>(*it);
      p->order.erase(it);
      p->slot_of_key[p->key_of_slot[slot]] = -1;
      p->st.evictions += 1;
    }
    p->key_of_slot[slot] = key;
    p->slot_of_key[key] = slot;
    p->count[slot] = 1;
    p->last[slot] = p->tick;
    p->order.insert(std::make_tuple((int64_t)1, p->tick, slot));
    p->st.misses += 1;
    loads.emplace_back(experts[i], slot);
  }
  if (n_missed) *n_missed = (int32_t)loads.size();
  if ((p->flags & MOE_POOL_HOST_ONLY) || loads.empty()) return MOE_OK;
  for (const auto& ld : loads) {
    const uint8_t* src = p->host_pack + ((int64_t)layer * p->E + ld.first) * p->host_stride;
    uint8_t* dst = p->slab + (int64_t)ld.second * p->slab_stride;
    if (hipMemcpyAsync(dst, src, (size_t)p->blob_bytes, hipMemcpyHostToDevice, stream) !=
        hipSuccess)
      return MOE_ERR_LAUNCH;
    p->st.bytes_copied += p->blob_bytes;
  }
  int32_t* row = p->tables + (int64_t)layer * p->E;
  for (size_t i0 = 0; i0 < loads.size(); i0 += kTableUpdates) {
    TableUpdate u{};
    u.n = (int32_t)std::min<size_t>(kTableUpdates, loads.size() - i0);
    for (int32_t j = 0; j < u.n; ++j) {
      u.expert[j] = loads[i0 + j].first;
      u.slot[j] = loads[i0 + j].second;
    }
    hipLaunchKernelGGL(pool_table_kernel, dim3(1), dim3(kTableUpdates), 0, stream, row, u);
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

extern "C" int moe_pool_stats(const moe_pool* p, moe_pool_stats_t* out) {
  if (p == nullptr || out == nullptr) return MOE_ERR_INVALID_ARG;
  *out = p->st;
  return MOE_OK;
}

extern "C" int32_t moe_pool_slot(const moe_pool* p, int32_t layer, int32_t expert) {
  if (p == nullptr || layer < 0 || layer >= p->n_layers || expert < 0 || expert >= p->E)
    return -1;
  return p->slot_of_key[(int64_t)layer * p->E + expert];
}

extern "C" void moe_pool_destroy(moe_pool* p) { delete p; }
