// Expert pool: per-layer HBM slots for routed experts, an LRU planner and the
// fill pipeline that feeds the slots from a pinned host master copy.
//
// [P2] "SSD 专家卸载 · Prerouter 路由预测", expert-pool and prefetch
// paragraphs: recently used experts stay resident (least recently used ones
// are replaced), and the experts the Prerouter predicts for the next layer
// are loaded ahead of use.  Here the master copy is pinned host memory, the
// pool is a set of HBM slots per layer, and kernels find an expert through a
// device slot table (-1: not resident, read the host copy directly).
//
// Ordering.  A fill of slot s (evicting expert a, loading expert b) runs on a
// side stream as: (1) table row with a -> -1, (2) event inv[layer], (3) copy
// of b's blob into s, (4) table row with b -> s, (5) event filled[layer].  A
// kernel of that layer that starts after inv[layer] never maps a to s, and
// sees b -> s only once the copy is complete; kernels that used a were
// finished before the plan was made (the caller plans after the previous
// token completed).  A kernel that starts after filled[layer] finds every
// expert of the plan in its slot (prediction-as-routing waits for that).
// With a modeled storage latency, one wait kernel precedes the plan's copies.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <new>
#include <vector>

#include "moe_internal.h"
#include "status.h"

namespace {

struct LayerLru {
  std::vector<int32_t> slot_expert;  // [n_slots], -1 = free
  std::vector<int32_t> expert_slot;  // [E], -1 = not resident
  std::vector<uint64_t> last_use;    // [n_slots]
};

}  // namespace

struct moe_lru {
  int32_t n_layers = 0, E = 0, n_slots = 0;
  uint64_t clock = 0;
  std::vector<LayerLru> layers;
  unsigned long long fills = 0, evictions = 0;
};

struct moe_pool {
  moe_lru lru;
  size_t blob_bytes = 0;
  uint8_t* slots = nullptr;         // device [n_layers][n_slots][blob_bytes]
  int32_t* table = nullptr;         // device [n_layers][E]
  const uint8_t* host = nullptr;      // pinned [n_layers][E][blob_bytes] (host view)
  const uint8_t* host_dev = nullptr;  // the same memory as seen by kernels
  int32_t* staging = nullptr;       // pinned [2][n_layers][E]
  std::vector<hipEvent_t> inv;      // per layer
  std::vector<char> inv_pending;    // per layer: inv[layer] recorded since last wait
  std::vector<hipEvent_t> filled;   // per layer: after the fills and the final table row
  std::vector<char> filled_pending;
  uint32_t read_delay_ns = 0;       // modeled storage latency of the master copy
  std::vector<moe_pool_fill_t> plan;
};

namespace {

moe_status_t lru_init(moe_lru* l, int32_t n_layers, int32_t E, int32_t n_slots) {
  if (n_layers <= 0 || E <= 0 || n_slots <= 0 || n_slots > E)
    return fail(MOE_EINVAL, "moe_lru: need n_layers > 0, 0 < n_slots <= E (got %d, %d, %d)",
                n_layers, n_slots, E);
  l->n_layers = n_layers;
  l->E = E;
  l->n_slots = n_slots;
  l->layers.resize(n_layers);
  for (auto& L : l->layers) {
    L.slot_expert.assign(n_slots, -1);
    L.expert_slot.assign(E, -1);
    L.last_use.assign(n_slots, 0);
  }
  return MOE_OK;
}

// One planning step; see moe_lru_plan in the header for the rules.
moe_status_t lru_plan(moe_lru* l, const int32_t* executed, int32_t K, const int32_t* predicted,
                      int32_t Kp, int32_t max_fills, std::vector<moe_pool_fill_t>& out) {
  out.clear();
  if (K < 0 || Kp < 0 || (K > 0 && executed == nullptr) || (Kp > 0 && predicted == nullptr))
    return fail(MOE_EINVAL, "moe_lru_plan: bad executed/predicted arguments");
  for (int32_t ly = 0; ly < l->n_layers; ++ly)
    for (int32_t k = 0; k < K; ++k) {
      const int32_t e = executed[size_t(ly) * K + k];
      if (e < 0 || e >= l->E) return fail(MOE_EINVAL, "moe_lru_plan: executed expert %d out of range", e);
    }
  for (int32_t ly = 0; ly < l->n_layers; ++ly)
    for (int32_t k = 0; k < Kp; ++k)
      if (predicted[size_t(ly) * Kp + k] >= l->E)
        return fail(MOE_EINVAL, "moe_lru_plan: predicted expert %d out of range",
                    predicted[size_t(ly) * Kp + k]);
  const uint64_t now = ++l->clock;
  std::vector<char> prot;
  std::vector<int32_t> want;
  for (int32_t ly = 0; ly < l->n_layers; ++ly) {
    LayerLru& L = l->layers[ly];
    prot.assign(l->E, 0);
    // executed experts: mark used (resident ones get the new time stamp)
    for (int32_t k = 0; k < K; ++k) {
      const int32_t e = executed[size_t(ly) * K + k];
      prot[e] = 1;
      if (L.expert_slot[e] >= 0) L.last_use[L.expert_slot[e]] = now;
    }
    // fill candidates: predicted experts first, then this token's misses
    want.clear();
    for (int32_t k = 0; k < Kp; ++k) {
      const int32_t e = predicted[size_t(ly) * Kp + k];
      if (e < 0) continue;  // no prediction
      prot[e] = 1;
      if (L.expert_slot[e] >= 0)
        L.last_use[L.expert_slot[e]] = now;  // predicted and resident: keep it
      else if (std::find(want.begin(), want.end(), e) == want.end())
        want.push_back(e);
    }
    for (int32_t k = 0; k < K; ++k) {
      const int32_t e = executed[size_t(ly) * K + k];
      if (L.expert_slot[e] < 0 && std::find(want.begin(), want.end(), e) == want.end()) want.push_back(e);
    }
    int32_t n_fill = 0;
    for (int32_t e : want) {
      if (max_fills >= 0 && n_fill >= max_fills) break;
      // victim: a free slot, else the least recently used slot whose expert
      // is not protected (ties: lowest slot index)
      int32_t victim = -1;
      for (int32_t s = 0; s < l->n_slots; ++s)
        if (L.slot_expert[s] < 0) {
          victim = s;
          break;
        }
      if (victim < 0)
        for (int32_t s = 0; s < l->n_slots; ++s) {
          if (prot[L.slot_expert[s]]) continue;
          if (victim < 0 || L.last_use[s] < L.last_use[victim]) victim = s;
        }
      if (victim < 0) break;  // every slot holds a protected expert
      const int32_t old = L.slot_expert[victim];
      if (old >= 0) {
        L.expert_slot[old] = -1;
        ++l->evictions;
      }
      L.slot_expert[victim] = e;
      L.expert_slot[e] = victim;
      L.last_use[victim] = now;
      prot[e] = 1;
      ++l->fills;
      ++n_fill;
      out.push_back(moe_pool_fill_t{ly, e, victim, old});
    }
  }
  return MOE_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// LRU planner (host only)
// ---------------------------------------------------------------------------
extern "C" {

MOE_API moe_status_t moe_lru_create(int32_t n_layers, int32_t E, int32_t n_slots, moe_lru_t** out) {
  if (out == nullptr) return fail(MOE_EINVAL, "moe_lru_create: out is NULL");
  *out = nullptr;
  moe_lru* l = new (std::nothrow) moe_lru();
  if (l == nullptr) return fail(MOE_EINVAL, "moe_lru_create: out of host memory");
  const moe_status_t st = lru_init(l, n_layers, E, n_slots);
  if (st != MOE_OK) {
    delete l;
    return st;
  }
  *out = l;
  return MOE_OK;
}

MOE_API void moe_lru_destroy(moe_lru_t* l) { delete l; }

MOE_API moe_status_t moe_lru_plan(moe_lru_t* l, const int32_t* executed, int32_t K,
                                  const int32_t* predicted, int32_t Kp, int32_t max_fills,
                                  moe_pool_fill_t* fills, int32_t max_out, int32_t* n_out) {
  if (l == nullptr || n_out == nullptr) return fail(MOE_EINVAL, "moe_lru_plan: NULL argument");
  std::vector<moe_pool_fill_t> plan;
  const moe_status_t st = lru_plan(l, executed, K, predicted, Kp, max_fills, plan);
  if (st != MOE_OK) return st;
  *n_out = int32_t(plan.size());
  if (int32_t(plan.size()) > max_out)
    return fail(MOE_EINVAL, "moe_lru_plan: %zu fills do not fit in %d entries", plan.size(), max_out);
  if (!plan.empty()) std::memcpy(fills, plan.data(), plan.size() * sizeof(moe_pool_fill_t));
  return MOE_OK;
}

MOE_API moe_status_t moe_lru_table(const moe_lru_t* l, int32_t layer, int32_t* expert_to_slot) {
  if (l == nullptr || expert_to_slot == nullptr || layer < 0 || layer >= l->n_layers)
    return fail(MOE_EINVAL, "moe_lru_table: bad arguments");
  std::memcpy(expert_to_slot, l->layers[layer].expert_slot.data(), size_t(l->E) * sizeof(int32_t));
  return MOE_OK;
}

MOE_API moe_status_t moe_lru_stats(const moe_lru_t* l, unsigned long long* fills,
                                   unsigned long long* evictions) {
  if (l == nullptr) return fail(MOE_EINVAL, "moe_lru_stats: NULL pool");
  if (fills) *fills = l->fills;
  if (evictions) *evictions = l->evictions;
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// Pool: planner + fills on a side stream
// ---------------------------------------------------------------------------
MOE_API moe_status_t moe_pool_create(int32_t n_layers, int32_t E, int32_t n_slots, size_t blob_bytes,
                                     void* device_slots, int32_t* device_table,
                                     const void* host_blobs, void* stream, moe_pool_t** out) {
  if (out == nullptr) return fail(MOE_EINVAL, "moe_pool_create: out is NULL");
  *out = nullptr;
  if (device_slots == nullptr || device_table == nullptr || host_blobs == nullptr || blob_bytes == 0)
    return fail(MOE_EINVAL, "moe_pool_create: slots, table and host blobs are required");
  moe_pool* p = new (std::nothrow) moe_pool();
  if (p == nullptr) return fail(MOE_EINVAL, "moe_pool_create: out of host memory");
  moe_status_t st = lru_init(&p->lru, n_layers, E, n_slots);
  if (st != MOE_OK) {
    delete p;
    return st;
  }
  p->blob_bytes = blob_bytes;
  p->slots = static_cast<uint8_t*>(device_slots);
  p->table = device_table;
  p->host = static_cast<const uint8_t*>(host_blobs);
  // kernels read non-resident experts through the device view of the pinned
  // host copy; memory that is not pinned and mapped is rejected here
  void* dview = nullptr;
  hipError_t e = hipHostGetDevicePointer(&dview, const_cast<void*>(host_blobs), 0);
  if (e != hipSuccess || dview == nullptr) {
    (void)hipGetLastError();
    delete p;
    return fail(MOE_EINVAL, "moe_pool_create: host_blobs is not pinned, device-visible memory (%s)",
                hipGetErrorString(e));
  }
  p->host_dev = static_cast<const uint8_t*>(dview);
  const size_t rows = size_t(2) * n_layers * E;
  e = hipHostMalloc(reinterpret_cast<void**>(&p->staging), rows * sizeof(int32_t),
                    hipHostMallocDefault);
  if (e != hipSuccess) {
    delete p;
    return fail(MOE_EHIP, "moe_pool_create: hipHostMalloc: %s", hipGetErrorString(e));
  }
  for (size_t i = 0; i < rows; ++i) p->staging[i] = -1;
  p->inv.assign(n_layers, nullptr);
  p->inv_pending.assign(n_layers, 0);
  p->filled.assign(n_layers, nullptr);
  p->filled_pending.assign(n_layers, 0);
  for (int32_t ly = 0; ly < n_layers && e == hipSuccess; ++ly) {
    e = hipEventCreateWithFlags(&p->inv[ly], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&p->filled[ly], hipEventDisableTiming);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(p->table, p->staging, size_t(n_layers) * E * sizeof(int32_t),
                       hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    moe_pool_destroy(p);
    return fail(MOE_EHIP, "moe_pool_create: %s", hipGetErrorString(e));
  }
  *out = p;
  return MOE_OK;
}

MOE_API void moe_pool_destroy(moe_pool_t* p) {
  if (p == nullptr) return;
  for (hipEvent_t ev : p->inv)
    if (ev) (void)hipEventDestroy(ev);
  for (hipEvent_t ev : p->filled)
    if (ev) (void)hipEventDestroy(ev);
  if (p->staging) (void)hipHostFree(p->staging);
  delete p;
}

MOE_API moe_status_t moe_pool_layer(const moe_pool_t* p, int32_t layer, unsigned long long* counters,
                                    moe_experts_t* out) {
  if (p == nullptr || out == nullptr || layer < 0 || layer >= p->lru.n_layers)
    return fail(MOE_EINVAL, "moe_pool_layer: bad arguments");
  out->slots = p->slots + size_t(layer) * p->lru.n_slots * p->blob_bytes;
  out->n_slots = p->lru.n_slots;
  out->expert_to_slot = p->table + size_t(layer) * p->lru.E;
  out->host_blobs = p->host_dev + size_t(layer) * p->lru.E * p->blob_bytes;
  out->counters = counters;
  out->read_delay_ns = p->read_delay_ns;
  return MOE_OK;
}

MOE_API moe_status_t moe_pool_set_read_delay(moe_pool_t* p, uint32_t ns) {
  if (p == nullptr) return fail(MOE_EINVAL, "moe_pool_set_read_delay: NULL pool");
  if (ns > MOE_MAX_READ_DELAY_NS)
    return fail(MOE_EINVAL, "moe_pool_set_read_delay: %u ns exceeds %u", ns, MOE_MAX_READ_DELAY_NS);
  p->read_delay_ns = ns;
  return MOE_OK;
}

MOE_API moe_status_t moe_pool_update(moe_pool_t* p, const int32_t* executed, int32_t K,
                                     const int32_t* predicted, int32_t Kp, int32_t max_fills,
                                     void* side_stream, int32_t* n_fills) {
  if (p == nullptr) return fail(MOE_EINVAL, "moe_pool_update: NULL pool");
  hipStream_t s = static_cast<hipStream_t>(side_stream);
  // the staging rows of the previous update must have been consumed
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(MOE_EHIP, "moe_pool_update: %s", hipGetErrorString(e));
  moe_status_t st = lru_plan(&p->lru, executed, K, predicted, Kp, max_fills, p->plan);
  if (st != MOE_OK) return st;
  if (n_fills) *n_fills = int32_t(p->plan.size());
  const int32_t E = p->lru.E;
  const size_t row_bytes = size_t(E) * sizeof(int32_t);
  if (!p->plan.empty() && p->read_delay_ns) {
    // the step's reads are issued together: one storage latency before the copies
    e = moe::launch_storage_delay(moe::wall_ticks(p->read_delay_ns), s);
    if (e != hipSuccess) return fail(MOE_EHIP, "moe_pool_update: %s", hipGetErrorString(e));
  }
  size_t i = 0;
  while (i < p->plan.size()) {
    const int32_t ly = p->plan[i].layer;
    size_t j = i;
    while (j < p->plan.size() && p->plan[j].layer == ly) ++j;
    int32_t* inv_row = p->staging + size_t(ly) * E;
    int32_t* pub_row = p->staging + size_t(p->lru.n_layers + ly) * E;
    // pub_row: the planner's new table; inv_row: the old table minus evictions
    std::memcpy(pub_row, p->lru.layers[ly].expert_slot.data(), row_bytes);
    std::memcpy(inv_row, pub_row, row_bytes);
    for (size_t f = i; f < j; ++f) inv_row[p->plan[f].expert] = -1;
    int32_t* dev_row = p->table + size_t(ly) * E;
    e = hipMemcpyAsync(dev_row, inv_row, row_bytes, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipEventRecord(p->inv[ly], s);
    for (size_t f = i; f < j && e == hipSuccess; ++f) {
      const moe_pool_fill_t& fl = p->plan[f];
      uint8_t* dst = p->slots + (size_t(ly) * p->lru.n_slots + fl.slot) * p->blob_bytes;
      const uint8_t* src = p->host + (size_t(ly) * E + fl.expert) * p->blob_bytes;
      e = hipMemcpyAsync(dst, src, p->blob_bytes, hipMemcpyHostToDevice, s);
    }
    if (e == hipSuccess) e = hipMemcpyAsync(dev_row, pub_row, row_bytes, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipEventRecord(p->filled[ly], s);
    if (e != hipSuccess) return fail(MOE_EHIP, "moe_pool_update: %s", hipGetErrorString(e));
    p->inv_pending[ly] = 1;
    p->filled_pending[ly] = 1;
    i = j;
  }
  return MOE_OK;
}

MOE_API moe_status_t moe_pool_wait_layer(moe_pool_t* p, int32_t layer, void* stream) {
  if (p == nullptr || layer < 0 || layer >= p->lru.n_layers)
    return fail(MOE_EINVAL, "moe_pool_wait_layer: bad arguments");
  if (!p->inv_pending[layer]) return MOE_OK;
  const hipError_t e = hipStreamWaitEvent(static_cast<hipStream_t>(stream), p->inv[layer], 0);
  if (e != hipSuccess) return fail(MOE_EHIP, "moe_pool_wait_layer: %s", hipGetErrorString(e));
  p->inv_pending[layer] = 0;
  return MOE_OK;
}

MOE_API moe_status_t moe_pool_wait_layer_filled(moe_pool_t* p, int32_t layer, void* stream) {
  if (p == nullptr || layer < 0 || layer >= p->lru.n_layers)
    return fail(MOE_EINVAL, "moe_pool_wait_layer_filled: bad arguments");
  if (!p->filled_pending[layer]) return MOE_OK;
  const hipError_t e = hipStreamWaitEvent(static_cast<hipStream_t>(stream), p->filled[layer], 0);
  if (e != hipSuccess)
    return fail(MOE_EHIP, "moe_pool_wait_layer_filled: %s", hipGetErrorString(e));
  p->filled_pending[layer] = 0;
  p->inv_pending[layer] = 0;  // the fills follow the invalidation on the same stream
  return MOE_OK;
}

MOE_API moe_status_t moe_pool_sync(moe_pool_t* p, void* side_stream) {
  if (p == nullptr) return fail(MOE_EINVAL, "moe_pool_sync: NULL pool");
  const hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(side_stream));
  if (e != hipSuccess) return fail(MOE_EHIP, "moe_pool_sync: %s", hipGetErrorString(e));
  return MOE_OK;
}

MOE_API const moe_lru_t* moe_pool_lru(const moe_pool_t* p) { return p ? &p->lru : nullptr; }

}  // extern "C"
