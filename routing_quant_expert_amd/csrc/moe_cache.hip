// Expert streaming beyond HBM: an expert cache of a fixed number of device
// slots over host-resident expert blocks [device_route.rs, module doc,
// fn route_device_m1, fn slot_table_update; moe_v41.rs, module doc: the LRU
// gathers the picked experts' raw blocks into its device slots, misses read
// from storage]. Per layer:
//   1. the routing runs on the device against the layer's row of the device
//      slot table: the header gets the picks, their weights, the picks'
//      slots in plan order (-1 = absent) and the miss flag;
//   2. the header is read back, once;
//   3. the LRU makes every pick resident: a hit is touched, a miss takes the
//      least recently used slot outside the call's protected set and its
//      blocks are copied there from host memory; the slot table rows that
//      changed are uploaded;
//   4. the experts, the shared expert and the combine run from the slots.
// With prefetch_k > 0 the next layer's router also runs on this layer's
// input (the pages' predictor: pred_logits, prefetch_k), and the first
// prefetch_k predicted experts of each token are copied into slots on a copy
// stream of the cache's own while this layer computes; the next layer's
// demand copies wait for them.
// The copies, table uploads and kernels of one layer are ordered on the
// caller's stream, so a slot is only overwritten after the kernels that read
// its previous expert; prefetch copies only take slots that no enqueued
// kernel reads.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <vector>

#include "moe_host.h"
#include "moe_internal.h"

struct moe_cache;

namespace moe {

// Least-recently-used assignment of keys (layer * n_routed + expert) to
// slots. A batch is the set of keys one step needs at once: every key of it
// ends up resident, and no slot taken for it, or touched by it, is evicted
// before the batch is over. protect_from: slots last used by a batch at or
// after this epoch are not evicted either (the batch of kernels still in
// flight, when prefetching).
class SlotLru {
 public:
  struct Change {
    int64_t key;
    int32_t slot;   // -1: the key was evicted
  };

  SlotLru(int n_slots, int64_t n_keys)
      : slot_of_key_(n_keys, -1), key_of_slot_(n_slots, -1), last_use_(n_slots, 0), epoch_of_(n_slots, 0) {}

  int64_t n_keys() const { return (int64_t)slot_of_key_.size(); }
  int n_slots() const { return (int)key_of_slot_.size(); }
  const int32_t* table() const { return slot_of_key_.data(); }
  uint64_t epoch() const { return epoch_; }

  // Opens a new batch; returns its epoch.
  uint64_t begin() { return ++epoch_; }

  // Makes `key` resident within the current batch. Returns its slot, or -1
  // when every slot is protected. *miss: the key was not resident.
  int32_t acquire(int64_t key, uint64_t protect_from, bool* miss, std::vector<Change>& changes) {
    int32_t s = slot_of_key_[key];
    *miss = s < 0;
    if (s < 0) {
      int best = -1;
      for (int i = 0; i < n_slots(); ++i) {   // the least recently used unprotected slot (never used: 0)
        if (epoch_of_[i] >= protect_from && epoch_of_[i] != 0) continue;
        if (best < 0 || last_use_[i] < last_use_[best]) best = i;
      }
      if (best < 0) return -1;
      s = best;
      const int64_t old = key_of_slot_[s];
      if (old >= 0) {
        slot_of_key_[old] = -1;
        changes.push_back({old, -1});
      }
      key_of_slot_[s] = key;
      slot_of_key_[key] = s;
      changes.push_back({key, s});
    }
    last_use_[s] = ++clock_;
    epoch_of_[s] = epoch_;
    return s;
  }

  // A whole batch: the keys already resident are touched first, so that no
  // miss of the batch evicts a key the batch needs; then the misses take slots.
  void acquire_batch(const int64_t* keys, int n, uint64_t protect_from, int32_t* slots, char* miss,
                     std::vector<Change>& changes) {
    bool m = false;
    for (int i = 0; i < n; ++i) {
      slots[i] = -1;
      miss[i] = 0;
      if (slot_of_key_[keys[i]] >= 0) slots[i] = acquire(keys[i], protect_from, &m, changes);
    }
    for (int i = 0; i < n; ++i)
      if (slots[i] < 0) {   // a miss, or a repeat of a key placed earlier in this pass (then a hit)
        slots[i] = acquire(keys[i], protect_from, &m, changes);
        miss[i] = m;
      }
  }

 private:
  std::vector<int32_t> slot_of_key_;
  std::vector<int64_t> key_of_slot_;
  std::vector<uint64_t> last_use_;
  std::vector<uint64_t> epoch_of_;   // epoch of the batch that last used the slot (0: never)
  uint64_t clock_ = 0, epoch_ = 0;
};

}  // namespace moe

using namespace moe;

struct moe_cache {
  moe_cfg cfg;
  int n_layers = 0, n_slots = 0, max_m = 0;
  std::vector<const uint8_t*> host;   // each layer's host arena: expert e at host[l] + e * stride
  uint64_t stride = 0, gate_off = 0, up_off = 0, down_off = 0;
  int device = 0;
  uint8_t* pool = nullptr;            // device: n_slots * stride
  int32_t* table = nullptr;           // device: [n_layers][n_routed] slot of each expert, -1 absent
  int32_t* pred_hdr = nullptr;        // device: the predicted next-layer headers [max_m][hw]
  int32_t* hdr_host = nullptr;        // pinned: a layer's headers, then the predicted ones
  int32_t* stage = nullptr;           // pinned: staging of the slot table rows uploaded between two read-backs
  int stage_rows = 0, stage_used = 0;
  hipStream_t copy = nullptr;         // prefetch copies
  hipEvent_t copy_done = nullptr;
  bool copy_pending = false;
  uint64_t demand_epoch = 0;          // the LRU epoch of the last layer's demand batch
  std::vector<char> prefetched;       // per slot: filled by a prefetch and not demanded since
  SlotLru lru;
  moe_cache_stats stats{};

  moe_cache(int n_slots_, int64_t n_keys) : lru(n_slots_, n_keys) {}
};

namespace {

int cache_fail(hipError_t e, const char* where) { return hip_fail(e, where); }

void free_cache(moe_cache* c) {
  if (!c) return;
  if (c->pool) (void)hipFree(c->pool);
  if (c->table) (void)hipFree(c->table);
  if (c->pred_hdr) (void)hipFree(c->pred_hdr);
  if (c->hdr_host) (void)hipHostFree(c->hdr_host);
  if (c->stage) (void)hipHostFree(c->stage);
  if (c->copy_done) (void)hipEventDestroy(c->copy_done);
  if (c->copy) (void)hipStreamDestroy(c->copy);
  delete c;
}

// Uploads the slot-table rows of the keys in `changes` on stream `s`, each
// row staged in pinned memory that stays untouched until the next read-back.
int upload_rows(moe_cache* c, const std::vector<SlotLru::Change>& changes, hipStream_t s) {
  const int n = c->cfg.n_routed;
  std::vector<int> rows;
  for (const auto& ch : changes) {
    const int l = (int)(ch.key / n);
    bool seen = false;
    for (int r : rows) seen |= r == l;
    if (!seen) rows.push_back(l);
  }
  for (int l : rows) {
    if (c->stage_used == c->stage_rows) {   // every staged row may still be read: drain, then reuse
      hipError_t e = hipStreamSynchronize(s);
      if (e != hipSuccess) return cache_fail(e, "cache staging");
      c->stage_used = 0;
    }
    int32_t* st = c->stage + (int64_t)c->stage_used++ * n;
    std::memcpy(st, c->lru.table() + (int64_t)l * n, (size_t)n * 4);
    hipError_t e = hipMemcpyAsync(c->table + (int64_t)l * n, st, (size_t)n * 4, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return cache_fail(e, "slot table upload");
  }
  return MOE_OK;
}

// Acquires `keys` (one batch) and copies the misses' blocks into their slots
// on `s`. protect_from: as SlotLru::acquire. prefetch: a miss that finds no
// free slot is skipped instead of failing.
int fetch(moe_cache* c, const std::vector<int64_t>& keys, uint64_t protect_from, bool prefetch, hipStream_t s,
          std::vector<SlotLru::Change>& changes) {
  const int n = c->cfg.n_routed;
  const int nk = (int)keys.size();
  std::vector<int32_t> slots(nk, -1);
  std::vector<char> misses(nk, 0);
  c->lru.acquire_batch(keys.data(), nk, protect_from, slots.data(), misses.data(), changes);
  for (int q = 0; q < nk; ++q) {
    const int64_t key = keys[q];
    const bool miss = misses[q] != 0;
    const int32_t slot = slots[q];
    if (slot < 0) {
      if (prefetch) continue;
      return fail(MOE_EUNSUPPORTED, "expert cache: a layer's picks need more slots than the cache has%s (%lld)", "",
                  (long long)c->n_slots);
    }
    if (prefetch) {
      if (miss) {
        c->prefetched[slot] = 1;
        c->stats.prefetched += 1;
      }
    } else if (miss) {
      c->stats.misses += 1;
    } else {
      c->stats.hits += 1;
      if (c->prefetched[slot]) c->stats.prefetch_used += 1;
    }
    if (!prefetch) c->prefetched[slot] = 0;
    if (miss) {
      const int l = (int)(key / n), e = (int)(key % n);
      hipError_t err = hipMemcpyAsync(c->pool + (uint64_t)slot * c->stride, c->host[l] + (uint64_t)e * c->stride,
                                      c->stride, hipMemcpyHostToDevice, s);
      if (err != hipSuccess) return cache_fail(err, "expert copy");
      c->stats.bytes_copied += (int64_t)c->stride;
    }
  }
  return MOE_OK;
}

}  // namespace

extern "C" {

static int moe_cache_create_body(const moe_cfg* cfg, int32_t n_layers, const void* const* host_experts,
                                 uint64_t stride, uint64_t gate_off, uint64_t up_off, uint64_t down_off,
                                 int32_t n_slots, int32_t max_m, moe_cache** out) {
  if (int r = check_cfg(cfg)) return r;
  if (!out || !host_experts || n_layers < 1 || n_slots < 1)
    return fail(MOE_EINVAL, "expert cache: out, host_experts non-NULL, n_layers >= 1, n_slots >= 1%s%lld");
  if (int r = check_m(*cfg, max_m)) return r;
  for (int l = 0; l < n_layers; ++l)
    if (!host_experts[l]) return fail(MOE_EINVAL, "expert cache: host arena of layer %s%lld is NULL", "", l);
  moe_experts probe{reinterpret_cast<const void*>(16), stride, gate_off, up_off, down_off};
  if (int r = check_experts(&probe)) return r;
  const uint64_t gate_bytes = (uint64_t)cfg->inter * (cfg->dim / 256) * kQ2KBytes;
  const uint64_t down_bytes = (uint64_t)cfg->dim * (cfg->inter / 256) * kQ3KBytes;
  if (gate_off + gate_bytes > stride || up_off + gate_bytes > stride || down_off + down_bytes > stride)
    return fail(MOE_EINVAL, "expert cache: an expert's matrices must fit in its stride%s (%lld bytes)", "",
                (long long)stride);
  const int64_t n_keys = (int64_t)n_layers * cfg->n_routed;
  moe_cache* c = new moe_cache(n_slots, n_keys);
  c->cfg = *cfg;
  c->n_layers = n_layers;
  c->n_slots = n_slots;
  c->max_m = max_m;
  c->stride = stride;
  c->gate_off = gate_off;
  c->up_off = up_off;
  c->down_off = down_off;
  c->prefetched.assign(n_slots, 0);
  for (int l = 0; l < n_layers; ++l) c->host.push_back(static_cast<const uint8_t*>(host_experts[l]));
  const int hw = 1 + 3 * cfg->topk;
  c->stage_rows = 2 * n_layers + 16;
  hipError_t e;
  if ((e = hipGetDevice(&c->device)) != hipSuccess ||
      (e = hipMalloc(&c->pool, (size_t)n_slots * stride)) != hipSuccess ||
      (e = hipMalloc(&c->table, (size_t)n_keys * 4)) != hipSuccess ||
      (e = hipMalloc(&c->pred_hdr, (size_t)max_m * hw * 4)) != hipSuccess ||
      (e = hipHostMalloc(&c->hdr_host, (size_t)2 * max_m * hw * 4, hipHostMallocDefault)) != hipSuccess ||
      (e = hipHostMalloc(&c->stage, (size_t)c->stage_rows * cfg->n_routed * 4, hipHostMallocDefault)) != hipSuccess ||
      (e = hipStreamCreateWithFlags(&c->copy, hipStreamNonBlocking)) != hipSuccess ||
      (e = hipEventCreateWithFlags(&c->copy_done, hipEventDisableTiming)) != hipSuccess ||
      (e = hipMemcpy(c->table, c->lru.table(), (size_t)n_keys * 4, hipMemcpyHostToDevice)) != hipSuccess) {
    free_cache(c);
    return cache_fail(e, "expert cache set-up");
  }
  *out = c;
  return MOE_OK;
}

int moe_cache_destroy(moe_cache* cache) {
  if (!cache) return MOE_OK;
  if (cache->copy) (void)hipStreamSynchronize(cache->copy);
  free_cache(cache);
  return MOE_OK;
}

static int moe_cache_forward_body(moe_cache* cache, const moe_cfg* cfg, const moe_layer* layers, int32_t first_layer,
                                  int32_t n_layers, uint16_t* xs, int32_t m, float* out_f32, int32_t* headers,
                                  int32_t prefetch_k, void* ws, size_t ws_bytes, void* stream) {
  if (!cache) return fail(MOE_EINVAL, "expert cache is NULL%s%lld");
  if (int r = check_cfg(cfg)) return r;
  if (int r = check_score_mode(*cfg)) return r;
  moe_cache* c = cache;
  if (std::memcmp(cfg, &c->cfg, sizeof(moe_cfg)) != 0)
    return fail(MOE_EINVAL, "expert cache: cfg differs from the one the cache was made for%s%lld");
  if (!layers || !xs) return fail(MOE_EINVAL, "layers and xs must be non-NULL%s%lld");
  if (n_layers < 1 || first_layer < 0 || first_layer + n_layers > c->n_layers)
    return fail(MOE_EINVAL, "expert cache: layers outside the cache%s (first %lld)", "", first_layer);
  if (int r = check_m(*cfg, m)) return r;
  if (m > c->max_m) return fail(MOE_EINVAL, "expert cache: m above the cache's max_m%s (%lld)", "", m);
  if (prefetch_k < 0 || prefetch_k > cfg->topk) return fail(MOE_EINVAL, "prefetch_k outside 0..topk%s (%lld)", "", prefetch_k);
  if (!a16(xs) || ((int64_t)m * cfg->dim * 2) % 16) return fail(MOE_EINVAL, "xs must be 16-byte aligned%s%lld");
  for (int l = 0; l < n_layers; ++l)
    if (int r = check_layer(&layers[l], false)) return r;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev != c->device)
    return fail(MOE_EINVAL, "expert cache: called with another device current%s%lld");
  moe_ws_layout L;
  if (int r = check_ws(*cfg, m, ws, ws_bytes, &L)) return r;
  Ws w = ws_view(ws, L, *cfg, m);
  int32_t* grp = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) + L.grp);
  const hipStream_t s = (hipStream_t)stream;
  const int n = cfg->n_routed, k = cfg->topk, hw = 1 + 3 * k;
  const int64_t row = (int64_t)m * cfg->dim;
  hipError_t e;
  for (int i = 0; i < n_layers; ++i) {
    const int l = first_layer + i;
    const moe_layer& layer = layers[i];
    const int32_t* slot_row = c->table + (int64_t)l * n;
    int32_t* hdr = headers ? headers + (int64_t)i * m * hw : w.status + 4;
    const uint16_t* x = xs + i * row;
    // 1. routing against the slot table (and, for prefetching, the next layer's router on the same input)
    if ((e = route_launches(*cfg, x, m, layer.gate_w, layer.bias, hdr, w, slot_row, s)) != hipSuccess)
      return hip_fail(e, "cache routing");
    const bool predict = prefetch_k > 0 && l + 1 < c->n_layers && i + 1 < n_layers;
    if (predict && (e = route_launches(*cfg, x, m, layers[i + 1].gate_w, layers[i + 1].bias, c->pred_hdr, w,
                                       nullptr, s)) != hipSuccess)
      return hip_fail(e, "cache prediction");
    // 2. the one read-back
    if ((e = hipMemcpyAsync(c->hdr_host, hdr, (size_t)m * hw * 4, hipMemcpyDeviceToHost, s)) != hipSuccess ||
        (predict && (e = hipMemcpyAsync(c->hdr_host + (int64_t)m * hw, c->pred_hdr, (size_t)m * hw * 4,
                                        hipMemcpyDeviceToHost, s)) != hipSuccess) ||
        (e = hipStreamSynchronize(s)) != hipSuccess)
      return hip_fail(e, "cache header read-back");
    c->stats.reads_back += 1;
    c->stage_used = 0;   // every earlier upload has run
    // 3. the picks made resident (after the last prefetch's copies)
    if (c->copy_pending) {
      if ((e = hipStreamWaitEvent(s, c->copy_done, 0)) != hipSuccess) return hip_fail(e, "cache join");
      c->copy_pending = false;
    }
    std::vector<int64_t> keys;
    for (int t = 0; t < m; ++t)
      for (int r = 0; r < k; ++r) {
        const int32_t pick = c->hdr_host[t * hw + 1 + r];
        if (pick < 0 || pick >= n) return fail(MOE_EINVAL, "expert cache: a pick outside 0..n_routed%s (%lld)", "", pick);
        const int64_t key = (int64_t)l * n + pick;
        bool seen = false;
        for (int64_t q : keys) seen |= q == key;
        if (!seen) keys.push_back(key);
      }
    std::vector<SlotLru::Change> changes;
    c->demand_epoch = c->lru.begin();
    if (int r = fetch(c, keys, c->demand_epoch, false, s, changes)) return r;
    if (int r = upload_rows(c, changes, s)) return r;
    // 4. the experts from the slots, the shared expert and the combine
    moe_experts pool{c->pool, c->stride, c->gate_off, c->up_off, c->down_off};
    const XArena ar = arena_of(pool, n, shared_bf16(layer) ? nullptr : &layer.shared_q, slot_row);
    LayerOut o{out_f32 ? out_f32 + i * row : nullptr, nullptr, x, xs + (i + 1) * row};
    if (int r = layer_launches_hdr(*cfg, layer, ar, x, m, hdr, o, w, grp, s)) return r;
    // the next layer's predicted experts, copied while this layer computes
    if (predict) {
      std::vector<int64_t> pkeys;
      const int32_t* ph = c->hdr_host + (int64_t)m * hw;
      for (int t = 0; t < m; ++t)
        for (int r = 0; r < prefetch_k; ++r) {
          const int32_t pick = ph[t * hw + 1 + r];
          if (pick < 0 || pick >= n) continue;
          const int64_t key = (int64_t)(l + 1) * n + pick;
          bool seen = false;
          for (int64_t q : pkeys) seen |= q == key;
          if (!seen) pkeys.push_back(key);
        }
      std::vector<SlotLru::Change> pchanges;
      c->lru.begin();
      if (int r = fetch(c, pkeys, c->demand_epoch, true, c->copy, pchanges)) return r;
      if ((e = hipEventRecord(c->copy_done, c->copy)) != hipSuccess) return hip_fail(e, "cache prefetch event");
      c->copy_pending = true;
      if (int r = upload_rows(c, pchanges, s)) return r;
    }
  }
  return MOE_OK;
}

static int moe_cache_prefetch_body(moe_cache* cache, int32_t layer, const int32_t* experts, int32_t n, void* stream) {
  if (!cache || (n > 0 && !experts)) return fail(MOE_EINVAL, "expert cache and experts must be non-NULL%s%lld");
  moe_cache* c = cache;
  if (layer < 0 || layer >= c->n_layers) return fail(MOE_EINVAL, "expert cache: layer outside the cache%s (%lld)", "", layer);
  std::vector<int64_t> keys;
  for (int i = 0; i < n; ++i) {
    if (experts[i] < 0 || experts[i] >= c->cfg.n_routed)
      return fail(MOE_EINVAL, "expert cache: expert outside 0..n_routed%s (%lld)", "", experts[i]);
    keys.push_back((int64_t)layer * c->cfg.n_routed + experts[i]);
  }
  const hipStream_t s = (hipStream_t)stream;
  std::vector<SlotLru::Change> changes;
  const uint64_t ep = c->lru.begin();
  // on the caller's stream: ordered after every kernel enqueued there before
  if (int r = fetch(c, keys, ep, true, s, changes)) return r;
  return upload_rows(c, changes, s);
}

int moe_cache_get_stats(const moe_cache* cache, moe_cache_stats* out) {
  if (!cache || !out) return fail(MOE_EINVAL, "expert cache and out must be non-NULL%s%lld");
  *out = cache->stats;
  return MOE_OK;
}

int moe_cache_resident(const moe_cache* cache, int32_t layer, int32_t* slots) {
  if (!cache || !slots) return fail(MOE_EINVAL, "expert cache and slots must be non-NULL%s%lld");
  if (layer < 0 || layer >= cache->n_layers)
    return fail(MOE_EINVAL, "expert cache: layer outside the cache%s (%lld)", "", layer);
  std::memcpy(slots, cache->lru.table() + (int64_t)layer * cache->cfg.n_routed, (size_t)cache->cfg.n_routed * 4);
  return MOE_OK;
}

static int moe_lru_simulate_body(int32_t n_slots, int64_t n_keys, const int64_t* keys, const int32_t* batch_len,
                                 int32_t n_batches, int32_t* slots_out, int32_t* miss_out) {
  if (n_slots < 1 || n_keys < 1 || n_batches < 0 || (n_batches > 0 && (!keys || !batch_len || !slots_out || !miss_out)))
    return fail(MOE_EINVAL, "bad LRU simulation arguments%s%lld");
  SlotLru lru(n_slots, n_keys);
  std::vector<SlotLru::Change> changes;
  int64_t q = 0;
  for (int b = 0; b < n_batches; ++b) {
    const int nb = batch_len[b];
    if (nb < 0) return fail(MOE_EINVAL, "LRU simulation: negative batch length%s%lld");
    for (int i = 0; i < nb; ++i)
      if (keys[q + i] < 0 || keys[q + i] >= n_keys)
        return fail(MOE_EINVAL, "LRU simulation: key out of range%s (%lld)", "", keys[q + i]);
    std::vector<int32_t> sl(nb, -1);
    std::vector<char> ms(nb, 0);
    lru.acquire_batch(keys + q, nb, lru.begin(), sl.data(), ms.data(), changes);
    for (int i = 0; i < nb; ++i, ++q) {
      slots_out[q] = sl[i];
      miss_out[q] = ms[i];
    }
  }
  return MOE_OK;
}

int moe_cache_create(const moe_cfg* cfg, int32_t n_layers, const void* const* host_experts, uint64_t stride,
                     uint64_t gate_off, uint64_t up_off, uint64_t down_off, int32_t n_slots, int32_t max_m,
                     moe_cache** out) {
  return guarded([&] {
    return moe_cache_create_body(cfg, n_layers, host_experts, stride, gate_off, up_off, down_off, n_slots, max_m,
                                 out);
  });
}

int moe_cache_forward(moe_cache* cache, const moe_cfg* cfg, const moe_layer* layers, int32_t first_layer,
                      int32_t n_layers, uint16_t* xs, int32_t m, float* out_f32, int32_t* headers, int32_t prefetch_k,
                      void* ws, size_t ws_bytes, void* stream) {
  return guarded([&] {
    return moe_cache_forward_body(cache, cfg, layers, first_layer, n_layers, xs, m, out_f32, headers, prefetch_k, ws,
                                  ws_bytes, stream);
  });
}

int moe_cache_prefetch(moe_cache* cache, int32_t layer, const int32_t* experts, int32_t n, void* stream) {
  return guarded([&] { return moe_cache_prefetch_body(cache, layer, experts, n, stream); });
}

int moe_lru_simulate(int32_t n_slots, int64_t n_keys, const int64_t* keys, const int32_t* batch_len,
                     int32_t n_batches, int32_t* slots_out, int32_t* miss_out) {
  return guarded([&] {
    return moe_lru_simulate_body(n_slots, n_keys, keys, batch_len, n_batches, slots_out, miss_out);
  });
}

}  // extern "C"
