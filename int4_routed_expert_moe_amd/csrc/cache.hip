// Expert cache in HBM for models whose experts do not all fit on the GPU.
//
// "Show HN: 遅いコンピュータで GLM 5.2 を実行する", section ディスクストリーミング
// ベースの MoE 実行方式: experts are loaded on demand through a per-layer LRU
// cache with an optional pinned hot store; section Learning cache とハードウェア
// 別の期待値: the experts routed in real use are recorded and the hottest ones
// are pinned at start-up.  On this machine the cold tier is pinned host
// memory and the cache is a set of record slots in HBM:
//
//   - moe_layer_ptrs reads each routed expert through a device table of
//     record pointers; an entry points at an HBM slot (hit) or at the
//     record in pinned host memory, which the kernels then stream over the
//     host link (miss).  A step never waits for the host.
//   - After each layer call, moe_cache_step copies that call's idx to pinned
//     memory (event-ordered on the caller's stream) and, once it has landed,
//     counts hits and misses against the table as that call saw it, and
//     promotes missed experts into LRU slots: the victim's entry is turned
//     back to host memory on the caller's stream first, the record copy runs
//     on the device's copy stream after that, and the new entry is
//     written on the caller's stream once the copy has completed.  So no
//     kernel ever reads a slot that is being overwritten, and the caller's
//     stream never waits for a copy.
//   - Slots [0, n_pinned) hold the experts with the largest recorded usage
//     (the learning cache's pinning), loaded at creation; the others are LRU.
//   - Routing one layer ahead ("Comment exécuter un réseau de neurones de 744
//     milliards de paramètres...", section "Comment fonctionne le moteur",
//     step 1: a prefetch thread routes the next layer early, a prediction
//     right about 71 % of the time, so that its reads overlap compute):
//     moe_cache_prefetch takes a predicted idx for this cache's layer (the
//     caller routes it with this layer's router on the previous layer's
//     input) and starts promotions of the predicted experts at once, so their
//     copies run while the previous layer computes; moe_cache_publish, just
//     before this layer's call, makes the caller's stream wait for the
//     copies still in flight and points their entries at the slots.  A
//     wrong prediction costs a copy and an LRU slot, never a result: the
//     layer reads whatever the table points at.
//
// The policy (Policy below) is plain host code, also run by
// moe_cache_simulate for tests without a GPU.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <vector>

#include "kernels.h"

// read-backs outstanding before moe_cache_step waits: promotions are decided
// when a read-back lands and their copies queue behind the layer calls
// already enqueued, so a host far ahead of the GPU promotes too late (a
// 4-layer stack at 192 of 256 slots: 15 % hits with 32, 63 % with 4; 2 is
// no better than 4, which still keeps several calls queued)
#ifndef MOE_CACHE_RING
#define MOE_CACHE_RING 4
#endif

namespace moe {

// ------------------------------------------------------------------ policy

struct Promotion {
  int expert, slot, evicted;  // evicted: previous occupant (-1: the slot was empty)
};

struct Policy {
  int E = 0, S = 0, P = 0, max_promote = 0;
  std::vector<int> slot_of;     // [E] slot holding the expert, -1 (host)
  std::vector<int> expert_in;   // [S] occupant (resident or being copied), -1 empty
  std::vector<char> pending;    // [S] copy in flight
  std::vector<uint64_t> last_use;  // [S] last step that hit (or claimed) the slot
  std::vector<uint64_t> usage;     // [E] steps that routed the expert
  uint64_t step = 0;
  moe_cache_stats st{};

  void init(int E_, int S_, int P_, int max_promote_) {
    E = E_, S = S_, P = P_, max_promote = max_promote_;
    slot_of.assign(E, -1);
    expert_in.assign(S, -1);
    pending.assign(S, 0);
    last_use.assign(S, 0);
    usage.assign(E, 0);
    step = 0;
    st = moe_cache_stats{};
  }

  // The pinned hot store: the P experts with the largest recorded usage
  // (ties: lower id; experts never used are not pinned).
  std::vector<int> pin_order(const uint64_t *recorded) const {
    std::vector<int> ids;
    if (!recorded) return ids;
    for (int e = 0; e < E; e++)
      if (recorded[e] > 0) ids.push_back(e);
    std::stable_sort(ids.begin(), ids.end(),
                     [&](int a, int b) { return recorded[a] > recorded[b]; });
    if ((int)ids.size() > P) ids.resize(P);
    return ids;
  }

  void place(int e, int s) {  // a resident expert (pinned at start-up)
    slot_of[e] = s;
    expert_in[s] = e;
  }

  // LRU victim among the unpinned slots that are not being copied (nor
  // marked in keep): an empty one first (lowest index), else the least
  // recently used (ties: lower).
  int victim(const std::vector<char> *keep = nullptr) const {
    int best = -1;
    for (int s = P; s < S; s++) {
      if (pending[s] || (keep && (*keep)[s])) continue;
      if (expert_in[s] < 0) return s;
      if (best < 0 || last_use[s] < last_use[best]) best = s;
    }
    return best;
  }

  // One step's routed experts (idx entries, any order, -1 = dropped) against
  // the residency the step saw (resident[e] != 0: read from HBM).  Updates
  // usage, LRU times and counters; appends the promotions to start.
  void account(const int32_t *idx, int n, const std::vector<char> &resident,
               std::vector<Promotion> &out) {
    step++;
    std::vector<int> U;
    for (int i = 0; i < n; i++)
      if (idx[i] >= 0 && idx[i] < E) U.push_back(idx[i]);
    std::sort(U.begin(), U.end());
    U.erase(std::unique(U.begin(), U.end()), U.end());
    st.steps++;
    // first every routed expert's count and LRU time, so that no promotion
    // below evicts an expert this step used while an older one stays
    for (int e : U) {
      usage[e]++;
      st.routed++;
      if (resident[e]) {
        st.hits++;
      } else {
        st.misses++;
      }
      if (slot_of[e] >= 0) last_use[slot_of[e]] = step;  // resident now
    }
    int promoted = 0;
    for (int e : U) {
      if (slot_of[e] >= 0) continue;
      bool in_flight = false;
      for (int t = 0; t < S; t++) in_flight |= (pending[t] && expert_in[t] == e);
      if (in_flight || promoted >= max_promote) continue;
      const int v = victim();
      if (v < 0) continue;
      const int old = expert_in[v];
      if (old >= 0) slot_of[old] = -1;
      expert_in[v] = e;
      pending[v] = 1;
      last_use[v] = step;
      out.push_back(Promotion{e, v, old});
      promoted++;
      st.promotions++;
    }
  }

  // Predicted experts of the layer's next call (any order, -1 skipped):
  // resident ones are marked used now and are no victims of this prefetch;
  // the others that are not being copied take LRU victims, at most
  // max_promote.  No usage or hit counts: the call has not happened.
  void prefetch(const int32_t *idx, int n, std::vector<Promotion> &out) {
    std::vector<int> U;
    for (int i = 0; i < n; i++)
      if (idx[i] >= 0 && idx[i] < E) U.push_back(idx[i]);
    std::sort(U.begin(), U.end());
    U.erase(std::unique(U.begin(), U.end()), U.end());
    std::vector<char> keep(S, 0);
    for (int e : U)
      if (slot_of[e] >= 0) {
        last_use[slot_of[e]] = step;
        keep[slot_of[e]] = 1;
      }
    int promoted = 0;
    for (int e : U) {
      if (slot_of[e] >= 0) continue;
      bool in_flight = false;
      for (int t = 0; t < S; t++) in_flight |= (pending[t] && expert_in[t] == e);
      if (in_flight || promoted >= max_promote) continue;
      const int v = victim(&keep);
      if (v < 0) continue;
      const int old = expert_in[v];
      if (old >= 0) slot_of[old] = -1;
      expert_in[v] = e;
      pending[v] = 1;
      last_use[v] = step;
      out.push_back(Promotion{e, v, old});
      promoted++;
      st.promotions++;
      st.prefetched++;
    }
  }

  void complete(int s) {  // the copy into slot s has landed
    pending[s] = 0;
    slot_of[expert_in[s]] = s;
    st.completed++;
  }

  std::vector<char> residency() const {
    std::vector<char> r(E, 0);
    for (int e = 0; e < E; e++) r[e] = slot_of[e] >= 0;
    return r;
  }
};

// ------------------------------------------------------------------ device side

struct PtrUpdates {
  static constexpr int N = 16;
  int n;
  int idx[N];
  const void *ptr[N];
};

__global__ void k_set_ptrs(const void **table, PtrUpdates u) {
  const int i = threadIdx.x;
  if (i < u.n) table[u.idx[i]] = u.ptr[i];
}

static hipError_t set_ptrs(const void **table, const std::vector<std::pair<int, const void *>> &v,
                           hipStream_t st) {
  for (size_t b = 0; b < v.size(); b += PtrUpdates::N) {
    PtrUpdates u{};
    u.n = (int)std::min<size_t>(PtrUpdates::N, v.size() - b);
    for (int i = 0; i < u.n; i++) {
      u.idx[i] = v[b + i].first;
      u.ptr[i] = v[b + i].second;
    }
    hipLaunchKernelGGL(k_set_ptrs, dim3(1), dim3(64), 0, st, table, u);
  }
  return hipGetLastError();
}

}  // namespace moe

struct moe_cache {
  moe::Policy pol;
  size_t blob_bytes = 0;
  int max_pairs = 0;
  std::vector<const void *> host;  // [E] device-readable records in host memory
  uint8_t *slots = nullptr;        // [S][blob_bytes] in HBM
  const void **table = nullptr;    // [E] device table of record pointers
  hipStream_t copy = nullptr;  // the device's copy stream (shared, not owned)
  // idx read-back ring: the host waits once R read-backs are outstanding
  static constexpr int R = MOE_CACHE_RING;
  int32_t *ring = nullptr;  // pinned [R][max_pairs]
  hipEvent_t ring_ev[R] = {};
  int ring_n[R] = {};
  std::vector<char> ring_res[R];
  uint64_t head = 0, tail = 0;  // entries [tail, head) are in flight
  int32_t *pred = nullptr;      // pinned [max_pairs]: a predicted idx read back
  hipEvent_t pred_ev = nullptr;
  struct Copy {
    int slot;
    hipEvent_t after_table, done;
    bool published;  // entry already written on a stream that waited for the copy
  };
  std::vector<Copy> copies;
};

namespace {

int hip_fail(const char *what, hipError_t e) {
  char buf[256];
  snprintf(buf, sizeof(buf), "%s: %s", what, hipGetErrorString(e));
  return moe::set_error(MOE_EHIP, buf);
}

// Promotions decided for one read-back step: victims' entries back to host
// memory on the caller's stream, then each record copy on the copy stream
// after an event that follows those entries (and every earlier kernel).
int start_promotions(moe_cache *c, const std::vector<moe::Promotion> &pr, hipStream_t st) {
  if (pr.empty()) return MOE_OK;
  std::vector<std::pair<int, const void *>> back;
  for (const auto &p : pr)
    if (p.evicted >= 0) back.push_back({p.evicted, c->host[p.evicted]});
  hipError_t e = moe::set_ptrs(c->table, back, st);
  if (e != hipSuccess) return hip_fail("moe_cache_step (table)", e);
  for (const auto &p : pr) {
    moe_cache::Copy cp{p.slot, nullptr, nullptr, false};
    if ((e = hipEventCreateWithFlags(&cp.after_table, hipEventDisableTiming)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&cp.done, hipEventDisableTiming)) != hipSuccess ||
        (e = hipEventRecord(cp.after_table, st)) != hipSuccess ||
        (e = hipStreamWaitEvent(c->copy, cp.after_table, 0)) != hipSuccess ||
        (e = hipMemcpyAsync(c->slots + (size_t)p.slot * c->blob_bytes, c->host[p.expert],
                            c->blob_bytes, hipMemcpyHostToDevice, c->copy)) != hipSuccess ||
        (e = hipEventRecord(cp.done, c->copy)) != hipSuccess)
      return hip_fail("moe_cache_step (copy)", e);
    c->copies.push_back(cp);
    c->pol.st.bytes_copied += c->blob_bytes;
  }
  return MOE_OK;
}

// Copies that have landed (all of them when wait): their experts' entries
// now point at the slots, written on the caller's stream.
int finish_copies(moe_cache *c, bool wait, hipStream_t st) {
  std::vector<std::pair<int, const void *>> upd;
  std::vector<moe_cache::Copy> keep;
  for (const auto &cp : c->copies) {
    hipError_t e = wait ? hipEventSynchronize(cp.done) : hipEventQuery(cp.done);
    if (e == hipErrorNotReady) {
      keep.push_back(cp);
      continue;
    }
    if (e != hipSuccess) return hip_fail("moe_cache_step (copy event)", e);
    if (!cp.published) {
      c->pol.complete(cp.slot);
      upd.push_back({c->pol.expert_in[cp.slot], c->slots + (size_t)cp.slot * c->blob_bytes});
    }
    hipEventDestroy(cp.after_table);
    hipEventDestroy(cp.done);
  }
  c->copies.swap(keep);
  hipError_t e = moe::set_ptrs(c->table, upd, st);
  return e == hipSuccess ? MOE_OK : hip_fail("moe_cache_step (table)", e);
}

// Read-back entries whose idx has landed (the oldest one at least when
// force, all of them when wait), in step order.
int drain(moe_cache *c, bool force, bool wait, hipStream_t st) {
  while (c->tail < c->head) {
    const int r = (int)(c->tail % moe_cache::R);
    hipError_t e = (force || wait) ? hipEventSynchronize(c->ring_ev[r])
                                   : hipEventQuery(c->ring_ev[r]);
    if (e == hipErrorNotReady) break;
    if (e != hipSuccess) return hip_fail("moe_cache_step (idx event)", e);
    std::vector<moe::Promotion> pr;
    c->pol.account(c->ring + (size_t)r * c->max_pairs, c->ring_n[r], c->ring_res[r], pr);
    c->tail++;
    force = false;
    int rc = start_promotions(c, pr, st);
    if (rc) return rc;
  }
  return MOE_OK;
}

// One copy stream per device, shared by every cache on it and kept until the
// process ends: promotions of all layers go out in order over the one host
// link, and the process stays within a few hardware queues (with a stream
// per cache, eight layers' caches shared the compute stream's queue, and
// their copies waited behind every layer call already queued).
hipError_t device_copy_stream(hipStream_t *out) {
  static std::mutex mu;
  static std::map<int, hipStream_t> streams;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  auto it = streams.find(dev);
  if (it == streams.end()) {
    hipStream_t s = nullptr;
    if ((e = hipStreamCreate(&s)) != hipSuccess) return e;
    it = streams.emplace(dev, s).first;
  }
  *out = it->second;
  return hipSuccess;
}

// Every copy of this cache has landed (its slots may be freed after this).
void release(moe_cache *c) {
  for (auto &cp : c->copies) {
    hipEventSynchronize(cp.done);
    hipEventDestroy(cp.after_table);
    hipEventDestroy(cp.done);
  }
  for (int r = 0; r < moe_cache::R; r++)
    if (c->ring_ev[r]) hipEventDestroy(c->ring_ev[r]);
  if (c->ring) hipHostFree(c->ring);
  if (c->pred_ev) hipEventDestroy(c->pred_ev);
  if (c->pred) hipHostFree(c->pred);
  delete c;
}

}  // namespace

extern "C" {

int moe_host_device_ptr(const void *host, void **dev) {
  if (!host || !dev) return moe::set_error(MOE_EINVAL, "moe_host_device_ptr: NULL argument");
  hipError_t e = hipHostGetDevicePointer(dev, const_cast<void *>(host), 0);
  if (e != hipSuccess) return hip_fail("moe_host_device_ptr (not pinned host memory?)", e);
  return MOE_OK;
}

int moe_cache_create(const moe_cfg *cfg, int32_t n_slots, int32_t n_pinned, int32_t max_promote,
                     int32_t max_pairs, const void *const *host_records, void *slots,
                     void *table, const uint64_t *usage, void *stream, moe_cache **out) {
  (void)hipGetLastError();  // a failure reported below is then this call's own
  if (!out) return moe::set_error(MOE_EINVAL, "moe_cache_create: out is NULL");
  *out = nullptr;
  const size_t bb = moe_expert_blob_bytes(cfg);
  if (bb == 0) return MOE_EINVAL;  // message set by the cfg check
  const int E = cfg->n_experts;
  if (n_slots < 0 || n_pinned < 0 || n_pinned > n_slots || max_promote < 0 || max_pairs < 1)
    return moe::set_error(MOE_EINVAL,
                          "moe_cache_create: need 0 <= n_pinned <= n_slots, max_promote >= 0, "
                          "max_pairs >= 1");
  if (!host_records || !table || (n_slots > 0 && !slots))
    return moe::set_error(MOE_EINVAL, "moe_cache_create: NULL host_records, table or slots");
  if (((uintptr_t)slots % 256) || ((uintptr_t)table % 8))
    return moe::set_error(MOE_EALIGN, "moe_cache_create: slots 256-byte, table 8-byte aligned");
  for (int e = 0; e < E; e++)
    if (!host_records[e] || ((uintptr_t)host_records[e] % 256))
      return moe::set_error(MOE_EALIGN, "moe_cache_create: host record NULL or not 256-byte "
                                        "aligned");
  hipStream_t st = (hipStream_t)stream;
  moe_cache *c = new moe_cache();
  c->pol.init(E, n_slots, n_pinned, max_promote);
  c->blob_bytes = bb;
  c->max_pairs = max_pairs;
  c->host.assign(host_records, host_records + E);
  c->slots = static_cast<uint8_t *>(slots);
  c->table = static_cast<const void **>(table);
  hipError_t e;
  if ((e = device_copy_stream(&c->copy)) != hipSuccess) {
    release(c);
    return hip_fail("moe_cache_create (copy stream)", e);
  }
  if ((e = hipHostMalloc((void **)&c->ring, sizeof(int32_t) * moe_cache::R * max_pairs)) !=
      hipSuccess) {
    c->ring = nullptr;
    release(c);
    return hip_fail("moe_cache_create (pinned ring)", e);
  }
  for (int r = 0; r < moe_cache::R; r++)
    if ((e = hipEventCreateWithFlags(&c->ring_ev[r], hipEventDisableTiming)) != hipSuccess) {
      release(c);
      return hip_fail("moe_cache_create (events)", e);
    }
  if ((e = hipHostMalloc((void **)&c->pred, sizeof(int32_t) * max_pairs)) != hipSuccess) {
    c->pred = nullptr;
    release(c);
    return hip_fail("moe_cache_create (pinned prediction buffer)", e);
  }
  if ((e = hipEventCreateWithFlags(&c->pred_ev, hipEventDisableTiming)) != hipSuccess) {
    c->pred_ev = nullptr;
    release(c);
    return hip_fail("moe_cache_create (events)", e);
  }
  // every entry to host memory, then the pinned hot store
  std::vector<std::pair<int, const void *>> init;
  for (int x = 0; x < E; x++) init.push_back({x, c->host[x]});
  const std::vector<int> pin = c->pol.pin_order(usage);
  for (size_t i = 0; i < pin.size(); i++) {
    const int x = pin[i];
    if ((e = hipMemcpyAsync(c->slots + i * bb, c->host[x], bb, hipMemcpyHostToDevice, st)) !=
        hipSuccess) {
      release(c);
      return hip_fail("moe_cache_create (pin copy)", e);
    }
    c->pol.place(x, (int)i);
    init[x].second = c->slots + i * bb;
  }
  if ((e = moe::set_ptrs(c->table, init, st)) != hipSuccess ||
      (e = hipStreamSynchronize(st)) != hipSuccess) {
    release(c);
    return hip_fail("moe_cache_create (table)", e);
  }
  if (usage) c->pol.usage.assign(usage, usage + E);
  *out = c;
  return MOE_OK;
}

int moe_cache_step(moe_cache *c, const int32_t *idx, int32_t n, int32_t wait, void *stream) {
  (void)hipGetLastError();  // a failure reported below is then this call's own
  if (!c || !idx) return moe::set_error(MOE_EINVAL, "moe_cache_step: NULL argument");
  if (n < 0 || n > c->max_pairs)
    return moe::set_error(MOE_EINVAL, "moe_cache_step: n outside [0, max_pairs]");
  hipStream_t st = (hipStream_t)stream;
  int rc = MOE_OK;
  if (c->head - c->tail == (uint64_t)moe_cache::R && (rc = drain(c, true, false, st))) return rc;
  const int r = (int)(c->head % moe_cache::R);
  hipError_t e;
  if ((e = hipMemcpyAsync(c->ring + (size_t)r * c->max_pairs, idx, sizeof(int32_t) * n,
                          hipMemcpyDeviceToHost, st)) != hipSuccess ||
      (e = hipEventRecord(c->ring_ev[r], st)) != hipSuccess)
    return hip_fail("moe_cache_step (idx read-back)", e);
  c->ring_n[r] = n;
  c->ring_res[r] = c->pol.residency();  // what the call just enqueued reads
  c->head++;
  if ((rc = finish_copies(c, false, st))) return rc;
  if ((rc = drain(c, false, wait != 0, st))) return rc;
  if (wait && (rc = finish_copies(c, true, st))) return rc;
  return MOE_OK;
}

int moe_cache_prefetch(moe_cache *c, const int32_t *idx, int32_t n, void *stream) {
  (void)hipGetLastError();  // a failure reported below is then this call's own
  if (!c || (n > 0 && !idx)) return moe::set_error(MOE_EINVAL, "moe_cache_prefetch: NULL argument");
  if (n < 0 || n > c->max_pairs)
    return moe::set_error(MOE_EINVAL, "moe_cache_prefetch: n outside [0, max_pairs]");
  if (n == 0) return MOE_OK;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if ((e = hipMemcpyAsync(c->pred, idx, sizeof(int32_t) * n, hipMemcpyDeviceToHost, st)) !=
          hipSuccess ||
      (e = hipEventRecord(c->pred_ev, st)) != hipSuccess ||
      (e = hipEventSynchronize(c->pred_ev)) != hipSuccess)
    return hip_fail("moe_cache_prefetch (idx read-back)", e);
  int rc = finish_copies(c, false, st);  // landed copies free their slots' pending state
  if (rc) return rc;
  std::vector<moe::Promotion> pr;
  c->pol.prefetch(c->pred, n, pr);
  return start_promotions(c, pr, st);
}

int moe_cache_publish(moe_cache *c, void *stream) {
  (void)hipGetLastError();  // a failure reported below is then this call's own
  if (!c) return moe::set_error(MOE_EINVAL, "moe_cache_publish: NULL argument");
  hipStream_t st = (hipStream_t)stream;
  std::vector<std::pair<int, const void *>> upd;
  for (auto &cp : c->copies) {
    if (cp.published) continue;
    hipError_t e = hipStreamWaitEvent(st, cp.done, 0);
    if (e != hipSuccess) return hip_fail("moe_cache_publish (wait)", e);
    cp.published = true;
    c->pol.complete(cp.slot);
    upd.push_back({c->pol.expert_in[cp.slot], c->slots + (size_t)cp.slot * c->blob_bytes});
  }
  hipError_t e = moe::set_ptrs(c->table, upd, st);
  return e == hipSuccess ? MOE_OK : hip_fail("moe_cache_publish (table)", e);
}

int moe_cache_get_stats(const moe_cache *c, moe_cache_stats *s) {
  if (!c || !s) return moe::set_error(MOE_EINVAL, "moe_cache_get_stats: NULL argument");
  *s = c->pol.st;
  s->resident = 0;
  for (int x = 0; x < c->pol.E; x++) s->resident += c->pol.slot_of[x] >= 0;
  return MOE_OK;
}

int moe_cache_usage(const moe_cache *c, uint64_t *usage) {
  if (!c || !usage) return moe::set_error(MOE_EINVAL, "moe_cache_usage: NULL argument");
  std::copy(c->pol.usage.begin(), c->pol.usage.end(), usage);
  return MOE_OK;
}

int moe_cache_slot_of(const moe_cache *c, int32_t *slot_of) {
  if (!c || !slot_of) return moe::set_error(MOE_EINVAL, "moe_cache_slot_of: NULL argument");
  std::copy(c->pol.slot_of.begin(), c->pol.slot_of.end(), slot_of);
  return MOE_OK;
}

int moe_cache_destroy(moe_cache *c) {
  if (!c) return MOE_OK;
  release(c);
  return MOE_OK;
}

int moe_cache_simulate(int32_t n_experts, int32_t n_slots, int32_t n_pinned, int32_t max_promote,
                       const uint64_t *usage, const int32_t *idx, const int32_t *pred,
                       int32_t n_steps, int32_t n, int32_t *hits, int32_t *misses,
                       int32_t *slot_of) {
  if (n_experts < 1 || n_slots < 0 || n_pinned < 0 || n_pinned > n_slots || max_promote < 0 ||
      n_steps < 0 || n < 0 || (n_steps > 0 && !idx) || !hits || !misses || !slot_of)
    return moe::set_error(MOE_EINVAL, "moe_cache_simulate: bad argument");
  moe::Policy p;
  p.init(n_experts, n_slots, n_pinned, max_promote);
  const std::vector<int> pin = p.pin_order(usage);
  for (size_t i = 0; i < pin.size(); i++) p.place(pin[i], (int)i);
  if (usage) p.usage.assign(usage, usage + n_experts);
  for (int t = 0; t < n_steps; t++) {
    if (pred) {  // the step's prediction, its copies landed before the step
      std::vector<moe::Promotion> pp;
      p.prefetch(pred + (size_t)t * n, n, pp);
      for (const auto &x : pp) p.complete(x.slot);
    }
    const moe_cache_stats before = p.st;
    std::vector<moe::Promotion> pr;
    p.account(idx + (size_t)t * n, n, p.residency(), pr);
    for (const auto &x : pr) p.complete(x.slot);  // copies land before the next step
    hits[t] = (int32_t)(p.st.hits - before.hits);
    misses[t] = (int32_t)(p.st.misses - before.misses);
  }
  std::copy(p.slot_of.begin(), p.slot_of.end(), slot_of);
  return MOE_OK;
}

}  // extern "C"
