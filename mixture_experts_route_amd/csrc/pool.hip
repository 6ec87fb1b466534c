// Host service of a per-layer expert-slot pool (decode path).
//
// Betelgeuse news article, section "mechanism: VRAM expert-slot pool, in-stream doorbell and
// victim cache": each layer keeps a fixed number of HBM slots; the GPU-side check finds the
// misses and rings the host only then; a miss is filled from host memory, and the HBM and host
// copies of an expert are exclusive (the expert a fill displaces moves to the host).  The policy
// is unnamed there; this service uses least-recently-used over slots not selected in the step,
// ties to the lower slot, misses placed in ascending id order (the oracle's SlotPoolLRU).
//
// One call of the layer with this pool:
//   moe_pool_arm      -> the doorbell for the next call (epoch + 1);
//   moe_layer_forward -> enqueues route + check (the check kernel writes the miss list, the
//                        step's selections and the epoch into host-mapped memory; with no miss it
//                        also writes *ready = epoch), a stream wait on *ready >= epoch, the FFNs;
//   moe_pool_serve    -> polls the epoch, places the misses, and per miss enqueues one
//                        device->host copy of the victim into a spare host buffer (on the d2h
//                        stream) and one host->device copy of the missing expert into the victim's
//                        slot (on the h2d stream, after that slot's device->host copy), then on the
//                        h2d stream the updated slot table and *ready = epoch.  The spare buffer
//                        and the filled expert's old host buffer trade places (the exclusive
//                        swap); with several spares (a FIFO) and two streams the victims' copies
//                        out and the misses' copies in overlap on the two PCIe directions.
// The FFN kernels read the slot of a missed expert from the table when they run, after the wait.
#include <algorithm>
#include <atomic>
#include <cstdio>
#include <chrono>
#include <cstring>
#include <deque>
#include <new>
#include <thread>
#include <utility>
#include <vector>

#include "kernels.hpp"

namespace moe {
__global__ void k_set_error_bits(int32_t* ctrl, int bits) {
  if (threadIdx.x == 0) atomicOr(&ctrl[kCtrlError], bits);
}
}  // namespace moe

using namespace moe;

struct moe_pool {
  int E = 0, k = 0;
  int64_t blob_bytes = 0, stride = 0;
  int n_slots = 0;
  uint8_t* arena = nullptr;
  int32_t* table_dev = nullptr;
  int32_t* table_host = nullptr;  // pinned mirror, copied to table_dev after fills
  std::vector<int32_t> holder;    // expert in each slot
  std::vector<int64_t> last_use;  // recency stamp of each slot
  int64_t clock = 0;
  std::vector<uint8_t*> home;     // pinned host blob of every expert not in a slot
  // pinned host blobs holding no expert, oldest first, each with the ring event (or -1) of the
  // host->device copy that last read it (a device->host copy into it waits for that event)
  std::deque<std::pair<uint8_t*, int>> spares;
  std::vector<hipEvent_t> ev_ring;  // n_spares + 1 events, used round robin
  int ev_next = 0;
  hipEvent_t ev_d2h = nullptr;      // a miss's device->host copy (its slot's host->device copy waits)
  hipEvent_t ev_end = nullptr;      // the h2d stream after a serve's copies (the next serve's d2h waits)
  bool ev_end_set = false;
  int32_t* host_miss_ids = nullptr;
  int32_t* host_counts = nullptr;
  int32_t* host_step_ids = nullptr;
  uint32_t* ready = nullptr;
  uint32_t epoch = 0;
  bool armed = false;
  moe_pool_stats stats{};
  std::vector<int64_t> profile;   // selections seen per expert (hits and misses)
  int lent = 0;                   // slots n_slots - lent .. n_slots - 1 are lent out
  uint8_t* lent_bufs = nullptr;   // their experts' host copies while lent
  int fail_after = -1;            // test hook: copy enqueues that succeed before one is failed
};

// A copy enqueue of the pool, or the failure the test hook injects in its place.
static hipError_t pool_copy(moe_pool* p, void* dst, const void* src, size_t n, hipMemcpyKind kind, hipStream_t s) {
  if (p->fail_after == 0) return hipErrorInvalidValue;
  if (p->fail_after > 0) --p->fail_after;
  return hipMemcpyAsync(dst, src, n, kind, s);
}

static bool hip_ok(hipError_t e) { return e == hipSuccess; }

extern "C" {

static void destroy_events(moe_pool* p) {
  for (hipEvent_t e : p->ev_ring)
    if (e) (void)hipEventDestroy(e);
  p->ev_ring.clear();
  if (p->ev_d2h) (void)hipEventDestroy(p->ev_d2h);
  if (p->ev_end) (void)hipEventDestroy(p->ev_end);
  p->ev_d2h = p->ev_end = nullptr;
}

MOE_API int moe_pool_create(const moe_dims* dims, uint8_t* arena, int64_t slot_stride, int32_t n_slots, int32_t* table,
                            const int32_t* initial, uint8_t* const* host_home, uint8_t* spares, int32_t n_spares,
                            int32_t* host_miss_ids, int32_t* host_counts, int32_t* host_step_ids, uint32_t* ready,
                            moe_pool** pool_out) {
  if (!pool_out) return MOE_EINVAL;
  *pool_out = nullptr;
  const size_t blob = moe_expert_blob_bytes(dims);
  if (!blob) return MOE_EINVAL;
  if (!arena || !table || !initial || !host_home || !spares || n_spares < 1 || n_spares > MOE_POOL_MAX_SPARES ||
      !host_miss_ids || !host_counts || !host_step_ids || !ready)
    return MOE_EINVAL;
  if (n_slots < 1 || n_slots > dims->n_experts || slot_stride < (int64_t)blob || slot_stride % 4096) return MOE_EINVAL;
  const int E = dims->n_experts;
  std::vector<int32_t> tab(E, -1);
  for (int s = 0; s < n_slots; ++s) {
    const int e = initial[s];
    if (e < 0 || e >= E || tab[e] >= 0) return MOE_EINVAL;  // each slot holds a distinct expert
    tab[e] = s;
  }
  for (int e = 0; e < E; ++e)
    if ((tab[e] < 0) != (host_home[e] != nullptr)) return MOE_EINVAL;  // exactly one home per expert
  moe_pool* p = new (std::nothrow) moe_pool();
  if (!p) return MOE_EINVAL;
  p->E = E;
  p->k = dims->top_k;
  p->blob_bytes = (int64_t)blob;
  p->stride = slot_stride;
  p->n_slots = n_slots;
  p->arena = arena;
  p->table_dev = table;
  p->holder.assign(initial, initial + n_slots);
  p->last_use.resize(n_slots);
  for (int s = 0; s < n_slots; ++s) p->last_use[s] = -(int64_t)(s + 1);  // hottest first: colder evicted first
  p->home.assign(host_home, host_home + E);
  p->profile.assign(E, 0);
  for (int i = 0; i < n_spares; ++i) p->spares.emplace_back(spares + (int64_t)i * slot_stride, -1);
  p->ev_ring.assign(n_spares + 1, nullptr);
  bool ev_ok = true;
  for (hipEvent_t& e : p->ev_ring) ev_ok = ev_ok && hip_ok(hipEventCreateWithFlags(&e, hipEventDisableTiming));
  ev_ok = ev_ok && hip_ok(hipEventCreateWithFlags(&p->ev_d2h, hipEventDisableTiming)) &&
          hip_ok(hipEventCreateWithFlags(&p->ev_end, hipEventDisableTiming));
  if (!ev_ok) {
    destroy_events(p);
    delete p;
    return MOE_EHIP;
  }
  p->host_miss_ids = host_miss_ids;
  p->host_counts = host_counts;
  p->host_step_ids = host_step_ids;
  p->ready = ready;
  if (!hip_ok(hipHostMalloc((void**)&p->table_host, sizeof(int32_t) * E, hipHostMallocDefault))) {
    destroy_events(p);
    delete p;
    return MOE_EHIP;
  }
  std::memcpy(p->table_host, tab.data(), sizeof(int32_t) * E);
  const uint32_t zero = 0;
  if (!hip_ok(hipMemcpy(table, p->table_host, sizeof(int32_t) * E, hipMemcpyHostToDevice)) ||
      !hip_ok(hipMemcpy(ready, &zero, sizeof(zero), hipMemcpyHostToDevice))) {
    (void)hipHostFree(p->table_host);
    destroy_events(p);
    delete p;
    return MOE_EHIP;
  }
  host_counts[1] = 0;
  *pool_out = p;
  return MOE_OK;
}

MOE_API int moe_pool_destroy(moe_pool* pool) {
  if (!pool) return MOE_EINVAL;
  (void)hipHostFree(pool->table_host);
  destroy_events(pool);
  delete pool;
  return MOE_OK;
}

MOE_API int moe_pool_arm(moe_pool* pool, moe_doorbell* bell_out) {
  if (!pool || !bell_out) return MOE_EINVAL;
  if (pool->armed) return MOE_EINVAL;  // the previous call was not served
  if (pool->lent) return MOE_EINVAL;   // slots are lent out: return them first
  pool->epoch += 1;
  pool->armed = true;
  bell_out->host_miss_ids = pool->host_miss_ids;
  bell_out->host_miss_count = pool->host_counts;
  bell_out->ready = pool->ready;
  bell_out->epoch = pool->epoch;
  bell_out->host_step_ids = pool->host_step_ids;
  return MOE_OK;
}

// Releases the waiting stream with the fill error flagged (and the table as it stands); the reason
// goes to stderr (the return code is the same for every reason).
static int release_with_error(moe_pool* p, void* ws, hipStream_t cs, const char* why, long v0 = 0, long v1 = 0) {
  fprintf(stderr, "moe_pool_serve: epoch %u: %s (%ld, %ld)\n", p->epoch, why, v0, v1);
  if (ws) k_set_error_bits<<<1, 64, 0, cs>>>((int32_t*)ws, MOE_DERR_FILL);
  (void)hipStreamWriteValue32(cs, p->ready, p->epoch, 0);
  // the copies already enqueued on `cs` still order the next serve's device->host copies
  p->ev_end_set = hip_ok(hipEventRecord(p->ev_end, cs));
  if (!p->ev_end_set) (void)hipStreamSynchronize(cs);
  p->armed = false;
  return MOE_EFILL;
}

MOE_API int moe_pool_serve(moe_pool* pool, void* ws_or_null, void* d2h_stream, void* h2d_stream_or_null,
                           int32_t* fills_out, int32_t* n_fills_out, int64_t timeout_us) {
  if (!pool || !pool->armed) return MOE_EINVAL;
  moe_pool* p = pool;
  hipStream_t sd = (hipStream_t)d2h_stream;
  hipStream_t cs = h2d_stream_or_null ? (hipStream_t)h2d_stream_or_null : sd;  // h2d stream: table, release
  const bool two = cs != sd;
  if (n_fills_out) *n_fills_out = 0;
  // wait for the check kernel's doorbell (the epoch is written after the lists)
  volatile int32_t* counts = p->host_counts;
  const auto t0 = std::chrono::steady_clock::now();
  while ((uint32_t)counts[1] != p->epoch) {
    if (timeout_us > 0 &&
        std::chrono::duration_cast<std::chrono::microseconds>(std::chrono::steady_clock::now() - t0).count() >
            timeout_us)
      return release_with_error(p, ws_or_null, cs,
                                "no doorbell before the timeout (precondition: the compute and copy streams were "
                                "created together before other streams, so no copy stream shares a hardware queue "
                                "with the compute stream's wait)",
                                (long)counts[1], (long)p->epoch);
    std::this_thread::yield();
  }
  std::atomic_thread_fence(std::memory_order_acquire);
  const int n_miss = counts[0];
  const int n_sel = counts[2];
  if (n_miss < 0 || n_miss > p->E || n_sel < 0 || n_sel > kMaxDecodeTok * kMaxK)
    return release_with_error(p, ws_or_null, cs, "counts out of range", n_miss, n_sel);
  std::vector<int32_t> miss(n_miss), sel(n_sel);
  for (int i = 0; i < n_miss; ++i) miss[i] = ((volatile int32_t*)p->host_miss_ids)[i];
  for (int i = 0; i < n_sel; ++i) sel[i] = ((volatile int32_t*)p->host_step_ids)[i];
  std::vector<char> selected(p->E, 0);
  for (int e : sel) {
    if (e < 0 || e >= p->E) return release_with_error(p, ws_or_null, cs, "selected id out of range", e, n_sel);
    selected[e] = 1;
  }
  int n_fills = 0;
  // the victims of this serve may be slots the previous serve filled (its h2d stream ends at ev_end)
  if (n_miss > 0 && p->ev_end_set && !hip_ok(hipStreamWaitEvent(sd, p->ev_end, 0)))
    return release_with_error(p, ws_or_null, cs, "copy enqueue failed", -1, -1);
  for (int e : miss) {
    if (e < 0 || e >= p->E || p->table_host[e] >= 0 || !p->home[e])
      return release_with_error(p, ws_or_null, cs, "miss id not away", e, (e >= 0 && e < p->E) ? p->table_host[e] : -9);
    selected[e] = 1;
    // victim: the least recently used slot whose expert is not selected in this step
    int best = -1;
    for (int s = 0; s < p->n_slots; ++s) {
      if (selected[p->holder[s]]) continue;
      if (best < 0 || p->last_use[s] < p->last_use[best]) best = s;
    }
    if (best < 0) return release_with_error(p, ws_or_null, cs, "no victim slot", n_miss, n_sel);
    const int old = p->holder[best];
    uint8_t* slot = p->arena + (int64_t)best * p->stride;
    // exclusive swap: the victim goes to the oldest spare host buffer, the missing expert to the
    // slot (after the victim's copy out); the expert's old host buffer becomes the newest spare
    const auto [buf, buf_ev] = p->spares.front();
    bool ok = !two || buf_ev < 0 || hip_ok(hipStreamWaitEvent(sd, p->ev_ring[buf_ev], 0));
    ok = ok && hip_ok(pool_copy(p, buf, slot, p->blob_bytes, hipMemcpyDeviceToHost, sd));
    if (two) ok = ok && hip_ok(hipEventRecord(p->ev_d2h, sd)) && hip_ok(hipStreamWaitEvent(cs, p->ev_d2h, 0));
    ok = ok && hip_ok(pool_copy(p, slot, p->home[e], p->blob_bytes, hipMemcpyHostToDevice, cs));
    // nothing was placed if an enqueue failed: the slot still holds the victim, the buffer stays spare
    if (!ok) return release_with_error(p, ws_or_null, cs, "copy enqueue failed", e, best);
    int read_ev = -1;
    if (two) {
      read_ev = p->ev_next;
      p->ev_next = (p->ev_next + 1) % (int)p->ev_ring.size();
      // without the event the buffer is guarded by draining the h2d stream
      if (!hip_ok(hipEventRecord(p->ev_ring[read_ev], cs))) {
        read_ev = -1;
        ok = hip_ok(hipStreamSynchronize(cs));
      }
    }
    p->spares.pop_front();
    p->spares.emplace_back(p->home[e], read_ev);
    p->home[old] = buf;
    p->home[e] = nullptr;
    p->table_host[old] = -1;
    p->table_host[e] = best;
    p->holder[best] = e;
    if (!ok) return release_with_error(p, ws_or_null, cs, "event record failed", e, best);
    if (fills_out) {
      fills_out[3 * n_fills + 0] = e;
      fills_out[3 * n_fills + 1] = best;
      fills_out[3 * n_fills + 2] = old;
    }
    ++n_fills;
    p->stats.bytes_h2d += p->blob_bytes;
    p->stats.bytes_d2h += p->blob_bytes;
  }
  if (n_miss > 0) {
    if (!hip_ok(hipMemcpyAsync(p->table_dev, p->table_host, sizeof(int32_t) * p->E, hipMemcpyHostToDevice, cs)) ||
        !hip_ok(hipStreamWriteValue32(cs, p->ready, p->epoch, 0)))
      return release_with_error(p, ws_or_null, cs, "table copy or release enqueue failed");
    if (!hip_ok(hipEventRecord(p->ev_end, cs))) return release_with_error(p, ws_or_null, cs, "event record failed");
    p->ev_end_set = true;
  }
  // recency: every selection of the step, in (token, choice) order; the profile counts them
  for (int e : sel) {
    p->last_use[p->table_host[e]] = ++p->clock;
    ++p->profile[e];
  }
  if (n_sel == 0)
    for (int i = 0; i < n_miss; ++i) p->last_use[p->table_host[miss[i]]] = ++p->clock;
  p->stats.calls += 1;
  p->stats.selections += n_sel;
  p->stats.misses += n_miss;
  if (n_fills_out) *n_fills_out = n_fills;
  p->armed = false;
  return MOE_OK;
}

MOE_API int moe_pool_get_stats(const moe_pool* pool, moe_pool_stats* out) {
  if (!pool || !out) return MOE_EINVAL;
  *out = pool->stats;
  return MOE_OK;
}

MOE_API int moe_pool_get_table(const moe_pool* pool, int32_t* table_out) {
  if (!pool || !table_out) return MOE_EINVAL;
  std::memcpy(table_out, pool->table_host, sizeof(int32_t) * pool->E);
  return MOE_OK;
}

MOE_API int moe_pool_get_profile(const moe_pool* pool, int64_t* counts_out) {
  if (!pool || !counts_out) return MOE_EINVAL;
  std::memcpy(counts_out, pool->profile.data(), sizeof(int64_t) * pool->E);
  return MOE_OK;
}

MOE_API int moe_profile_seed(const int64_t* counts, int32_t n_experts, int32_t n_slots, int32_t* initial_out) {
  if (!counts || !initial_out || n_experts < 1 || n_slots < 1 || n_slots > n_experts) return MOE_EINVAL;
  std::vector<int32_t> order(n_experts);
  for (int e = 0; e < n_experts; ++e) order[e] = e;
  // hottest first: more selections first, the lower id first among equal counts
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return counts[a] > counts[b]; });
  std::memcpy(initial_out, order.data(), sizeof(int32_t) * n_slots);
  return MOE_OK;
}

MOE_API int moe_pool_lend(moe_pool* pool, int32_t n, uint8_t* host_bufs, void* stream, uint8_t** region_out) {
  if (!pool || !host_bufs || !region_out || n < 1 || n > pool->n_slots) return MOE_EINVAL;
  moe_pool* p = pool;
  if (p->armed || p->lent) return MOE_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  const int first = p->n_slots - n;
  // the last serve's copies into these slots come first
  if (p->ev_end_set && !hip_ok(hipStreamWaitEvent(st, p->ev_end, 0))) return MOE_EHIP;
  for (int i = 0; i < n; ++i) {
    const int s = first + i;
    if (!hip_ok(pool_copy(p, host_bufs + (int64_t)i * p->stride, p->arena + (int64_t)s * p->stride, p->blob_bytes,
                          hipMemcpyDeviceToHost, st))) {
      (void)hipStreamSynchronize(st);  // nothing changed hands: the slots keep their experts
      return MOE_EFILL;
    }
  }
  for (int i = 0; i < n; ++i) {
    const int e = p->holder[first + i];
    p->table_host[e] = -1;
    p->home[e] = host_bufs + (int64_t)i * p->stride;
  }
  if (!hip_ok(hipMemcpyAsync(p->table_dev, p->table_host, sizeof(int32_t) * p->E, hipMemcpyHostToDevice, st)))
    return MOE_EHIP;
  p->lent = n;
  p->lent_bufs = host_bufs;
  *region_out = p->arena + (int64_t)first * p->stride;
  return MOE_OK;
}

MOE_API int moe_pool_unlend(moe_pool* pool, void* stream) {
  if (!pool || !pool->lent) return MOE_EINVAL;
  moe_pool* p = pool;
  hipStream_t st = (hipStream_t)stream;
  const int n = p->lent, first = p->n_slots - n;
  for (int i = 0; i < n; ++i) {
    const int s = first + i;
    if (!hip_ok(pool_copy(p, p->arena + (int64_t)s * p->stride, p->lent_bufs + (int64_t)i * p->stride, p->blob_bytes,
                          hipMemcpyHostToDevice, st)))
      return MOE_EFILL;  // still lent: the call can be repeated
  }
  for (int i = 0; i < n; ++i) {
    const int e = p->holder[first + i];
    p->table_host[e] = first + i;
    p->home[e] = nullptr;
  }
  if (!hip_ok(hipMemcpyAsync(p->table_dev, p->table_host, sizeof(int32_t) * p->E, hipMemcpyHostToDevice, st)))
    return MOE_EHIP;
  // the next serve's copies out of these slots wait for the restore
  p->ev_end_set = hip_ok(hipEventRecord(p->ev_end, st));
  if (!p->ev_end_set) (void)hipStreamSynchronize(st);
  p->lent = 0;
  p->lent_bufs = nullptr;
  return MOE_OK;
}

MOE_API int moe_pool_debug_fail_copies(moe_pool* pool, int32_t after_n) {
  if (!pool) return MOE_EINVAL;
  pool->fail_after = after_n < 0 ? -1 : after_n;
  return MOE_OK;
}

}  // extern "C"
