// Router, top-k selection and the in-stream residency check.
//
// Router and selection: Betelgeuse news article, section "mechanism" (each token takes 10 of
// 512 routed experts + 1 shared) and "what bit-exact means" (the top-10 is exact).
// Residency: same article, "mechanism" table, scheduling row (expert id -> HBM slot decided on
// the GPU in the stream; the host is rung only on a miss).
#include "kernels.hpp"
#include "select.hpp"

namespace moe {

template <int NPER>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, int T, int E, int k,
                                               int32_t* __restrict__ ids, float* __restrict__ w,
                                               int32_t* __restrict__ ctrl) {
  const int t = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (t >= T) return;
  select_topk_wave<NPER>(logits + (size_t)t * E, E, k, ids + (size_t)t * k, w + (size_t)t * k, ctrl);
}

// ------------------------------------------------------------------------------------------
// Block-wide exclusive scan of one int per thread (blockDim.x <= 1024, multiple of 64).
// ------------------------------------------------------------------------------------------
MOE_DEV int block_exclusive_scan(int v, int* lds_wave_sums, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, n_waves = blockDim.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) lds_wave_sums[wave] = incl;
  __syncthreads();
  int base = 0, tot = 0;
  for (int i = 0; i < n_waves; ++i) {
    const int s = lds_wave_sums[i];
    if (i < wave) base += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + incl - v;
}

// The same scan with DPP lane moves (no LDS crossbar round trips inside the wave): inclusive
// within each row of 16 by shifts of 1, 2, 4, 8, then rows 1 and 3 add lane 15 of the row
// before, rows 2 and 3 add lane 31.
MOE_DEV int block_exclusive_scan_dpp(int v, int* lds_wave_sums, int* total) {
  const int wave = threadIdx.x >> 6, n_waves = blockDim.x >> 6;
  int incl = v;
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x111, 0xF, 0xF, false);  // row_shr:1
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x112, 0xF, 0xF, false);  // row_shr:2
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x114, 0xF, 0xF, false);  // row_shr:4
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x118, 0xF, 0xF, false);  // row_shr:8
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x142, 0xA, 0xF, false);  // row_bcast:15
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x143, 0xC, 0xF, false);  // row_bcast:31
  const int wave_total = __builtin_amdgcn_readlane(incl, 63);
  if ((threadIdx.x & 63) == 0) lds_wave_sums[wave] = wave_total;
  __syncthreads();
  int base = 0, tot = 0;
  for (int i = 0; i < n_waves; ++i) {
    const int s = lds_wave_sums[i];
    if (i < wave) base += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + incl - v;
}

// ------------------------------------------------------------------------------------------
// Doorbell: publish the miss list to host-mapped memory, then the count, then the epoch;
// with no miss, release the stream's wait directly.
// ------------------------------------------------------------------------------------------
MOE_DEV void ring_doorbell(const DoorbellArgs& bell, const int32_t* miss_ids, int n_miss, const int32_t* step_ids,
                           int n_sel) {
  if (!bell.active) return;
  volatile int32_t* hids = bell.host_miss_ids;
  for (int i = threadIdx.x; i < n_miss; i += blockDim.x) hids[i] = miss_ids[i];
  if (bell.host_step_ids && step_ids) {
    volatile int32_t* hs = bell.host_step_ids;
    for (int i = threadIdx.x; i < n_sel; i += blockDim.x) hs[i] = step_ids[i];
  }
  __threadfence_system();
  __syncthreads();
  if (threadIdx.x == 0) {
    volatile int32_t* hcnt = bell.host_miss_count;
    hcnt[0] = n_miss;
    hcnt[2] = (bell.host_step_ids && step_ids) ? n_sel : 0;
    __threadfence_system();
    hcnt[1] = (int32_t)bell.epoch;
    __threadfence_system();
    if (n_miss == 0) {
      *(volatile uint32_t*)bell.ready = bell.epoch;
      __threadfence_system();
    }
  }
}

// ------------------------------------------------------------------------------------------
// Residency check for any number of (token, choice) pairs, pass 1: slots and miss flags.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_lookup_pairs(const int32_t* __restrict__ ids, int n_pairs, int E,
                                                       const int32_t* __restrict__ table, int n_slots,
                                                       int32_t* __restrict__ slots, uint8_t* __restrict__ miss_flag,
                                                       int32_t* __restrict__ ctrl) {
  extern __shared__ int32_t tab[];
  for (int e = threadIdx.x; e < E; e += blockDim.x) tab[e] = table ? table[e] : e;
  __syncthreads();
  int bad = 0;
  for (int p = blockIdx.x * blockDim.x + threadIdx.x; p < n_pairs; p += gridDim.x * blockDim.x) {
    const int e = ids[p];
    int s = -1;
    if (e < 0 || e >= E) {
      bad |= MOE_DERR_EXPERT_ID;
    } else {
      s = tab[e];
      if (s >= n_slots) {
        bad |= MOE_DERR_SLOT;
        s = -1;
      } else if (s < 0) {
        miss_flag[e] = 1;
      }
    }
    if (slots) slots[p] = s;
  }
  if (bad) set_error(ctrl, bad);
}

// Pass 2 (one workgroup): ascending unique miss list from the flags, doorbell, clear flags.
__global__ __launch_bounds__(1024) void k_lookup_compact(int E, uint8_t* __restrict__ miss_flag,
                                                          int32_t* __restrict__ miss_ids,
                                                          int32_t* __restrict__ miss_count,
                                                          int32_t* __restrict__ ctrl, DoorbellArgs bell) {
  __shared__ int wave_sums[16];
  const int e = threadIdx.x;
  const int f = (e < E && miss_flag[e]) ? 1 : 0;
  int total;
  const int pos = block_exclusive_scan(f, wave_sums, &total);
  if (f) miss_ids[pos] = e;
  if (e < E) miss_flag[e] = 0;
  if (threadIdx.x == 0) {
    *miss_count = total;
    ctrl[kCtrlMissCount] = total;
  }
  if (bell.active) {
    __threadfence();
    __syncthreads();
    ring_doorbell(bell, miss_ids, total, nullptr, 0);
  }
}

// Both passes in one workgroup for a few pairs (n_pairs <= blockDim.x, E <= blockDim.x): one launch
// instead of two.  Thread p looks up pair p and flags a miss in LDS; thread e then reads flag e, and
// one block scan places the misses in ascending id.
__global__ __launch_bounds__(1024) void k_lookup_small(const int32_t* __restrict__ ids, int n_pairs, int E,
                                                       const int32_t* __restrict__ table, int n_slots,
                                                       int32_t* __restrict__ slots, int32_t* __restrict__ miss_ids,
                                                       int32_t* __restrict__ miss_count, int32_t* __restrict__ ctrl,
                                                       DoorbellArgs bell) {
  __shared__ uint32_t flag[kMaxExperts];
  __shared__ int wave_sums[16];
  const int t = threadIdx.x;
  if (t < E) flag[t] = 0u;
  __syncthreads();
  int bad = 0;
  if (t < n_pairs) {
    const int e = ids[t];
    int s = -1;
    if (e < 0 || e >= E) {
      bad = MOE_DERR_EXPERT_ID;
    } else {
      s = table ? table[e] : e;
      if (s >= n_slots) {
        bad = MOE_DERR_SLOT;
        s = -1;
      } else if (s < 0) {
        flag[e] = 1u;  // every writer of e writes the same value
      }
    }
    if (slots) slots[t] = s;
  }
  if (bad) set_error(ctrl, bad);
  __syncthreads();
  const int f = (t < E && flag[t]) ? 1 : 0;
  int total;
  const int pos = block_exclusive_scan(f, wave_sums, &total);
  if (f) miss_ids[pos] = t;
  if (t == 0) {
    *miss_count = total;
    ctrl[kCtrlMissCount] = total;
  }
  if (bell.active) {
    // the selections go with the miss list (a pool's recency policy needs the hits); a doorbell
    // comes only with a decode-sized call (n_pairs <= kMaxDecodeTok * kMaxK, checked on the host)
    __threadfence();
    __syncthreads();
    ring_doorbell(bell, miss_ids, total, ids, n_pairs);
  }
}

// ------------------------------------------------------------------------------------------
// Decode plan (one workgroup of 256 threads, <= 16 tokens): residency check + one task per
// distinct expert (ascending id) with the tokens that chose it, then the shared expert over all
// tokens.  A task whose expert missed keeps slot -1 and the FFN kernels read the table entry when
// they run, so slots filled after this check (doorbell path) are seen.
// ------------------------------------------------------------------------------------------
struct alignas(16) PlanShared {
  uint32_t tok_mask[kMaxExperts];
  int32_t slot_of[kMaxExperts];
  uint32_t choice[kMaxExperts];     // 4 bits per token t < 8: position j of the expert in its top-k
  uint32_t choice_hi[kMaxExperts];  // tokens 8..15
  int wave_sums[16];
  int bad;
};

// ids: the step's [T][k] selections (LDS or global).  One thread per pair fills the per-expert
// token masks and slots in LDS; then each thread owns a run of consecutive experts, so tasks and
// misses come out in ascending expert id.
MOE_DEV void build_plan(const int32_t* ids, int T, int k, int E, int n_shared, const int32_t* table, int n_slots,
                        int32_t* miss_ids, DecodeTask* tasks, int32_t* ctrl, const DoorbellArgs& bell,
                        PlanShared& sh, bool slots_staged = false) {
  for (int e = threadIdx.x; e < E; e += blockDim.x) sh.tok_mask[e] = sh.choice[e] = sh.choice_hi[e] = 0;
  if (threadIdx.x == 0) sh.bad = 0;
  __syncthreads();
  const int n_pairs = T * k;
  for (int p = threadIdx.x; p < n_pairs; p += blockDim.x) {
    const int e = ids[p];
    const int t = p / k, j = p - t * k;
    if (e < 0 || e >= E) {
      atomicOr(&sh.bad, MOE_DERR_EXPERT_ID);
    } else {
      // a token naming e twice: reported, and only its first choice keeps a pair row
      if (atomicOr(&sh.tok_mask[e], 1u << t) & (1u << t)) atomicOr(&sh.bad, MOE_DERR_DUP_ID);
      else atomicOr(t < 8 ? &sh.choice[e] : &sh.choice_hi[e], (uint32_t)j << (4 * (t & 7)));
      const int s = slots_staged ? sh.slot_of[e] : table ? table[e] : e;
      if (!slots_staged) sh.slot_of[e] = s;  // every writer of e writes the same value
      if (s >= n_slots) atomicOr(&sh.bad, MOE_DERR_SLOT);
    }
  }
  __syncthreads();
  const int per = (E + blockDim.x - 1) / blockDim.x;
  const int e0 = threadIdx.x * per;
  int n_sub = 0, n_mis = 0;
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e >= E) break;
    if (sh.tok_mask[e]) {
      ++n_sub;
      if (sh.slot_of[e] < 0) ++n_mis;
    }
  }
  // task and miss positions from one scan of the packed pair (n_sub, n_mis): totals stay < 2^16
  int packed_total;
  const int packed = block_exclusive_scan_dpp(n_sub | (n_mis << 16), sh.wave_sums, &packed_total);
  int tpos = packed & 0xFFFF, mpos = packed >> 16;
  const int n_tasks = packed_total & 0xFFFF, n_miss = packed_total >> 16;
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e >= E) break;
    const uint32_t m = sh.tok_mask[e];
    if (!m) continue;
    const int s = sh.slot_of[e];
    if (s < 0) miss_ids[mpos++] = e;
    tasks[tpos++] = make_task(e, s, m, sh.choice[e], sh.choice_hi[e]);
  }
  if (threadIdx.x == 0) {
    int n_all = n_tasks;
    if (n_shared) tasks[n_all++] = shared_task(T);
    ctrl[kCtrlNTasks] = n_all;
    ctrl[kCtrlMissCount] = n_miss;
    if (sh.bad) set_error(ctrl, sh.bad);
  }
  if (bell.active) {
    // the host reads the miss list as soon as the doorbell rings: publish it first.  Without a
    // doorbell the kernel boundary publishes everything (an agent-scope fence here would write
    // back every XCD's L2).
    __threadfence();
    __syncthreads();
    ring_doorbell(bell, miss_ids, n_miss, ids, T * k);
  }
}

__global__ __launch_bounds__(256) void k_decode_plan(const int32_t* __restrict__ ids, int T, int k, int E,
                                                      int n_shared, const int32_t* __restrict__ table,
                                                      int n_slots, int32_t* __restrict__ miss_ids,
                                                      DecodeTask* __restrict__ tasks, int32_t* __restrict__ ctrl,
                                                      DoorbellArgs bell) {
  __shared__ PlanShared sh;
  build_plan(ids, T, k, E, n_shared, table, n_slots, miss_ids, tasks, ctrl, bell, sh);
}

// ------------------------------------------------------------------------------------------
// Decode route (<= 16 tokens): a router GEMV over all workgroups (each wave's first router row
// is loaded before the activations are staged); the last workgroup to finish then selects and
// plans, in the same launch.  The logits cross the XCDs through agent-scope stores and an
// agent-scope acquire in that workgroup (a release fence in every workgroup would write back each
// XCD's L2 many times over).
// ------------------------------------------------------------------------------------------
struct RouteArgs {
  const void* x;
  const void* Wr;
  const float* bias;
  int T, E, H, k, n_shared;
  float* logits;   // [T][E]
  int32_t* ids;    // [T][k]
  float* w;        // [T][k]
  int32_t* ctrl;
  int plan;        // also build the decode plan
  const int32_t* table;
  int n_slots;
  int32_t* miss_ids;
  DecodeTask* tasks;
  DoorbellArgs bell;
};


// The decode plan by one wave, from the step's selections in LDS (s_ids, [T][k], valid ids):
// lane l owns experts NPER*l .. NPER*l + NPER - 1.  The wave clears its experts' token masks and
// top-k positions, sets them with LDS atomics per (token, choice), reads its experts back, and one
// wave scan of the packed (tasks, misses) counts places tasks and misses in ascending expert id.
// A wave's LDS operations take effect in the order it issues them, so no barrier is needed.
template <int NPER>
MOE_DEV void plan_wave(const RouteArgs& a, PlanShared& sh, const int32_t* s_ids, int32_t* s_miss, int* s_nmiss) {
  const int lane = threadIdx.x & 63;
  const int e0 = NPER * lane;
#pragma unroll
  for (int i = 0; i < NPER; i += 4) {
    *(uint4*)&sh.tok_mask[e0 + i] = make_uint4(0u, 0u, 0u, 0u);
    *(uint4*)&sh.choice[e0 + i] = make_uint4(0u, 0u, 0u, 0u);
    *(uint4*)&sh.choice_hi[e0 + i] = make_uint4(0u, 0u, 0u, 0u);
  }
  asm volatile("" ::: "memory");  // keep the LDS phases in program order
  const int n_pairs = a.T * a.k;
  bool dup = false;
  for (int p = lane; p < n_pairs; p += 64) {
    const int e = s_ids[p];
    const int t = p / a.k, j = p - t * a.k;
    // (the selection's ids are distinct; a repeat would be reported, its choice dropped)
    const uint32_t old =
        __hip_atomic_fetch_or(&sh.tok_mask[e], 1u << t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    dup |= (old >> t) & 1u;
    if (!((old >> t) & 1u))
      __hip_atomic_fetch_or(t < 8 ? &sh.choice[e] : &sh.choice_hi[e], (uint32_t)j << (4 * (t & 7)), __ATOMIC_RELAXED,
                            __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  asm volatile("" ::: "memory");
  uint32_t m[NPER], c[NPER], ch[NPER];
  int32_t sl[NPER];
#pragma unroll
  for (int i = 0; i < NPER; i += 4) {
    const uint4 mv = *(const uint4*)&sh.tok_mask[e0 + i];
    const uint4 cv = *(const uint4*)&sh.choice[e0 + i];
    const uint4 hv = *(const uint4*)&sh.choice_hi[e0 + i];
    const int4 sv = *(const int4*)&sh.slot_of[e0 + i];
    m[i] = mv.x, m[i + 1] = mv.y, m[i + 2] = mv.z, m[i + 3] = mv.w;
    c[i] = cv.x, c[i + 1] = cv.y, c[i + 2] = cv.z, c[i + 3] = cv.w;
    ch[i] = hv.x, ch[i + 1] = hv.y, ch[i + 2] = hv.z, ch[i + 3] = hv.w;
    sl[i] = sv.x, sl[i + 1] = sv.y, sl[i + 2] = sv.z, sl[i + 3] = sv.w;
  }
  int n_sub = 0, n_mis = 0;
  bool bad = false;
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const bool used = m[i] != 0u;  // experts >= E are never selected
    n_sub += used;
    n_mis += used && sl[i] < 0;
    bad |= used && sl[i] >= a.n_slots;
  }
  // wave exclusive scan of the packed counts (totals stay < 2^16)
  const int v = n_sub | (n_mis << 16);
  int incl = v;
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x111, 0xF, 0xF, false);  // row_shr:1
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x112, 0xF, 0xF, false);  // row_shr:2
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x114, 0xF, 0xF, false);  // row_shr:4
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x118, 0xF, 0xF, false);  // row_shr:8
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x142, 0xA, 0xF, false);  // row_bcast:15
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x143, 0xC, 0xF, false);  // row_bcast:31
  const int total = __builtin_amdgcn_readlane(incl, 63);
  const int excl = incl - v;
  int tpos = excl & 0xFFFF, mpos = excl >> 16;
  const int n_tasks = total & 0xFFFF, n_miss = total >> 16;
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    if (m[i] != 0u) {
      const int e = e0 + i;
      if (sl[i] < 0) {
        a.miss_ids[mpos] = e;
        s_miss[mpos] = e;
        ++mpos;
      }
      a.tasks[tpos++] = make_task(e, sl[i], m[i], c[i], ch[i]);
    }
  }
  const bool any_bad = __any(bad);
  const bool any_dup = __any(dup);
  if (lane == 0) {
    int n_all = n_tasks;
    if (a.n_shared) a.tasks[n_all++] = shared_task(a.T);
    a.ctrl[kCtrlNTasks] = n_all;
    a.ctrl[kCtrlMissCount] = n_miss;
    if (any_bad || any_dup) set_error(a.ctrl, (any_bad ? MOE_DERR_SLOT : 0) | (any_dup ? MOE_DERR_DUP_ID : 0));
    *s_nmiss = n_miss;
  }
}

// One workgroup: the top-k of every token (one wave per token, DPP arg-max) and, if asked, the
// decode plan (residency check, task list, miss list, doorbell).  Needs >= 256 threads.
template <int NPER>
MOE_DEV void select_and_plan(const RouteArgs& a) {
  __shared__ PlanShared sh;
  __shared__ int32_t s_ids[kMaxDecodeTok * kMaxK];
  __shared__ float s_w[kMaxDecodeTok * kMaxK];
  __shared__ int32_t s_miss[kMaxDecodeTok * kMaxK];
  __shared__ int s_nmiss;
  const int wave = threadIdx.x >> 6;
  // the slot table is loaded with the logits (issued first: one wait covers both) and goes to LDS
  // after the selections, so the plan makes no dependent global load
  constexpr int kTabPer = kMaxExperts / 256;  // blockDim.x >= 256
  int32_t tab[kTabPer];
#pragma unroll
  for (int i = 0; i < kTabPer; ++i) {
    const int e = min((int)(threadIdx.x + i * blockDim.x), a.E - 1);
    tab[i] = a.table ? a.table[e] : e;
  }
  // The slots go to LDS as soon as the wait for the logits has covered them.  The selections
  // stay in LDS until the plan has read its LDS: a store still in flight when a later LDS read
  // reuses its data register makes the compiler wait for every outstanding memory operation.
  auto stage_slots = [&]() {
#pragma unroll
    for (int i = 0; i < kTabPer; ++i) {
      const int e = threadIdx.x + i * blockDim.x;
      if (e < a.E) sh.slot_of[e] = tab[i];
    }
  };
  if (wave < a.T) {
    select_topk_wave<NPER>(a.logits + (size_t)wave * a.E, a.E, a.k, nullptr, nullptr, a.ctrl, s_ids + wave * a.k,
                           s_w + wave * a.k, stage_slots);
    for (int t = wave + (blockDim.x >> 6); t < a.T; t += blockDim.x >> 6) {
      select_topk_wave<NPER>(a.logits + (size_t)t * a.E, a.E, a.k, nullptr, nullptr, a.ctrl, s_ids + t * a.k,
                             s_w + t * a.k);
    }
  } else {
    stage_slots();
  }
  __syncthreads();
  if (wave == 0) {
    if (a.plan) plan_wave<NPER>(a, sh, s_ids, s_miss, &s_nmiss);
    for (int p = threadIdx.x; p < a.T * a.k; p += 64) {
      a.ids[p] = s_ids[p];
      a.w[p] = s_w[p];
    }
  }
  if (!a.plan) return;
  if (a.bell.active) {
    // the host reads the miss list and the selections as soon as the doorbell rings: both go
    // to host memory from LDS before the count and the epoch
    __syncthreads();
    ring_doorbell(a.bell, s_miss, s_nmiss, s_ids, a.T * a.k);
  }
}

// End of a router workgroup: its logits went out as agent-scope stores (written through to the
// coherence point the XCDs share); it waits for them and counts itself; the workgroup that
// completes the count (every router row is then written) acquires at agent scope and runs the
// selection and the plan.  No workgroup waits on another.
// Invariant this rests on: every logit the selecting workgroup reads is written by such an
// agent-scope store (store_logit), completed before the relaxed counter increment.  There is no
// release fence: a plain store to the logits would stay in its XCD's L2, unseen by the selection.
MOE_DEV void store_logit(float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

template <int NPER>
MOE_DEV void route_tail(const RouteArgs& a) {
  __shared__ int s_last;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's logit stores are complete
  __syncthreads();
  if (threadIdx.x == 0) {
    const int old = __hip_atomic_fetch_add(&a.ctrl[kCtrlRouteDone], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = old == (int)gridDim.x - 1;
  }
  __syncthreads();
  if (!s_last) return;
  if (threadIdx.x == 0) __hip_atomic_store(&a.ctrl[kCtrlRouteDone], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  select_and_plan<NPER>(a);
}

template <bool X_BF16, bool R_BF16, int NPER>
__global__ __launch_bounds__(256) void k_router_gemv(RouteArgs a) {
  extern __shared__ float xs[];  // [T][H]
  const int T = a.T, E = a.E, H = a.H;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int waves_total = gridDim.x * (blockDim.x >> 6);
  constexpr int kPer = R_BF16 ? 8 : 4;  // elements per 16-byte load
  const int n_chunks = H / kPer;
  const int e_first = blockIdx.x * (blockDim.x >> 6) + wave;
  // first router row's loads go out before the activations are staged
  constexpr int kMaxChunkPerLane = R_BF16 ? 8 : 16;  // H <= 4096
  uint4 wpre[kMaxChunkPerLane];
#pragma unroll
  for (int i = 0; i < kMaxChunkPerLane; ++i) {
    const int c = lane + 64 * i;
    if (e_first < E && c < n_chunks) wpre[i] = *((const uint4*)((const uint8_t*)a.Wr + (size_t)e_first * H * (R_BF16 ? 2 : 4)) + c);
  }
  for (int i = threadIdx.x; i < T * H; i += blockDim.x) {
    float v;
    if (X_BF16) v = __uint_as_float(((uint32_t)((const uint16_t*)a.x)[i]) << 16);
    else v = ((const float*)a.x)[i];
    xs[i] = v;
  }
  __syncthreads();
  for (int e = e_first; e < E; e += waves_total) {
    float acc[kMaxDecodeTok];
#pragma unroll
    for (int t = 0; t < kMaxDecodeTok; ++t) acc[t] = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxChunkPerLane; ++i) {
      const int c = lane + 64 * i;
      if (c >= n_chunks) break;
      const uint4 q = e == e_first ? wpre[i]
                                   : *((const uint4*)((const uint8_t*)a.Wr + (size_t)e * H * (R_BF16 ? 2 : 4)) + c);
      float wv[kPer];
      if constexpr (R_BF16) {
        const uint32_t p[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          wv[2 * j] = bf16_lo(p[j]);
          wv[2 * j + 1] = bf16_hi(p[j]);
        }
      } else {
        wv[0] = __uint_as_float(q.x);
        wv[1] = __uint_as_float(q.y);
        wv[2] = __uint_as_float(q.z);
        wv[3] = __uint_as_float(q.w);
      }
#pragma unroll
      for (int t = 0; t < kMaxDecodeTok; ++t) {
        if (t < T) {
          const float* xr = xs + t * H + c * kPer;
#pragma unroll
          for (int j = 0; j < kPer; ++j) acc[t] = fmaf(xr[j], wv[j], acc[t]);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < kMaxDecodeTok; ++t) {
      if (t < T) {
        const float sum = group_sum_dpp(acc[t], 64);
        if (lane == 63) store_logit(a.logits + (size_t)t * E + e, sum + (a.bias ? a.bias[e] : 0.f));
      }
    }
  }
  route_tail<NPER>(a);
}

// Router GEMV on the matrix cores (bf16 router): one workgroup per kRouterRows router rows (8: 64
// workgroups share the 2 MB of weights, so each CU reads 32 KB), its 8 waves split the H inputs and
// reduce through LDS.  A = activation rows (one per token; fp32 inputs as bf16 hi + lo rows), B = the
// router rows in the MFMA's first kRouterRows columns, 32 inputs per v_mfma_f32_16x16x32_bf16 step;
// each lane loads 16 contiguous bytes of its router row per step (the row's 4 lanes read 64 bytes).
constexpr int kRouterWaves = 8;
constexpr int kRouterRows = 8;  // router rows per workgroup (of the MFMA's 16 columns)
constexpr int kRouterMaxSteps = 4096 / 32 / kRouterWaves;  // H <= 4096

MOE_DEV uint4 split_bf16_part(const float4& a, const float4& b, int part) {
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t q[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t hi = f32_to_bf16_rne(v[e]);
    q[e] = part ? f32_to_bf16_rne(v[e] - __uint_as_float(hi << 16)) : hi;
  }
  return make_uint4(q[0] | (q[1] << 16), q[2] | (q[3] << 16), q[4] | (q[5] << 16), q[6] | (q[7] << 16));
}

// TAIL false: the logits only (the one-token gate/up launch selects for itself).
template <bool X_BF16, int NPER, bool TAIL = true, int ROWS = kRouterRows>
__global__ __launch_bounds__(64 * kRouterWaves) void k_router_mfma(RouteArgs a) {
  __shared__ float red[kRouterWaves][16][16];  // [wave][A row][router row]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int T = a.T, E = a.E, H = a.H;
  const int e0 = blockIdx.x * ROWS;
  const int e = n < ROWS ? e0 + n : E;  // B columns past the workgroup's rows stay zero
  const int NB = H / 32;
  const int spw = (NB + kRouterWaves - 1) / kRouterWaves;  // 32-input steps per wave
  const int b0 = wave * spw;
  const int nb = min(spw, NB - b0);
  const int rows = X_BF16 ? T : 2 * T;
  const int m = n;  // A row of this lane
  const bool live = m < rows;
  const int tok = X_BF16 ? m : (m >> 1);
  const uint16_t* wr = (const uint16_t*)a.Wr + (size_t)(e < E ? e : 0) * H + 8 * g;
  uint4 wb[kRouterMaxSteps];
  uint4 xa[X_BF16 ? kRouterMaxSteps : 1];
#pragma unroll
  for (int j = 0; j < kRouterMaxSteps; ++j) {
    if (j < nb) {
      if constexpr (X_BF16)
        xa[j] = live ? *(const uint4*)((const uint16_t*)a.x + (size_t)tok * H + (b0 + j) * 32 + 8 * g)
                     : make_uint4(0u, 0u, 0u, 0u);
      wb[j] = e < E ? *(const uint4*)(wr + (size_t)(b0 + j) * 32) : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kRouterMaxSteps; ++j) {
    if (j < nb) {
      uint4 av;
      if constexpr (X_BF16) {
        av = xa[j];
      } else {
        av = make_uint4(0u, 0u, 0u, 0u);
        if (live) {
          const float* xr = (const float*)a.x + (size_t)tok * H + (b0 + j) * 32 + 8 * g;
          av = split_bf16_part(*(const float4*)xr, *(const float4*)(xr + 4), m & 1);
        }
      }
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, wb[j]),
                                                    acc, 0, 0, 0);
    }
  }
  // lane (g, n) holds A rows 4g + r of router row n
#pragma unroll
  for (int r = 0; r < 4; ++r) red[wave][4 * g + r][n] = acc[r];
  __syncthreads();
  if ((int)threadIdx.x < 16 * T) {
    const int t = threadIdx.x >> 4, c = threadIdx.x & 15;
    const int ee = e0 + c;
    if (c < ROWS && ee < E) {
      float sum = 0.f;
      for (int w = 0; w < kRouterWaves; ++w) {
        if constexpr (X_BF16) sum += red[w][t][c];
        else sum += red[w][2 * t][c] + red[w][2 * t + 1][c];
      }
      store_logit(a.logits + (size_t)t * E + ee, sum + (a.bias ? a.bias[ee] : 0.f));
    }
  }
  if constexpr (TAIL) route_tail<NPER>(a);
}

// ------------------------------------------------------------------------------------------
// Launchers
// ------------------------------------------------------------------------------------------
hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w, int32_t* ctrl,
                       hipStream_t st) {
  const int grid = (T + 3) / 4;
  if (E <= 512) k_topk<8><<<grid, 256, 0, st>>>(logits, T, E, k, ids, w, ctrl);
  else k_topk<16><<<grid, 256, 0, st>>>(logits, T, E, k, ids, w, ctrl);
  return hipGetLastError();
}

hipError_t launch_lookup(const int32_t* ids, int n_pairs, int E, const int32_t* table, int n_slots,
                         int32_t* slots, uint8_t* miss_flag, int32_t* miss_ids, int32_t* miss_count,
                         int32_t* ctrl, const DoorbellArgs& bell, hipStream_t st) {
  if (n_pairs <= 1024 && E <= kMaxExperts && E <= 1024) {
    // a decode-sized check: one launch
    k_lookup_small<<<1, 1024, 0, st>>>(ids, n_pairs, E, table, n_slots, slots, miss_ids, miss_count, ctrl, bell);
    return hipGetLastError();
  }
  if (n_pairs > 0) {
    int grid = (n_pairs + 255) / 256;
    if (grid > 1024) grid = 1024;
    k_lookup_pairs<<<grid, 256, (size_t)E * sizeof(int32_t), st>>>(ids, n_pairs, E, table, n_slots, slots,
                                                                   miss_flag, ctrl);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  k_lookup_compact<<<1, 1024, 0, st>>>(E, miss_flag, miss_ids, miss_count, ctrl, bell);
  return hipGetLastError();
}

hipError_t launch_decode_plan(const int32_t* ids, int T, int k, int E, int n_shared, const int32_t* table,
                              int n_slots, int32_t* miss_ids, DecodeTask* tasks, int32_t* ctrl,
                              const DoorbellArgs& bell, hipStream_t st) {
  k_decode_plan<<<1, 256, 0, st>>>(ids, T, k, E, n_shared, table, n_slots, miss_ids, tasks, ctrl, bell);
  return hipGetLastError();
}

template <int NPER>
static hipError_t launch_router(const RouteArgs& a, int x_dtype, int r_dtype, hipStream_t st) {
  if (r_dtype == MOE_BF16) {
    // bf16 router: matrix-core GEMV
    const int grid = (a.E + kRouterRows - 1) / kRouterRows;
    if (x_dtype == MOE_BF16)
      return launch_timed(kTimeDecodeRoute, k_router_mfma<true, NPER>, grid, 64 * kRouterWaves, 0, st, a);
    return launch_timed(kTimeDecodeRoute, k_router_mfma<false, NPER>, grid, 64 * kRouterWaves, 0, st, a);
  }
  // fp32 router: exact fp32 FMA GEMV
  const int grid = (a.E + 3) / 4;
  const uint32_t lds = (uint32_t)(a.T * a.H * sizeof(float));
  if (x_dtype == MOE_BF16) return launch_timed(kTimeDecodeRoute, k_router_gemv<true, false, NPER>, grid, 256, lds, st, a);
  return launch_timed(kTimeDecodeRoute, k_router_gemv<false, false, NPER>, grid, 256, lds, st, a);
}

hipError_t launch_router_logits_bf16(const void* x, const void* Wr, const float* bias, int E, int H, float* logits,
                                     hipStream_t st) {
  RouteArgs a{};
  a.x = x;
  a.Wr = Wr;
  a.bias = bias;
  a.T = 1;
  a.E = E;
  a.H = H;
  a.logits = logits;
  // with no hand-over at the end, more and smaller workgroups: 4 router rows each
  constexpr int kRows = 4;
  const int grid = (E + kRows - 1) / kRows;
  return launch_timed(kTimeDecodeRoute, k_router_mfma<true, 8, false, kRows>, grid, 64 * kRouterWaves, 0, st, a);
}

hipError_t launch_decode_route(const void* x, int x_dtype, const void* Wr, int r_dtype, const float* bias, int T,
                               int E, int H, int k, int n_shared, float* logits, int32_t* ids, float* w,
                               int32_t* ctrl, bool plan, const int32_t* table, int n_slots, int32_t* miss_ids,
                               DecodeTask* tasks, const DoorbellArgs& bell, hipStream_t st) {
  RouteArgs a{};
  a.x = x;
  a.Wr = Wr;
  a.bias = bias;
  a.T = T;
  a.E = E;
  a.H = H;
  a.k = k;
  a.n_shared = n_shared;
  a.logits = logits;
  a.ids = ids;
  a.w = w;
  a.ctrl = ctrl;
  a.plan = plan ? 1 : 0;
  a.table = table;
  a.n_slots = n_slots;
  a.miss_ids = miss_ids;
  a.tasks = tasks;
  a.bell = bell;
  // the router launch also selects and plans (its last workgroup); 8 or 16 logits per lane
  if (E <= 512) return launch_router<8>(a, x_dtype, r_dtype, st);
  return launch_router<16>(a, x_dtype, r_dtype, st);
}

}  // namespace moe
