// Router, top-k selection and the in-stream residency check.
//
// Router and selection: Betelgeuse news article, section "mechanism" (each token takes 10 of
// 512 routed experts + 1 shared) and "what bit-exact means" (the top-10 is exact).
// Residency: same article, "mechanism" table, scheduling row (expert id -> HBM slot decided on
// the GPU in the stream; the host is rung only on a miss).
#include "kernels.hpp"

namespace moe {

// ------------------------------------------------------------------------------------------
// Router GEMV for <= 8 tokens: logits[t][e] = sum_h x[t][h] * Wr[e][h] + bias[e].
// x is staged once per workgroup in LDS as fp32 (exact widening of bf16/fp32); each wave
// streams router rows with 16-byte loads (8 bf16 or 4 fp32 per lane per load), accumulates
// in fp32 and reduces across the wave.  Bandwidth-bound on the router rows.
// ------------------------------------------------------------------------------------------
template <bool X_BF16, bool R_BF16>
__global__ __launch_bounds__(256) void k_router_gemv(const void* __restrict__ x, const void* __restrict__ Wr,
                                                      const float* __restrict__ bias, int T, int E, int H,
                                                      float* __restrict__ logits) {
  extern __shared__ float xs[];  // [T][H]
  for (int i = threadIdx.x; i < T * H; i += blockDim.x) {
    float v;
    if (X_BF16) v = __uint_as_float(((uint32_t)((const uint16_t*)x)[i]) << 16);
    else v = ((const float*)x)[i];
    xs[i] = v;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int waves_total = gridDim.x * (blockDim.x >> 6);
  constexpr int kPer = R_BF16 ? 8 : 4;  // elements per 16-byte load
  const int n_chunks = H / kPer;
  for (int e = blockIdx.x * (blockDim.x >> 6) + wave; e < E; e += waves_total) {
    float acc[kMaxDecodeTok];
#pragma unroll
    for (int t = 0; t < kMaxDecodeTok; ++t) acc[t] = 0.f;
    for (int c = lane; c < n_chunks; c += 64) {
      float wv[kPer];
      if (R_BF16) {
        uint4 q = *((const uint4*)((const uint16_t*)Wr + (size_t)e * H) + c);
        uint32_t p[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          wv[2 * i] = bf16_lo(p[i]);
          wv[2 * i + 1] = bf16_hi(p[i]);
        }
      } else {
        float4 q = *((const float4*)((const float*)Wr + (size_t)e * H) + c);
        wv[0] = q.x; wv[1] = q.y; wv[2] = q.z; wv[3] = q.w;
      }
#pragma unroll
      for (int t = 0; t < kMaxDecodeTok; ++t) {
        if (t < T) {
          const float* xr = xs + t * H + c * kPer;
#pragma unroll
          for (int i = 0; i < kPer; ++i) acc[t] = fmaf(xr[i], wv[i], acc[t]);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < kMaxDecodeTok; ++t) {
      if (t < T) {
        float s = wave_sum(acc[t]);
        if (lane == 0) logits[(size_t)t * E + e] = s + (bias ? bias[e] : 0.f);
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// Top-k of E logits per token, one wave per token.  Each lane holds E/64 logits; k rounds of
// (local best, wave arg-max on (value desc, id asc)) pick the experts in rank order.  The
// weights are a softmax over the selected logits, summed in selection order.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, int T, int E, int k,
                                               int32_t* __restrict__ ids, float* __restrict__ w,
                                               int32_t* __restrict__ ctrl) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (t >= T) return;
  constexpr int kPerLane = kMaxExperts / 64;
  float v[kPerLane];
  const float* row = logits + (size_t)t * E;
  bool nan_seen = false;
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const int e = lane + 64 * i;
    float val = -INFINITY;
    if (e < E) {
      val = row[e];
      if (val != val) {
        nan_seen = true;
        val = -INFINITY;
      }
    }
    v[i] = val;
  }
  if (__any(nan_seen) && lane == 0) set_error(ctrl, MOE_DERR_NAN);
  uint32_t taken = 0;
  float my_v = 0.f;
  int my_i = 0;
  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      const int e = lane + 64 * i;
      if (!(taken & (1u << i)) && e < E && (v[i] > bv || (v[i] == bv && e < bi))) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == r) {
      my_v = bv;
      my_i = bi;
    }
  }
  const float m = __shfl(my_v, 0, 64);
  const float ex = lane < k ? expf(my_v - m) : 0.f;
  float s = 0.f;
  for (int r = 0; r < k; ++r) s += __shfl(ex, r, 64);
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_i;
    w[(size_t)t * k + lane] = ex / s;
  }
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

// ------------------------------------------------------------------------------------------
// Doorbell: publish the miss list to host-mapped memory, then the count, then the epoch;
// with no miss, release the stream's wait directly.
// ------------------------------------------------------------------------------------------
MOE_DEV void ring_doorbell(const DoorbellArgs& bell, const int32_t* miss_ids, int n_miss) {
  if (!bell.active) return;
  volatile int32_t* hids = bell.host_miss_ids;
  for (int i = threadIdx.x; i < n_miss; i += blockDim.x) hids[i] = miss_ids[i];
  __threadfence_system();
  __syncthreads();
  if (threadIdx.x == 0) {
    volatile int32_t* hcnt = bell.host_miss_count;
    hcnt[0] = n_miss;
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
  __threadfence();
  __syncthreads();
  ring_doorbell(bell, miss_ids, total);
}

// ------------------------------------------------------------------------------------------
// Decode plan (one workgroup, <= 8 tokens): residency check + the list of distinct experts
// (ascending id) with the tokens that chose each, then the shared expert over all tokens.
// The FFN kernels resolve each task's slot from the table when they run, so slots filled
// after this check (doorbell path) are seen.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_decode_plan(const int32_t* __restrict__ ids, int T, int k, int E,
                                                       int n_shared, const int32_t* __restrict__ table,
                                                       int n_slots, int32_t* __restrict__ slots_out,
                                                       int32_t* __restrict__ miss_ids,
                                                       int32_t* __restrict__ miss_count_out,
                                                       DecodeTask* __restrict__ tasks,
                                                       int32_t* __restrict__ ctrl, DoorbellArgs bell) {
  __shared__ uint32_t tok_mask[kMaxExperts];
  __shared__ uint8_t choice[kMaxExperts][kMaxDecodeTok];
  __shared__ int wave_sums[16];
  __shared__ int s_bad;
  for (int e = threadIdx.x; e < E; e += blockDim.x) tok_mask[e] = 0;
  if (threadIdx.x == 0) s_bad = 0;
  __syncthreads();
  const int n_pairs = T * k;
  for (int p = threadIdx.x; p < n_pairs; p += blockDim.x) {
    const int e = ids[p];
    const int t = p / k, j = p - t * k;
    int s = -1;
    if (e < 0 || e >= E) {
      atomicOr(&s_bad, MOE_DERR_EXPERT_ID);
    } else {
      atomicOr(&tok_mask[e], 1u << t);
      choice[e][t] = (uint8_t)j;
      s = table ? table[e] : e;
      if (s >= n_slots) {
        atomicOr(&s_bad, MOE_DERR_SLOT);
        s = -1;
      }
    }
    if (slots_out) slots_out[p] = s;
  }
  __syncthreads();
  const int e = threadIdx.x;
  const uint32_t m = e < E ? tok_mask[e] : 0u;
  const int n_e = __popc(m);
  const bool used = n_e > 0;
  int slot_e = -1;
  if (used) slot_e = table ? table[e] : e;
  const bool miss = used && slot_e < 0;
  int n_tasks, n_miss;
  const int n_sub = (n_e + kTaskTok - 1) / kTaskTok;  // tasks of at most kTaskTok tokens
  const int tpos = block_exclusive_scan(n_sub, wave_sums, &n_tasks);
  const int mpos = block_exclusive_scan(miss ? 1 : 0, wave_sums, &n_miss);
  if (used) {
    DecodeTask tk;
    tk.expert = e;
    int n = 0, task = tpos;
    for (int t = 0; t < T; ++t) {
      if (m & (1u << t)) {
        tk.tok[n] = t;
        tk.pair[n] = t * k + choice[e][t];
        if (++n == kTaskTok) {
          tk.n_tok = n;
          tasks[task++] = tk;
          n = 0;
        }
      }
    }
    if (n > 0) {
      tk.n_tok = n;
      tasks[task] = tk;
    }
  }
  if (miss) miss_ids[mpos] = e;
  if (threadIdx.x == 0) {
    int n_all = n_tasks;
    if (n_shared) {
      for (int t0 = 0; t0 < T; t0 += kTaskTok) {
        DecodeTask tk;
        tk.expert = -1;
        tk.n_tok = min(kTaskTok, T - t0);
        for (int n = 0; n < tk.n_tok; ++n) {
          tk.tok[n] = t0 + n;
          tk.pair[n] = T * k + t0 + n;
        }
        tasks[n_all++] = tk;
      }
    }
    ctrl[kCtrlNTasks] = n_all;
    ctrl[kCtrlMissCount] = n_miss;
    if (miss_count_out) *miss_count_out = n_miss;
    if (s_bad) set_error(ctrl, s_bad);
  }
  __threadfence();
  __syncthreads();
  ring_doorbell(bell, miss_ids, n_miss);
}

// ------------------------------------------------------------------------------------------
// Launchers
// ------------------------------------------------------------------------------------------
hipError_t launch_router_gemv(const void* x, int x_dtype, const void* Wr, int r_dtype, const float* bias,
                              int T, int E, int H, float* logits, hipStream_t st) {
  const int waves_per_wg = 4;
  int grid = (E + waves_per_wg - 1) / waves_per_wg;
  if (grid > 512) grid = 512;
  const size_t lds = (size_t)T * H * sizeof(float);
  if (x_dtype == MOE_BF16 && r_dtype == MOE_BF16)
    k_router_gemv<true, true><<<grid, 256, lds, st>>>(x, Wr, bias, T, E, H, logits);
  else if (x_dtype == MOE_BF16)
    k_router_gemv<true, false><<<grid, 256, lds, st>>>(x, Wr, bias, T, E, H, logits);
  else if (r_dtype == MOE_BF16)
    k_router_gemv<false, true><<<grid, 256, lds, st>>>(x, Wr, bias, T, E, H, logits);
  else
    k_router_gemv<false, false><<<grid, 256, lds, st>>>(x, Wr, bias, T, E, H, logits);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w, int32_t* ctrl,
                       hipStream_t st) {
  const int grid = (T + 3) / 4;
  k_topk<<<grid, 256, 0, st>>>(logits, T, E, k, ids, w, ctrl);
  return hipGetLastError();
}

hipError_t launch_lookup(const int32_t* ids, int n_pairs, int E, const int32_t* table, int n_slots,
                         int32_t* slots, uint8_t* miss_flag, int32_t* miss_ids, int32_t* miss_count,
                         int32_t* ctrl, const DoorbellArgs& bell, hipStream_t st) {
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
                              int n_slots, int32_t* slots_out, int32_t* miss_ids, int32_t* miss_count_out,
                              DecodeTask* tasks, int32_t* ctrl, const DoorbellArgs& bell, hipStream_t st) {
  k_decode_plan<<<1, 1024, 0, st>>>(ids, T, k, E, n_shared, table, n_slots, slots_out, miss_ids,
                                    miss_count_out, tasks, ctrl, bell);
  return hipGetLastError();
}

}  // namespace moe
