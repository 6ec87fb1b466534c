// Grouping of (token, choice) pairs by expert for the prefill path: a stable counting sort.
//
// halogen-flash-server README, "Measured": the step that orders the tokens was changed between
// releases and moved prefill speed; here it is the bucketing that turns the routed pairs into one
// dense row block per expert for the grouped GEMM.
//
// Stable and deterministic without a sort: each expert e keeps a bitmap over tokens (bit t set
// when token t chose e; a token chooses an expert at most once, so the pairs of bucket e in pair
// order are its tokens in increasing order; a second choice of the same expert finds its bit set
// and is reported as MOE_DERR_DUP_ID).  Setting bits with atomicOr is order-independent.
// The rank of (t, e) inside bucket e is the popcount of the bits below t: a per-bucket prefix of
// word popcounts plus a popcount of the masked word.  The shared expert is bucket E and holds
// every token in order.
#include "kernels.hpp"

namespace moe {

__global__ __launch_bounds__(256) void k_group_setbits(const int32_t* __restrict__ ids, int T, int k, int E, int W,
                                                        uint32_t* __restrict__ bits, int32_t* __restrict__ ctrl) {
  const int n = T * k;
  int bad = 0;
  for (int p = blockIdx.x * blockDim.x + threadIdx.x; p < n; p += gridDim.x * blockDim.x) {
    const int e = ids[p];
    if (e < 0 || e >= E) {
      bad |= MOE_DERR_EXPERT_ID;
      continue;
    }
    const int t = p / k;
    const uint32_t bit = 1u << (t & 31);
    // a bit already set: the token named expert e twice (its pairs would share one sorted row)
    if (atomicOr(&bits[(size_t)e * W + (t >> 5)], bit) & bit) bad |= MOE_DERR_DUP_ID;
  }
  if (bad) set_error(ctrl, bad);
}

// One workgroup per routed bucket: exclusive prefix of word popcounts and the bucket count.
__global__ __launch_bounds__(256) void k_group_bucket_scan(const uint32_t* __restrict__ bits, int W,
                                                            int32_t* __restrict__ prefix, int32_t* __restrict__ count) {
  __shared__ int wave_sums[4];
  const int e = blockIdx.x;
  const uint32_t* row = bits + (size_t)e * W;
  int32_t* pre = prefix + (size_t)e * W;
  const int per = (W + blockDim.x - 1) / blockDim.x;
  const int w0 = threadIdx.x * per;
  int local = 0;
  for (int i = 0; i < per; ++i) {
    const int w = w0 + i;
    if (w < W) local += __popc(row[w]);
  }
  // block exclusive scan of `local`
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) wave_sums[wave] = incl;
  __syncthreads();
  int base = 0, tot = 0;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) {
    if (i < wave) base += wave_sums[i];
    tot += wave_sums[i];
  }
  int run = base + incl - local;
  for (int i = 0; i < per; ++i) {
    const int w = w0 + i;
    if (w < W) {
      pre[w] = run;
      run += __popc(row[w]);
    }
  }
  if (threadIdx.x == 0) count[e] = tot;
}

// One workgroup (1024 threads): bucket offsets, the GEMM tile list, the public counts/offsets.
__global__ __launch_bounds__(1024) void k_group_offsets(const int32_t* __restrict__ count, int E, int n_shared, int T,
                                                         int item_rows, int32_t* __restrict__ offsets,
                                                         TileItem* __restrict__ items, int32_t* __restrict__ ctrl,
                                                         int32_t* __restrict__ counts_out,
                                                         int32_t* __restrict__ offsets_out) {
  __shared__ int wave_sums[16];
  const int e = threadIdx.x;
  const int c = e < E ? count[e] : 0;
  const int n_it = (c + item_rows - 1) / item_rows;
  int total_rows, total_items;
  // block-wide exclusive scans (blockDim.x == 1024 >= E)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  auto scan = [&](int v, int* tot) {
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl, o, 64);
      if (lane >= o) incl += u;
    }
    if (lane == 63) wave_sums[wave] = incl;
    __syncthreads();
    int base = 0, t = 0;
    for (int i = 0; i < 16; ++i) {
      if (i < wave) base += wave_sums[i];
      t += wave_sums[i];
    }
    __syncthreads();
    *tot = t;
    return base + incl - v;
  };
  const int off = scan(c, &total_rows);
  const int ipos = scan(n_it, &total_items);
  if (e < E) {
    offsets[e] = off;
    if (counts_out) counts_out[e] = c;
    if (offsets_out) offsets_out[e] = off;
    for (int i = 0; i < n_it; ++i) {
      TileItem it;
      it.bucket = e;
      it.row0 = off + i * item_rows;
      it.rows = min(item_rows, c - i * item_rows);
      it.pad = n_it == 1 ? kItemOnly : 0;
      items[ipos + i] = it;
    }
  }
  if (threadIdx.x == 0) {
    offsets[E] = total_rows;
    if (offsets_out) offsets_out[E] = total_rows;
    int n_all = total_items;
    if (n_shared) {
      offsets[E + 1] = total_rows + T;
      for (int r0 = 0; r0 < T; r0 += item_rows) {
        TileItem it;
        it.bucket = E;
        it.row0 = total_rows + r0;
        it.rows = min(item_rows, T - r0);
        it.pad = T <= item_rows ? kItemOnly : 0;
        items[n_all++] = it;
      }
    } else {
      offsets[E + 1] = total_rows;
    }
    ctrl[kCtrlNTiles] = n_all;
  }
}

// Position of every pair in bucket order, the token and router weight of each sorted row, and
// the inverse map used by the combine.
__global__ __launch_bounds__(256) void k_group_scatter(const int32_t* __restrict__ ids, const float* __restrict__ topk_w,
                                                        int T, int k, int E, int n_shared, int W,
                                                        const uint32_t* __restrict__ bits,
                                                        const int32_t* __restrict__ prefix,
                                                        const int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ perm, int32_t* __restrict__ row_tok,
                                                        float* __restrict__ row_w, int32_t* __restrict__ inv) {
  const int n_routed = T * k;
  const int n = n_routed + (n_shared ? T : 0);
  for (int p = blockIdx.x * blockDim.x + threadIdx.x; p < n; p += gridDim.x * blockDim.x) {
    if (p < n_routed) {
      const int e = ids[p];
      if (e < 0 || e >= E) {
        inv[p] = -1;
        continue;
      }
      const int t = p / k;
      const int w = t >> 5;
      const uint32_t word = bits[(size_t)e * W + w];
      const int pos = offsets[e] + prefix[(size_t)e * W + w] + __popc(word & ((1u << (t & 31)) - 1u));
      perm[pos] = p;
      row_tok[pos] = t;
      row_w[pos] = topk_w ? topk_w[p] : 1.0f;
      inv[p] = pos;
    } else {
      const int t = p - n_routed;
      const int pos = offsets[E] + t;
      perm[pos] = p;
      row_tok[pos] = t;
      row_w[pos] = 1.0f;
      inv[p] = pos;
    }
  }
}

hipError_t launch_group(const int32_t* ids, const float* topk_w, int T, int k, int E, int n_shared,
                        const GroupBuffers& g, int32_t* ctrl, int32_t* counts_out, int32_t* offsets_out,
                        hipStream_t st, int item_rows) {
  const int W = (T + 31) / 32;
  hipError_t err = launch_fill_zero(g.bits, sizeof(uint32_t) * (size_t)E * W, st);
  if (err != hipSuccess) return err;
  const int n = T * k;
  int grid = (n + 255) / 256;
  if (grid > 2048) grid = 2048;
  k_group_setbits<<<grid, 256, 0, st>>>(ids, T, k, E, W, g.bits, ctrl);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  k_group_bucket_scan<<<E, 256, 0, st>>>(g.bits, W, g.prefix, g.count);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  k_group_offsets<<<1, 1024, 0, st>>>(g.count, E, n_shared, T, item_rows, g.offsets, g.items, ctrl, counts_out,
                                      offsets_out);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const int np = n + (n_shared ? T : 0);
  grid = (np + 255) / 256;
  if (grid > 4096) grid = 4096;
  k_group_scatter<<<grid, 256, 0, st>>>(ids, topk_w, T, k, E, n_shared, W, g.bits, g.prefix, g.offsets, g.perm,
                                        g.row_tok, g.row_w, g.inv);
  return hipGetLastError();
}

}  // namespace moe
