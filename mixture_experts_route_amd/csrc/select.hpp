// One wave's exact top-k of a row of logits (used by the router launch and by the one-token
// gate/up launch that selects for itself).  Betelgeuse news article, sections "mechanism" (10 of
// 512 routed experts per token) and "what bit-exact means" (the top-10 is exact).
#pragma once

#include "kernels.hpp"

namespace moe {

// ------------------------------------------------------------------------------------------
// Top-k of E logits per token, one wave per token.  Each lane holds the logits lane + 64 i;
// k rounds of (local best, DPP wave arg-max on (value desc, id asc)) pick the experts in rank
// order.  The weights are a softmax over the selected logits, summed in selection order.  NaN
// logits are flagged and never selected.
// ------------------------------------------------------------------------------------------
// NPER = logits per lane, 64 * NPER >= E (8 for E <= 512, 16 for E <= 1024).
struct NoOp {
  MOE_DEV void operator()() const {}
};

// Results go to ids_out / w_out, or (ids_out null) to lds_ids / lds_w.  after_loads() runs once
// the row's logits are in registers: work on other loads issued before the call waits there.
template <int NPER, typename AfterLoads = NoOp>
MOE_DEV void select_topk_wave(const float* row, int E, int k, int32_t* ids_out, float* w_out, int32_t* ctrl,
                              int32_t* lds_ids = nullptr, float* lds_w = nullptr, AfterLoads&& after_loads = NoOp{}) {
  constexpr int kPerLane = NPER;
  const int lane = threadIdx.x & 63;
  float v[kPerLane];
  // all loads are issued before any value is looked at: a clamped index instead of a branch keeps
  // the compiler from waiting on each load in turn
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const int e = lane + 64 * i;
    v[i] = row[e < E ? e : E - 1];
  }
  // key = (order-preserving value bits, ~id): a larger key is a larger logit, then a lower id.
  // NaN ranks as -inf (and is reported); ids >= E get key 0, below every real key.
  uint64_t key[kPerLane];
  bool nan_seen = false;
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const int e = lane + 64 * i;
    const bool nan = v[i] != v[i];
    nan_seen |= nan && e < E;
    const float f = nan ? -INFINITY : v[i];
    key[i] = e < E ? (((uint64_t)f32_order_key(f) << 32) | (uint32_t)~e) : 0ull;
  }
  after_loads();
  if (__any(nan_seen) && lane == 0) set_error(ctrl, MOE_DERR_NAN);
  uint64_t mine = 0;  // lane r keeps the r-th selection
  if constexpr (kPerLane == 8) {
    // each lane sorts its 8 keys (descending, odd-even merge network); a round takes the wave
    // maximum of the lanes' heads and the winning lane shifts its list by one.
    auto cx = [&](int a, int b) {
      const uint64_t hi = key[a] > key[b] ? key[a] : key[b];
      const uint64_t lo = key[a] > key[b] ? key[b] : key[a];
      key[a] = hi;
      key[b] = lo;
    };
    cx(0, 1); cx(2, 3); cx(4, 5); cx(6, 7);
    cx(0, 2); cx(1, 3); cx(4, 6); cx(5, 7);
    cx(1, 2); cx(5, 6);
    cx(0, 4); cx(1, 5); cx(2, 6); cx(3, 7);
    cx(2, 4); cx(3, 5);
    cx(1, 2); cx(3, 4); cx(5, 6);
    // A round reduces the heads' high words (the values) only; the lanes holding that value are
    // a ballot, and only when there are several (equal logits) does a second reduction over their
    // low words (the complemented ids) pick the lowest id.
    uint32_t hi[kPerLane], lo[kPerLane];
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      hi[i] = (uint32_t)(key[i] >> 32);
      lo[i] = (uint32_t)key[i];
    }
    for (int r = 0; r < k; ++r) {
      const uint32_t wh = wave_max_u32(hi[0]);
      const uint64_t tied = __builtin_amdgcn_ballot_w64(hi[0] == wh);
      int win_lane;
      if (__builtin_popcountll(tied) == 1) {
        win_lane = __builtin_ctzll(tied);
      } else {
        const uint32_t wl = wave_max_u32(hi[0] == wh ? lo[0] : 0u);
        win_lane = __builtin_ctzll(__builtin_amdgcn_ballot_w64(hi[0] == wh && lo[0] == wl));
      }
      const uint32_t wlo = (uint32_t)__builtin_amdgcn_readlane((int)lo[0], win_lane);
      mine = lane == r ? (((uint64_t)wh << 32) | wlo) : mine;
      const bool took = lane == win_lane;
#pragma unroll
      for (int i = 0; i < kPerLane - 1; ++i) {
        hi[i] = took ? hi[i + 1] : hi[i];
        lo[i] = took ? lo[i + 1] : lo[i];
      }
      hi[kPerLane - 1] = took ? 0u : hi[kPerLane - 1];
      lo[kPerLane - 1] = took ? 0u : lo[kPerLane - 1];
    }
  } else {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) best = key[i] > best ? key[i] : best;
    for (int r = 0; r < k; ++r) {
      const uint64_t win = wave_max_u64(best);
      mine = lane == r ? win : mine;
      // the lane holding the winner drops it; every lane recomputes its best (no branches)
      best = 0;
#pragma unroll
      for (int i = 0; i < kPerLane; ++i) {
        key[i] = key[i] == win ? 0ull : key[i];
        best = key[i] > best ? key[i] : best;
      }
    }
  }
  const int my_i = (int)~(uint32_t)mine;
  const float my_v = f32_from_order_key((uint32_t)(mine >> 32));
  // weights: softmax over the selected logits, denominator summed in selection order
  const float m = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(my_v)));
  const float ex = lane < k ? expf(my_v - m) : 0.f;
  float sum = 0.f;
  for (int r = 0; r < k; ++r) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), r));
  if (lane < k) {
    if (ids_out) {
      ids_out[lane] = my_i;
      w_out[lane] = ex / sum;
    } else {
      lds_ids[lane] = my_i;
      lds_w[lane] = ex / sum;
    }
  }
}

}  // namespace moe
