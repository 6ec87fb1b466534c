// Declarations shared between the kernel sources and the C-ABI host layer.
#pragma once

#include <hip/hip_ext.h>

#include "common.hpp"

namespace moe {

// Profiling aid (moe_debug_kernel_events): launches of kernel `which` record `start` / `stop`
// around the kernel itself through hipExtLaunchKernelGGL.
enum TimedKernel { kTimeNone = 0, kTimeDecodeGateUp = 1, kTimeDecodeDown = 2, kTimePrefillGateUp = 3,
                   kTimePrefillDown = 4, kTimeDecodeRoute = 5 };
struct KernelEvents {
  int which;
  hipEvent_t start, stop;
};
extern KernelEvents g_kernel_events;

template <typename K, typename... Args>
hipError_t launch_timed(int which, K kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t st, Args... args) {
  if (which != kTimeNone && g_kernel_events.which == which)
    hipExtLaunchKernelGGL(kernel, grid, block, lds, st, g_kernel_events.start, g_kernel_events.stop, 0u, args...);
  else
    kernel<<<grid, block, lds, st>>>(args...);
  return hipGetLastError();
}

// One expert's work in a decode step: the tokens that chose it (a bitmask; a task holds every
// token of the step that chose its expert, so each expert's weights are read once) and, for a
// routed expert, the position j of the expert in each token's top-k list (4 bits per token).
// Token t of a routed task owns FFN output row (pair) t*k + j; of the shared task, T*k + t.
constexpr int kTaskTok = kMaxDecodeTok;

struct alignas(16) DecodeTask {
  int32_t expert;      // routed expert id, or -1 for the shared expert
  int32_t slot;        // slot resolved by the plan, or -1: look the table up when the FFN runs (a miss)
  uint32_t tok_mask;   // bit t: token t chose the expert
  uint32_t choice;     // bits 4t..4t+3: j of token t < 8 (routed tasks)
  uint32_t choice_hi;  // bits 4(t-8)..4(t-8)+3: j of token t >= 8
  uint32_t pad[3];
};

__host__ __device__ inline DecodeTask make_task(int32_t expert, int32_t slot, uint32_t tok_mask, uint32_t choice,
                                                uint32_t choice_hi) {
  DecodeTask t;
  t.expert = expert;
  t.slot = slot;
  t.tok_mask = tok_mask;
  t.choice = choice;
  t.choice_hi = choice_hi;
  t.pad[0] = t.pad[1] = t.pad[2] = 0u;
  return t;
}

// The shared expert's task over T tokens.
__host__ __device__ inline DecodeTask shared_task(int T) {
  return make_task(-1, -1, T >= 32 ? 0xFFFFFFFFu : ((1u << T) - 1u), 0u, 0u);
}

// Position j of token t in a routed task's expert list.
__host__ __device__ inline int task_choice(const DecodeTask& tk, int t) {
  return (int)(((t < 8 ? tk.choice : tk.choice_hi) >> (4 * (t & 7))) & 15u);
}

// Upper bound on decode tasks for T tokens: every routed task holds >= 1 pair, plus one task
// for the shared expert.
inline int decode_max_tasks(int T, int k, int n_shared) { return T * k + (n_shared ? 1 : 0); }

struct DoorbellArgs {
  int active;
  int32_t* host_miss_ids;
  int32_t* host_miss_count;
  int32_t* host_step_ids;  // may be null
  uint32_t* ready;
  uint32_t epoch;
};

// Where each expert blob lives: routed expert e in slot table[e] (identity without a table).
struct ExpertSource {
  const uint8_t* arena;
  int64_t slot_stride;
  int32_t n_slots;
  const int32_t* table;  // may be null
  const uint8_t* shared_blob;
  int32_t fmt;           // moe_format
  Codebook cb;           // MOE_FMT_CB4
};

// Prefill: one grouped-GEMM work item = up to item_rows (64 or 128, the plan's choice) consecutive
// rows of one bucket (bucket E = the shared expert) in bucket-sorted order.
constexpr int kTileRows = 128;    // the largest item
constexpr int kMinItemRows = 64;  // the smallest item a plan takes

struct TileItem {
  int32_t bucket;
  int32_t row0;  // first sorted row
  int32_t rows;  // 1..kTileRows
  int32_t pad;   // flags: kItemOnly
};
// The item holds all of its bucket's rows: its works are the only readers of the bucket's weights
// in the call, so they load them with the non-temporal hint.
constexpr int32_t kItemOnly = 1;

// Upper bound on work items: sum over non-empty buckets of ceil(c / item_rows).
inline int prefill_max_items(int T, int k, int E, int n_shared, int item_rows = kMinItemRows) {
  const long long rows = (long long)T * (k + n_shared);
  return (int)((rows + item_rows - 1) / item_rows) + E + 1;
}

// How a prefill call runs (moe_prefill_plan): the item size, the grouped-GEMM kernel of each
// projection and the router GEMM's rows per work.
enum GemmKernel { kGemmPipe128 = 0, kGemmPipe64Deep = 1, kGemmGeneral = 2 };
struct PrefillPlan {
  int item_rows;
  int gate_up;
  int down;
  int router_rows;
};

struct GroupBuffers {
  uint32_t* bits;    // [E][W] token bitmaps, W = ceil(T / 32)
  int32_t* prefix;   // [E][W] exclusive popcount prefix per bucket
  int32_t* count;    // [E]
  int32_t* offsets;  // [E + 2]
  TileItem* items;   // [prefill_max_items]
  int32_t* perm;     // [P] pair index of each sorted row
  int32_t* row_tok;  // [P] token of each sorted row
  float* row_w;      // [P] router weight of each sorted row (1 for the shared expert)
  int32_t* inv;      // [P] sorted row of each pair (-1 = invalid id)
};

// route.hip
hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w, int32_t* ctrl,
                       hipStream_t st);
hipError_t launch_lookup(const int32_t* ids, int n_pairs, int E, const int32_t* table, int n_slots,
                         int32_t* slots, uint8_t* miss_flag, int32_t* miss_ids, int32_t* miss_count,
                         int32_t* ctrl, const DoorbellArgs& bell, hipStream_t st);
hipError_t launch_decode_plan(const int32_t* ids, int T, int k, int E, int n_shared, const int32_t* table,
                              int n_slots, int32_t* miss_ids, DecodeTask* tasks, int32_t* ctrl,
                              const DoorbellArgs& bell, hipStream_t st);
hipError_t launch_decode_route(const void* x, int x_dtype, const void* Wr, int r_dtype, const float* bias, int T,
                               int E, int H, int k, int n_shared, float* logits, int32_t* ids, float* w,
                               int32_t* ctrl, bool plan, const int32_t* table, int n_slots, int32_t* miss_ids,
                               DecodeTask* tasks, const DoorbellArgs& bell, hipStream_t st);

// ffn_decode.hip
// One bf16 token, the whole-layer call without a doorbell: the router launch writes only the logits
// and the gate/up launch selects (each workgroup for itself) and plans.
hipError_t launch_router_logits_bf16(const void* x, const void* Wr, const float* bias, int E, int H, float* logits,
                                     hipStream_t st);
bool decode_select1_supported(int H, int F, int k, int n_shared, int E);
hipError_t launch_decode_ffn_select1(int H, int F, int k, int n_shared, int E, const ExpertSource& src,
                                     const void* x, const float* logits, DecodeTask* tasks, int32_t* ids_out,
                                     float* w_out, uint16_t* h_hi, uint16_t* h_lo, float* y, int32_t* ctrl,
                                     hipStream_t st);
hipError_t launch_decode_ffn(int H, int F, int k, int n_shared, int T, int max_tasks, const ExpertSource& src,
                             const void* x, int x_dtype, const DecodeTask* tasks, const float* topk_w,
                             uint16_t* h_hi, uint16_t* h_lo, float* y_pairs, float* y, int32_t* ctrl,
                             hipStream_t st);
// group.hip
hipError_t launch_group(const int32_t* ids, const float* topk_w, int T, int k, int E, int n_shared,
                        const GroupBuffers& g, int32_t* ctrl, int32_t* counts_out, int32_t* offsets_out,
                        hipStream_t st, int item_rows = kTileRows);

// ffn_prefill.hip
struct PrefillBuffers {
  _Float16* x16;   // [T][H]
  _Float16* h16;   // [P][F]
  _Float16* y_rows;  // [P][H] router-weighted expert outputs (fp16)
};
hipError_t launch_prefill_ffn(int H, int F, int k, int E, int n_shared, int T, const ExpertSource& src,
                              const void* x_bf16, const GroupBuffers& g, const PrefillBuffers& b, float* y,
                              int32_t* ctrl, const PrefillPlan& plan, hipStream_t st);
hipError_t launch_router_gemm(const void* x_bf16, const void* Wr_bf16, const float* bias, int T, int E, int H,
                              float* logits, int rows_per_work, hipStream_t st);
// Whether a grouped-GEMM kernel is built for these widths and this format.
bool prefill_kernel_fits(int kernel, int mode_down, int H, int F, int fmt, int item_rows);

hipError_t launch_debug_dequant(int H, int F, int fmt, const Codebook& cb, const uint8_t* blob, int matrix, float* out,
                                hipStream_t st);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st);

}  // namespace moe
