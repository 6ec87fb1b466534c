// The C interface (include/moe_route.h): host-side validation, workspace carving and launches.
// Nothing here allocates device memory; every error is reported before anything is enqueued.
#include <mutex>

#include "kernels.hpp"

namespace moe {

KernelEvents g_kernel_events = {kTimeNone, nullptr, nullptr};

// Workspace carve-up for up to `T` tokens.  The first kCtrlBytes hold the control words
// (error word, counters) and, at byte 3072, the residency miss flags (one byte per expert).
struct WsLayout {
  size_t tasks, h, y_pairs, logits, ids, w, slots, miss_ids, miss_flag;
  // prefill region
  size_t x16, bits, prefix, count, offsets, items, perm, row_tok, row_w, inv, h16, y_rows;
  size_t total;
};

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Pairs of a decode step of T tokens (routed t*k + j, then shared T*k + t).
static int decode_pairs(const moe_dims* d, int T) {
  const int Td = T < kMaxDecodeTok ? T : kMaxDecodeTok;
  return Td * (d->top_k + d->n_shared);
}

static WsLayout ws_layout(const moe_dims* d, int T) {
  WsLayout L{};
  const int Td = T < kMaxDecodeTok ? T : kMaxDecodeTok;
  const int pairs_d = decode_pairs(d, T);
  size_t off = kCtrlBytes;
  L.miss_flag = 3072;
  L.tasks = off;
  off = align256(off + sizeof(DecodeTask) * (size_t)decode_max_tasks(Td, d->top_k, d->n_shared));
  L.h = off;
  off = align256(off + sizeof(float) * (size_t)pairs_d * d->ffn);
  L.y_pairs = off;
  off = align256(off + sizeof(float) * (size_t)pairs_d * d->hidden);
  L.logits = off;
  off = align256(off + sizeof(float) * (size_t)T * d->n_experts);
  L.ids = off;
  off = align256(off + sizeof(int32_t) * (size_t)T * d->top_k);
  L.w = off;
  off = align256(off + sizeof(float) * (size_t)T * d->top_k);
  L.slots = off;
  off = align256(off + sizeof(int32_t) * (size_t)T * d->top_k);
  L.miss_ids = off;
  off = align256(off + sizeof(int32_t) * (size_t)d->n_experts);
  // prefill: grouping and grouped-GEMM buffers for T tokens
  const size_t W = ((size_t)T + 31) / 32;
  const size_t P = (size_t)T * (d->top_k + d->n_shared);
  L.x16 = off;
  off = align256(off + 2 * (size_t)T * d->hidden);
  L.bits = off;
  off = align256(off + 4 * (size_t)d->n_experts * W);
  L.prefix = off;
  off = align256(off + 4 * (size_t)d->n_experts * W);
  L.count = off;
  off = align256(off + 4 * (size_t)d->n_experts);
  L.offsets = off;
  off = align256(off + 4 * ((size_t)d->n_experts + 2));
  L.items = off;
  off = align256(off + sizeof(TileItem) * (size_t)prefill_max_items(T, d->top_k, d->n_experts, d->n_shared));
  L.perm = off;
  off = align256(off + 4 * P);
  L.row_tok = off;
  off = align256(off + 4 * P);
  L.row_w = off;
  off = align256(off + 4 * P);
  L.inv = off;
  off = align256(off + 4 * P);
  L.h16 = off;
  off = align256(off + 2 * P * d->ffn);
  L.y_rows = off;
  off = align256(off + 2 * P * d->hidden);
  L.total = off;
  return L;
}

// Largest decode batch of the FFN kernels for these activations: 16 bf16 tokens when F <= 2048
// (the down launch stages every token's h rows, hi and lo, in LDS), else 8 (an fp32 token takes
// two matrix-core rows).
static int decode_limit(const moe_dims* d, int x_dtype) {
  return (x_dtype == MOE_BF16 && d->ffn <= kMaxDecodeF16Tok) ? kMaxDecodeTok : kMaxDecodeTokNarrow;
}
// ... and of the routing launch (the router GEMV's rows: one per bf16 token, two per fp32 token;
// an fp32 router stages the tokens in LDS as fp32).
static int route_decode_limit(int x_dtype, int r_dtype) {
  return (x_dtype == MOE_BF16 && r_dtype == MOE_BF16) ? kMaxDecodeTok : kMaxDecodeTokNarrow;
}
static int layer_decode_limit(const moe_dims* d, int x_dtype, int r_dtype) {
  const int a = decode_limit(d, x_dtype), b = route_decode_limit(x_dtype, r_dtype);
  return a < b ? a : b;
}

// ---- prefill plans: the tuned table, a default, and a process-wide override for the tuner -------
struct TunedPlanRow {
  int H, F, E, k, fmt, t_lo, t_hi;
  PrefillPlan plan;
};
static const TunedPlanRow kTunedPlans[] = {
#include "tuned_plans.inc"
    {0, 0, 0, 0, 0, 0, 0, {0, 0, 0, 0}}  // end marker
};

static PrefillPlan g_forced_plan;
static bool g_plan_forced = false;

// Without a table row: 128-row items, the pipelined kernels where they are built, and the router
// GEMM's token rows per work where each router kernel was measured faster: 64-row works from 3,072
// tokens with the pipelined router kernel (E a multiple of 128, H / 128 = 8, 16 or 32), from 16K
// tokens with the general one (half the router-weight re-reads, still thousands of works).
static PrefillPlan default_plan(const moe_dims* d, int T) {
  PrefillPlan p;
  p.item_rows = 128;
  p.gate_up = p.down = kGemmPipe128;
  const int nk = d->hidden / 128;
  const bool pipe_router = d->n_experts % 128 == 0 && d->hidden % 128 == 0 && (nk == 8 || nk == 16 || nk == 32);
  p.router_rows = T >= (pipe_router ? 3072 : 16385) ? 64 : 32;
  return p;
}

static PrefillPlan plan_for(const moe_dims* d, int T) {
  if (g_plan_forced) return g_forced_plan;
  for (const TunedPlanRow& r : kTunedPlans) {
    if (r.H == 0) break;
    if (r.H == d->hidden && r.F == d->ffn && r.E == d->n_experts && r.k == d->top_k && r.fmt == d->format &&
        T >= r.t_lo && T <= r.t_hi)
      return r.plan;
  }
  return default_plan(d, T);
}

static int check_plan(const moe_prefill_plan* p) {
  if (p->item_rows != 64 && p->item_rows != 128) return MOE_EINVAL;
  if (p->router_rows != 32 && p->router_rows != 64) return MOE_EINVAL;
  for (int k : {p->gate_up_kernel, p->down_kernel}) {
    if (k < kGemmPipe128 || k > kGemmGeneral) return MOE_EINVAL;
    if (k == kGemmPipe64Deep && p->item_rows != 64) return MOE_EINVAL;
  }
  return MOE_OK;
}

static int check_dims(const moe_dims* d) {
  if (!d) return MOE_EINVAL;
  if (d->hidden <= 0 || d->ffn <= 0 || d->n_experts <= 0 || d->top_k <= 0) return MOE_EINVAL;
  if (d->n_shared != 0 && d->n_shared != 1) return MOE_EINVAL;
  if (d->top_k > d->n_experts) return MOE_EINVAL;
  if (d->block != kBlock) return MOE_EUNSUPPORTED;
  if (d->format != MOE_FMT_Q4_0 && d->format != MOE_FMT_CB4 && d->format != MOE_FMT_AFFINE4) return MOE_EUNSUPPORTED;
  // rows are whole groups of 4 blocks (the interleaved code layout)
  if (d->hidden % kGroupElems || d->ffn % kGroupElems) return MOE_EINVAL;
  if (d->hidden > 4096 || d->ffn > 4096) return MOE_EUNSUPPORTED;
  if (d->top_k > kMaxK || d->n_experts > kMaxExperts) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

static int check_ws(const moe_dims* d, int T, const void* ws, size_t ws_bytes) {
  if (!ws || ((uintptr_t)ws & 255)) return MOE_EWORKSPACE;
  if (ws_bytes < ws_layout(d, T).total) return MOE_EWORKSPACE;
  return MOE_OK;
}

static int check_weights(const moe_dims* d, const moe_layer_weights* w, const int32_t* table) {
  if (!w || !w->arena) return MOE_EINVAL;
  if (w->n_slots <= 0) return MOE_EINVAL;
  if (w->slot_stride < blob_layout(d->hidden, d->ffn, d->format).total || (w->slot_stride % 4096)) return MOE_EINVAL;
  if (((uintptr_t)w->arena & 255)) return MOE_EINVAL;
  if (d->n_shared == 1 && (!w->shared_blob || ((uintptr_t)w->shared_blob & 15))) return MOE_EINVAL;
  if (d->n_shared == 0 && w->shared_blob) return MOE_EINVAL;
  if (!table && w->n_slots < d->n_experts) return MOE_EINVAL;
  return MOE_OK;
}

static int check_dtype(int dt) { return (dt == MOE_F32 || dt == MOE_BF16) ? MOE_OK : MOE_EUNSUPPORTED; }

// Activations, outputs and the router matrix are moved with 16-byte vector accesses.
static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

static int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

static int32_t* ctrl_of(void* ws) { return (int32_t*)ws; }

template <typename T>
static T* at(void* ws, size_t off) {
  return (T*)((uint8_t*)ws + off);
}

static DoorbellArgs bell_args(const moe_doorbell* b) {
  DoorbellArgs a{};
  if (b) {
    a.active = 1;
    a.host_miss_ids = b->host_miss_ids;
    a.host_miss_count = b->host_miss_count;
    a.host_step_ids = b->host_step_ids;
    a.ready = b->ready;
    a.epoch = b->epoch;
  }
  return a;
}

static int check_bell(const moe_doorbell* b) {
  if (!b) return MOE_OK;
  if (!b->host_miss_ids || !b->host_miss_count || !b->ready) return MOE_EINVAL;
  return MOE_OK;
}

// route: logits + top-k.  Inputs validated by the caller.
static int do_route(const moe_dims* d, const void* x, int x_dtype, int T, const void* router, int r_dtype,
                    const float* bias, int32_t* ids, float* w, float* logits, void* ws, hipStream_t st) {
  const WsLayout L = ws_layout(d, T);
  float* lg = logits ? logits : at<float>(ws, L.logits);
  int rc;
  if (T > route_decode_limit(x_dtype, r_dtype)) {
    // long batches: router GEMM on MFMA (bf16 x bf16, fp32 accumulation)
    if (x_dtype != MOE_BF16 || r_dtype != MOE_BF16 || d->hidden % 128) return MOE_EUNSUPPORTED;
    rc = hip_status(launch_router_gemm(x, router, bias, T, d->n_experts, d->hidden, lg, plan_for(d, T).router_rows, st));
    if (rc) return rc;
    return hip_status(launch_topk(lg, T, d->n_experts, d->top_k, ids, w, ctrl_of(ws), st));
  }
  // short batches: router GEMV whose last workgroup selects the top-k
  return hip_status(launch_decode_route(x, x_dtype, router, r_dtype, bias, T, d->n_experts, d->hidden, d->top_k,
                                        d->n_shared, lg, ids, w, ctrl_of(ws), false, nullptr, 0, nullptr, nullptr,
                                        DoorbellArgs{}, st));
}

static Codebook codebook_of(const moe_dims* d) {
  Codebook cb;
  for (int i = 0; i < 4; ++i)
    cb.w[i] = (uint32_t)(uint8_t)d->codebook[4 * i] | ((uint32_t)(uint8_t)d->codebook[4 * i + 1] << 8) |
              ((uint32_t)(uint8_t)d->codebook[4 * i + 2] << 16) | ((uint32_t)(uint8_t)d->codebook[4 * i + 3] << 24);
  return cb;
}

static ExpertSource source_of(const moe_dims* d, const moe_layer_weights* w, const int32_t* table) {
  ExpertSource s;
  s.arena = w->arena;
  s.slot_stride = w->slot_stride;
  s.n_slots = w->n_slots;
  s.table = table;
  s.shared_blob = w->shared_blob;
  s.fmt = d->format;
  s.cb = codebook_of(d);
  return s;
}

// decode FFN; with `plan_done` the plan is already in the workspace (fused route), otherwise it
// is built from `ids` here.  `bell` (may be null) was or is rung by the planning kernel.
static int do_decode_ffn(const moe_dims* d, const moe_layer_weights* w, const int32_t* table,
                         const moe_doorbell* bell, const void* x, int x_dtype, int T, const int32_t* ids,
                         const float* topk_w, float* y, void* ws, hipStream_t st, bool plan_done) {
  const WsLayout L = ws_layout(d, T);
  int32_t* ctrl = ctrl_of(ws);
  DecodeTask* tasks = at<DecodeTask>(ws, L.tasks);
  int rc;
  if (!plan_done) {
    rc = hip_status(launch_decode_plan(ids, T, d->top_k, d->n_experts, d->n_shared, table, w->n_slots,
                                       at<int32_t>(ws, L.miss_ids), tasks, ctrl, bell_args(bell), st));
    if (rc) return rc;
  }
  if (bell) {
    if (hipStreamWaitValue32(st, bell->ready, bell->epoch, hipStreamWaitValueGte, 0xFFFFFFFFu) != hipSuccess)
      return MOE_EHIP;
  }
  // h: bf16 hi parts of every pair, then the lo parts
  uint16_t* h_hi = at<uint16_t>(ws, L.h);
  uint16_t* h_lo = h_hi + (size_t)decode_pairs(d, T) * d->ffn;
  return hip_status(launch_decode_ffn(d->hidden, d->ffn, d->top_k, d->n_shared, T,
                                      decode_max_tasks(T, d->top_k, d->n_shared), source_of(d, w, table), x, x_dtype,
                                      tasks, topk_w, h_hi, h_lo, at<float>(ws, L.y_pairs), y, ctrl, st));
}

static GroupBuffers group_buffers(const WsLayout& L, void* ws) {
  GroupBuffers g;
  g.bits = at<uint32_t>(ws, L.bits);
  g.prefix = at<int32_t>(ws, L.prefix);
  g.count = at<int32_t>(ws, L.count);
  g.offsets = at<int32_t>(ws, L.offsets);
  g.items = at<TileItem>(ws, L.items);
  g.perm = at<int32_t>(ws, L.perm);
  g.row_tok = at<int32_t>(ws, L.row_tok);
  g.row_w = at<float>(ws, L.row_w);
  g.inv = at<int32_t>(ws, L.inv);
  return g;
}

// The prefill kernels address activation rows with 32-bit element offsets: T H < 2^31.
static int prefill_shape_ok(const moe_dims* d, int T) {
  if ((int64_t)T * d->hidden > INT32_MAX) return MOE_EUNSUPPORTED;
  return (d->hidden % 256 == 0 && d->ffn % 128 == 0) ? MOE_OK : MOE_EUNSUPPORTED;
}

// prefill FFN after routing (and after any residency wait).
static int do_prefill_ffn(const moe_dims* d, const moe_layer_weights* w, const int32_t* table, const void* x, int T,
                          const int32_t* ids, const float* topk_w, float* y, void* ws, hipStream_t st) {
  const WsLayout L = ws_layout(d, T);
  int32_t* ctrl = ctrl_of(ws);
  const GroupBuffers g = group_buffers(L, ws);
  const PrefillPlan plan = plan_for(d, T);
  int rc = hip_status(
      launch_group(ids, topk_w, T, d->top_k, d->n_experts, d->n_shared, g, ctrl, nullptr, nullptr, st, plan.item_rows));
  if (rc) return rc;
  PrefillBuffers b;
  b.x16 = at<_Float16>(ws, L.x16);
  b.h16 = at<_Float16>(ws, L.h16);
  b.y_rows = at<_Float16>(ws, L.y_rows);
  return hip_status(launch_prefill_ffn(d->hidden, d->ffn, d->top_k, d->n_experts, d->n_shared, T, source_of(d, w, table),
                                       x, g, b, y, ctrl, plan, st));
}

// Host-side validation of a whole-layer call (everything but the workspace).
static int check_layer_args(const moe_dims* dims, const moe_layer_weights* w, const int32_t* table,
                            const moe_doorbell* bell, const void* x, int x_dtype, int n_tokens, const float* y) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (!x || !y || n_tokens < 1) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(y)) return MOE_EINVAL;
  if ((rc = check_dtype(x_dtype))) return rc;
  if ((rc = check_weights(dims, w, table))) return rc;
  if (!w->router || (rc = check_dtype(w->router_dtype))) return rc ? rc : MOE_EINVAL;
  if (!aligned16(w->router)) return MOE_EINVAL;
  if ((rc = check_bell(bell))) return rc;
  if (bell && !table) return MOE_EINVAL;
  // a doorbell goes with a decode-sized call, whose plan publishes the step's selections
  const int limit = layer_decode_limit(dims, x_dtype, w->router_dtype);
  if (bell && n_tokens > limit) return MOE_EUNSUPPORTED;
  if (n_tokens > limit) {
    if (x_dtype != MOE_BF16 || w->router_dtype != MOE_BF16) return MOE_EUNSUPPORTED;
    if ((rc = prefill_shape_ok(dims, n_tokens))) return rc;
  }
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" {

MOE_API size_t moe_expert_blob_bytes(const moe_dims* dims) {
  if (check_dims(dims) != MOE_OK) return 0;
  return (size_t)blob_layout(dims->hidden, dims->ffn, dims->format).total;
}

MOE_API size_t moe_workspace_bytes(const moe_dims* dims, int32_t max_tokens) {
  if (check_dims(dims) != MOE_OK || max_tokens < 1) return 0;
  return ws_layout(dims, max_tokens).total;
}

MOE_API const char* moe_strerror(int code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "unsupported dtype, block size or shape";
    case MOE_EWORKSPACE: return "workspace missing, misaligned or too small";
    case MOE_EHIP: return "HIP runtime call failed";
    case MOE_EDEVICE: return "the device reported an error (see moe_check_device_error bits)";
    case MOE_EFILL: return "slot-pool fill failed";
    default: return "unknown status code";
  }
}

MOE_API int moe_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws || ((uintptr_t)ws & 255) || ws_bytes < (size_t)kCtrlBytes) return MOE_EWORKSPACE;
  return hip_status(launch_fill_zero(ws, kCtrlBytes, (hipStream_t)stream));
}

MOE_API int moe_check_device_error(void* ws, void* stream, int32_t* bits_out) {
  if (!ws || ((uintptr_t)ws & 255)) return MOE_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  int32_t bits = 0;
  if (hipMemcpyAsync(&bits, ws, sizeof(int32_t), hipMemcpyDeviceToHost, st) != hipSuccess) return MOE_EHIP;
  if (hipStreamSynchronize(st) != hipSuccess) return MOE_EHIP;
  if (bits_out) *bits_out = bits;
  if (bits) {
    if (launch_fill_zero(ws, sizeof(int32_t), st) != hipSuccess) return MOE_EHIP;
    if (hipStreamSynchronize(st) != hipSuccess) return MOE_EHIP;
    return MOE_EDEVICE;
  }
  return MOE_OK;
}

MOE_API int moe_debug_kernel_events(int32_t which, void* start_event, void* stop_event) {
  if (which < kTimeNone || which > kTimeDecodeRoute) return MOE_EINVAL;
  if (which != kTimeNone && (!start_event || !stop_event)) return MOE_EINVAL;
  g_kernel_events.which = which;
  g_kernel_events.start = (hipEvent_t)start_event;
  g_kernel_events.stop = (hipEvent_t)stop_event;
  return MOE_OK;
}

MOE_API int moe_prefill_plan_get(const moe_dims* dims, int32_t n_tokens, moe_prefill_plan* out) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (!out || n_tokens < 1) return MOE_EINVAL;
  const PrefillPlan p = plan_for(dims, n_tokens);
  out->item_rows = p.item_rows;
  out->gate_up_kernel =
      prefill_kernel_fits(p.gate_up, 0, dims->hidden, dims->ffn, dims->format, p.item_rows) ? p.gate_up : kGemmGeneral;
  out->down_kernel =
      prefill_kernel_fits(p.down, 1, dims->hidden, dims->ffn, dims->format, p.item_rows) ? p.down : kGemmGeneral;
  out->router_rows = p.router_rows;
  return MOE_OK;
}

MOE_API int moe_debug_force_prefill_plan(const moe_prefill_plan* plan_or_null) {
  if (!plan_or_null) {
    g_plan_forced = false;
    return MOE_OK;
  }
  const int rc = check_plan(plan_or_null);
  if (rc) return rc;
  g_forced_plan.item_rows = plan_or_null->item_rows;
  g_forced_plan.gate_up = plan_or_null->gate_up_kernel;
  g_forced_plan.down = plan_or_null->down_kernel;
  g_forced_plan.router_rows = plan_or_null->router_rows;
  g_plan_forced = true;
  return MOE_OK;
}

MOE_API int moe_debug_dequant(const moe_dims* dims, const uint8_t* blob, int32_t matrix, float* out,
                              void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (!blob || !out || matrix < 0 || matrix > 2 || ((uintptr_t)blob & 3)) return MOE_EINVAL;
  return hip_status(launch_debug_dequant(dims->hidden, dims->ffn, dims->format, codebook_of(dims), blob, matrix, out,
                                         (hipStream_t)stream));
}

MOE_API int moe_route(const moe_dims* dims, const void* x, int32_t x_dtype, int32_t n_tokens, const void* router,
                      int32_t router_dtype, const float* bias, int32_t* topk_ids, float* topk_w,
                      float* logits_or_null, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (!x || !router || !topk_ids || !topk_w || n_tokens < 1) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(router)) return MOE_EINVAL;
  if ((rc = check_dtype(x_dtype)) || (rc = check_dtype(router_dtype))) return rc;
  if ((rc = check_ws(dims, n_tokens, ws, ws_bytes))) return rc;
  return do_route(dims, x, x_dtype, n_tokens, router, router_dtype, bias, topk_ids, topk_w, logits_or_null, ws,
                  (hipStream_t)stream);
}

MOE_API int moe_slot_lookup(const moe_dims* dims, const int32_t* layer_table, int32_t n_slots,
                            const int32_t* topk_ids, int32_t n_tokens, int32_t* slots, int32_t* miss_ids,
                            int32_t* miss_count, const moe_doorbell* bell_or_null, void* ws, size_t ws_bytes,
                            void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (!layer_table || !topk_ids || !slots || !miss_ids || !miss_count || n_tokens < 1 || n_slots < 1)
    return MOE_EINVAL;
  if ((rc = check_bell(bell_or_null))) return rc;
  // a doorbell publishes the step's selections too (the pool's recency policy needs the hits):
  // decode-sized calls only
  if (bell_or_null && n_tokens > kMaxDecodeTok) return MOE_EUNSUPPORTED;
  if ((rc = check_ws(dims, n_tokens, ws, ws_bytes))) return rc;
  const WsLayout L = ws_layout(dims, n_tokens);
  return hip_status(launch_lookup(topk_ids, n_tokens * dims->top_k, dims->n_experts, layer_table, n_slots, slots,
                                  at<uint8_t>(ws, L.miss_flag), miss_ids, miss_count, ctrl_of(ws),
                                  bell_args(bell_or_null), (hipStream_t)stream));
}

MOE_API int moe_group_tokens(const moe_dims* dims, const int32_t* topk_ids, int32_t n_tokens, int32_t* counts,
                             int32_t* offsets, int32_t* perm, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (!topk_ids || !counts || !offsets || !perm || n_tokens < 1) return MOE_EINVAL;
  if ((rc = check_ws(dims, n_tokens, ws, ws_bytes))) return rc;
  const WsLayout L = ws_layout(dims, n_tokens);
  GroupBuffers g = group_buffers(L, ws);
  g.perm = perm;  // routed pairs only (no shared bucket): perm[0 .. T*k) is the public output
  return hip_status(launch_group(topk_ids, nullptr, n_tokens, dims->top_k, dims->n_experts, 0, g, ctrl_of(ws), counts,
                                 offsets, (hipStream_t)stream));
}

MOE_API int moe_expert_ffn_decode(const moe_dims* dims, const moe_layer_weights* w, const int32_t* layer_table_or_null,
                                  const void* x, int32_t x_dtype, int32_t n_tokens, const int32_t* topk_ids,
                                  const float* topk_w, float* y, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (!x || !topk_ids || !topk_w || !y) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(y)) return MOE_EINVAL;
  if ((rc = check_dtype(x_dtype))) return rc;
  if (n_tokens < 1 || n_tokens > decode_limit(dims, x_dtype)) return MOE_EINVAL;
  if ((rc = check_weights(dims, w, layer_table_or_null))) return rc;
  if ((rc = check_ws(dims, n_tokens, ws, ws_bytes))) return rc;
  return do_decode_ffn(dims, w, layer_table_or_null, nullptr, x, x_dtype, n_tokens, topk_ids, topk_w, y, ws,
                       (hipStream_t)stream, false);
}

MOE_API int moe_expert_ffn_prefill(const moe_dims* dims, const moe_layer_weights* w,
                                   const int32_t* layer_table_or_null, const void* x, int32_t x_dtype,
                                   int32_t n_tokens, const int32_t* topk_ids, const float* topk_w, float* y, void* ws,
                                   size_t ws_bytes, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (!x || !topk_ids || !topk_w || !y || n_tokens < 1) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(y)) return MOE_EINVAL;
  if (x_dtype != MOE_BF16) return MOE_EUNSUPPORTED;
  if ((rc = check_weights(dims, w, layer_table_or_null))) return rc;
  if ((rc = prefill_shape_ok(dims, n_tokens))) return rc;
  if ((rc = check_ws(dims, n_tokens, ws, ws_bytes))) return rc;
  return do_prefill_ffn(dims, w, layer_table_or_null, x, n_tokens, topk_ids, topk_w, y, ws, (hipStream_t)stream);
}

MOE_API int moe_layer_forward(const moe_dims* dims, const moe_layer_weights* w, const int32_t* layer_table_or_null,
                              const moe_doorbell* bell_or_null, const void* x, int32_t x_dtype, int32_t n_tokens,
                              float* y, int32_t* topk_ids_out_or_null, float* topk_w_out_or_null, void* ws,
                              size_t ws_bytes, void* stream) {
  int rc = check_layer_args(dims, w, layer_table_or_null, bell_or_null, x, x_dtype, n_tokens, y);
  if (rc) return rc;
  if ((rc = check_ws(dims, n_tokens, ws, ws_bytes))) return rc;
  const bool prefill = n_tokens > layer_decode_limit(dims, x_dtype, w->router_dtype);
  hipStream_t st = (hipStream_t)stream;
  const WsLayout L = ws_layout(dims, n_tokens);
  int32_t* ids = topk_ids_out_or_null ? topk_ids_out_or_null : at<int32_t>(ws, L.ids);
  float* tw = topk_w_out_or_null ? topk_w_out_or_null : at<float>(ws, L.w);
  if (!prefill && n_tokens == 1 && !bell_or_null && x_dtype == MOE_BF16 && w->router_dtype == MOE_BF16 &&
      decode_select1_supported(dims->hidden, dims->ffn, dims->top_k, dims->n_shared, dims->n_experts)) {
    // one token, no doorbell: the router launch ends with its logits; the gate/up launch selects,
    // checks residency and plans (the router launch's last-workgroup step is off the path)
    float* logits = at<float>(ws, L.logits);
    rc = hip_status(launch_router_logits_bf16(x, w->router, w->router_bias, dims->n_experts, dims->hidden, logits, st));
    if (rc) return rc;
    uint16_t* h_hi = at<uint16_t>(ws, L.h);
    uint16_t* h_lo = h_hi + (size_t)decode_pairs(dims, 1) * dims->ffn;
    return hip_status(launch_decode_ffn_select1(dims->hidden, dims->ffn, dims->top_k, dims->n_shared,
                                                dims->n_experts, source_of(dims, w, layer_table_or_null), x, logits,
                                                at<DecodeTask>(ws, L.tasks), ids, tw, h_hi, h_lo, y, ctrl_of(ws),
                                                st));
  }
  if (!prefill) {
    // fused route: router GEMV, top-k, residency check, plan and doorbell in one kernel
    rc = hip_status(launch_decode_route(x, x_dtype, w->router, w->router_dtype, w->router_bias, n_tokens,
                                        dims->n_experts, dims->hidden, dims->top_k, dims->n_shared,
                                        at<float>(ws, L.logits), ids, tw, ctrl_of(ws), true, layer_table_or_null,
                                        w->n_slots, at<int32_t>(ws, L.miss_ids), at<DecodeTask>(ws, L.tasks),
                                        bell_args(bell_or_null), st));
    if (rc) return rc;
    return do_decode_ffn(dims, w, layer_table_or_null, bell_or_null, x, x_dtype, n_tokens, ids, tw, y, ws, st, true);
  }
  rc = do_route(dims, x, x_dtype, n_tokens, w->router, w->router_dtype, w->router_bias, ids, tw, nullptr, ws, st);
  if (rc) return rc;
  if (layer_table_or_null) {
    // residency check over all pairs (no doorbell at this size: a missing expert is an error)
    rc = hip_status(launch_lookup(ids, n_tokens * dims->top_k, dims->n_experts, layer_table_or_null, w->n_slots,
                                  at<int32_t>(ws, L.slots), at<uint8_t>(ws, L.miss_flag), at<int32_t>(ws, L.miss_ids),
                                  ctrl_of(ws) + kCtrlMissCount, ctrl_of(ws), DoorbellArgs{}, st));
    if (rc) return rc;
  }
  return do_prefill_ffn(dims, w, layer_table_or_null, x, n_tokens, ids, tw, y, ws, st);
}

}  // extern "C"

// ---- the layer without a caller workspace (moe_layer_forward_static) ----------------------------
// Its workspace is a file-scope device array, one per GPU, of kScratchBytes.  Host code never uses
// the array's name as an address: on the first call on a device (with that device current) its
// device address is looked up once with hipGetSymbolAddress and kept per device.
namespace moe {

constexpr size_t kScratchBytes = (size_t)MOE_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// Copies the call's device error word out to the caller and clears it (one thread).
__global__ void k_take_error(int32_t* ctrl, int32_t* out) {
  if (threadIdx.x == 0) {
    out[0] = ctrl[kCtrlError];
    ctrl[kCtrlError] = 0;
  }
}

// The current device's scratch address; the first call on a device looks it up and clears the
// control area on `st` (a fill kernel), so the counters and the error word start at zero.
static int scratch_for_current_device(hipStream_t st, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_EHIP;
    if (launch_fill_zero(p, kCtrlBytes, st) != hipSuccess) return MOE_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace moe

extern "C" MOE_API int moe_layer_forward_static(const moe_dims* dims, const moe_layer_weights* w,
                                                const int32_t* layer_table_or_null, const moe_doorbell* bell_or_null,
                                                const void* x, int32_t x_dtype, int32_t n_tokens, float* y,
                                                int32_t* topk_ids_out_or_null, float* topk_w_out_or_null,
                                                int32_t* device_error_out, void* stream) {
  int rc = check_layer_args(dims, w, layer_table_or_null, bell_or_null, x, x_dtype, n_tokens, y);
  if (rc) return rc;
  if (!device_error_out) return MOE_EINVAL;
  if (ws_layout(dims, n_tokens).total > kScratchBytes) return MOE_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  void* ws = nullptr;
  if ((rc = scratch_for_current_device(st, &ws))) return rc;
  rc = moe_layer_forward(dims, w, layer_table_or_null, bell_or_null, x, x_dtype, n_tokens, y, topk_ids_out_or_null,
                         topk_w_out_or_null, ws, kScratchBytes, stream);
  if (rc) return rc;
  k_take_error<<<1, 64, 0, st>>>(ctrl_of(ws), device_error_out);
  return hip_status(hipGetLastError());
}
