/*
 * moe_route.h -- C interface of the MI355X (gfx950) routed mixture-of-experts layer.
 *
 * The layer, as the pages describe it:
 *   - Betelgeuse news article (fanjiajia.top, "Betelgeuse: RTX 3060 12GB + 16GB ..."),
 *     section "mechanism: VRAM expert-slot pool, in-stream doorbell and victim cache":
 *     48 layers x 512 routed experts; each token takes 10 routed experts + 1 shared one;
 *     router and shared expert always resident; routed experts sit in a per-layer pool
 *     of HBM slots; a GPU-side check finds the misses and rings the host only on a miss;
 *     HBM and host copies of an expert are exclusive.  Section "what bit-exact means":
 *     the top-10 selection is exact and never altered; a failed expert read is an error,
 *     never a silent zero weight.
 *   - halogen-flash-server README, section "Bring your own GGUF": expert weights are a
 *     small set of values times a per-block scale (the Q4_0 family), repacked losslessly
 *     into the kernels' own layout; unsupported formats are refused by name.
 *   - Basalt README, section "The .basalt model file": quantized bytes used as stored.
 *
 * Readings where the pages are silent: router weights = softmax over the k selected
 * logits (they sum to 1 over the chosen experts); equal logits -> lower expert id first;
 * the optional per-expert bias is added to the logits before selection; the shared expert
 * has weight 1; the expert FFN is SwiGLU, y_e = Wd (silu(Wg x) * (Wu x)); the layer output
 * is y = sum_j w_j y_{e_j} (j = 0..k-1, selection order) + y_shared, with no residual.
 *
 * Conventions for every entry point
 *   - Tensor pointers are device pointers owned by the caller (allocated by any means);
 *     the library never allocates or frees device memory.  The activations x, the outputs y
 *     and the router matrix are moved with 16-byte vector accesses and must be 16-byte
 *     aligned (a hipMalloc'd buffer, and a whole-token slice of one, is); a misaligned one is
 *     MOE_EINVAL.  Its only process-wide state is
 *     the profiling selection of moe_debug_kernel_events (off unless a caller sets it).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work is
 *     enqueued asynchronously on it; the call returns once it is enqueued.
 *   - Every call validates its arguments on the host first and enqueues nothing when
 *     it returns an error.  Return value: MOE_OK (0) or a negative MOE_E* code.
 *   - n_tokens >= 1 wherever a token count is taken: an empty batch is MOE_EINVAL.
 *   - `ws` is a caller-owned device workspace of `ws_bytes` bytes (256-byte aligned),
 *     at least moe_workspace_bytes(dims, n_tokens).  It must be cleared once with
 *     moe_workspace_init before its first use; calls leave it reusable.  Calls that
 *     share one workspace must be ordered on one stream.
 *   - Faults the device detects (an expert id out of range, a slot index out of range,
 *     a selected expert that is not resident when its weights are needed, a NaN logit,
 *     an expert named twice in one token's top-k list, a value outside the fp16 range on
 *     the prefill path) set bits of an error word in `ws`; the outputs of that call are
 *     then invalid, never silently computed (Betelgeuse article, "what bit-exact means":
 *     a failed expert read is an error, not a zero weight).  moe_check_device_error reads
 *     and clears the word.
 *
 * Expert blob (one routed or shared expert; H = hidden, F = ffn), six sections in this order:
 *   [gate codes F*H/2][up codes F*H/2][down codes H*F/2]
 *   [gate scales F*H/16][up scales F*H/16][down scales H*F/16]          (bytes)
 * Gate and up have R = F rows over K = H inputs, down R = H rows over K = F inputs.  A code
 * u (0..15) stands for q = u - 8; blocks of 32 consecutive inputs of a row share one fp16
 * scale (little-endian), and the weight is q * scale (halogen README, "Bring your own GGUF":
 * a small set of values times a per-block scale, moved losslessly into the kernels' layout).
 * Each row is cut into K/128 groups of 128 inputs (four blocks), stored group-major:
 *   - codes of group c of row r: the 64-byte record at byte 64 * (c * R + r) of the section,
 *     sixteen little-endian 32-bit words.  Word 4g + i (g, i = 0..3) holds slice g of block i,
 *     that is inputs 128c + 32i + 8g .. 128c + 32i + 8g + 7: input 128c + 32i + 8g + 2j in bits
 *     4j..4j+3 and input 128c + 32i + 8g + 2j + 1 in bits 16+4j..16+4j+3 (j = 0..3);
 *   - scales of group c of row r: four fp16 values (blocks 4c .. 4c+3 of the row) at byte
 *     8 * (c * R + r) of the scale section.
 * With MOE_FMT_AFFINE4 three more sections follow, [gate mins][up mins][down mins], laid out
 * as the scales.  Model shape (H 2048, F 768): 2,654,208 bytes = 648 x 4 KiB (affine: 2,949,120).
 */
#ifndef MOE_ROUTE_H
#define MOE_ROUTE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_API __attribute__((visibility("default")))

enum moe_status {
  MOE_OK = 0,
  MOE_EINVAL = -1,        /* a NULL pointer, a size out of range, inconsistent dimensions */
  MOE_EUNSUPPORTED = -2,  /* valid request this library does not implement (dtype, block, shape) */
  MOE_EWORKSPACE = -3,    /* ws NULL, misaligned or smaller than moe_workspace_bytes */
  MOE_EHIP = -4,          /* a HIP runtime call failed (launch, copy, stream wait) */
  MOE_EDEVICE = -5,       /* the device error word was set (moe_check_device_error) */
  MOE_EFILL = -6          /* a slot-pool fill (host -> HBM expert copy) failed */
};

enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 };

/* Device error word bits (moe_check_device_error). */
enum moe_device_error {
  MOE_DERR_EXPERT_ID = 1,     /* a selected / given expert id outside [0, n_experts) */
  MOE_DERR_SLOT = 2,          /* a slot-table entry >= n_slots */
  MOE_DERR_NOT_RESIDENT = 4,  /* an expert needed by an FFN call has no slot (-1) */
  MOE_DERR_NAN = 8,           /* a NaN logit reached the selection */
  MOE_DERR_FILL = 16,         /* the slot-pool service reported a failed fill */
  MOE_DERR_DUP_ID = 32,       /* a token's top-k list names one expert twice */
  MOE_DERR_RANGE = 64         /* prefill: an activation, SwiGLU output or weighted expert row
                                 beyond the fp16 range (|v| > 65504) or not finite */
};

/* Largest token count of a decode call.  The pages' decode batches: concurrent streams (Basalt
 * README, "Concurrent requests: --parallel N", N = 1..8) and speculative verify batches, whose
 * tokens must come out byte-identical to the same request decoded alone and serially (halogen
 * README, "Quality: what is measured, and what is not", identity properties).  On the decode
 * path a token's output is bitwise the same at every batch size up to the limit:
 *   MOE_DECODE_MAX_TOKENS (16) with bf16 activations (and a bf16 router, for the calls that
 *   route) and F <= 2048;
 *   MOE_DECODE_MAX_TOKENS_NARROW (8) otherwise: an fp32 token takes two matrix-core rows, and 16
 *   tokens' SwiGLU rows of a wider F do not fit a workgroup's LDS.
 * Above the limit moe_layer_forward takes the prefill kernels. */
#define MOE_DECODE_MAX_TOKENS 16
#define MOE_DECODE_MAX_TOKENS_NARROW 8

/* Layer dimensions.  hidden = H, ffn = F (expert FFN width, shared expert too),
 * n_experts = E routed experts, top_k = k, n_shared = 0 or 1, block = 32 (the only
 * supported quantization block; anything else is MOE_EUNSUPPORTED).
 * Supported: H and F multiples of 128 (whole groups of the code layout; else MOE_EINVAL)
 * and at most 4096; 1 <= k <= 16; k <= E <= 1024 (beyond: MOE_EUNSUPPORTED).  The prefill
 * path (more than MOE_DECODE_MAX_TOKENS tokens) further needs H % 256 == 0, bf16
 * activations and router, and n_tokens * H < 2^31 (1,048,575 tokens at H = 2048; beyond:
 * MOE_EUNSUPPORTED). */
typedef struct moe_dims {
  int32_t hidden;
  int32_t ffn;
  int32_t n_experts;
  int32_t top_k;
  int32_t n_shared;
  int32_t block;
  int32_t format;        /* weight format (moe_format); 0 = MOE_FMT_Q4_0, so a zeroed tail is the default */
  int8_t codebook[16];   /* MOE_FMT_CB4: the 16 values a code stands for (times the block scale) */
} moe_dims;

/* Weight formats (halogen README, "Bring your own GGUF": the engine reads the IQ4_NL / IQ4_XS /
 * IQ3_S / Q4_0 family as a small set of values times a per-block scale, and Q4_K / Q5_K / Q5_1
 * as exact affine planes; other block layouts are refused by name).  With a block scale s (fp16):
 *   MOE_FMT_Q4_0     w = (u - 8) * s;
 *   MOE_FMT_CB4      w = codebook[u] * s, codebook = dims.codebook (16 signed 8-bit values);
 *   MOE_FMT_AFFINE4  w = u * s - m, with a second fp16 plane m per block (the blob's mins).
 * Any other value of dims.format is MOE_EUNSUPPORTED.  Q4_0 runs on every kernel; the other two
 * run on the general (non-pipelined) decode and prefill kernels. */
enum moe_format { MOE_FMT_Q4_0 = 0, MOE_FMT_CB4 = 1, MOE_FMT_AFFINE4 = 2 };

/* One layer's weights (all device pointers).
 *   router       [E][H], dtype router_dtype (MOE_F32 or MOE_BF16); row e scores expert e.
 *   router_bias  [E] fp32 added to the logits, or NULL.
 *   arena        expert blobs; the blob in slot s starts at arena + s * slot_stride.
 *   slot_stride  bytes; >= moe_expert_blob_bytes and a multiple of 4096 (the Betelgeuse
 *                article stores each expert as one 4 KB-aligned blob).
 *   n_slots      number of slots in the arena.
 *   shared_blob  the shared expert's blob when n_shared == 1 (always resident), else NULL. */
typedef struct moe_layer_weights {
  const void* router;
  int32_t router_dtype;
  const float* router_bias;
  const uint8_t* arena;
  int64_t slot_stride;
  int32_t n_slots;
  const uint8_t* shared_blob;
} moe_layer_weights;

/* Miss notification for a slot pool served by the host (Betelgeuse article, "mechanism":
 * the in-stream check rings a host doorbell only on a miss).
 *   host_miss_ids    host-mapped pinned int32[E]: the step's miss list (ascending ids).
 *   host_miss_count  host-mapped pinned int32[3]: [0] = number of misses, [2] = number of
 *                    selections written to host_step_ids, [1] = epoch, written last (the
 *                    host polls [1] == epoch, then reads the rest).
 *   ready            device-visible uint32 the stream waits on: work after the check
 *                    runs once *ready >= epoch.  With no miss the check kernel writes
 *                    *ready = epoch itself; otherwise the host writes it after the fills.
 *   epoch            this call's epoch (strictly increasing over calls).
 *   host_step_ids    optional host-mapped pinned int32[n_tokens * k] (or NULL): the step's
 *                    selections in (token, choice) order, written by the decode path
 *                    (<= MOE_DECODE_MAX_TOKENS tokens) before the epoch; a pool's
 *                    recency policy needs the hits as well as the misses. */
typedef struct moe_doorbell {
  int32_t* host_miss_ids;
  int32_t* host_miss_count;
  uint32_t* ready;
  uint32_t epoch;
  int32_t* host_step_ids;
} moe_doorbell;

/* Bytes of one expert blob (layout above) for `dims`; 0 if dims are invalid. */
MOE_API size_t moe_expert_blob_bytes(const moe_dims* dims);

/* Workspace bytes that every entry point below needs for up to `max_tokens` tokens;
 * 0 if dims are invalid or max_tokens < 1. */
MOE_API size_t moe_workspace_bytes(const moe_dims* dims, int32_t max_tokens);

/* Static message for a status code (never NULL). */
MOE_API const char* moe_strerror(int code);

/* Clears the control area at the start of `ws` (its first 4 KiB: error word, counters, miss
 * flags) with a fill kernel on `stream`.  Call once before the workspace's first use. */
MOE_API int moe_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Synchronizes `stream`, reads the device error word of `ws` into *bits_out (may be NULL)
 * and clears it.  Returns MOE_OK when the word was 0, MOE_EDEVICE otherwise. */
MOE_API int moe_check_device_error(void* ws, void* stream, int32_t* bits_out);

/* Profiling aid.  Until the next call, every launch of kernel `which` (1 = decode gate/up GEMV,
 * 2 = decode down GEMV, 3 = prefill gate/up grouped GEMM, 4 = prefill down grouped
 * GEMM, 5 = decode router GEMV; 0 = off) records the hipEvent_t `start_event` / `stop_event` (created by the caller with
 * timing enabled) around that kernel alone, via hipExtLaunchKernel.  Process-wide setting,
 * not for concurrent use from several threads. */
MOE_API int moe_debug_kernel_events(int32_t which, void* start_event, void* stop_event);

/* Prefill plan (halogen README, "Measured": the engine's GEMM plan carries choices measured on
 * the hardware).  How a prefill call of n_tokens runs: the rows per grouped-GEMM work item (64 or
 * 128), the grouped-GEMM kernel of the gate/up and of the down projection, and the router GEMM's
 * rows per work (32 or 64).  The library takes the plan from a table measured on MI355X per shape
 * and token range (tune.py in the package writes it), else a default.  Kernels:
 *   MOE_GEMM_PIPE128      8 waves x 512 weight rows, up to 128-row items, weights 1 chunk ahead;
 *   MOE_GEMM_PIPE64_DEEP  the same with up to 64-row items and weights 3 chunks ahead;
 *   MOE_GEMM_GENERAL      4 waves x 256 weight rows, every width and weight format.
 * The pipelined kernels exist at the model's reduction widths (gate/up over H = 2048, down over
 * F = 768), for every weight format except the affine one on MOE_GEMM_PIPE128; elsewhere the
 * general kernel runs whatever the plan says. */
enum moe_gemm_kernel { MOE_GEMM_PIPE128 = 0, MOE_GEMM_PIPE64_DEEP = 1, MOE_GEMM_GENERAL = 2 };
typedef struct moe_prefill_plan {
  int32_t item_rows;
  int32_t gate_up_kernel;
  int32_t down_kernel;
  int32_t router_rows;
} moe_prefill_plan;

/* The plan a prefill call of n_tokens with these dims runs (the kernels as they will run). */
MOE_API int moe_prefill_plan_get(const moe_dims* dims, int32_t n_tokens, moe_prefill_plan* out);

/* Tuning aid: every prefill call of the process runs `plan` (validated: item_rows 64 or 128,
 * MOE_GEMM_PIPE64_DEEP only with 64, router_rows 32 or 64; else MOE_EINVAL) until the next call;
 * NULL returns to the table.  Process-wide, not for concurrent use from several threads. */
MOE_API int moe_debug_force_prefill_plan(const moe_prefill_plan* plan_or_null);

/* Test entry point: dequantizes matrix `matrix` (0 = gate [F][H], 1 = up [F][H],
 * 2 = down [H][F]) of the expert blob at `blob` into fp32 `out` (row-major), exactly
 * (q * scale is exact in fp32).  Follows halogen README "Bring your own GGUF" (a small
 * set of values times a per-block scale). */
MOE_API int moe_debug_dequant(const moe_dims* dims, const uint8_t* blob, int32_t matrix,
                              float* out, void* stream);

/* Router and top-k selection (Betelgeuse article, "mechanism": 10 routed experts of 512
 * per token; "what bit-exact means": the selection is exact).
 *   x        [n_tokens][H], dtype x_dtype (MOE_F32 or MOE_BF16).
 *   router   [E][H], dtype router_dtype; bias [E] fp32 or NULL.
 *   topk_ids [n_tokens][k] int32 out: ids ranked by (logit desc, id asc).
 *   topk_w   [n_tokens][k] fp32 out: softmax over the k selected logits.
 *   logits   [n_tokens][E] fp32 out (x . router_e + bias_e), or NULL.
 * Logits accumulate in fp32 (bf16 x bf16 products are exact).  With more than
 * MOE_DECODE_MAX_TOKENS_NARROW tokens both x and router must be bf16. */
MOE_API int moe_route(const moe_dims* dims, const void* x, int32_t x_dtype, int32_t n_tokens,
                      const void* router, int32_t router_dtype, const float* bias,
                      int32_t* topk_ids, float* topk_w, float* logits_or_null,
                      void* ws, size_t ws_bytes, void* stream);

/* In-stream residency check (Betelgeuse article, "mechanism", scheduling row: expert id ->
 * slot on the GPU, host notified only on a miss).
 *   layer_table [E] int32: slot of each expert, -1 = not resident (cached in LDS).
 *   topk_ids    [n_tokens][k].
 *   slots       [n_tokens][k] int32 out: layer_table[id] (-1 for a miss).
 *   miss_ids    [E] int32 out: the distinct missing ids, ascending; miss_count [1] out.
 *   bell        optional doorbell (see moe_doorbell), or NULL.  With a doorbell the call also
 *               publishes the selections to bell->host_step_ids (when not NULL), so a pool
 *               knows the step's hits; it then takes at most MOE_DECODE_MAX_TOKENS tokens
 *               (more: MOE_EUNSUPPORTED).
 * Entries >= n_slots set MOE_DERR_SLOT; ids outside [0, E) set MOE_DERR_EXPERT_ID. */
MOE_API int moe_slot_lookup(const moe_dims* dims, const int32_t* layer_table, int32_t n_slots,
                            const int32_t* topk_ids, int32_t n_tokens, int32_t* slots,
                            int32_t* miss_ids, int32_t* miss_count, const moe_doorbell* bell_or_null,
                            void* ws, size_t ws_bytes, void* stream);

/* Grouping of the (token, choice) pairs p = t*k + j by expert: a stable counting sort.
 *   counts [E] out, offsets [E+1] out (exclusive prefix sums), perm [n_tokens*k] out:
 *   pair indices in (expert, p) order.  (halogen README, "Measured": the ordering step
 *   of the tokens moves prefill speed.)  A token's k ids must be distinct (as moe_route
 *   writes them); a repeated id sets MOE_DERR_DUP_ID and the outputs are invalid. */
MOE_API int moe_group_tokens(const moe_dims* dims, const int32_t* topk_ids, int32_t n_tokens,
                             int32_t* counts, int32_t* offsets, int32_t* perm,
                             void* ws, size_t ws_bytes, void* stream);

/* Expert FFNs + combine for a small batch (1..MOE_DECODE_MAX_TOKENS tokens with bf16 x and
 * F <= 2048, else 1..MOE_DECODE_MAX_TOKENS_NARROW; more: MOE_EINVAL).  Betelgeuse
 * article, "mechanism": every token runs its 10 routed experts and the shared expert, all of
 * them, none dropped; halogen README, "Bring your own GGUF": decode pays per byte of weights
 * read.  So each distinct selected expert's blob is streamed once per call, whatever the
 * number of tokens that chose it: 4-bit GEMVs, codes entering the matrix cores exactly,
 * fp32 accumulation, bandwidth-bound.
 *   layer_table [E] or NULL (NULL: expert e sits in slot e, all resident).
 *   x [n_tokens][H] (MOE_F32 or MOE_BF16); topk_ids / topk_w [n_tokens][k] (as moe_route
 *   writes them: a token's ids distinct, else MOE_DERR_DUP_ID); y [n_tokens][H] fp32 out.
 * Every expert a token selected must be resident (else MOE_DERR_NOT_RESIDENT). */
MOE_API int moe_expert_ffn_decode(const moe_dims* dims, const moe_layer_weights* w,
                                  const int32_t* layer_table_or_null, const void* x, int32_t x_dtype,
                                  int32_t n_tokens, const int32_t* topk_ids, const float* topk_w,
                                  float* y, void* ws, size_t ws_bytes, void* stream);

/* Expert FFNs + combine for a long batch (prefill).  halogen README, "Measured": prefill is
 * compute-bound and the ordering of tokens moves its speed; Basalt README, "Prompt chunks":
 * a chunk's cost per token keeps falling up to a few thousand tokens.  Tokens are grouped by
 * expert (a stable counting sort), and each expert's rows run as a grouped GEMM on MFMA with
 * dequantized fp16 tiles and fp32 accumulation, SwiGLU fused into the gate/up epilogue.
 * x must be MOE_BF16.  Arguments as moe_expert_ffn_decode, any n_tokens >= 1.  The fp16
 * operands and intermediates hold |v| <= 65504: a bf16 activation, a SwiGLU output or a
 * router-weighted expert row beyond that sets MOE_DERR_RANGE (the output is then invalid). */
MOE_API int moe_expert_ffn_prefill(const moe_dims* dims, const moe_layer_weights* w,
                                   const int32_t* layer_table_or_null, const void* x, int32_t x_dtype,
                                   int32_t n_tokens, const int32_t* topk_ids, const float* topk_w,
                                   float* y, void* ws, size_t ws_bytes, void* stream);

/* The whole layer (Betelgeuse article, "mechanism": router and shared expert resident, 10
 * routed experts of 512 per token, the residency check in the stream and the host rung only
 * on a miss): route -> residency check -> (wait for fills) -> expert FFNs -> combine.
 * Uses the decode kernels up to the decode limit (MOE_DECODE_MAX_TOKENS for bf16 x and router
 * and F <= 2048, else MOE_DECODE_MAX_TOKENS_NARROW) and the prefill kernels above.  With a layer_table and a doorbell, misses are reported to the host and the FFNs
 * run after *bell->ready >= bell->epoch (the host fills the slots and updates the table
 * meanwhile); a doorbell is taken only by a decode-sized call (n_tokens within the decode
 * limit; more: MOE_EUNSUPPORTED), since the host's recency policy needs the
 * step's selections.  topk_ids_out / topk_w_out [n_tokens][k] receive the routing if not
 * NULL. */
MOE_API int moe_layer_forward(const moe_dims* dims, const moe_layer_weights* w,
                              const int32_t* layer_table_or_null, const moe_doorbell* bell_or_null,
                              const void* x, int32_t x_dtype, int32_t n_tokens, float* y,
                              int32_t* topk_ids_out_or_null, float* topk_w_out_or_null,
                              void* ws, size_t ws_bytes, void* stream);

/* The whole layer without a caller workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).  Same
 * arguments and results as moe_layer_forward, with two differences:
 *   - the workspace is a library-owned static device array of MOE_STATIC_SCRATCH_BYTES per GPU
 *     (held from the first call on that GPU until the process ends); a call whose workspace
 *     would exceed it (moe_workspace_bytes(dims, n_tokens) > MOE_STATIC_SCRATCH_BYTES; the
 *     model shape fits up to about 100 tokens) returns MOE_EWORKSPACE, enqueueing nothing;
 *   - device_error_out (device int32[1], required) receives the call's device error bits
 *     (0 = none; the moe_device_error bits otherwise), copied from the array and cleared there
 *     by the call's last kernel.
 * It calls no hipMalloc, hipFree or allocating routine.  Every call on one GPU shares that GPU's
 * array: calls that may overlap on one GPU (different streams, or other threads) race and must be
 * ordered by the caller.  The first call on a GPU looks the array up and clears its control words
 * on `stream`. */
#define MOE_STATIC_SCRATCH_BYTES (8u << 20)
MOE_API int moe_layer_forward_static(const moe_dims* dims, const moe_layer_weights* w,
                                     const int32_t* layer_table_or_null, const moe_doorbell* bell_or_null,
                                     const void* x, int32_t x_dtype, int32_t n_tokens, float* y,
                                     int32_t* topk_ids_out_or_null, float* topk_w_out_or_null,
                                     int32_t* device_error_out, void* stream);

/* ---- Host service of a per-layer expert-slot pool (decode calls) ----------------------------
 * Betelgeuse news article, section "mechanism: VRAM expert-slot pool, in-stream doorbell and
 * victim cache": a layer keeps a fixed number of HBM slots, the in-stream check rings the host
 * only on a miss, a miss is filled from host memory, and the HBM and host copies of an expert
 * are exclusive.  Policy (the article names none): least recently used among the slots whose
 * expert is not selected in the step, ties to the lower slot; misses placed in ascending id
 * order; recency stamped per selection in (token, choice) order.
 *
 * Use per layer call: moe_pool_arm -> moe_layer_forward(..., table, &bell, ...) on the compute
 * stream -> moe_pool_serve on the host (it blocks until the call's check has run, then
 * enqueues the copies, the table update and the release of the compute stream on its copy
 * streams).  Several layers' calls may be enqueued before their serves; serve them in the
 * same order.  A pool is used from one host thread and one pair of copy streams (or one).
 *
 * The compute stream's wait stalls whatever the runtime has queued behind it on the same
 * hardware queue, and the runtime spreads streams over a few such queues (4 by default).
 * Create the compute stream and the copy streams together, non-blocking, before other
 * streams (a framework's stream pool, graph capture streams) exist: a copy stream that ends
 * up behind the wait never runs, and the next serve then times out.  Each serve failure is
 * also reported on stderr with its epoch and reason. */
typedef struct moe_pool moe_pool;

#define MOE_POOL_MAX_SPARES 64

typedef struct moe_pool_stats {
  int64_t calls;       /* served calls */
  int64_t selections;  /* (token, choice) selections seen */
  int64_t misses;      /* distinct misses filled */
  int64_t bytes_h2d;   /* expert bytes copied host -> HBM */
  int64_t bytes_d2h;   /* expert bytes copied HBM -> host (exclusive swap) */
} moe_pool_stats;

/* Creates the service for one layer.  All memory is the caller's and must outlive the pool:
 *   arena, slot_stride, n_slots  device slots (as in moe_layer_weights), n_slots <= E;
 *   table          device int32[E]: written here (slot of each expert, -1 elsewhere) and kept
 *                  up to date by moe_pool_serve; pass it as the layer_table of the calls;
 *   initial        host int32[n_slots]: the distinct expert held by each slot, hottest first
 *                  (colder ones are evicted first); their blobs must already be in the slots;
 *   host_home      host array [E] of pinned host pointers: the blob of every expert not in
 *                  `initial`, NULL for those in it (the pool permutes these buffers);
 *   spares, n_spares  n_spares (1..MOE_POOL_MAX_SPARES) pinned host buffers holding no
 *                  expert, at spares + i * slot_stride; the pool permutes them with host_home
 *                  (a miss's victim goes to the oldest, the missed expert's buffer becomes the
 *                  newest); more spares let the copies out run ahead of the copies in;
 *   host_miss_ids  host-mapped pinned int32[E]; host_counts host-mapped pinned int32[3];
 *   host_step_ids  host-mapped pinned int32[MOE_DECODE_MAX_TOKENS * k];
 *   ready          device uint32 (set to 0 here).
 * Copies the table and the ready word synchronously.  Returns MOE_EINVAL on inconsistent
 * arguments (a slot holding an id out of range or twice, an expert with no or two homes). */
MOE_API int moe_pool_create(const moe_dims* dims, uint8_t* arena, int64_t slot_stride, int32_t n_slots,
                            int32_t* table, const int32_t* initial, uint8_t* const* host_home, uint8_t* spares,
                            int32_t n_spares, int32_t* host_miss_ids, int32_t* host_counts,
                            int32_t* host_step_ids, uint32_t* ready, moe_pool** pool_out);

/* Frees the pool object and its events (not the caller's memory).  Synchronize the pool's copy
 * streams first: the copies it enqueued and their event waits must have completed. */
MOE_API int moe_pool_destroy(moe_pool* pool);

/* The doorbell of the pool's next call (next epoch).  MOE_EINVAL if the previous call was
 * armed but not served. */
MOE_API int moe_pool_arm(moe_pool* pool, moe_doorbell* bell_out);

/* Serves the armed call: waits on the host until the check kernel has written the epoch
 * (polling host memory, at most timeout_us microseconds if > 0), places every miss, and
 * enqueues per miss a device->host copy of the victim into a spare buffer on d2h_stream and a
 * host->device copy of the missed expert into the victim's slot on h2d_stream (ordered after
 * that device->host copy by an event), then on h2d_stream the table and *ready = epoch.
 * h2d_stream_or_null NULL puts everything on d2h_stream.  With two streams the copies of the
 * two PCIe directions overlap; a device->host copy into a buffer waits for the host->device
 * copy that last read it, and a serve's first one waits for the previous serve's copies in
 * (its victims may be slots those filled).  fills_out (host int32[E][3] or NULL)
 * receives (expert, slot, evicted expert) per fill, n_fills_out their number.  On a timeout,
 * a bad doorbell or a failed copy the compute stream is still released (*ready = epoch), the
 * fill error bit is set in ws (when not NULL) and MOE_EFILL is returned. */
MOE_API int moe_pool_serve(moe_pool* pool, void* ws_or_null, void* d2h_stream, void* h2d_stream_or_null,
                           int32_t* fills_out, int32_t* n_fills_out, int64_t timeout_us);

/* Counters since creation. */
MOE_API int moe_pool_get_stats(const moe_pool* pool, moe_pool_stats* out);

/* The pool's current slot table (host int32[E]). */
MOE_API int moe_pool_get_table(const moe_pool* pool, int32_t* table_out);

/* Hot-expert profile (Betelgeuse article, "limits and licence": a profile file only seeds the
 * cache with hot experts; "mechanism": the package carries a hot-expert profile).
 * moe_pool_get_profile: host int64[E], the selections of every expert the pool has served
 * (hits and misses) since creation.
 * moe_profile_seed: from such counts, the initial residency of a pool of n_slots slots: the
 * n_slots experts with the most selections, hottest first (ties: lower id first), as
 * moe_pool_create's `initial` takes it (host int32[n_slots] out).  1 <= n_slots <= n_experts. */
MOE_API int moe_pool_get_profile(const moe_pool* pool, int64_t* counts_out);
MOE_API int moe_profile_seed(const int64_t* counts, int32_t n_experts, int32_t n_slots, int32_t* initial_out);

/* Slot lending (Basalt README, "Prompt chunks: --prefill": a prompt chunk's buffers are carved
 * from the expert cache's last slots for the length of the prompt, and the experts in those slots
 * are copied back afterwards).  moe_pool_lend lends the pool's last n slots (n_slots - n ..
 * n_slots - 1, one contiguous region of n * slot_stride bytes at *region_out, e.g. another call's
 * workspace): on `stream` it copies their experts out to host_bufs (caller's pinned host memory,
 * n * slot_stride bytes, which holds them meanwhile: the tiers stay exclusive) and marks them not
 * resident in the table.  Use the region only after those copies (same stream, or an event).
 * moe_pool_unlend copies the experts back on `stream` (after the caller's last use of the region
 * in that stream's order) and restores the table; the recency policy is as if nothing had been
 * lent.  Neither may be called while a call is armed; moe_pool_arm refuses while slots are lent
 * (MOE_EINVAL).  A failed copy enqueue returns MOE_EFILL with the lend state unchanged. */
MOE_API int moe_pool_lend(moe_pool* pool, int32_t n, uint8_t* host_bufs, void* stream, uint8_t** region_out);
MOE_API int moe_pool_unlend(moe_pool* pool, void* stream);

/* Test hook for the failure path: after `after_n` more successful copy enqueues, the pool treats
 * the next one as failed (the copy is not enqueued), as a failed hipMemcpyAsync would be: serve
 * then releases the compute stream with MOE_DERR_FILL set and returns MOE_EFILL (Betelgeuse article,
 * "what bit-exact means": a failed expert read is an error, never zero weights).  -1 = off. */
MOE_API int moe_pool_debug_fail_copies(moe_pool* pool, int32_t after_n);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ROUTE_H */
