// Expert FFNs for a small batch of tokens (decode): 4-bit GEMVs on the matrix cores.
//
// Weights: halogen-flash-server README, "Bring your own GGUF" (small set of values x one scale
// per block, used as stored).  The layer: Betelgeuse news article, "mechanism" (10 routed + 1
// shared expert per token).  Decode pays per byte of weights read (halogen README, "Bring your
// own GGUF": an 8-bit trunk costs 2 GB more per token at 240 GB/s), so each selected expert's blob
// is streamed once from HBM per step, whatever the number of tokens (1 to 16) that chose it.
//
// Design (gfx950).  A VALU GEMV over 4-bit weights spends ~2 vector instructions per weight
// (unpack, dot, scale) and at one token that is as long as the weight stream itself.  Here the
// dot products run on the matrix cores: for a 16-row tile of a weight matrix and one block of 32
// inputs, one v_mfma_f32_16x16x32_bf16 takes
//   A = the activation rows (one row per token; fp32 inputs as two bf16 rows hi + lo, which
//       together carry 16 significant bits),
//   B = the block's codes as bf16 (128 + u) = q + 136, built with one shift and one mask-or per
//       code pair (exact),
//   C = -136 * sum_k A[m][k], itself one MFMA of A against a constant -136 operand,
// so D[m][n] = sum_k A[m][k] * q[n][k] (products exact, fp32 sums), and the block's scale is
// applied with one FMA per live D register.  The interleaved code layout gives each lane, with
// one 16-byte load, slice g of four consecutive blocks of its row: its share of four MFMA steps.
// What is left on the VALU is ~7 instructions per 8 weights of a lane plus the scale FMAs.
//
// Kernels of a step; no workgroup waits on another:
//   gate/up: the general kernel takes one workgroup per (task, 16-row tile of the F rows); its
//     waves split the H inputs in runs of 4 groups (512 inputs) and reduce through LDS.  The
//     pipelined kernel (4 to 16 bf16 tokens) gives each wave a whole 16-row tile over all H inputs,
//     its weight loads one or two chunks ahead; the single-token kernel also selects the token's
//     top-k from the logits itself.  Each applies SwiGLU and stores h = silu(g) * u of the task's
//     tokens as bf16 hi + lo, ready to be the down projection's A operand.
//   down: 16 output rows of a task per wave over all F inputs (general and pipelined kernels), or,
//     for one token, the output rows outermost with the combine in the same workgroup.  A rows are
//     the (hi, lo) row pairs of the task's tokens (a 16-row A block per 8 tokens), so one MFMA per
//     block covers both parts.  Writes each pair's output row y_e.
//   combine: y[t] = sum_j w[t][j] * y_{e_j}[t] (j = 0..k-1), then + y_shared[t]: fixed order,
//     done inside the down launch by the last workgroup to finish each row tile (a counter per
//     tile; the pair rows go through agent-scope stores and loads).
#include "kernels.hpp"
#include "select.hpp"

namespace moe {

constexpr int kGuQuadsPerWave = 4;  // gate/up: groups of 128 inputs per wave
constexpr int kGuRG = 2;            // gate/up: row groups of 16 per workgroup
constexpr int kGuRG1 = 1;           // gate/up, one token: row groups of 16 per workgroup
constexpr int kDnQuadsPerPass = 6;  // down: groups per load batch
constexpr int kDnWaves = 8;         // down: waves per workgroup
// down: row groups of 16 per wave (more output rows per staged activation tile when the tasks
// carry more tokens)
template <int MAXTOK>
constexpr int kDnRGW = MAXTOK >= 4 ? 2 : 1;
// down: h chunks (16 bytes) per thread held in registers while staging; sized so that F <= 1536
// needs no second pass
template <int MAXTOK>
constexpr int kDnStageChunks = (2 * MAXTOK * (1536 / 8) + 64 * kDnWaves - 1) / (64 * kDnWaves);
constexpr uint32_t kMagicPair = 0x43004300u;                         // bf16 pair (128, 128)
constexpr uint32_t kNeg136Pair = 0xC308C308u;                        // bf16 pair (-136, -136)

// A task's blob: the shared expert, the slot the plan resolved, or (for an expert that missed when
// the plan ran and was filled since) the table entry read now.
MOE_DEV const uint8_t* task_blob(const ExpertSource& s, const DecodeTask& tk) {
  if (tk.expert < 0) return s.shared_blob;
  int slot = tk.slot;
  if (slot < 0) slot = s.table ? s.table[tk.expert] : tk.expert;
  if (slot < 0 || slot >= s.n_slots) return nullptr;
  return s.arena + (int64_t)slot * s.slot_stride;
}

// The two constants of the code unpacking, held in registers (the nibble mask in a scalar register,
// the bf16 pair (128, 128) in a vector register) so that each output register is one
// v_and_or_b32 (plus a shift): with literal operands the compiler splits it into an and and an or.
struct Unpack {
  uint32_t mask, magic;
};
MOE_DEV Unpack make_unpack() {
  Unpack u;
  asm("s_mov_b32 %0, 0xf000f" : "=s"(u.mask));
  asm("v_mov_b32 %0, 0x43004300" : "=v"(u.magic));
  return u;
}

// One code word (8 elements of a slice) -> B operand: 8 bf16 values q + 136 = 128 + u.  Pair j of
// the word (its elements 2j and 2j+1 in bits 4j and 16 + 4j) becomes register j.
MOE_DEV bf16x8 codes_q136(uint32_t w, const Unpack& k) {
  uint4 p;
  p.x = (w & k.mask) | k.magic;
  p.y = ((w >> 4) & k.mask) | k.magic;
  p.z = ((w >> 8) & k.mask) | k.magic;
  p.w = ((w >> 12) & k.mask) | k.magic;
  return __builtin_bit_cast(bf16x8, p);
}
MOE_DEV bf16x8 codes_q136(uint32_t w) {
  uint4 p;
  p.x = (w & 0x000F000Fu) | kMagicPair;
  p.y = ((w >> 4) & 0x000F000Fu) | kMagicPair;
  p.z = ((w >> 8) & 0x000F000Fu) | kMagicPair;
  p.w = ((w >> 12) & 0x000F000Fu) | kMagicPair;
  return __builtin_bit_cast(bf16x8, p);
}

MOE_DEV bf16x8 const_neg136() {
  const uint4 p = make_uint4(kNeg136Pair, kNeg136Pair, kNeg136Pair, kNeg136Pair);
  return __builtin_bit_cast(bf16x8, p);
}

// ---- weight formats on the matrix cores -------------------------------------------------------
// One block of 32 inputs is one MFMA D = A B + C, and the block's scale s then multiplies D:
//   MOE_FMT_Q4_0:    B = 128 + u (= q + 136), C = -136 sum_k A  ->  D = sum A q;  acc += s D
//   MOE_FMT_AFFINE4: B = 128 + u,             C = -128 sum_k A  ->  D = sum A u;  acc += s D, and
//                    the block's -m sum_k A is (m / 128) C:      acc += (m / 128) C
//   MOE_FMT_CB4:     B = codebook[u] (8-bit integers are exact bf16), C = 0 ->  D = sum A cb[u]
// Products are exact in every format; the sums are fp32.
template <int FMT>
MOE_DEV bf16x8 fmt_offset() {
  constexpr uint32_t p = FMT == MOE_FMT_AFFINE4 ? 0xC300C300u : kNeg136Pair;  // bf16 pair -128 / -136
  return __builtin_bit_cast(bf16x8, make_uint4(p, p, p, p));
}
template <int FMT>
MOE_DEV float4v fmt_c(const bf16x8& A, const float4v& zero) {
  if constexpr (FMT == MOE_FMT_CB4) return zero;
  else return __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, fmt_offset<FMT>(), zero, 0, 0, 0);
}
// The B operand of one code word: 8 values, pair j (codes in bits 4j, 16 + 4j) in register j.
template <int FMT>
MOE_DEV bf16x8 fmt_b(uint32_t w, const uint32_t* cbt) {
  if constexpr (FMT == MOE_FMT_CB4) {
    uint4 p;
    p.x = cbt[code_pair_index(w, 0)];
    p.y = cbt[code_pair_index(w, 1)];
    p.z = cbt[code_pair_index(w, 2)];
    p.w = cbt[code_pair_index(w, 3)];
    return __builtin_bit_cast(bf16x8, p);
  } else {
    return codes_q136(w);
  }
}
// The same operand with the unpacking constants in registers (the pipelined kernels).
template <int FMT>
MOE_DEV bf16x8 pipe_b(uint32_t w, const Unpack& uk, const uint32_t* cbt) {
  if constexpr (FMT == MOE_FMT_CB4) return fmt_b<FMT>(w, cbt);
  else return codes_q136(w, uk);
}
// The 256-entry LDS table of the codebook format: entry (c1 << 4 | c0) = (bf16 cb[c0], bf16 cb[c1]).
MOE_DEV void fill_codebook_bf16(const Codebook& cb, uint32_t* cbt) {
  for (int i = threadIdx.x; i < 256; i += blockDim.x) {
    const uint32_t lo = f32_to_bf16_rne((float)codebook_value(cb, i & 15));
    const uint32_t hi = f32_to_bf16_rne((float)codebook_value(cb, i >> 4));
    cbt[i] = lo | (hi << 16);
  }
}

MOE_DEV uint32_t word_at(const uint4& c, int i) { return i == 0 ? c.x : i == 1 ? c.y : i == 2 ? c.z : c.w; }
MOE_DEV uint32_t word_at(const u32x4& c, int i) { return c[i]; }

// fp16 scale i (0..3) of a group's four block scales.
MOE_DEV float scale_at(const uint2& s, int i) {
  const uint32_t w = i < 2 ? s.x : s.y;
  return fp16_bits_to_f32((i & 1) ? (w >> 16) : (w & 0xFFFFu));
}
MOE_DEV float scale_at(const u32x2& s, int i) {
  const uint32_t w = s[i >> 1];
  return fp16_bits_to_f32((i & 1) ? (w >> 16) : (w & 0xFFFFu));
}


// Token of slot m of a task: the m-th set bit of its token mask (m < popcount(mask)).
MOE_DEV int task_token(uint32_t mask, int m) {
  uint32_t x = mask;
#pragma unroll
  for (int j = 0; j < kTaskTok - 1; ++j) x = j < m ? (x & (x - 1u)) : x;
  return __builtin_ctz(x);
}

// FFN output row (pair) of token t in a task.
MOE_DEV int task_pair(const DecodeTask& tk, int t, int T, int k) {
  return tk.expert < 0 ? T * k + t : t * k + task_choice(tk, t);
}

// Keeps every load above it ahead of the code below it: the loads of a wave's whole tile go out
// together, and the waits the compiler inserts before each group's MFMA steps then cover only
// that group's data (loads complete in order).
MOE_DEV void issue_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

MOE_DEV float4v mfma_bf16(const bf16x8& a, const bf16x8& b, const float4v& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Eight fp32 activations -> one bf16 part (0 = hi, 1 = lo) as an A operand; hi = RNE(x),
// lo = RNE(x - hi).
MOE_DEV uint4 split_part(const float4& a, const float4& b, int part) {
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t q[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t hi = f32_to_bf16_rne(v[e]);
    q[e] = part ? f32_to_bf16_rne(v[e] - __uint_as_float(hi << 16)) : hi;
  }
  return make_uint4(q[0] | (q[1] << 16), q[2] | (q[3] << 16), q[4] | (q[5] << 16), q[6] | (q[7] << 16));
}

struct DecodeArgs {
  ExpertSource src;
  const DecodeTask* tasks;
  int32_t* ctrl;
  const void* x;        // [T][H] bf16 or fp32
  uint16_t* h_hi;       // [P][F] bf16: SwiGLU output, high part
  uint16_t* h_lo;       // [P][F] bf16: low part
  float* y_pairs;       // [P][H] each pair's expert output
  const float* topk_w;  // [T][k]
  float* y;             // [T][H]
  int H, F, T, k, n_shared;
  int tiles_gu;  // workgroups per task, gate/up
  int tiles_dn;  // workgroups per task, down
  int32_t* tile_done;  // per down row tile: workgroups finished (control words, zero between calls)
  // one token, selection inside the gate/up launch: the router's logits [E], and where the plan
  // and the routing go (tasks for the down launch, the token's ids and weights)
  const float* sel_logits;
  DecodeTask* sel_tasks;
  int32_t* sel_ids;
  int E;
};

// One token: every gate/up workgroup selects the token's top-k from the router's logits itself (one
// wave, the router launch's algorithm), so the router launch ends with its logits.  Tasks are the k
// selected experts in ascending id, then the shared expert; the workgroup takes task blockIdx / tiles
// and workgroup 0 also writes the plan, the ids and the weights for the down launch and the caller.
MOE_DEV DecodeTask select_own_task(const DecodeArgs& a, int task) {
  __shared__ int32_t s_ids[kMaxK];
  __shared__ float s_w[kMaxK];
  __shared__ int32_t s_slot[8 * 64];
  __shared__ DecodeTask s_tk;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int E = a.E, k = a.k;
    // the slot of every expert, loaded with the logits (one wait covers both) and kept in LDS
    int32_t tab[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = min(lane + 64 * i, E - 1);
      tab[i] = a.src.table ? a.src.table[e] : e;
    }
    auto stage_slots = [&]() {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int e = lane + 64 * i;
        if (e < E) s_slot[e] = tab[i];
      }
    };
    select_topk_wave<8>(a.sel_logits, E, k, nullptr, nullptr, a.ctrl, s_ids, s_w, stage_slots);
    asm volatile("" ::: "memory");  // one wave: its LDS operations take effect in issue order
    const int my_id = lane < k ? s_ids[lane] : 0x7FFFFFFF;
    int rank = 0;  // position of selection `lane` in ascending expert id (ids are distinct)
#pragma unroll
    for (int i = 0; i < kMaxK; ++i) rank += (i < k && s_ids[i] < my_id) ? 1 : 0;
    const int my_slot = lane < k ? s_slot[lane < k ? my_id : 0] : -1;  // index clamped for the other lanes
    if (task < k) {
      const int j = __builtin_ctzll(__builtin_amdgcn_ballot_w64(lane < k && rank == task));
      if (lane == j) s_tk = make_task(my_id, my_slot, 1u, (uint32_t)j, 0u);
    } else if (lane == 0) {
      s_tk = shared_task(1);
    }
    if (blockIdx.x == 0) {
      if (lane < k) {
        a.sel_tasks[rank] = make_task(my_id, my_slot, 1u, (uint32_t)lane, 0u);
        a.sel_ids[lane] = my_id;
        ((float*)a.topk_w)[lane] = s_w[lane];
      }
      const bool bad = lane < k && my_slot >= a.src.n_slots;
      const int n_miss = __builtin_popcountll(__builtin_amdgcn_ballot_w64(lane < k && my_slot < 0));
      const bool any_bad = __any(bad);
      if (lane == 0) {
        int n_all = k;
        if (a.n_shared) a.sel_tasks[n_all++] = shared_task(1);
        a.ctrl[kCtrlNTasks] = n_all;
        a.ctrl[kCtrlMissCount] = n_miss;
        if (any_bad) set_error(a.ctrl, MOE_DERR_SLOT);
      }
    }
  }
  __syncthreads();
  return s_tk;
}

// ---- activation rows in LDS -----------------------------------------------------------------
// A task's A-operand rows (bf16) are copied once per workgroup into LDS, row m at m * (K + 8)
// elements: the 16-byte pad puts the 16 rows an MFMA fragment reads into 16 different bank
// groups.  Each thread loads its chunks (8 elements, 16 bytes) into registers before the weight
// loads are issued and writes them to LDS after: waiting for these loads (loads complete in order)
// then leaves the weight loads in flight.  (LDS DMA would save the registers, but the compiler
// cannot tell which outstanding load wrote LDS and waits for all of them before any LDS read.)
MOE_DEV int lds_row_stride(int K) { return K + 8; }


// Chunk c of this thread: index threadIdx.x + c * blockDim.x over rows * K / 8 chunks; row m,
// column col.
MOE_DEV void chunk_pos(int idx, int K, int& m, int& col) {
  m = idx / (K / 8);
  col = (idx - m * (K / 8)) * 8;
}

// Loads this thread's first MAXC chunks (clamped: no load under a branch).  Row m of the staged
// operand comes from src_row(m) (K bf16 elements).
template <int MAXC, typename SrcRow>
MOE_DEV void stage_load(u32x4 (&v)[MAXC], int rows, int K, SrcRow src_row) {
  const int n_chunks = rows * (K / 8);
  static_for<MAXC>([&](auto c) {
    const int idx = min((int)(threadIdx.x + c.value * blockDim.x), n_chunks - 1);
    int m, col;
    chunk_pos(idx, K, m, col);
    v[c.value] = *(const u32x4*)(src_row(m) + col);
  });
  __builtin_amdgcn_sched_barrier(0);  // these loads go out before the weight loads
}

// Writes the chunks to LDS (with MAY_OVERFLOW, any beyond MAXC per thread are copied directly), then a plain
// workgroup barrier (__syncthreads would also wait for every weight load still in flight).
template <bool MAY_OVERFLOW, int MAXC, typename SrcRow>
MOE_DEV void stage_store_sync(const u32x4 (&v)[MAXC], uint16_t* lds, int rows, int K, SrcRow src_row) {
  const int n_chunks = rows * (K / 8);
  static_for<MAXC>([&](auto c) {
    const int idx = threadIdx.x + c.value * blockDim.x;
    int m, col;
    chunk_pos(min(idx, n_chunks - 1), K, m, col);
    if (idx < n_chunks) *(u32x4*)(lds + m * lds_row_stride(K) + col) = v[c.value];
  });
  if constexpr (MAY_OVERFLOW) {
    for (int idx = threadIdx.x + MAXC * blockDim.x; idx < n_chunks; idx += blockDim.x) {
      int m, col;
      chunk_pos(idx, K, m, col);
      *(u32x4*)(lds + m * lds_row_stride(K) + col) = *(const u32x4*)(src_row(m) + col);
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// A fragment for one 16x16x32 step: lane (g, m) takes inputs k0 + 8 g .. +7 of row m (zero for
// rows >= rows).
MOE_DEV bf16x8 lds_fragment(const uint16_t* lds, int rows, int K, int m, int g, int k0) {
  const int mr = m < rows ? m : 0;
  uint4 v = *(const uint4*)(lds + mr * lds_row_stride(K) + k0 + 8 * g);
  if (m >= rows) v = make_uint4(0u, 0u, 0u, 0u);
  return __builtin_bit_cast(bf16x8, v);
}

// ---- gate/up: h[pair][r] = silu(Wg[r] . x) * (Wu[r] . x) for one task and 32 rows r ------------
// Workgroup = RG row groups of 16 rows x KS waves splitting the H inputs in runs of 4 groups
// (KS = H / 512).  A rows: token slot m of the task (bf16 x) or 2 m + part (fp32 x, hi / lo).
template <int MAXTOK, bool X_BF16, int RG, bool SEL = false, int FMT = MOE_FMT_Q4_0>
__global__ __launch_bounds__(1024) void k_decode_gate_up(DecodeArgs a) {
  constexpr int ROWS = X_BF16 ? MAXTOK : 2 * MAXTOK;
  constexpr int NR = ROWS < 4 ? ROWS : 4;                    // live D registers per lane
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  __shared__ uint32_t cbt[FMT == MOE_FMT_CB4 ? 256 : 1];

  const int task = blockIdx.x / a.tiles_gu;
  const int tile = blockIdx.x - task * a.tiles_gu;
  const int H = a.H, F = a.F;
  // ---- bf16 activations: the rows of every token of the step (row t = token t) are loaded
  // before the task is known (they do not depend on it) and stored to LDS once the weight loads
  // are issued; a lane picks its token slot's row when it reads its fragment.  fp32 rows (small
  // shapes only) are split into hi / lo bf16 rows of the task's tokens by the threads below.
  auto x_row = [&](int m) { return (const uint16_t*)a.x + (size_t)(m < a.T ? m : 0) * H; };
  // bf16: ROWS * H / 8 chunks over 64 RG KS threads, KS >= H / (128 kGuQuadsPerWave) waves per row
  // group, is at most MAXTOK kGuQuadsPerWave / (4 RG) per thread
  u32x4 xv[(MAXTOK * kGuQuadsPerWave / 4 + RG - 1) / RG];
  if constexpr (X_BF16) stage_load(xv, ROWS, H, x_row);
  DecodeTask tk;
  if constexpr (SEL) {
    static_assert(MAXTOK == 1 && X_BF16, "selection inside the launch: one bf16 token");
    tk = select_own_task(a, task);  // every task of the grid exists (k distinct experts + shared)
  } else {
    // the descriptor slot always exists (max_tasks of them): load it together with the count
    tk = a.tasks[task];
    if (task >= a.ctrl[kCtrlNTasks]) return;
  }
  const uint8_t* blob = task_blob(a.src, tk);
  if (!blob) {
    if (threadIdx.x == 0) set_error(a.ctrl, MOE_DERR_NOT_RESIDENT);
    return;
  }
  const BlobLayout lay = blob_layout(H, F, FMT);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int NQ = H / kGroupElems;
  const int KS = (NQ + kGuQuadsPerWave - 1) / kGuQuadsPerWave;  // waves per row group
  if constexpr (FMT == MOE_FMT_CB4) fill_codebook_bf16(a.src.cb, cbt);  // visible after the barrier below
  const int rg = wave / KS, kq = wave - rg * KS;
  const int row = (tile * RG + rg) * 16 + n;
  const int q0 = kq * kGuQuadsPerWave;
  const int nq = min(kGuQuadsPerWave, NQ - q0);
  const int n_tok = __builtin_popcount(tk.tok_mask);
  // A row of this lane in LDS: bf16, the token of slot n (none past the task's tokens); fp32, row n
  const int arow = X_BF16 ? (n < n_tok ? task_token(tk.tok_mask, n) : ROWS) : n;

  if constexpr (!X_BF16) {
    for (int c = threadIdx.x; c < ROWS * (H / 8); c += blockDim.x) {
      const int m = c / (H / 8), col = (c - m * (H / 8)) * 8;
      const int slot = m >> 1;
      const int tok = task_token(tk.tok_mask, slot < n_tok ? slot : 0);
      const float* xf = (const float*)a.x + (size_t)tok * H + col;
      *(uint4*)(smem + m * lds_row_stride(H) + col) = split_part(*(const float4*)xf, *(const float4*)(xf + 4), m & 1);
    }
  }

  // ---- weights: slice g of each group record of row `row` in this wave's K range, both
  // matrices, and the records' scales; unconditional (clamped groups), all issued now
  const uint8_t* gcode = blob + lay.gate_codes + (size_t)row * kGroupBytes + 16 * g;
  const uint8_t* ucode = blob + lay.up_codes + (size_t)row * kGroupBytes + 16 * g;
  const uint8_t* gscale = blob + lay.gate_scales + (size_t)row * kGroupScaleBytes;
  const uint8_t* uscale = blob + lay.up_scales + (size_t)row * kGroupScaleBytes;
  uint4 cg[kGuQuadsPerWave], cu[kGuQuadsPerWave];
  uint2 sg[kGuQuadsPerWave], su[kGuQuadsPerWave];
  uint2 mg[kGuQuadsPerWave], mu[kGuQuadsPerWave];  // affine format: the records' mins
#pragma unroll
  for (int qi = 0; qi < kGuQuadsPerWave; ++qi) {
    const int qq = min(q0 + qi, NQ - 1);  // record (qq, row) at 64 (qq F + row)
    cg[qi] = ld16_nt_u4(gcode + (size_t)qq * F * kGroupBytes);
    cu[qi] = ld16_nt_u4(ucode + (size_t)qq * F * kGroupBytes);
    sg[qi] = ld8_nt_u2(gscale + (size_t)qq * F * kGroupScaleBytes);
    su[qi] = ld8_nt_u2(uscale + (size_t)qq * F * kGroupScaleBytes);
    if constexpr (FMT == MOE_FMT_AFFINE4) {
      mg[qi] = ld8_nt_u2(gscale - lay.gate_scales + lay.gate_mins + (size_t)qq * F * kGroupScaleBytes);
      mu[qi] = ld8_nt_u2(uscale - lay.up_scales + lay.up_mins + (size_t)qq * F * kGroupScaleBytes);
    }
    __builtin_amdgcn_sched_barrier(0);  // group order kept: the waits below are per group
  }
  issue_fence();
  if constexpr (X_BF16) {
    stage_store_sync<false>(xv, smem, ROWS, H, x_row);
  } else {
    __syncthreads();
  }

  const float4v zero = {0.f, 0.f, 0.f, 0.f};
  float accg[NR], accu[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) accg[r] = accu[r] = 0.f;
#pragma unroll
  for (int qi = 0; qi < kGuQuadsPerWave; ++qi) {
    if (qi >= nq) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x8 A = lds_fragment(smem, ROWS, H, arow, g, (q0 + qi) * kGroupElems + 32 * i);
      const float4v O = fmt_c<FMT>(A, zero);
      const float4v Dg = mfma_bf16(A, fmt_b<FMT>(word_at(cg[qi], i), cbt), O);
      const float4v Du = mfma_bf16(A, fmt_b<FMT>(word_at(cu[qi], i), cbt), O);
      const float s_g = scale_at(sg[qi], i), s_u = scale_at(su[qi], i);
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        accg[r] = fmaf(s_g, Dg[r], accg[r]);
        accu[r] = fmaf(s_u, Du[r], accu[r]);
      }
      if constexpr (FMT == MOE_FMT_AFFINE4) {
        const float m_g = scale_at(mg[qi], i) * 0.0078125f, m_u = scale_at(mu[qi], i) * 0.0078125f;
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          accg[r] = fmaf(m_g, O[r], accg[r]);
          accu[r] = fmaf(m_u, O[r], accu[r]);
        }
      }
    }
  }

  // ---- reduce the K waves of each row group (LDS reused), SwiGLU, store h as bf16 hi + lo ----
  __syncthreads();
  float* red = (float*)smem;  // [wave][2][ROWS][16]
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int mr = 4 * g + r;  // lane (g, n) holds rows 4g + r of column n
    if (mr < ROWS) {
      red[((wave * 2 + 0) * ROWS + mr) * 16 + n] = accg[r];
      red[((wave * 2 + 1) * ROWS + mr) * 16 + n] = accu[r];
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < RG * 16 * MAXTOK; idx += blockDim.x) {
    const int r16 = idx / (16 * MAXTOK), rem = idx - r16 * 16 * MAXTOK;
    const int ts = rem >> 4, c = rem & 15;
    if (ts >= n_tok) continue;
    float gs = 0.f, us = 0.f;
    for (int w = r16 * KS; w < (r16 + 1) * KS; ++w) {
      if constexpr (X_BF16) {
        gs += red[((w * 2 + 0) * ROWS + ts) * 16 + c];
        us += red[((w * 2 + 1) * ROWS + ts) * 16 + c];
      } else {
        gs += red[((w * 2 + 0) * ROWS + 2 * ts) * 16 + c] + red[((w * 2 + 0) * ROWS + 2 * ts + 1) * 16 + c];
        us += red[((w * 2 + 1) * ROWS + 2 * ts) * 16 + c] + red[((w * 2 + 1) * ROWS + 2 * ts + 1) * 16 + c];
      }
    }
    const float h = silu(gs) * us;
    const uint32_t hi = f32_to_bf16_rne(h);
    const uint32_t lo = f32_to_bf16_rne(h - __uint_as_float(hi << 16));
    const size_t o = (size_t)task_pair(tk, task_token(tk.tok_mask, ts), a.T, a.k) * F + (tile * RG + r16) * 16 + c;
    a.h_hi[o] = (uint16_t)hi;
    a.h_lo[o] = (uint16_t)lo;
  }
}

static size_t gate_up_lds_bytes(int H, int rows, int waves) {
  const size_t xs = (size_t)rows * (H + 8) * 2;
  const size_t red = (size_t)waves * 2 * rows * 16 * 4;
  return xs > red ? xs : red;
}

// ---- combine inside the down kernels ------------------------------------------------------------
// Each down workgroup writes its rows of every pair with agent-scope stores (written through to
// the coherence point the XCDs share), waits for them, and counts itself in its row tile's
// counter; the workgroup that completes a tile's count (every task's workgroup for those rows has
// finished) combines the tile's rows after an agent-scope acquire:
// y[t][o] = sum_j w[t][j] * y_pair[t k + j][o], then + y_pair[T k + t][o], in that order.
// No workgroup waits on another.
// Invariant this rests on: every pair-row write the combining workgroup reads is such an
// agent-scope store, completed (s_waitcnt vmcnt(0)) before the relaxed counter increment.  There
// is no release fence: a plain store added to the pair rows would stay in its XCD's L2, and the
// combine could read stale rows.
MOE_DEV void store_pair(float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

// n_tasks: the step's task count (one counting workgroup per task for this tile; the slots past
// it return at once).
MOE_DEV void combine_tile_if_last(const DecodeArgs& a, int tile, int tile_rows, int n_tasks) {
  __shared__ int s_last;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's pair stores are complete
  __syncthreads();
  if (threadIdx.x == 0) {
    const int old = __hip_atomic_fetch_add(&a.tile_done[tile], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = old == n_tasks - 1;
  }
  __syncthreads();
  if (!s_last) return;
  if (threadIdx.x == 0) __hip_atomic_store(&a.tile_done[tile], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // acquire: drop this XCD's cached copies, so the plain loads below see the pairs just written
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  const int r0 = tile * tile_rows;
  const int rr4 = min(tile_rows, a.H - r0) / 4;
  for (int i = threadIdx.x; i < a.T * rr4; i += blockDim.x) {
    const int t = i / rr4, o = r0 + 4 * (i - t * rr4);
    // every load in flight at once (rows and weights past k clamped to j = 0, then not used)
    float4 v[kMaxK + 1];
    float w[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      const int jj = j < a.k ? j : 0;
      w[j] = a.topk_w[t * a.k + jj];
      v[j] = *(const float4*)(a.y_pairs + (size_t)(t * a.k + jj) * a.H + o);
    }
    v[kMaxK] = *(const float4*)(a.y_pairs + (size_t)(a.T * a.k + (a.n_shared ? t : 0)) * a.H + o);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      const bool use = j < a.k;
      acc.x = use ? fmaf(w[j], v[j].x, acc.x) : acc.x;
      acc.y = use ? fmaf(w[j], v[j].y, acc.y) : acc.y;
      acc.z = use ? fmaf(w[j], v[j].z, acc.z) : acc.z;
      acc.w = use ? fmaf(w[j], v[j].w, acc.w) : acc.w;
    }
    if (a.n_shared) {
      acc.x += v[kMaxK].x;
      acc.y += v[kMaxK].y;
      acc.z += v[kMaxK].z;
      acc.w += v[kMaxK].w;
    }
    *(float4*)(a.y + (size_t)t * a.H + o) = acc;
  }
}

// ---- down: y_e[pair][o] = Wd[o] . h[pair] for one task; RGW row groups of 16 per wave ----------
// A rows 2 s + part: token slot s, part 0 = h_hi, 1 = h_lo, staged in LDS once per workgroup.
template <int MAXTOK, int RGW, int FMT = MOE_FMT_Q4_0>
MOE_DEV void down_body(const DecodeArgs& a, int task, int tile, uint16_t* smem, uint32_t* cbt) {
  constexpr int ROWS = 2 * MAXTOK;
  constexpr int NR = ROWS < 4 ? ROWS : 4;
  constexpr int MB = (ROWS + 15) / 16;  // 16-row A blocks: a second one holds token slots 8..15
  const DecodeTask tk = a.tasks[task];
  const uint8_t* blob = task_blob(a.src, tk);
  if (!blob) {
    if (threadIdx.x == 0) set_error(a.ctrl, MOE_DERR_NOT_RESIDENT);
    return;
  }
  const int H = a.H, F = a.F;
  const BlobLayout lay = blob_layout(H, F, FMT);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int NQ = F / kGroupElems;
  const int n_tok = __builtin_popcount(tk.tok_mask);
  if constexpr (FMT == MOE_FMT_CB4) fill_codebook_bf16(a.src.cb, cbt);  // visible after the staging barrier

  auto h_row = [&](int m) {
    const int slot = m >> 1;
    const int pair = task_pair(tk, task_token(tk.tok_mask, slot < n_tok ? slot : 0), a.T, a.k);
    return (const uint16_t*)((m & 1) ? a.h_lo : a.h_hi) + (size_t)pair * F;
  };
  u32x4 hv[kDnStageChunks<MAXTOK>];
  stage_load(hv, ROWS, F, h_row);

  int rows[RGW];
  const uint8_t* dcode[RGW];
  const uint8_t* dscale[RGW];
  bool rg_live[RGW];  // row groups past H (a ragged last workgroup) load row 0 and store nothing
#pragma unroll
  for (int r = 0; r < RGW; ++r) {
    const int r0 = ((tile * kDnWaves + wave) * RGW + r) * 16;
    rg_live[r] = r0 < H;
    rows[r] = (rg_live[r] ? r0 : 0) + n;
    // record (q, row) of the down matrix (H rows) is at 64 (q H + row)
    dcode[r] = blob + lay.down_codes + (size_t)rows[r] * kGroupBytes + 16 * g;
    dscale[r] = blob + lay.down_scales + (size_t)rows[r] * kGroupScaleBytes;
  }
  const float4v zero = {0.f, 0.f, 0.f, 0.f};
  float acc[MB][RGW][NR / 2];  // per token slot: sum over groups of (hi + lo) group partials
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < RGW; ++r)
#pragma unroll
      for (int j = 0; j < NR / 2; ++j) acc[mb][r][j] = 0.f;
  // one batch of kDnQuadsPerPass groups: every load issued, then the MFMA steps group by group
  auto batch = [&](int q0, bool first) {
    const int nq = min(kDnQuadsPerPass, NQ - q0);
    uint4 cd[RGW][kDnQuadsPerPass];
    uint2 sd[RGW][kDnQuadsPerPass];
    uint2 md[RGW][kDnQuadsPerPass];  // affine format: the records' mins
#pragma unroll
    for (int qi = 0; qi < kDnQuadsPerPass; ++qi) {
      const int qq = min(q0 + qi, NQ - 1);
#pragma unroll
      for (int r = 0; r < RGW; ++r) {
        cd[r][qi] = ld16_nt_u4(dcode[r] + (size_t)qq * H * kGroupBytes);
        sd[r][qi] = ld8_nt_u2(dscale[r] + (size_t)qq * H * kGroupScaleBytes);
        if constexpr (FMT == MOE_FMT_AFFINE4)
          md[r][qi] = ld8_nt_u2(dscale[r] - lay.down_scales + lay.down_mins + (size_t)qq * H * kGroupScaleBytes);
      }
      __builtin_amdgcn_sched_barrier(0);  // group order kept: the waits below are per group
    }
    issue_fence();
    if (first) stage_store_sync<true>(hv, smem, ROWS, F, h_row);
#pragma unroll
    for (int qi = 0; qi < kDnQuadsPerPass; ++qi) {
      if (qi >= nq) continue;
      float part[MB][RGW][NR];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < RGW; ++r)
#pragma unroll
          for (int j = 0; j < NR; ++j) part[mb][r][j] = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16x8 A[MB];
        float4v O[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          A[mb] = lds_fragment(smem, ROWS, F, 16 * mb + n, g, (q0 + qi) * kGroupElems + 32 * i);
          O[mb] = fmt_c<FMT>(A[mb], zero);
        }
#pragma unroll
        for (int r = 0; r < RGW; ++r) {
          const bf16x8 B = fmt_b<FMT>(word_at(cd[r][qi], i), cbt);
          const float s = scale_at(sd[r][qi], i);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            const float4v D = mfma_bf16(A[mb], B, O[mb]);
#pragma unroll
            for (int j = 0; j < NR; ++j) part[mb][r][j] = fmaf(s, D[j], part[mb][r][j]);
            if constexpr (FMT == MOE_FMT_AFFINE4) {
              const float m = scale_at(md[r][qi], i) * 0.0078125f;
#pragma unroll
              for (int j = 0; j < NR; ++j) part[mb][r][j] = fmaf(m, O[mb][j], part[mb][r][j]);
            }
          }
        }
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < RGW; ++r)
#pragma unroll
          for (int j = 0; j < NR / 2; ++j) acc[mb][r][j] += part[mb][r][2 * j] + part[mb][r][2 * j + 1];
    }
  };
  batch(0, true);  // peeled: a loop head would wait for every outstanding load, the staging too
  for (int q0 = kDnQuadsPerPass; q0 < NQ; q0 += kDnQuadsPerPass) batch(q0, false);
  // lane (g, n) holds rows 4g + j of each A block: token slots 8 mb + 2g (j = 0, 1) and
  // 8 mb + 2g + 1 (j = 2, 3)
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int r = 0; r < RGW; ++r) {
#pragma unroll
      for (int s2 = 0; s2 < NR / 2; ++s2) {
        const int slot = 8 * mb + 2 * g + s2;
        if (rg_live[r] && slot < n_tok)
          store_pair(a.y_pairs + (size_t)task_pair(tk, task_token(tk.tok_mask, slot), a.T, a.k) * H + rows[r],
                     acc[mb][r][s2]);
      }
    }
  }
}

template <int MAXTOK, int RGW, int FMT = MOE_FMT_Q4_0>
__global__ __launch_bounds__(64 * kDnWaves) void k_decode_down(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  __shared__ uint32_t cbt[FMT == MOE_FMT_CB4 ? 256 : 1];
  const int task = blockIdx.x / a.tiles_dn;
  const int tile = blockIdx.x - task * a.tiles_dn;
  const int n_tasks = a.ctrl[kCtrlNTasks];
  if (task >= n_tasks) return;  // task slots past the step's count neither compute nor count
  down_body<MAXTOK, RGW, FMT>(a, task, tile, smem, cbt);
  combine_tile_if_last(a, tile, 16 * kDnWaves * RGW, n_tasks);
}

// ---- down for one token: output rows outermost, every task inside, no pair rows -------------------
// One workgroup of NWV waves per RT (8 or 16) output rows.  The work is (task, group of 128 F inputs)
// items; wave w takes items w, w + NWV, ... (at most MAXI), so each wave issues all of its weight
// loads (one 16-byte code load and one 8-byte scale load per lane per item) at once and the waves
// carry equal shares (16 waves of 4-5 items at the model shape: four waves per SIMD hide each
// other's MFMA chains).  A rows 0 and 1 are the token's h_hi and h_lo (the other rows zero).  An item's result is
// the group partial of its task's pair value; the workgroup then forms every pair value and the
// combine in the same order as the per-pair rows and the combine of the other decode kernels, and
// stores y directly: no per-pair rows and no cross-workgroup combine.
template <int MAXT, int MAXI, int RT, int NWV, int FMT = MOE_FMT_Q4_0>
__global__ __launch_bounds__(64 * NWV) void k_decode_down_rows1(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t hs[NWV][MAXI][2][kGroupElems];  // [wave][item][part][input]
  __shared__ float red[8][MAXT + 1][16];  // [group][task][row]: group partials (task MAXT: unused items)
  __shared__ float pv[MAXT][16];      // [task][row]: pair values
  __shared__ int s_inv[kMaxK];        // task of each top-k position j
  __shared__ uint32_t cbt[FMT == MOE_FMT_CB4 ? 256 : 1];
  constexpr bool kAff = FMT == MOE_FMT_AFFINE4;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int H = a.H, F = a.F;
  if constexpr (FMT == MOE_FMT_CB4) {
    // the codebook's pair table, before any load is in flight (the barrier would wait for them)
    fill_codebook_bf16(a.src.cb, cbt);
    __syncthreads();
  }
  const int NW = F / kGroupElems;  // groups of F inputs (<= 8)
  // RT output rows per workgroup; with RT = 8 lanes n and n + 8 load the same row (the upper
  // half of D is not used)
  const int row = blockIdx.x * RT + (n & (RT - 1));
  const BlobLayout lay = blob_layout(H, F, FMT);
  // task descriptors: lane t loads task t (the task list always has room for MAXT entries), so one
  // vector load brings them all; the per-task values are then read from those lanes
  const int n_tasks = min(a.ctrl[kCtrlNTasks], MAXT);
  const u32x4 tv = *(const u32x4*)&a.tasks[lane < MAXT ? lane : MAXT - 1];
  const float l_w = a.topk_w[lane < a.k ? lane : 0];  // lane j: the token's weight j
  const int l_expert = (int)tv[0];
  int l_slot = (int)tv[1];
  // an expert that missed when the plan ran: its table entry now (filled by the pool since)
  const bool l_routed = lane < n_tasks && l_expert >= 0;
  if (__any(l_routed && l_slot < 0)) {
    if (l_routed && l_slot < 0) l_slot = a.src.table ? a.src.table[l_expert] : l_expert;
  }
  const bool l_ok = l_routed && l_slot >= 0 && l_slot < a.src.n_slots;
  if (__any(l_routed && !l_ok) && threadIdx.x == 0) set_error(a.ctrl, MOE_DERR_NOT_RESIDENT);
  // items past the count (and experts not resident, reported above) load a valid blob and row
  // and are not computed
  const uint8_t* const fallback = a.src.shared_blob ? a.src.shared_blob : a.src.arena;
  const int n_items = n_tasks * NW;
  const uint8_t* blob[MAXI];
  int it_t[MAXI], it_q[MAXI], it_pair[MAXI];
  bool use[MAXI];
  static_for<MAXI>([&](auto c) {
    constexpr int m = c.value;
    const int i = wave + NWV * m;
    const bool live = i < n_items;
    const int t = live ? i / NW : 0;
    it_t[m] = t;
    it_q[m] = live ? i - t * NW : 0;
    const int expert = __builtin_amdgcn_readlane(l_expert, t);
    const int slot = __builtin_amdgcn_readlane(l_slot, t);
    const int ok = __builtin_amdgcn_readlane((int)l_ok, t);
    const int choice = __builtin_amdgcn_readlane((int)tv[3], t);
    const bool routed = live && expert >= 0;
    const bool shared = live && expert < 0 && a.src.shared_blob;
    blob[m] = live && ok ? a.src.arena + (int64_t)slot * a.src.slot_stride : fallback;
    it_pair[m] = routed ? (choice & 15) : shared ? a.T * a.k : 0;
    use[m] = live && (ok || shared);
  });
  // h slices of the items: chunk c = lane + 64 i is item c / 32, part (c / 16) & 1, 8 inputs
  constexpr int HC = (MAXI * 32 + 63) / 64;
  u32x4 hv[HC];
  static_for<HC>([&](auto c) {
    constexpr int i = c.value;
    constexpr int m0 = 2 * i < MAXI ? 2 * i : MAXI - 1, m1 = 2 * i + 1 < MAXI ? 2 * i + 1 : MAXI - 1;
    const int pr = lane < 32 ? it_pair[m0] : it_pair[m1];
    const int qq = lane < 32 ? it_q[m0] : it_q[m1];
    const int part = (lane >> 4) & 1;
    hv[i] = *(const u32x4*)((part ? a.h_lo : a.h_hi) + (size_t)pr * F + qq * kGroupElems + (lane & 15) * 8);
  });
  __builtin_amdgcn_sched_barrier(0);
  // weights of every item: record (q, row) of the down matrix
  u32x4 cd[MAXI];
  u32x2 sd[MAXI];
  u32x2 md[kAff ? MAXI : 1];  // affine format: the records' mins
  static_for<MAXI>([&](auto c) {
    constexpr int m = c.value;
    cd[m] = ld16_nt(blob[m] + lay.down_codes + ((size_t)it_q[m] * H + row) * kGroupBytes + 16 * g);
    sd[m] = ld8_nt(blob[m] + lay.down_scales + ((size_t)it_q[m] * H + row) * kGroupScaleBytes);
    if constexpr (kAff) md[m] = ld8_nt(blob[m] + lay.down_mins + ((size_t)it_q[m] * H + row) * kGroupScaleBytes);
  });
  issue_fence();
  static_for<HC>([&](auto c) {
    constexpr int i = c.value;
    const int cc = lane + 64 * i;
    if (cc < MAXI * 32) *(u32x4*)&hs[wave][cc >> 5][(cc >> 4) & 1][(cc & 15) * 8] = hv[i];
  });
  asm volatile("" ::: "memory");  // the wave reads back only its own slices: LDS order suffices
  if (wave == 0 && lane < n_tasks && l_expert >= 0) s_inv[tv[3] & 15u] = lane;
  const Unpack uk = make_unpack();
  const float4v zero = {0.f, 0.f, 0.f, 0.f};
  // every item is computed (one basic block, so the MFMA chains of different items interleave);
  // unused items write their result to the spare task row
  static_for<MAXI>([&](auto c) {
    constexpr int m = c.value;
    float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint4 av = *(const uint4*)&hs[wave][m][n & 1][32 * i + 8 * g];
      if (n >= 2) av = make_uint4(0u, 0u, 0u, 0u);
      const bf16x8 A = __builtin_bit_cast(bf16x8, av);
      const float4v O = fmt_c<FMT>(A, zero);
      const float4v D = mfma_bf16(A, pipe_b<FMT>(word_at(cd[m], i), uk, cbt), O);
      const float sc = scale_at(sd[m], i);
      acc0 = fmaf(sc, D[0], acc0);
      acc1 = fmaf(sc, D[1], acc1);
      if constexpr (kAff) {
        const float mn = scale_at(md[m], i) * 0.0078125f;
        acc0 = fmaf(mn, O[0], acc0);
        acc1 = fmaf(mn, O[1], acc1);
      }
    }
    // lanes 0..15 hold rows 0 and 1 of D (the token's hi and lo parts) for output row n
    if (lane < RT) red[use[m] ? it_q[m] : 0][use[m] ? it_t[m] : MAXT][n] = acc0 + acc1;
  });
  __syncthreads();
  // the same arithmetic as the per-pair rows and the combine of the other decode kernels: a pair
  // value is the sum of its group partials in group order; y = sum_j w_j * pair_j in j order, then
  // + the shared expert's pair
  // (every load of a step is issued before the sums that use it)
  for (int idx = threadIdx.x; idx < 16 * MAXT; idx += blockDim.x) {
    const int t = idx >> 4, r = idx & 15;
    if (r >= RT) continue;
    float v[8];
#pragma unroll
    for (int w = 0; w < 8; ++w) v[w] = red[w < NW ? w : 0][t][r];
    float p = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) p = w < NW ? p + v[w] : p;
    pv[t][r] = p;
  }
  __syncthreads();
  if (threadIdx.x < RT) {
    int inv[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) inv[j] = s_inv[j < a.k ? j : 0];
    float v[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) v[j] = pv[inv[j]][threadIdx.x];
    const float vs = pv[a.n_shared ? n_tasks - 1 : 0][threadIdx.x];
    float y = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      y = j < a.k ? fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(l_w), j)), v[j], y) : y;
    if (a.n_shared) y += vs;
    a.y[blockIdx.x * RT + threadIdx.x] = y;
  }
}

// ---- pipelined variants for tasks of up to 4 or 8 bf16 tokens ----------------------------------
// Each wave owns whole row groups (16 output rows over the full input range), so there is no
// reduction across waves, and walks the input range in UNITS chunks whose loads go out one chunk
// ahead of the MFMA work: the wave always has weight loads in flight, and the grid (a workgroup per
// 64 gate/up rows or 256 down rows of one task) fits the chip in one round.
constexpr int kPipeGuWaves = 4;   // gate/up: waves (= row groups of 16) per workgroup
constexpr int kPipeGuGroups = 2;  // gate/up: groups of 128 inputs per chunk
constexpr int kPipeGuBufs = 3;    // gate/up: chunks in flight
constexpr int kPipeDnWaves = 8;   // down: waves per workgroup
constexpr int kPipeDnRGW = 2;     // down: row groups per wave (at most 2: one offset register each)
static_assert(kPipeDnRGW >= 1 && kPipeDnRGW <= 2, "down row groups per wave");
constexpr int kPipeDnGroups = 3;  // down: groups of 128 inputs per chunk
constexpr int kPipeDnBufs = 2;    // down: chunks in flight
// Waves per SIMD the pipelined kernels are compiled for: 4 (128 registers each) up to 8 tokens;
// 2 (256 registers) at 16, whose staged activation rows would not fit beside the weight ring.
constexpr int pipe_waves_per_eu(int maxtok) { return maxtok > 8 ? 2 : 4; }

// gate/up: H = 128 kPipeGuGroups UNITS; A rows = token slots of the task (bf16 x).  Every weight
// format, with the operands, the C term and the affine min term of the general kernel.
template <int MAXTOK, int UNITS, int FMT = MOE_FMT_Q4_0>
__global__ __launch_bounds__(64 * kPipeGuWaves) __attribute__((amdgpu_waves_per_eu(pipe_waves_per_eu(MAXTOK)))) void k_decode_gate_up_pipe(DecodeArgs a) {
  constexpr int ROWS = MAXTOK;
  constexpr int NR = ROWS < 4 ? ROWS : 4;
  constexpr int QG = kPipeGuGroups;
  constexpr bool kAff = FMT == MOE_FMT_AFFINE4;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  __shared__ uint32_t cbt[FMT == MOE_FMT_CB4 ? 256 : 1];
  const int task = blockIdx.x / a.tiles_gu;
  const int tile = blockIdx.x - task * a.tiles_gu;
  constexpr int H = 128 * QG * UNITS;
  constexpr int NT = 64 * kPipeGuWaves;  // threads
  // up to ROWS * H / 8 chunks of 16 bytes over the threads
  constexpr int XC = (ROWS * (H / 8) + NT - 1) / NT;
  u32x4 xv[XC];
  // chunks in flight (fewer when the staged rows, or the affine format's min records, need many
  // registers)
  constexpr int NBUF = (XC > 8 || kAff) ? 2 : kPipeGuBufs;
  const DecodeTask tk = a.tasks[task];
  if (task >= a.ctrl[kCtrlNTasks]) return;
  const uint8_t* blob = task_blob(a.src, tk);
  if (!blob) {
    if (threadIdx.x == 0) set_error(a.ctrl, MOE_DERR_NOT_RESIDENT);
    return;
  }
  const int F = a.F;
  const BlobLayout lay = blob_layout(H, F, FMT);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int row = (tile * kPipeGuWaves + wave) * 16 + n;
  const int n_tok = __builtin_popcount(tk.tok_mask);
  const int arow = n < n_tok ? n : ROWS;  // LDS row of this lane's token slot (ROWS: a zero row)
  // Only the task's own token rows are staged, in slot order (most tasks of a step carry one
  // token): n_tok H / 8 chunks; a round of chunks is loaded only if some thread has one (the
  // condition is uniform across the workgroup, so no load sits under a per-lane branch).
  auto x_row = [&](int m) { return (const uint16_t*)a.x + (size_t)task_token(tk.tok_mask, m < n_tok ? m : 0) * H; };
  const int n_chunks = n_tok * (H / 8);
  static_for<XC>([&](auto c) {
    if (c.value * NT < n_chunks) {
      int m, col;
      chunk_pos(min((int)threadIdx.x + c.value * NT, n_chunks - 1), H, m, col);
      xv[c.value] = *(const u32x4*)(x_row(m) + col);
    }
  });
  __builtin_amdgcn_sched_barrier(0);  // these loads go out before the weight loads
  const Unpack uk = make_unpack();
  if constexpr (FMT == MOE_FMT_CB4) fill_codebook_bf16(a.src.cb, cbt);  // visible after the staging barrier

  const __amdgpu_buffer_rsrc_t rs = blob_rsrc(blob, lay.total);
  const int voff_c = row * kGroupBytes + 16 * g, voff_s = row * kGroupScaleBytes;
  u32x4 cg[NBUF][QG], cu[NBUF][QG];
  u32x2 sg[NBUF][QG], su[NBUF][QG];
  u32x2 mg[kAff ? NBUF : 1][QG], mu[kAff ? NBUF : 1][QG];  // affine format: the records' mins
  // chunk u into buffer b: record (q, row) at 64 (q F + row), its scales at 8 (q F + row) (and
  // its mins likewise in the min planes)
  auto load_chunk = [&](auto bc, int u) {
    constexpr int b = decltype(bc)::value;
#pragma unroll
    for (int qi = 0; qi < QG; ++qi) {
      const int q = (u * QG + qi) * F;
      cg[b][qi] = buf_load16_nt(rs, voff_c, (int)lay.gate_codes + q * kGroupBytes);
      cu[b][qi] = buf_load16_nt(rs, voff_c, (int)lay.up_codes + q * kGroupBytes);
      sg[b][qi] = buf_load8_nt(rs, voff_s, (int)lay.gate_scales + q * kGroupScaleBytes);
      su[b][qi] = buf_load8_nt(rs, voff_s, (int)lay.up_scales + q * kGroupScaleBytes);
      if constexpr (kAff) {
        mg[b][qi] = buf_load8_nt(rs, voff_s, (int)lay.gate_mins + q * kGroupScaleBytes);
        mu[b][qi] = buf_load8_nt(rs, voff_s, (int)lay.up_mins + q * kGroupScaleBytes);
      }
      __builtin_amdgcn_sched_barrier(0);  // group order kept: the waits below are per group
    }
  };
  // the first chunks go out before the staged rows are stored (the store waits for the staging
  // loads only, issued first)
  static_for<(NBUF < UNITS ? NBUF : UNITS)>([&](auto uc) { load_chunk(uc, decltype(uc)::value); });
  issue_fence();
  stage_store_sync<false>(xv, smem, n_tok, H, x_row);

  const float4v zero = {0.f, 0.f, 0.f, 0.f};
  // Summation order of the split kernel above (a partial sum per range of kGuQuadsPerWave groups,
  // the partials added in range order), so a token's h is bitwise the same whichever kernel the
  // size of its step selects.
  constexpr int CPR = kGuQuadsPerWave / QG;  // chunks per range
  static_assert(kGuQuadsPerWave % QG == 0 && UNITS % CPR == 0, "whole ranges per chunk walk");
  float accg[NR], accu[NR], totg[NR], totu[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) accg[r] = accu[r] = totg[r] = totu[r] = 0.f;
  static_for<UNITS>([&](auto uc) {
    constexpr int u = decltype(uc)::value;
    constexpr int b = u % NBUF;
    if constexpr (u % CPR == 0) {
#pragma unroll
      for (int r = 0; r < NR; ++r) accg[r] = accu[r] = 0.f;
    }
#pragma unroll
    for (int qi = 0; qi < QG; ++qi) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8 A = lds_fragment(smem, ROWS, H, arow, g, (u * QG + qi) * kGroupElems + 32 * i);
        const float4v O = fmt_c<FMT>(A, zero);
        const float4v Dg = mfma_bf16(A, pipe_b<FMT>(word_at(cg[b][qi], i), uk, cbt), O);
        const float4v Du = mfma_bf16(A, pipe_b<FMT>(word_at(cu[b][qi], i), uk, cbt), O);
        const float s_g = scale_at(sg[b][qi], i), s_u = scale_at(su[b][qi], i);
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          accg[r] = fmaf(s_g, Dg[r], accg[r]);
          accu[r] = fmaf(s_u, Du[r], accu[r]);
        }
        if constexpr (kAff) {
          const float m_g = scale_at(mg[b][qi], i) * 0.0078125f, m_u = scale_at(mu[b][qi], i) * 0.0078125f;
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            accg[r] = fmaf(m_g, O[r], accg[r]);
            accu[r] = fmaf(m_u, O[r], accu[r]);
          }
        }
      }
      // one group at a time: an unbounded schedule hoists every MFMA and spills their results
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (u % CPR == CPR - 1) {
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        totg[r] += accg[r];
        totu[r] += accu[r];
      }
    }
    if constexpr (u + NBUF < UNITS) {
      load_chunk(std::integral_constant<int, b>{}, u + NBUF);
      issue_fence();
    }
  });

  // The sums are final here: without this the compiler sinks the whole accumulation chain into
  // the conditional stores below, after every MFMA, and spills the MFMA results.
#pragma unroll
  for (int r = 0; r < NR; ++r) asm volatile("" : "+v"(totg[r]), "+v"(totu[r]));
  // lane (g, n) holds token slots 4 g + r of row `row`: SwiGLU, h as bf16 hi + lo
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int slot = 4 * g + r;
    if (slot < n_tok) {
      const float h = silu(totg[r]) * totu[r];
      const uint32_t hi = f32_to_bf16_rne(h);
      const uint32_t lo = f32_to_bf16_rne(h - __uint_as_float(hi << 16));
      const size_t o = (size_t)task_pair(tk, task_token(tk.tok_mask, slot), a.T, a.k) * F + row;
      a.h_hi[o] = (uint16_t)hi;
      a.h_lo[o] = (uint16_t)lo;
    }
  }
}

// down: F = 128 kPipeDnGroups UNITS; A rows 2 s + part (token slot s, h hi / lo).  Every weight
// format, as in the general down kernel.
template <int MAXTOK, int UNITS, int FMT = MOE_FMT_Q4_0>
MOE_DEV void down_pipe_body(const DecodeArgs& a, int task, int tile, uint16_t* smem, const uint32_t* cbt) {
  constexpr bool kAff = FMT == MOE_FMT_AFFINE4;
  constexpr int ROWS = 2 * MAXTOK;
  constexpr int NR = ROWS < 4 ? ROWS : 4;
  constexpr int MB = (ROWS + 15) / 16;  // 16-row A blocks: a second one holds token slots 8..15
  constexpr int QG = kPipeDnGroups;
  constexpr int RGW = kPipeDnRGW;
  const DecodeTask tk = a.tasks[task];
  const uint8_t* blob = task_blob(a.src, tk);
  if (!blob) {
    if (threadIdx.x == 0) set_error(a.ctrl, MOE_DERR_NOT_RESIDENT);
    return;
  }
  constexpr int F = 128 * QG * UNITS;
  const int H = a.H;
  const BlobLayout lay = blob_layout(H, F, FMT);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int n_tok = __builtin_popcount(tk.tok_mask);
  const Unpack uk = make_unpack();

  auto h_row = [&](int m) {
    const int slot = m >> 1;
    const int pair = task_pair(tk, task_token(tk.tok_mask, slot < n_tok ? slot : 0), a.T, a.k);
    return (const uint16_t*)((m & 1) ? a.h_lo : a.h_hi) + (size_t)pair * F;
  };
  constexpr int HC = (ROWS * (F / 8) + 64 * kPipeDnWaves - 1) / (64 * kPipeDnWaves);
  u32x4 hv[HC];
  stage_load(hv, ROWS, F, h_row);

  const __amdgpu_buffer_rsrc_t rs = blob_rsrc(blob, lay.total);
  // the wave's row groups are consecutive: row group r of the wave at voff + 16 r records
  const int r0 = ((tile * kPipeDnWaves + wave) * RGW) * 16;
  bool rg_live[RGW];  // row groups past H (a ragged last workgroup) load row 0 and store nothing
  int rows[RGW];
#pragma unroll
  for (int r = 0; r < RGW; ++r) {
    rg_live[r] = r0 + 16 * r < H;
    rows[r] = (rg_live[r] ? r0 + 16 * r : 0) + n;
  }
  const int voff_c0 = rows[0] * kGroupBytes + 16 * g, voff_s0 = rows[0] * kGroupScaleBytes;
  const int voff_c1 = rows[RGW - 1] * kGroupBytes + 16 * g, voff_s1 = rows[RGW - 1] * kGroupScaleBytes;
  u32x4 cd[kPipeDnBufs][RGW][QG];
  u32x2 sd[kPipeDnBufs][RGW][QG];
  u32x2 md[kAff ? kPipeDnBufs : 1][RGW][QG];  // affine format: the records' mins
  auto load_chunk = [&](auto bc, int u) {
    constexpr int b = decltype(bc)::value;
#pragma unroll
    for (int qi = 0; qi < QG; ++qi) {
      const int q = (u * QG + qi) * H;  // record (q, row) of the down matrix (H rows)
#pragma unroll
      for (int r = 0; r < RGW; ++r) {
        cd[b][r][qi] = buf_load16_nt(rs, r == 0 ? voff_c0 : voff_c1, (int)lay.down_codes + q * kGroupBytes);
        sd[b][r][qi] = buf_load8_nt(rs, r == 0 ? voff_s0 : voff_s1, (int)lay.down_scales + q * kGroupScaleBytes);
        if constexpr (kAff)
          md[b][r][qi] = buf_load8_nt(rs, r == 0 ? voff_s0 : voff_s1, (int)lay.down_mins + q * kGroupScaleBytes);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // the first chunks go out before the staged rows are stored (the store waits for the staging
  // loads only, issued first)
  static_for<(kPipeDnBufs < UNITS ? kPipeDnBufs : UNITS)>([&](auto uc) { load_chunk(uc, decltype(uc)::value); });
  issue_fence();
  stage_store_sync<false>(hv, smem, ROWS, F, h_row);

  const float4v zero = {0.f, 0.f, 0.f, 0.f};
  float acc[MB][RGW][NR / 2];  // per token slot: sum over groups of (hi + lo) group partials
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < RGW; ++r)
#pragma unroll
      for (int j = 0; j < NR / 2; ++j) acc[mb][r][j] = 0.f;
  static_for<UNITS>([&](auto uc) {
    constexpr int u = decltype(uc)::value;
    constexpr int b = u % kPipeDnBufs;
#pragma unroll
    for (int qi = 0; qi < QG; ++qi) {
      float part[MB][RGW][NR];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < RGW; ++r)
#pragma unroll
          for (int j = 0; j < NR; ++j) part[mb][r][j] = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16x8 A[MB];
        float4v O[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          A[mb] = lds_fragment(smem, ROWS, F, 16 * mb + n, g, (u * QG + qi) * kGroupElems + 32 * i);
          O[mb] = fmt_c<FMT>(A[mb], zero);
        }
#pragma unroll
        for (int r = 0; r < RGW; ++r) {
          const bf16x8 B = pipe_b<FMT>(word_at(cd[b][r][qi], i), uk, cbt);
          const float s = scale_at(sd[b][r][qi], i);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            const float4v D = mfma_bf16(A[mb], B, O[mb]);
#pragma unroll
            for (int j = 0; j < NR; ++j) part[mb][r][j] = fmaf(s, D[j], part[mb][r][j]);
            if constexpr (kAff) {
              const float m = scale_at(md[b][r][qi], i) * 0.0078125f;
#pragma unroll
              for (int j = 0; j < NR; ++j) part[mb][r][j] = fmaf(m, O[mb][j], part[mb][r][j]);
            }
          }
        }
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < RGW; ++r)
#pragma unroll
          for (int j = 0; j < NR / 2; ++j) acc[mb][r][j] += part[mb][r][2 * j] + part[mb][r][2 * j + 1];
      __builtin_amdgcn_sched_barrier(0);  // one group at a time
    }
    if constexpr (u + kPipeDnBufs < UNITS) {
      load_chunk(std::integral_constant<int, b>{}, u + kPipeDnBufs);
      issue_fence();
    }
  });
  // final accumulators (kept from being sunk into the conditional stores)
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < RGW; ++r)
#pragma unroll
      for (int j = 0; j < NR / 2; ++j) asm volatile("" : "+v"(acc[mb][r][j]));
  // lane (g, n) holds rows 4g + j of each A block: token slots 8 mb + 2g (j = 0, 1) and
  // 8 mb + 2g + 1 (j = 2, 3)
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int r = 0; r < RGW; ++r) {
#pragma unroll
      for (int s2 = 0; s2 < NR / 2; ++s2) {
        const int slot = 8 * mb + 2 * g + s2;
        if (rg_live[r] && slot < n_tok)
          store_pair(a.y_pairs + (size_t)task_pair(tk, task_token(tk.tok_mask, slot), a.T, a.k) * H + rows[r],
                     acc[mb][r][s2]);
      }
    }
  }
}

template <int MAXTOK, int UNITS, int FMT = MOE_FMT_Q4_0>
__global__ __launch_bounds__(64 * kPipeDnWaves) __attribute__((amdgpu_waves_per_eu(pipe_waves_per_eu(MAXTOK)))) void k_decode_down_pipe(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  __shared__ uint32_t cbt[FMT == MOE_FMT_CB4 ? 256 : 1];
  const int task = blockIdx.x / a.tiles_dn;
  const int tile = blockIdx.x - task * a.tiles_dn;
  const int n_tasks = a.ctrl[kCtrlNTasks];
  if (task >= n_tasks) return;  // task slots past the step's count neither compute nor count
  if constexpr (FMT == MOE_FMT_CB4) fill_codebook_bf16(a.src.cb, cbt);  // visible after the staging barrier
  down_pipe_body<MAXTOK, UNITS, FMT>(a, task, tile, smem, cbt);
  combine_tile_if_last(a, tile, 16 * kPipeDnWaves * kPipeDnRGW, n_tasks);
}

// ---- dequantization check: one thread per code word, the same operands as the FFN kernels ------
// The default and affine formats decode the word as the MFMA operand 128 + u; the codebook format
// through the same 256-entry pair table.  Q4_0: (128 + u - 136) s; CB4: cb[u] s (both exact in
// fp32); AFFINE4: fma(u, s, -m), the exact u s - m rounded once.
__global__ __launch_bounds__(256) void k_debug_dequant(int H, int F, int fmt, Codebook cb,
                                                        const uint8_t* __restrict__ blob, int matrix,
                                                        float* __restrict__ out) {
  __shared__ uint32_t cbt[256];
  fill_codebook_bf16(cb, cbt);
  __syncthreads();
  const BlobLayout lay = blob_layout(H, F, fmt);
  const int rows = matrix == 2 ? H : F, cols = matrix == 2 ? F : H;
  const int64_t codes = matrix == 0 ? lay.gate_codes : matrix == 1 ? lay.up_codes : lay.down_codes;
  const int64_t scales = matrix == 0 ? lay.gate_scales : matrix == 1 ? lay.up_scales : lay.down_scales;
  const int64_t mins = matrix == 0 ? lay.gate_mins : matrix == 1 ? lay.up_mins : lay.down_mins;
  const int n_words = rows * cols / 8;
  for (int wi = blockIdx.x * blockDim.x + threadIdx.x; wi < n_words; wi += gridDim.x * blockDim.x) {
    const int rec = wi >> 4, p = wi & 15, g = p >> 2, i = p & 3;  // word 4g + i of record rec
    const int grp = rec / rows, r = rec - grp * rows;            // record (grp, r)
    const int blk = 4 * grp + i;
    const int c0 = blk * kBlock + 8 * g;
    const uint32_t w = *(const uint32_t*)(blob + codes + (size_t)wi * 4);
    const float s = fp16_bits_to_f32(*(const uint16_t*)(blob + scales + (size_t)rec * kGroupScaleBytes + 2 * i));
    const float m = fmt == MOE_FMT_AFFINE4
                        ? fp16_bits_to_f32(*(const uint16_t*)(blob + mins + (size_t)rec * kGroupScaleBytes + 2 * i))
                        : 0.f;
    const uint4 q = fmt == MOE_FMT_CB4 ? __builtin_bit_cast(uint4, fmt_b<MOE_FMT_CB4>(w, cbt))
                                       : __builtin_bit_cast(uint4, codes_q136(w));
    const uint32_t pr[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float v0 = bf16_lo(pr[j]), v1 = bf16_hi(pr[j]);
      float w0, w1;
      if (fmt == MOE_FMT_CB4) {
        w0 = v0 * s;
        w1 = v1 * s;
      } else if (fmt == MOE_FMT_AFFINE4) {
        w0 = fmaf(v0 - 128.f, s, -m);
        w1 = fmaf(v1 - 128.f, s, -m);
      } else {
        w0 = (v0 - 136.f) * s;
        w1 = (v1 - 136.f) * s;
      }
      out[(size_t)r * cols + c0 + 2 * j] = w0;
      out[(size_t)r * cols + c0 + 2 * j + 1] = w1;
    }
  }
}

__global__ void k_fill_zero(uint32_t* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0u;
}

// ------------------------------------------------------------------------------------------
// Launchers
// ------------------------------------------------------------------------------------------
// Pipelined kernels: input ranges of 4, 8 or 16 gate/up chunks (H = 1024, 2048, 4096) and 2 or 4
// down chunks (F = 768, 1536); 0 = not covered.
static int gate_up_pipe_units(int H) {
  const int u = H / (kGroupElems * kPipeGuGroups);
  return H % (kGroupElems * kPipeGuGroups) == 0 && (u == 4 || u == 8 || u == 16) ? u : 0;
}
static int down_pipe_units(int F) {
  const int u = F / (kGroupElems * kPipeDnGroups);
  return F % (kGroupElems * kPipeDnGroups) == 0 && (u == 2 || u == 4) ? u : 0;
}

template <int MAXTOK, int FMT>
static hipError_t launch_gate_up_pipe(DecodeArgs a, int max_tasks, int units, hipStream_t st) {
  a.tiles_gu = a.F / (16 * kPipeGuWaves);
  const int grid = max_tasks * a.tiles_gu, threads = 64 * kPipeGuWaves;
  const uint32_t lds = (uint32_t)(MAXTOK * (a.H + 8) * 2);
  if (units == 4)
    return launch_timed(kTimeDecodeGateUp, k_decode_gate_up_pipe<MAXTOK, 4, FMT>, grid, threads, lds, st, a);
  if (units == 8)
    return launch_timed(kTimeDecodeGateUp, k_decode_gate_up_pipe<MAXTOK, 8, FMT>, grid, threads, lds, st, a);
  return launch_timed(kTimeDecodeGateUp, k_decode_gate_up_pipe<MAXTOK, 16, FMT>, grid, threads, lds, st, a);
}

template <int MAXTOK, int FMT>
static hipError_t launch_down_pipe(DecodeArgs a, int max_tasks, int units, hipStream_t st) {
  const int rows = 16 * kPipeDnWaves * kPipeDnRGW;
  a.tiles_dn = (a.H + rows - 1) / rows;
  const int grid = max_tasks * a.tiles_dn, threads = 64 * kPipeDnWaves;
  const uint32_t lds = (uint32_t)(2 * MAXTOK * (a.F + 8) * 2);
  if (units == 2) return launch_timed(kTimeDecodeDown, k_decode_down_pipe<MAXTOK, 2, FMT>, grid, threads, lds, st, a);
  return launch_timed(kTimeDecodeDown, k_decode_down_pipe<MAXTOK, 4, FMT>, grid, threads, lds, st, a);
}

template <int MAXTOK, int FMT>
static hipError_t launch_decode_ffn_t(DecodeArgs a, int max_tasks, bool xb, hipStream_t st) {
  hipError_t err = hipSuccess;
  // tasks of more than 2 tokens (bf16 x) at the covered shapes: the pipelined kernels
  const int gu_units = (MAXTOK >= 4 && xb) ? gate_up_pipe_units(a.H) : 0;
  if (gu_units) {
    if constexpr (MAXTOK >= 4) err = launch_gate_up_pipe<MAXTOK, FMT>(a, max_tasks, gu_units, st);
  } else {
    const int ks = (a.H / kGroupElems + kGuQuadsPerWave - 1) / kGuQuadsPerWave;
    auto launch_rg = [&](auto rgc) {
      constexpr int RG = decltype(rgc)::value;
      const int gu_threads = 64 * RG * ks;
      a.tiles_gu = a.F / (16 * RG);
      const int grid_gu = max_tasks * a.tiles_gu;
      if (xb)
        return launch_timed(kTimeDecodeGateUp, k_decode_gate_up<MAXTOK, true, RG, false, FMT>, grid_gu, gu_threads,
                            (uint32_t)gate_up_lds_bytes(a.H, MAXTOK, RG * ks), st, a);
      // fp32 tokens are two A rows (hi, lo) each: 8 of them fill the MFMA's 16 rows
      if constexpr (MAXTOK <= 8)
        return launch_timed(kTimeDecodeGateUp, k_decode_gate_up<MAXTOK, false, RG, false, FMT>, grid_gu, gu_threads,
                            (uint32_t)gate_up_lds_bytes(a.H, 2 * MAXTOK, RG * ks), st, a);
      return hipErrorInvalidValue;
    };
    if (MAXTOK == 1 && a.F % (16 * kGuRG1) == 0 && kGuRG1 * ks <= 16)
      err = launch_rg(std::integral_constant<int, kGuRG1>{});
    else
      err = launch_rg(std::integral_constant<int, kGuRG>{});
  }
  if (err != hipSuccess) return err;
  const int dn_units = MAXTOK >= 4 ? down_pipe_units(a.F) : 0;
  if (MAXTOK == 1 && a.F <= 8 * kGroupElems && max_tasks <= kMaxK + 1) {
    // one token: output rows outermost, (task, group) items spread over the waves, no pair rows
    const int items = max_tasks * (a.F / kGroupElems);
    if (max_tasks <= 11 && items <= 16 * 5)
      return launch_timed(kTimeDecodeDown, k_decode_down_rows1<11, 5, 16, 16, FMT>, a.H / 16, 1024, 0, st, a);
    return launch_timed(kTimeDecodeDown, k_decode_down_rows1<kMaxK + 1, kMaxK + 1, 16, 8, FMT>, a.H / 16, 512, 0, st,
                        a);
  }
  if (dn_units) {
    if constexpr (MAXTOK >= 4) err = launch_down_pipe<MAXTOK, FMT>(a, max_tasks, dn_units, st);
  } else {
    const int dn_rows = 16 * kDnWaves * kDnRGW<MAXTOK>;
    a.tiles_dn = (a.H + dn_rows - 1) / dn_rows;
    const uint32_t dn_lds = (uint32_t)(2 * MAXTOK * (a.F + 8) * 2);
    err = launch_timed(kTimeDecodeDown, k_decode_down<MAXTOK, kDnRGW<MAXTOK>, FMT>, max_tasks * a.tiles_dn,
                       64 * kDnWaves, dn_lds, st, a);
  }
  return err;
}

template <int FMT>
static hipError_t launch_decode_ffn_fmt(DecodeArgs a, int T, int max_tasks, bool xb, hipStream_t st) {
  if (T <= 1) return launch_decode_ffn_t<1, FMT>(a, max_tasks, xb, st);
  if (T <= 2) return launch_decode_ffn_t<2, FMT>(a, max_tasks, xb, st);
  if (T <= 4) return launch_decode_ffn_t<4, FMT>(a, max_tasks, xb, st);
  if (T <= 8) return launch_decode_ffn_t<8, FMT>(a, max_tasks, xb, st);
  if (!xb) return hipErrorInvalidValue;  // fp32 tokens take two A rows each: at most 8 (host-checked)
  return launch_decode_ffn_t<16, FMT>(a, max_tasks, xb, st);
}

hipError_t launch_decode_ffn(int H, int F, int k, int n_shared, int T, int max_tasks, const ExpertSource& src,
                             const void* x, int x_dtype, const DecodeTask* tasks, const float* topk_w,
                             uint16_t* h_hi, uint16_t* h_lo, float* y_pairs, float* y, int32_t* ctrl,
                             hipStream_t st) {
  DecodeArgs a{};
  a.src = src;
  a.tasks = tasks;
  a.ctrl = ctrl;
  a.x = x;
  a.h_hi = h_hi;
  a.h_lo = h_lo;
  a.y_pairs = y_pairs;
  a.topk_w = topk_w;
  a.y = y;
  a.H = H;
  a.F = F;
  a.T = T;
  a.k = k;
  a.n_shared = n_shared;
  a.tile_done = ctrl + kCtrlTileDone;
  const bool xb = x_dtype == MOE_BF16;
  static_assert(kTaskTok == kMaxDecodeTok, "a decode task holds every token of the step that chose its expert");
  if (src.fmt == MOE_FMT_CB4) return launch_decode_ffn_fmt<MOE_FMT_CB4>(a, T, max_tasks, xb, st);
  if (src.fmt == MOE_FMT_AFFINE4) return launch_decode_ffn_fmt<MOE_FMT_AFFINE4>(a, T, max_tasks, xb, st);
  return launch_decode_ffn_fmt<MOE_FMT_Q4_0>(a, T, max_tasks, xb, st);
}

bool decode_select1_supported(int H, int F, int k, int n_shared, int E) {
  const int ks = (H / kGroupElems + kGuQuadsPerWave - 1) / kGuQuadsPerWave;
  return E <= 8 * 64 && F % (16 * kGuRG1) == 0 && kGuRG1 * ks <= 16 && F <= 8 * kGroupElems &&
         k + (n_shared ? 1 : 0) <= 11 && (k + (n_shared ? 1 : 0)) * (F / kGroupElems) <= 16 * 5;
}

hipError_t launch_decode_ffn_select1(int H, int F, int k, int n_shared, int E, const ExpertSource& src,
                                     const void* x, const float* logits, DecodeTask* tasks, int32_t* ids_out,
                                     float* w_out, uint16_t* h_hi, uint16_t* h_lo, float* y, int32_t* ctrl,
                                     hipStream_t st) {
  if (!decode_select1_supported(H, F, k, n_shared, E)) return hipErrorInvalidValue;
  DecodeArgs a{};
  a.src = src;
  a.tasks = tasks;
  a.ctrl = ctrl;
  a.x = x;
  a.h_hi = h_hi;
  a.h_lo = h_lo;
  a.topk_w = w_out;
  a.y = y;
  a.H = H;
  a.F = F;
  a.T = 1;
  a.k = k;
  a.n_shared = n_shared;
  a.tile_done = ctrl + kCtrlTileDone;
  a.sel_logits = logits;
  a.sel_tasks = tasks;
  a.sel_ids = ids_out;
  a.E = E;
  const int n_tasks = k + (n_shared ? 1 : 0);
  const int ks = (H / kGroupElems + kGuQuadsPerWave - 1) / kGuQuadsPerWave;
  a.tiles_gu = F / (16 * kGuRG1);
  auto run = [&](auto fmt_c) -> hipError_t {
    constexpr int FMT = decltype(fmt_c)::value;
    hipError_t err = launch_timed(kTimeDecodeGateUp, k_decode_gate_up<1, true, kGuRG1, true, FMT>,
                                  n_tasks * a.tiles_gu, 64 * kGuRG1 * ks,
                                  (uint32_t)gate_up_lds_bytes(H, 1, kGuRG1 * ks), st, a);
    if (err != hipSuccess) return err;
    return launch_timed(kTimeDecodeDown, k_decode_down_rows1<11, 5, 16, 16, FMT>, H / 16, 1024, 0, st, a);
  };
  if (src.fmt == MOE_FMT_CB4) return run(std::integral_constant<int, MOE_FMT_CB4>{});
  if (src.fmt == MOE_FMT_AFFINE4) return run(std::integral_constant<int, MOE_FMT_AFFINE4>{});
  return run(std::integral_constant<int, MOE_FMT_Q4_0>{});
}

hipError_t launch_debug_dequant(int H, int F, int fmt, const Codebook& cb, const uint8_t* blob, int matrix, float* out,
                                hipStream_t st) {
  const int n_words = H * F / 8;
  int grid = (n_words + 255) / 256;
  if (grid > 2048) grid = 2048;
  k_debug_dequant<<<grid, 256, 0, st>>>(H, F, fmt, cb, blob, matrix, out);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st) {
  const size_t n = bytes / 4;
  int grid = (int)((n + 255) / 256);
  if (grid > 1024) grid = 1024;
  if (grid < 1) grid = 1;
  k_fill_zero<<<grid, 256, 0, st>>>((uint32_t*)p, n);
  return hipGetLastError();
}

}  // namespace moe
