// Expert FFNs for a small batch of tokens (decode): 4-bit GEMVs on the matrix cores.
//
// Weights: halogen-flash-server README, "Bring your own GGUF" (small set of values x one scale
// per block, used as stored).  The layer: Betelgeuse news article, "mechanism" (10 routed + 1
// shared expert per token).  Decode pays per byte of weights read (halogen README, "Bring your
// own GGUF": an 8-bit trunk costs 2 GB more per token at 240 GB/s), so each selected expert's blob
// is streamed once from HBM per step, whatever the number of tokens (1..8) that chose it.
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
//   gate/up: one workgroup per (task, 16-row tile of the F rows).  Its waves split the H inputs
//     in runs of 4 groups (512 inputs), reduce through LDS, apply SwiGLU and store h = silu(g) * u
//     of the task's tokens as bf16 hi + lo, ready to be the down projection's A operand.
//   down: one wave per (task, 16 output rows) over all F inputs.  A rows are the (hi, lo) row
//     pairs of the task's tokens (<= 8 tokens -> <= 16 rows), so one MFMA per block covers both
//     parts.  Writes each pair's output row y_e.
//   combine: y[t] = sum_j w[t][j] * y_{e_j}[t] (j = 0..k-1), then + y_shared[t]: fixed order.
#include "kernels.hpp"

namespace moe {

constexpr int kGuQuadsPerWave = 4;                                   // groups of 128 inputs per wave
constexpr int kMaxGuWaves = 4096 / (kGroupElems * kGuQuadsPerWave);  // H <= 4096
constexpr int kDnQuadsPerPass = 6;                                   // down: groups per load batch
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

// One code word (8 elements of a slice) -> B operand: 8 bf16 values q + 136 = 128 + u.  Pair j of
// the word (its elements 2j and 2j+1 in bits 4j and 16 + 4j) becomes register j.
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

MOE_DEV uint32_t word_at(const uint4& c, int i) { return i == 0 ? c.x : i == 1 ? c.y : i == 2 ? c.z : c.w; }

// fp16 scale i (0..3) of a group's four block scales.
MOE_DEV float scale_at(const uint2& s, int i) {
  const uint32_t w = i < 2 ? s.x : s.y;
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
  return tk.expert < 0 ? T * k + t : t * k + (int)((tk.choice >> (4 * t)) & 15u);
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
  int tiles_gu;  // F / 16
  int tiles_dn;  // H / 64
};

// ---- gate/up: h[pair][r] = silu(Wg[r] . x) * (Wu[r] . x) for one task and 16 rows r --------
// A rows: token slot m of the task (bf16 x) or 2 m + part (fp32 x).  ROWS <= 16.
template <int MAXTOK, bool X_BF16>
__global__ __launch_bounds__(64 * kMaxGuWaves) void k_decode_gate_up(DecodeArgs a) {
  constexpr int ROWS = X_BF16 ? MAXTOK : 2 * MAXTOK;
  constexpr int NR = ROWS < 4 ? ROWS : 4;  // live D registers per lane
  __shared__ float red[kMaxGuWaves][2][ROWS][16];

  const int task = blockIdx.x / a.tiles_gu;
  const int tile = blockIdx.x - task * a.tiles_gu;
  // the descriptor slot always exists (max_tasks of them): load it together with the count
  const DecodeTask tk = a.tasks[task];
  if (task >= a.ctrl[kCtrlNTasks]) return;
  const uint8_t* blob = task_blob(a.src, tk);
  if (!blob) {
    if (threadIdx.x == 0) set_error(a.ctrl, MOE_DERR_NOT_RESIDENT);
    return;
  }
  const int H = a.H, F = a.F;
  const BlobLayout lay = blob_layout(H, F);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int row = tile * 16 + n;
  const int q0 = wave * kGuQuadsPerWave;
  const int nq = min(kGuQuadsPerWave, H / kGroupElems - q0);

  // ---- loads, group by group in the order the MFMA steps use them: the activations of the
  // group (A row m = lane % 16, inputs 32 i + 8 g .. +7), then slice g of the group's record of
  // row `row` in both matrices, and the record's four scales.  No load sits under a branch (dead
  // lanes and groups past the wave's range load valid, clamped addresses and are masked after),
  // so the compiler can wait for each group's data alone.
  const int m = n;
  const int tslot = X_BF16 ? m : (m >> 1);
  const int n_tok = __builtin_popcount(tk.tok_mask);
  const bool live = m < ROWS && tslot < n_tok;
  const int tok = live ? task_token(tk.tok_mask, tslot) : 0;
  const uint8_t* gcode = blob + lay.gate_codes + (size_t)row * kGroupBytes + 16 * g;
  const uint8_t* ucode = blob + lay.up_codes + (size_t)row * kGroupBytes + 16 * g;
  const uint8_t* gscale = blob + lay.gate_scales + (size_t)row * kGroupScaleBytes;
  const uint8_t* uscale = blob + lay.up_scales + (size_t)row * kGroupScaleBytes;
  const uint16_t* xr = (const uint16_t*)a.x + (size_t)tok * H + 8 * g;
  const int NQ = H / kGroupElems;
  uint4 cg[kGuQuadsPerWave], cu[kGuQuadsPerWave];
  uint2 sg[kGuQuadsPerWave], su[kGuQuadsPerWave];
  uint4 xa[X_BF16 ? kGuQuadsPerWave : 1][4];
#pragma unroll
  for (int qi = 0; qi < kGuQuadsPerWave; ++qi) {
    const int qq = min(q0 + qi, NQ - 1);  // record (qq, row) at 64 (qq F + row)
    if constexpr (X_BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) xa[qi][i] = *(const uint4*)(xr + (size_t)qq * kGroupElems + 32 * i);
    }
    cg[qi] = *(const uint4*)(gcode + (size_t)qq * F * kGroupBytes);
    cu[qi] = *(const uint4*)(ucode + (size_t)qq * F * kGroupBytes);
    sg[qi] = *(const uint2*)(gscale + (size_t)qq * F * kGroupScaleBytes);
    su[qi] = *(const uint2*)(uscale + (size_t)qq * F * kGroupScaleBytes);
  }
  issue_fence();
  if constexpr (X_BF16) {
#pragma unroll
    for (int qi = 0; qi < kGuQuadsPerWave; ++qi)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (!live) xa[qi][i] = make_uint4(0u, 0u, 0u, 0u);
  }

  const bf16x8 neg = const_neg136();
  const float4v zero = {0.f, 0.f, 0.f, 0.f};
  float accg[NR], accu[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) accg[r] = accu[r] = 0.f;
#pragma unroll
  for (int qi = 0; qi < kGuQuadsPerWave; ++qi) {
    if (qi >= nq) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint4 av;
      if constexpr (X_BF16) {
        av = xa[qi][i];
      } else {
        av = make_uint4(0u, 0u, 0u, 0u);
        if (live) {
          const float* xf = (const float*)a.x + (size_t)tok * H + (size_t)(q0 + qi) * kGroupElems + 32 * i + 8 * g;
          av = split_part(*(const float4*)xf, *(const float4*)(xf + 4), m & 1);
        }
      }
      const bf16x8 A = __builtin_bit_cast(bf16x8, av);
      const float4v O = mfma_bf16(A, neg, zero);
      const float4v Dg = mfma_bf16(A, codes_q136(word_at(cg[qi], i)), O);
      const float4v Du = mfma_bf16(A, codes_q136(word_at(cu[qi], i)), O);
      const float s_g = scale_at(sg[qi], i), s_u = scale_at(su[qi], i);
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        accg[r] = fmaf(s_g, Dg[r], accg[r]);
        accu[r] = fmaf(s_u, Du[r], accu[r]);
      }
    }
  }

  // ---- reduce the waves' K ranges, SwiGLU, store h as bf16 hi + lo ---------------------------
  // lane (g, n) holds rows 4g + r of column n
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int mr = 4 * g + r;
    if (mr < ROWS) {
      red[wave][0][mr][n] = accg[r];
      red[wave][1][mr][n] = accu[r];
    }
  }
  __syncthreads();
  const int nw = blockDim.x >> 6;
  if ((int)threadIdx.x < 16 * MAXTOK) {
    const int ts = threadIdx.x >> 4, c = threadIdx.x & 15;
    if (ts < n_tok) {
      float gs = 0.f, us = 0.f;
      for (int w = 0; w < nw; ++w) {
        if constexpr (X_BF16) {
          gs += red[w][0][ts][c];
          us += red[w][1][ts][c];
        } else {
          gs += red[w][0][2 * ts][c] + red[w][0][2 * ts + 1][c];
          us += red[w][1][2 * ts][c] + red[w][1][2 * ts + 1][c];
        }
      }
      const float h = silu(gs) * us;
      const uint32_t hi = f32_to_bf16_rne(h);
      const uint32_t lo = f32_to_bf16_rne(h - __uint_as_float(hi << 16));
      const size_t o = (size_t)task_pair(tk, task_token(tk.tok_mask, ts), a.T, a.k) * F + tile * 16 + c;
      a.h_hi[o] = (uint16_t)hi;
      a.h_lo[o] = (uint16_t)lo;
    }
  }
}

// ---- down: y_e[pair][o] = Wd[o] . h[pair] for one task and 16 output rows per wave ----------
// A rows 2 s + part: token slot s, part 0 = h_hi, 1 = h_lo.
template <int MAXTOK>
__global__ __launch_bounds__(256) void k_decode_down(DecodeArgs a) {
  constexpr int ROWS = 2 * MAXTOK;
  constexpr int NR = ROWS < 4 ? ROWS : 4;
  const int task = blockIdx.x / a.tiles_dn;
  const int tile = blockIdx.x - task * a.tiles_dn;
  const DecodeTask tk = a.tasks[task];
  if (task >= a.ctrl[kCtrlNTasks]) return;
  const uint8_t* blob = task_blob(a.src, tk);
  if (!blob) {
    if (threadIdx.x == 0) set_error(a.ctrl, MOE_DERR_NOT_RESIDENT);
    return;
  }
  const int H = a.H, F = a.F;
  const BlobLayout lay = blob_layout(H, F);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int row = (tile * 4 + wave) * 16 + n;
  const int NQ = F / kGroupElems;

  // record (q, row) of the down matrix (H rows) is at 64 (q H + row)
  const uint8_t* dcode = blob + lay.down_codes + (size_t)row * kGroupBytes + 16 * g;
  const uint8_t* dscale = blob + lay.down_scales + (size_t)row * kGroupScaleBytes;
  const int m = n, ts = m >> 1;
  const int n_tok = __builtin_popcount(tk.tok_mask);
  const bool live = m < ROWS && ts < n_tok;
  const int hpair = live ? task_pair(tk, task_token(tk.tok_mask, ts), a.T, a.k) : 0;
  const uint16_t* hrow = ((m & 1) ? a.h_lo : a.h_hi) + (size_t)hpair * F + 8 * g;

  const bf16x8 neg = const_neg136();
  const float4v zero = {0.f, 0.f, 0.f, 0.f};
  float acc[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) acc[r] = 0.f;
  for (int q0 = 0; q0 < NQ; q0 += kDnQuadsPerPass) {
    const int nq = min(kDnQuadsPerPass, NQ - q0);
    uint4 cd[kDnQuadsPerPass], ha[kDnQuadsPerPass][4];
    uint2 sd[kDnQuadsPerPass];
    // loads group by group in the order of use: h (A operands), then the record and its scales;
    // unconditional (clamped addresses, dead lanes masked after) so each group is waited for alone
#pragma unroll
    for (int qi = 0; qi < kDnQuadsPerPass; ++qi) {
      const int qq = min(q0 + qi, NQ - 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) ha[qi][i] = *(const uint4*)(hrow + (size_t)qq * kGroupElems + 32 * i);
      cd[qi] = *(const uint4*)(dcode + (size_t)qq * H * kGroupBytes);
      sd[qi] = *(const uint2*)(dscale + (size_t)qq * H * kGroupScaleBytes);
    }
    issue_fence();
#pragma unroll
    for (int qi = 0; qi < kDnQuadsPerPass; ++qi)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (!live) ha[qi][i] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int qi = 0; qi < kDnQuadsPerPass; ++qi) {
      if (qi >= nq) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8 A = __builtin_bit_cast(bf16x8, ha[qi][i]);
        const float4v O = mfma_bf16(A, neg, zero);
        const float4v D = mfma_bf16(A, codes_q136(word_at(cd[qi], i)), O);
        const float s = scale_at(sd[qi], i);
#pragma unroll
        for (int r = 0; r < NR; ++r) acc[r] = fmaf(s, D[r], acc[r]);
      }
    }
  }
  // lane (g, n) holds rows 4g + r: token slots 2g (r = 0, 1) and 2g + 1 (r = 2, 3)
#pragma unroll
  for (int s2 = 0; s2 < NR / 2; ++s2) {
    const int slot = 2 * g + s2;
    if (slot < n_tok)
      a.y_pairs[(size_t)task_pair(tk, task_token(tk.tok_mask, slot), a.T, a.k) * H + row] = acc[2 * s2] + acc[2 * s2 + 1];
  }
}

// ---- combine: y[t][o] = sum_j w[t][j] * y_pairs[t k + j][o] (+ y_pairs[T k + t][o]) ----------
__global__ __launch_bounds__(256) void k_decode_combine(DecodeArgs a) {
  const int per_tok = a.H / 4;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= a.T * per_tok) return;
  const int t = i / per_tok, o = (i - t * per_tok) * 4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < a.k; ++j) {
    const float w = a.topk_w[t * a.k + j];
    const float4 v = *(const float4*)(a.y_pairs + (size_t)(t * a.k + j) * a.H + o);
    acc.x = fmaf(w, v.x, acc.x);
    acc.y = fmaf(w, v.y, acc.y);
    acc.z = fmaf(w, v.z, acc.z);
    acc.w = fmaf(w, v.w, acc.w);
  }
  if (a.n_shared) {
    const float4 v = *(const float4*)(a.y_pairs + (size_t)(a.T * a.k + t) * a.H + o);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  *(float4*)(a.y + (size_t)t * a.H + o) = acc;
}

// ---- dequantization check: one thread per code word, the same unpacking as the FFN kernels --
__global__ __launch_bounds__(256) void k_debug_dequant(int H, int F, const uint8_t* __restrict__ blob,
                                                        int matrix, float* __restrict__ out) {
  const BlobLayout lay = blob_layout(H, F);
  const int rows = matrix == 2 ? H : F, cols = matrix == 2 ? F : H;
  const int64_t codes = matrix == 0 ? lay.gate_codes : matrix == 1 ? lay.up_codes : lay.down_codes;
  const int64_t scales = matrix == 0 ? lay.gate_scales : matrix == 1 ? lay.up_scales : lay.down_scales;
  const int n_words = rows * cols / 8;
  for (int wi = blockIdx.x * blockDim.x + threadIdx.x; wi < n_words; wi += gridDim.x * blockDim.x) {
    const int rec = wi >> 4, p = wi & 15, g = p >> 2, i = p & 3;  // word 4g + i of record rec
    const int grp = rec / rows, r = rec - grp * rows;            // record (grp, r)
    const int blk = 4 * grp + i;
    const int c0 = blk * kBlock + 8 * g;
    const uint32_t w = *(const uint32_t*)(blob + codes + (size_t)wi * 4);
    const float s = fp16_bits_to_f32(*(const uint16_t*)(blob + scales + (size_t)rec * kGroupScaleBytes + 2 * i));
    const uint4 q = __builtin_bit_cast(uint4, codes_q136(w));
    const uint32_t pr[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      out[(size_t)r * cols + c0 + 2 * j] = (bf16_lo(pr[j]) - 136.f) * s;
      out[(size_t)r * cols + c0 + 2 * j + 1] = (bf16_hi(pr[j]) - 136.f) * s;
    }
  }
}

__global__ void k_fill_zero(uint32_t* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0u;
}

// ------------------------------------------------------------------------------------------
// Launchers
// ------------------------------------------------------------------------------------------
template <int MAXTOK>
static hipError_t launch_decode_ffn_t(const DecodeArgs& a, int max_tasks, bool xb, hipStream_t st) {
  const int gu_waves = (a.H / kGroupElems + kGuQuadsPerWave - 1) / kGuQuadsPerWave;
  const int grid_gu = max_tasks * a.tiles_gu, grid_dn = max_tasks * a.tiles_dn;
  hipError_t err;
  if (xb) err = launch_timed(kTimeDecodeGateUp, k_decode_gate_up<MAXTOK, true>, grid_gu, 64 * gu_waves, 0, st, a);
  else err = launch_timed(kTimeDecodeGateUp, k_decode_gate_up<MAXTOK, false>, grid_gu, 64 * gu_waves, 0, st, a);
  if (err != hipSuccess) return err;
  err = launch_timed(kTimeDecodeDown, k_decode_down<MAXTOK>, grid_dn, 256, 0, st, a);
  if (err != hipSuccess) return err;
  const int n4 = a.T * a.H / 4;
  k_decode_combine<<<(n4 + 255) / 256, 256, 0, st>>>(a);
  return hipGetLastError();
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
  a.tiles_gu = F / 16;
  a.tiles_dn = H / 64;
  const bool xb = x_dtype == MOE_BF16;
  static_assert(kTaskTok == kMaxDecodeTok, "a decode task holds every token of the step that chose its expert");
  if (T <= 1) return launch_decode_ffn_t<1>(a, max_tasks, xb, st);
  if (T <= 2) return launch_decode_ffn_t<2>(a, max_tasks, xb, st);
  if (T <= 4) return launch_decode_ffn_t<4>(a, max_tasks, xb, st);
  return launch_decode_ffn_t<8>(a, max_tasks, xb, st);
}

hipError_t launch_debug_dequant(int H, int F, const uint8_t* blob, int matrix, float* out, hipStream_t st) {
  const int n_words = H * F / 8;
  int grid = (n_words + 255) / 256;
  if (grid > 2048) grid = 2048;
  k_debug_dequant<<<grid, 256, 0, st>>>(H, F, blob, matrix, out);
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
