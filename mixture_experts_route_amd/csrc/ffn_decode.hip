// Expert FFNs for a small batch of tokens (decode): 4-bit GEMV, bandwidth-bound.
//
// Weights: halogen-flash-server README, "Bring your own GGUF" (small set of values x one scale
// per block, used as stored).  The layer: Betelgeuse news article, "mechanism" (10 routed + 1
// shared expert per token).  Decode pays per byte of weights read (halogen README, "Bring your
// own GGUF": an 8-bit trunk costs 2 GB more per token at 240 GB/s), so each selected expert's blob
// is streamed once from HBM per step.
//
// GEMV design (gfx950): one lane per quantization block of a row.  A row of K inputs has L = K/32
// blocks; the L lanes of a row group (L rounded up to a power of two Lp, so P = 64/Lp rows per
// wave pass) each load the block's 16 code bytes with one 128-bit load and its fp16 scale.  The
// activations of the lane's block live in registers as bf16 pairs, so the inner loop is: one mask
// per code pair (the pair becomes two bf16 values q + 136, exact), one v_dot2c_f32_bf16 per pair
// and token, and one scale FMA per block and token.  The +136 offset is removed by starting each
// block's chain at -136 * sum(x over the block).  fp32 inputs (the FFN intermediate h, fp32
// activations) are split into two bf16 parts hi + lo (16 significant bits), each run through the
// same chain.  Row sums are reduced across the Lp lanes with DPP.
//
// Two kernels run the FFN of a step and no workgroup depends on another: the gate/up kernel (one
// workgroup per (task, 16-row tile)) writes h; in the down kernel one workgroup owns a tile of
// output rows for every task of the step (its waves take the tasks in turn), keeps each pair's
// partial rows in LDS and combines them for every token in the fixed order j = 0..k-1, then the
// shared expert.
#include "kernels.hpp"

namespace moe {

constexpr int kDecodeWaves = 4;  // waves per workgroup
constexpr int kRowsPerWave = 4;  // wave passes per unit (each pass covers P rows)
constexpr int kDnPasses = 4;     // down: wave passes per task (each pass covers P rows)
constexpr int kMaxPairs = kMaxDecodeTok * (kMaxK + 1);

// A task's blob: the shared expert, the slot the plan resolved, or (for an expert that missed when
// the plan ran and was filled since) the table entry read now.
MOE_DEV const uint8_t* task_blob(const ExpertSource& s, const DecodeTask& tk) {
  if (tk.expert < 0) return s.shared_blob;
  int slot = tk.slot;
  if (slot < 0) slot = s.table ? s.table[tk.expert] : tk.expert;
  if (slot < 0 || slot >= s.n_slots) return nullptr;
  return s.arena + (int64_t)slot * s.slot_stride;
}

// The 32 activations of block `blk` of row `src` as bf16 pair words (pair i = elements 2i,
// 2i+1) in NPART parts, and each part's chain start -136 * sum(part over the block).
template <int NPART, bool SRC_BF16>
MOE_DEV void load_x_block(const void* src, int blk, uint32_t (&q)[NPART][16], float (&init)[NPART]) {
  if constexpr (SRC_BF16) {
    static_assert(NPART == 1, "bf16 activations are one part");
    const uint4* p = (const uint4*)((const uint16_t*)src + (size_t)blk * kBlock);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = p[i];
      q[0][4 * i + 0] = v.x;
      q[0][4 * i + 1] = v.y;
      q[0][4 * i + 2] = v.z;
      q[0][4 * i + 3] = v.w;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) s += bf16_lo(q[0][i]) + bf16_hi(q[0][i]);
    init[0] = -136.f * s;
  } else {
    const float4* p = (const float4*)((const float*)src + (size_t)blk * kBlock);
    float s[NPART];
#pragma unroll
    for (int pp = 0; pp < NPART; ++pp) s[pp] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 v = p[i];
      const float f[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t hi[2], lo[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float xv = f[2 * h + e];
          hi[e] = f32_to_bf16_rne(xv);
          const float hv = __uint_as_float(hi[e] << 16);
          lo[e] = f32_to_bf16_rne(xv - hv);
          s[0] += hv;
          if constexpr (NPART == 2) s[1] += __uint_as_float(lo[e] << 16);
        }
        q[0][2 * i + h] = hi[0] | (hi[1] << 16);
        if constexpr (NPART == 2) q[1][2 * i + h] = lo[0] | (lo[1] << 16);
      }
    }
#pragma unroll
    for (int pp = 0; pp < NPART; ++pp) init[pp] = -136.f * s[pp];
  }
}

// sum over the block of x * q, for one part: starts at init = -136 * sum(x).
MOE_DEV float block_dot(const uint4 c, const uint32_t (&xq)[16], float init) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  float acc = init;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = dot2_bf16(xq[4 * d + j], code_pair_bf16_q136(w[d], j), acc);
  }
  return acc;
}

struct DecodeArgs {
  ExpertSource src;
  const DecodeTask* tasks;
  int32_t* ctrl;
  const void* x;         // activations [T][H], bf16 or fp32
  float* h;              // [pairs][F]
  float* y_pairs;        // [pairs][H]
  const float* topk_w;   // [T][k]
  float* y;              // [T][H]
  int H, F, T, k, n_shared;
  int tiles_gu, tiles_dn, max_tasks;
};

MOE_DEV int lanes_per_row(int L) {
  int Lp = 1;
  while (Lp < L && Lp < 64) Lp <<= 1;
  return Lp;
}

// Sum over the Lp lanes of a row group; valid in the group's last lane.
MOE_DEV float row_sum(float v, int Lp) {
  if (Lp >= 16) return group_sum_dpp(v, Lp);
  return group_sum(v, Lp);  // narrow rows (small hidden sizes): shuffles, valid in every lane
}

MOE_DEV bool row_writer(int lane, int Lp) { return Lp >= 16 ? group_last_lane(lane, Lp) : (lane % Lp) == 0; }

// ---- gate/up unit: h[pair][r] = silu(Wg[r] . x) * (Wu[r] . x) for the unit's rows ------------
template <int MAXTOK, int NPART, int BPL, bool X_BF16>
MOE_DEV void gate_up_unit(const DecodeArgs& a, const DecodeTask* tk, int tile) {
  const uint8_t* blob = task_blob(a.src, *tk);
  if (!blob) {
    if (threadIdx.x == 0) set_error(a.ctrl, MOE_DERR_NOT_RESIDENT);
    return;
  }
  const int ntok = tk->n_tok;
  const int H = a.H, F = a.F, L = H / kBlock;
  const BlobLayout lay = blob_layout(H, F);
  const int Lp = lanes_per_row(L), P = 64 / Lp;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane / Lp, b0 = lane - sub * Lp;
  const bool active = b0 < L;
  const int row0 = (tile * kDecodeWaves + wave) * kRowsPerWave * P;

  // weights first: they do not depend on the activations
  uint4 gc[kRowsPerWave][BPL], uc[kRowsPerWave][BPL];
  float gs[kRowsPerWave][BPL], us[kRowsPerWave][BPL];
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    const int r = row0 + i * P + sub;
#pragma unroll
    for (int bb = 0; bb < BPL; ++bb) {
      const int blk = b0 + 64 * bb;
      if (active && blk < L && r < F) {
        gc[i][bb] = *(const uint4*)(blob + lay.gate_codes + (size_t)r * (H / 2) + (size_t)blk * 16);
        uc[i][bb] = *(const uint4*)(blob + lay.up_codes + (size_t)r * (H / 2) + (size_t)blk * 16);
        gs[i][bb] = fp16_bits_to_f32(*(const uint16_t*)(blob + lay.gate_scales + ((size_t)r * L + blk) * 2));
        us[i][bb] = fp16_bits_to_f32(*(const uint16_t*)(blob + lay.up_scales + ((size_t)r * L + blk) * 2));
      } else {
        gc[i][bb] = make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
        uc[i][bb] = gc[i][bb];
        gs[i][bb] = 0.f;
        us[i][bb] = 0.f;
      }
    }
  }

  uint32_t xq[MAXTOK][BPL][NPART][16];
  float xi[MAXTOK][BPL][NPART];
#pragma unroll
  for (int n = 0; n < MAXTOK; ++n) {
#pragma unroll
    for (int bb = 0; bb < BPL; ++bb) {
      if (n < ntok && active && b0 + 64 * bb < L) {
        const int t = tk->tok[n];
        const void* xrow = X_BF16 ? (const void*)((const uint16_t*)a.x + (size_t)t * H)
                                  : (const void*)((const float*)a.x + (size_t)t * H);
        load_x_block<NPART, X_BF16>(xrow, b0 + 64 * bb, xq[n][bb], xi[n][bb]);
      } else {
#pragma unroll
        for (int p = 0; p < NPART; ++p) {
          xi[n][bb][p] = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) xq[n][bb][p][i] = 0u;
        }
      }
    }
  }

#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    const int r = row0 + i * P + sub;
#pragma unroll
    for (int n = 0; n < MAXTOK; ++n) {
      if (n < ntok) {
        float g = 0.f, u = 0.f;
#pragma unroll
        for (int bb = 0; bb < BPL; ++bb) {
          float sg = 0.f, su = 0.f;
#pragma unroll
          for (int p = 0; p < NPART; ++p) {
            sg += block_dot(gc[i][bb], xq[n][bb][p], xi[n][bb][p]);
            su += block_dot(uc[i][bb], xq[n][bb][p], xi[n][bb][p]);
          }
          g = fmaf(sg, gs[i][bb], g);
          u = fmaf(su, us[i][bb], u);
        }
        const float gt = row_sum(g, Lp);
        const float ut = row_sum(u, Lp);
        if (row_writer(lane, Lp) && r < F) a.h[(size_t)tk->pair[n] * F + r] = silu(gt) * ut;
      }
    }
  }
}

template <int MAXTOK, int NPART_X, int BPL, bool X_BF16>
__global__ __launch_bounds__(256) void k_decode_gate_up(DecodeArgs a) {
  const int task = blockIdx.x / a.tiles_gu;
  // the descriptor slot always exists (max_tasks of them): load it together with the count
  const DecodeTask tk = a.tasks[task];
  if (task >= a.ctrl[kCtrlNTasks]) return;
  gate_up_unit<MAXTOK, NPART_X, BPL, X_BF16>(a, &tk, blockIdx.x - task * a.tiles_gu);
}

// ---- down + combine: rows [tile*RW, tile*RW + RW) of y for every token ----------------------
// RW = kDnPasses * P rows.  Wave w takes tasks w, w+4, ...; it issues the weight and h loads of
// TS of its tasks before computing any of them, so their latencies overlap.
template <int MAXTOK, int BPL, int TS>
__global__ __launch_bounds__(256) void k_decode_down(DecodeArgs a) {
  __shared__ float ys[kMaxPairs][kDnPasses * 16];
  const int n_tasks = a.ctrl[kCtrlNTasks];
  const int H = a.H, F = a.F, L = F / kBlock;
  const BlobLayout lay = blob_layout(H, F);
  const int Lp = lanes_per_row(L), P = 64 / Lp;
  const int RW = kDnPasses * P;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane / Lp, b0 = lane - sub * Lp;
  const bool active = b0 < L;
  constexpr int NPART = 2;
  const int row0 = blockIdx.x * RW;
  for (int base = wave; base < n_tasks; base += kDecodeWaves * TS) {
    int ntok[TS];
    const uint8_t* blob[TS];
    int pair[TS][MAXTOK];
    uint4 dc[TS][kDnPasses][BPL];
    float ds[TS][kDnPasses][BPL];
    uint32_t xq[TS][MAXTOK][BPL][NPART][16];
    float xi[TS][MAXTOK][BPL][NPART];
#pragma unroll
    for (int q = 0; q < TS; ++q) {
      const int task = base + kDecodeWaves * q;
      ntok[q] = 0;
      blob[q] = nullptr;
      if (task < n_tasks) {
        const DecodeTask* tk = a.tasks + task;
        blob[q] = task_blob(a.src, *tk);
        if (!blob[q]) {
          if (lane == 0) set_error(a.ctrl, MOE_DERR_NOT_RESIDENT);
        } else {
          ntok[q] = tk->n_tok;
        }
#pragma unroll
        for (int n = 0; n < MAXTOK; ++n) pair[q][n] = n < ntok[q] ? tk->pair[n] : 0;
      }
#pragma unroll
      for (int i = 0; i < kDnPasses; ++i) {
        const int r = row0 + i * P + sub;
#pragma unroll
        for (int bb = 0; bb < BPL; ++bb) {
          const int blk = b0 + 64 * bb;
          if (ntok[q] > 0 && active && blk < L && r < H) {
            dc[q][i][bb] = *(const uint4*)(blob[q] + lay.down_codes + (size_t)r * (F / 2) + (size_t)blk * 16);
            ds[q][i][bb] =
                fp16_bits_to_f32(*(const uint16_t*)(blob[q] + lay.down_scales + ((size_t)r * L + blk) * 2));
          } else {
            dc[q][i][bb] = make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
            ds[q][i][bb] = 0.f;
          }
        }
      }
    }
#pragma unroll
    for (int q = 0; q < TS; ++q) {
#pragma unroll
      for (int n = 0; n < MAXTOK; ++n) {
#pragma unroll
        for (int bb = 0; bb < BPL; ++bb) {
          if (n < ntok[q] && active && b0 + 64 * bb < L) {
            const float* hrow = a.h + (size_t)pair[q][n] * F;
            load_x_block<NPART, false>(hrow, b0 + 64 * bb, xq[q][n][bb], xi[q][n][bb]);
          } else {
#pragma unroll
            for (int p = 0; p < NPART; ++p) {
              xi[q][n][bb][p] = 0.f;
#pragma unroll
              for (int i = 0; i < 16; ++i) xq[q][n][bb][p][i] = 0u;
            }
          }
        }
      }
    }
#pragma unroll
    for (int q = 0; q < TS; ++q) {
#pragma unroll
      for (int i = 0; i < kDnPasses; ++i) {
#pragma unroll
        for (int n = 0; n < MAXTOK; ++n) {
          if (n < ntok[q]) {
            float yv = 0.f;
#pragma unroll
            for (int bb = 0; bb < BPL; ++bb) {
              float sd = 0.f;
#pragma unroll
              for (int p = 0; p < NPART; ++p) sd += block_dot(dc[q][i][bb], xq[q][n][bb][p], xi[q][n][bb][p]);
              yv = fmaf(sd, ds[q][i][bb], yv);
            }
            const float yt = row_sum(yv, Lp);
            if (row_writer(lane, Lp)) ys[pair[q][n]][i * P + sub] = yt;
          }
        }
      }
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < a.T * RW; idx += blockDim.x) {
    const int t = idx / RW, rr = idx - t * RW, o = row0 + rr;
    if (o >= H) continue;
    float acc = 0.f;
    for (int j = 0; j < a.k; ++j) acc = fmaf(a.topk_w[t * a.k + j], ys[t * a.k + j][rr], acc);
    if (a.n_shared) acc += ys[a.T * a.k + t][rr];
    a.y[(size_t)t * H + o] = acc;
  }
}

// ------------------------------------------------------------------------------------------
// Test entry: dequantize one matrix of a blob to fp32 (exact).
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_debug_dequant(int H, int F, const uint8_t* __restrict__ blob,
                                                        int matrix, float* __restrict__ out) {
  const BlobLayout lay = blob_layout(H, F);
  const int rows = matrix == 2 ? H : F, cols = matrix == 2 ? F : H;
  const int64_t codes = matrix == 0 ? lay.gate_codes : matrix == 1 ? lay.up_codes : lay.down_codes;
  const int64_t scales = matrix == 0 ? lay.gate_scales : matrix == 1 ? lay.up_scales : lay.down_scales;
  const int n_words = rows * cols / 8;
  for (int wi = blockIdx.x * blockDim.x + threadIdx.x; wi < n_words; wi += gridDim.x * blockDim.x) {
    const int r = wi / (cols / 8), d = wi - r * (cols / 8);
    const uint32_t w = *(const uint32_t*)(blob + codes + (size_t)wi * 4);
    const int c0 = d * 8;
    const float s = fp16_bits_to_f32(*(const uint16_t*)(blob + scales + ((size_t)r * (cols / kBlock) + c0 / kBlock) * 2));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t pr = code_pair_bf16_q136(w, j);
      out[(size_t)r * cols + c0 + 2 * j] = (bf16_lo(pr) - 136.f) * s;
      out[(size_t)r * cols + c0 + 2 * j + 1] = (bf16_hi(pr) - 136.f) * s;
    }
  }
}

__global__ void k_fill_zero(uint32_t* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0u;
}

// ------------------------------------------------------------------------------------------
// Launchers
// ------------------------------------------------------------------------------------------
static int lanes_per_row_host(int K) {
  const int L = K / kBlock;
  int Lp = 1;
  while (Lp < L && Lp < 64) Lp <<= 1;
  return Lp;
}

// gate/up: rows per workgroup; down: rows per workgroup (one tile of y for all tasks)
static int rows_per_unit(int K) { return kDecodeWaves * kRowsPerWave * (64 / lanes_per_row_host(K)); }
static int rows_per_down_tile(int F) { return kDnPasses * (64 / lanes_per_row_host(F)); }

int decode_tiles_dn(int H, int F) { return (H + rows_per_down_tile(F) - 1) / rows_per_down_tile(F); }

template <int MAXTOK>
static hipError_t launch_decode_ffn_t(const DecodeArgs& a, int bpl_gu, int bpl_dn, bool xb, hipStream_t st) {
  const int grid_gu = a.max_tasks * a.tiles_gu, grid_dn = a.tiles_dn;
  hipError_t err;
  if (xb) {
    if (bpl_gu == 1) err = launch_timed(kTimeDecodeGateUp, k_decode_gate_up<MAXTOK, 1, 1, true>, grid_gu, 256, 0, st, a);
    else err = launch_timed(kTimeDecodeGateUp, k_decode_gate_up<MAXTOK, 1, 2, true>, grid_gu, 256, 0, st, a);
  } else {
    if (bpl_gu == 1) err = launch_timed(kTimeDecodeGateUp, k_decode_gate_up<MAXTOK, 2, 1, false>, grid_gu, 256, 0, st, a);
    else err = launch_timed(kTimeDecodeGateUp, k_decode_gate_up<MAXTOK, 2, 2, false>, grid_gu, 256, 0, st, a);
  }
  if (err != hipSuccess) return err;
  // task slots per wave: as many as the registers allow for MAXTOK tokens per task
  constexpr int TS = MAXTOK == 1 ? 3 : MAXTOK == 2 ? 2 : 1;
  if (bpl_dn == 1) return launch_timed(kTimeDecodeDown, k_decode_down<MAXTOK, 1, TS>, grid_dn, 256, 0, st, a);
  return launch_timed(kTimeDecodeDown, k_decode_down<MAXTOK, 2, TS>, grid_dn, 256, 0, st, a);
}

hipError_t launch_decode_ffn(int H, int F, int k, int n_shared, int T, int max_tasks, const ExpertSource& src,
                             const void* x, int x_dtype, const DecodeTask* tasks, const float* topk_w,
                             float* h, float* y_pairs, float* y, int32_t* ctrl, hipStream_t st) {
  DecodeArgs a{};
  a.src = src;
  a.tasks = tasks;
  a.ctrl = ctrl;
  a.x = x;
  a.h = h;
  a.y_pairs = y_pairs;
  a.topk_w = topk_w;
  a.y = y;
  a.H = H;
  a.F = F;
  a.T = T;
  a.k = k;
  a.n_shared = n_shared;
  a.tiles_gu = (F + rows_per_unit(H) - 1) / rows_per_unit(H);
  a.tiles_dn = decode_tiles_dn(H, F);
  a.max_tasks = max_tasks;
  const int bpl_gu = (H / kBlock) > 64 ? 2 : 1;
  const int bpl_dn = (F / kBlock) > 64 ? 2 : 1;
  const bool xb = x_dtype == MOE_BF16;
  static_assert(kTaskTok == 4, "instantiations below cover tasks of up to 4 tokens");
  if (T <= 1) return launch_decode_ffn_t<1>(a, bpl_gu, bpl_dn, xb, st);
  if (T <= 2) return launch_decode_ffn_t<2>(a, bpl_gu, bpl_dn, xb, st);
  return launch_decode_ffn_t<4>(a, bpl_gu, bpl_dn, xb, st);
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
