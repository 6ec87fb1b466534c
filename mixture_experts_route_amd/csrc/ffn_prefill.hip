// Prefill: expert FFNs as grouped GEMMs on MFMA, plus the prefill router GEMM.
//
// The work is a dense contraction per expert once tokens are grouped by expert (halogen README,
// "Measured": prefill is compute-bound; Basalt README, "Prompt chunks": per-token cost keeps
// falling up to a few thousand tokens per call).  Weights: halogen README, "Bring your own GGUF"
// (small set of values x one scale per block, used as stored).
//
// Tile of one workgroup (4 waves): up to 128 rows of one expert (a TileItem, bucket-sorted rows)
// x 256 weight rows; each wave owns 64 weight rows (4 MFMA subtiles of 16) for all rows of the
// item.  Per 128-wide K chunk:
//   A (activations, fp16): staged global -> LDS (double-buffered, 16-byte padded rows), read
//     back as 16x16x32 MFMA fragments (one 16-byte LDS read per lane per MFMA, reused by the
//     wave's 4 subtiles);
//   B (weights): each lane loads 16 code bytes (slice g = lane / 16 of the chunk's four blocks,
//     the interleaved code layout) and the four block scales of its weight row straight into
//     registers and dequantizes to fp16 in registers, q * scale rounded once: two bit operations
//     build (1024 + u) in fp16, one packed subtract gives q exactly, one packed multiply applies
//     the scale.
//   MFMA v_mfma_f32_16x16x32_f16, fp32 accumulation.  MFMA d (0..3) of a chunk covers block d of
//   the chunk: word d of every lane's 16 bytes with activations 32 d + 8 g .. +7, so each B
//   register is used as loaded and each MFMA sees one scale per weight row.
// Rows of an item are processed in 16-row subtiles up to the item's row count (no work on
// padding beyond the last 16-row subtile).  fp16 (11 significant bits) instead of bf16 (8) for
// the dequantized weights and the SwiGLU intermediate keeps the layer within a 2e-3 relative
// error; the MFMA rate is the same.
// Work items are mapped XCD-aware: consecutive work indices (the n-tiles of one item, then the
// next item of the same expert) land on the same XCD and share its L2.
#include "kernels.hpp"

namespace moe {

constexpr int kKC = 128;                  // K per pipeline stage (4 quantization blocks)
constexpr int kAStride = kKC + 8;         // LDS row stride in 16-bit elements (16-byte pad)
constexpr int kMSub = kTileRows / 16;     // 16-row subtiles per item
constexpr int kNTileW = 256;              // weight rows per workgroup (4 waves x 64)

enum GemmMode { kGateUp = 0, kDown = 1, kRouter = 2 };
// Router GEMM token rows per work (the plan's choice): 32 or 64.  In the general kernel's router
// mode, 32-row works give a 4K-token call works enough to stream the router through every CU; the
// pipelined router kernel below (128 router rows per work) is faster with 64-row works from ~3K
// tokens (the default plan's thresholds follow these measurements).
constexpr int kRouterTileRows = 32;
constexpr int kRouterTallRows = 64;

struct GemmArgs {
  ExpertSource src;
  const TileItem* items;
  const int32_t* n_items;  // device count (ctrl word); null for the router (dense m-tiles)
  int32_t* ctrl;
  int n_ntiles;
  int n_works;             // items_max * n_ntiles
  int E;                   // bucket E = the shared expert
  int H, F;
  int T;                   // router: tokens
  const uint16_t* a16;     // gate/up: x16 [T][H]; down: h16 [P][F]; router: x bf16 [T][H]
  const int32_t* row_tok;  // gate/up: token of each sorted row
  const float* row_w;      // down: router weight of each sorted row
  const uint16_t* wr;      // router: Wr bf16 [E][H]
  const float* bias;       // router: bias [E] or null
  _Float16* h_out;         // gate/up: h16 [P][F]
  float* y_out;            // router: logits [T][E]
  _Float16* y16_out;       // down: y_rows [P][H], router-weighted, fp16
};

MOE_DEV const uint8_t* bucket_blob(const ExpertSource& s, int bucket, int E) {
  if (bucket == E) return s.shared_blob;
  const int slot = s.table ? s.table[bucket] : bucket;
  if (slot < 0 || slot >= s.n_slots) return nullptr;
  return s.arena + (int64_t)slot * s.slot_stride;
}

// One code word (8 elements of a slice) -> the 8 fp16 weights q * scale of an MFMA step.
MOE_DEV half8 dequant_word(uint32_t w, half2v s2) {
  const half2v off = {(_Float16)1032.0f, (_Float16)1032.0f};
  half8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t t = ((w >> (4 * j)) & 0x000F000Fu) | 0x64006400u;  // fp16 (1024 + u) pair
    const half2v q = __builtin_bit_cast(half2v, t) - off;              // q = u - 8, exact
    const half2v v = q * s2;                                           // fp16(q * scale)
    r[2 * j] = v.x;
    r[2 * j + 1] = v.y;
  }
  return r;
}

// The constants of dequant_word in registers (the nibble mask in a scalar register, the fp16 pair
// (1024, 1024) in a vector register): each pair is then one v_and_or_b32 (plus a shift), where
// literal operands make the compiler split it into an and and an or.
struct DequantConsts {
  uint32_t mask, magic, off;
};
MOE_DEV DequantConsts make_dequant_consts() {
  DequantConsts c;
  asm("s_mov_b32 %0, 0xf000f" : "=s"(c.mask));
  asm("v_mov_b32 %0, 0x64006400" : "=v"(c.magic));
  asm("s_mov_b32 %0, 0x64086408" : "=s"(c.off));  // fp16 pair (1032, 1032)
  return c;
}
MOE_DEV half8 dequant_word_k(uint32_t w, half2v s2, const DequantConsts& c) {
  const half2v off = __builtin_bit_cast(half2v, c.off);
  half8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t t = ((w >> (4 * j)) & c.mask) | c.magic;  // fp16 (1024 + u) pair
    const half2v q = __builtin_bit_cast(half2v, t) - off;   // q = u - 8, exact
    const half2v v = q * s2;                                // fp16(q * scale)
    r[2 * j] = v.x;
    r[2 * j + 1] = v.y;
  }
  return r;
}

MOE_DEV uint32_t word_of(const uint4& c, int d) { return d == 0 ? c.x : d == 1 ? c.y : d == 2 ? c.z : c.w; }

// The other weight formats, one rounding to fp16 each:
//   affine:   fp16(u * s - m) by one fp16 fma on the exact u (fp16 1024 + u minus 1024);
//   codebook: fp16(cb[u] * s), cb[u] exact in fp16, from a 256-entry table of fp16 pairs indexed by
//             a code pair (the pair j of a word: codes in bits 4j and 16 + 4j).
MOE_DEV half8 dequant_word_affine(uint32_t w, half2v s2, half2v nm2) {
  const half2v k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
  half8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t t = ((w >> (4 * j)) & 0x000F000Fu) | 0x64006400u;  // fp16 (1024 + u) pair
    const half2v u = __builtin_bit_cast(half2v, t) - k1024;           // u, exact
    const half2v v = __builtin_elementwise_fma(u, s2, nm2);           // fp16(u * s - m)
    r[2 * j] = v.x;
    r[2 * j + 1] = v.y;
  }
  return r;
}
MOE_DEV half8 dequant_word_cb(uint32_t w, half2v s2, const uint32_t* cbt16) {
  half8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const half2v v = __builtin_bit_cast(half2v, cbt16[code_pair_index(w, j)]) * s2;
    r[2 * j] = v.x;
    r[2 * j + 1] = v.y;
  }
  return r;
}
// The fp16 pair table of the codebook: entry (c1 << 4 | c0) = (fp16 cb[c0], fp16 cb[c1]).
MOE_DEV void fill_codebook_f16(const Codebook& cb, uint32_t* cbt16) {
  for (int i = threadIdx.x; i < 256; i += blockDim.x) {
    const _Float16 lo = (_Float16)(float)codebook_value(cb, i & 15), hi = (_Float16)(float)codebook_value(cb, i >> 4);
    cbt16[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
  }
}


MOE_DEV void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// fp16 operands and intermediates hold |v| <= 65504: a value beyond (or not finite) would be
// stored as an infinity, so it is reported instead (MOE_DERR_RANGE), once per wave.
MOE_DEV bool f16_out_of_range(float v) { return !(fabsf(v) <= 65504.0f); }
MOE_DEV void report_range(bool bad, int32_t* ctrl) {
  if (__any(bad) && (threadIdx.x & 63) == 0) set_error(ctrl, MOE_DERR_RANGE);
}

// RROWS: rows of a router work (the router's weights are read once per work: longer calls take
// taller works)
template <int MODE, int RROWS = kRouterTileRows, int FMT = MOE_FMT_Q4_0>
__global__ __launch_bounds__(256, 2) void k_expert_gemm(GemmArgs a) {
  __shared__ uint32_t cbt16[FMT == MOE_FMT_CB4 ? 256 : 1];
  // 16-row subtiles per work: a 128-row item, or a router work
  constexpr int MSUB = MODE == kRouter ? RROWS / 16 : kMSub;
  // A tile: 128 rows x 128 16-bit elements per stage, two stages.  16-byte chunk c of row r is
  // stored at chunk c ^ (r & 15) of the row, so the 16 lanes of a fragment read (16 rows, one
  // chunk) hit 16 different chunk slots.
  __shared__ __attribute__((aligned(1024))) uint16_t As0[kTileRows * kKC];
  __shared__ __attribute__((aligned(1024))) uint16_t As1[kTileRows * kKC];

  // XCD-aware work index: blockIdx i runs on XCD i % 8; each XCD gets a contiguous eighth of the
  // works that exist (the item count is known on the device only; the grid covers the bound).
  int n_works = a.n_works;
  if constexpr (MODE != kRouter) n_works = min(*a.n_items * a.n_ntiles, a.n_works);
  const int per_xcd = (n_works + 7) >> 3;
  const int local = (int)(blockIdx.x >> 3);
  const int work = (int)(blockIdx.x & 7) * per_xcd + local;
  if (local >= per_xcd || work >= n_works) return;
  const int item_id = work / a.n_ntiles;
  const int ntile = work - item_id * a.n_ntiles;

  TileItem it;
  const uint8_t* blob = nullptr;
  if constexpr (MODE == kRouter) {
    it.bucket = 0;
    it.row0 = item_id * RROWS;
    it.rows = min(RROWS, a.T - it.row0);
    if (it.rows <= 0) return;
  } else {
    it = a.items[item_id];
    blob = bucket_blob(a.src, it.bucket, a.E);
    if (!blob) {
      if (threadIdx.x == 0) set_error(a.ctrl, MOE_DERR_NOT_RESIDENT);
      return;
    }
  }

  const int H = a.H, F = a.F;
  const int K = MODE == kDown ? F : H;
  const int nk = K / kKC;
  const int wrows = MODE == kDown ? H : F;  // rows of the weight matrix
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int ms = (it.rows + 15) >> 4;

  // ---- this lane's 4 weight rows (one per subtile): byte offsets from one base --------------
  const uint8_t* bbase;
  uint32_t coff[4], soff[4];
  bool bvalid[4];
  if constexpr (MODE == kRouter) {
    bbase = (const uint8_t*)a.wr;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int e = ntile * kNTileW + wave * 64 + 16 * s + n;
      bvalid[s] = e < a.E;
      coff[s] = (uint32_t)(bvalid[s] ? e : 0) * (uint32_t)H * 2u;
      soff[s] = 0;
    }
  } else {
    const BlobLayout lay = blob_layout(H, F, FMT);
    bbase = blob;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      int row;
      int64_t cb, sb;
      if constexpr (MODE == kGateUp) {
        const bool up = s >= 2;
        row = ntile * (kNTileW / 2) + wave * 32 + 16 * (s & 1) + n;
        cb = up ? lay.up_codes : lay.gate_codes;
        sb = up ? lay.up_scales : lay.gate_scales;
      } else {
        row = ntile * kNTileW + wave * 64 + 16 * s + n;
        cb = lay.down_codes;
        sb = lay.down_scales;
      }
      bvalid[s] = true;
      // record (kc, row) of a matrix of R rows: codes at 64 (kc R + row), scales at 8 (kc R + row)
      coff[s] = (uint32_t)(cb + (int64_t)row * kGroupBytes);
      soff[s] = (uint32_t)(sb + (int64_t)row * kGroupScaleBytes);
    }
  }

  // ---- A staging by DMA: instruction i of wave w fills rows 16i + 4w + (lane >> 4) ---------
  const int a_ld = MODE == kDown ? F : H;
  const int a_pc = lane & 15;  // physical chunk written by this lane
  int32_t a_src[MSUB];        // source row (token or sorted row) of this lane's row per instruction
#pragma unroll
  for (int i = 0; i < MSUB; ++i) {
    const int r = 16 * i + 4 * wave + (lane >> 4);
    const int rr = r < it.rows ? r : 0;  // padding rows copy row 0 (their outputs are dropped)
    if constexpr (MODE == kGateUp) a_src[i] = a.row_tok[it.row0 + rr];
    else a_src[i] = it.row0 + rr;
  }
  const int a_lc = a_pc ^ ((4 * wave + (lane >> 4)) & 15);  // logical chunk: row & 15 = (4w + l/16) & 15
  auto issue_a = [&](int kc, uint16_t* buf) {
#pragma unroll
    for (int i = 0; i < MSUB; ++i) {
      if (i < ms)
        lds_dma16(a.a16 + (size_t)a_src[i] * a_ld + kc * kKC + a_lc * 8, buf + (16 * i + 4 * wave) * kKC);
    }
  };

  // ---- B registers --------------------------------------------------------------------------
  constexpr int kBW = MODE == kRouter ? 4 : 1;  // 16-byte loads per subtile per chunk
  uint4 braw[4][kBW];
  uint2 bsc[4];  // the four block scales (fp16) of the chunk
  uint2 bmn[4];  // affine format: the four block mins
  // distance from a scale record to its min record (the min planes follow the scale planes)
  int64_t min_from_scale = 0;
  if constexpr (MODE != kRouter && FMT == MOE_FMT_AFFINE4) {
    const BlobLayout lay = blob_layout(H, F, FMT);
    min_from_scale = MODE == kDown ? lay.down_mins - lay.down_scales : lay.gate_mins - lay.gate_scales;
  }
  auto load_b = [&](int kc) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if constexpr (MODE == kRouter) {
#pragma unroll
        for (int d = 0; d < 4; ++d)
          braw[s][d] = bvalid[s] ? *(const uint4*)(bbase + coff[s] + ((size_t)kc * kKC + 32 * d + 8 * g) * 2)
                                 : make_uint4(0u, 0u, 0u, 0u);
        bsc[s] = make_uint2(0u, 0u);
      } else {
        braw[s][0] = *(const uint4*)(bbase + coff[s] + (size_t)kc * wrows * kGroupBytes + 16 * g);
        bsc[s] = *(const uint2*)(bbase + soff[s] + (size_t)kc * wrows * kGroupScaleBytes);
        if constexpr (FMT == MOE_FMT_AFFINE4)
          bmn[s] = *(const uint2*)(bbase + soff[s] + min_from_scale + (size_t)kc * wrows * kGroupScaleBytes);
      }
    }
  };
  if constexpr (MODE != kRouter && FMT == MOE_FMT_CB4) fill_codebook_f16(a.src.cb, cbt16);  // before the barrier

  float4v acc[MSUB][4];
#pragma unroll
  for (int i = 0; i < MSUB; ++i)
#pragma unroll
    for (int s = 0; s < 4; ++s) acc[i][s] = (float4v){0.f, 0.f, 0.f, 0.f};

  issue_a(0, As0);
  load_b(0);
  wait_vm();
  __syncthreads();

  for (int kc = 0; kc < nk; ++kc) {
    uint16_t* Ab = (kc & 1) ? As1 : As0;
    uint4 bcur[4][kBW];
    uint2 scur[4], mcur[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int d = 0; d < kBW; ++d) bcur[s][d] = braw[s][d];
      scur[s] = bsc[s];
      if constexpr (FMT == MOE_FMT_AFFINE4) mcur[s] = bmn[s];
    }
    if (kc + 1 < nk) {
      issue_a(kc + 1, (kc & 1) ? As0 : As1);
      load_b(kc + 1);
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      // fragment read: row 16i + n, inputs 32 d + 8 g .. +7 = logical chunk 4d + g -> physical
      // chunk (4d + g) ^ n
      const int pcol = (((4 * d + g) ^ n) * 8);
      if constexpr (MODE == kRouter) {
#pragma unroll
        for (int i = 0; i < MSUB; ++i) {
          if (i < ms) {
            const bf16x8 af = *(const bf16x8*)(Ab + (16 * i + n) * kKC + pcol);
#pragma unroll
            for (int s = 0; s < 4; ++s)
              acc[i][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, __builtin_bit_cast(bf16x8, bcur[s][d]),
                                                                  acc[i][s], 0, 0, 0);
          }
        }
      } else {
        half8 bf[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint32_t sw = d < 2 ? scur[s].x : scur[s].y;
          const _Float16 sv = __builtin_bit_cast(_Float16, (uint16_t)((d & 1) ? (sw >> 16) : (sw & 0xFFFFu)));
          if constexpr (FMT == MOE_FMT_AFFINE4) {
            const uint32_t mw = d < 2 ? mcur[s].x : mcur[s].y;
            const _Float16 mv = __builtin_bit_cast(_Float16, (uint16_t)((d & 1) ? (mw >> 16) : (mw & 0xFFFFu)));
            bf[s] = dequant_word_affine(word_of(bcur[s][0], d), (half2v){sv, sv}, (half2v){-mv, -mv});
          } else if constexpr (FMT == MOE_FMT_CB4) {
            bf[s] = dequant_word_cb(word_of(bcur[s][0], d), (half2v){sv, sv}, cbt16);
          } else {
            bf[s] = dequant_word(word_of(bcur[s][0], d), (half2v){sv, sv});
          }
        }
#pragma unroll
        for (int i = 0; i < MSUB; ++i) {
          if (i < ms) {
            const half8 af = *(const half8*)(Ab + (16 * i + n) * kKC + pcol);
#pragma unroll
            for (int s = 0; s < 4; ++s)
              acc[i][s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[s], acc[i][s], 0, 0, 0);
          }
        }
      }
    }
    wait_vm();
    __syncthreads();
  }

  // ---- epilogue: lane holds D[16i + 4g + r][16s + n] -----------------------------------------
  bool range_bad = false;
#pragma unroll
  for (int i = 0; i < MSUB; ++i) {
    if (i >= ms) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * i + 4 * g + r;
      if (row >= it.rows) continue;
      if constexpr (MODE == kGateUp) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const float gv = acc[i][s][r], uv = acc[i][s + 2][r];
          const int col = ntile * (kNTileW / 2) + wave * 32 + 16 * s + n;
          const float hv = silu(gv) * uv;
          range_bad |= f16_out_of_range(hv);
          a.h_out[(size_t)(it.row0 + row) * F + col] = (_Float16)hv;
        }
      } else if constexpr (MODE == kDown) {
        const float wv = a.row_w[it.row0 + row];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int col = ntile * kNTileW + wave * 64 + 16 * s + n;
          const float yv = acc[i][s][r] * wv;
          range_bad |= f16_out_of_range(yv);
          a.y16_out[(size_t)(it.row0 + row) * H + col] = (_Float16)yv;
        }
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int e = ntile * kNTileW + wave * 64 + 16 * s + n;
          if (e < a.E)
            a.y_out[(size_t)(it.row0 + row) * a.E + e] = acc[i][s][r] + (a.bias ? a.bias[e] : 0.f);
        }
      }
    }
  }
  if constexpr (MODE != kRouter) report_range(range_bad, a.ctrl);
}

// ---- pipelined variant (the model's K: NK chunks of 128) ----------------------------------------
// Workgroup = 8 waves over 512 weight rows (gate/up: 256 gate + 256 up rows = 256 h columns; down:
// 512 output columns) of one item; each wave keeps the 128 x 64 tile of the scalar kernel above.
// The activation tile goes through a 3-stage LDS ring, loaded through registers 3 chunks before
// its MFMA work (written to LDS one chunk after its loads were issued, so the wait is for those
// loads alone); weights go through a 3-slot register ring, 2 chunks ahead.  One barrier per chunk
// and no wait for all loads: the weight stream never drains inside a work.
// Two shapes of it (a tuning choice, see the plan table): items of up to 128 rows with the weights
// 1 chunk ahead (MSUB 8, BD 2), or items of up to 64 rows, whose accumulators take half the registers,
// with the weights 3 chunks ahead (MSUB 4, BD 4): three times the weight bytes in flight per CU for
// the short items of a skewed routing, at the price of twice the weight reads of long groups.
constexpr int kPWaves = 8;
constexpr int kPNTile = 64 * kPWaves;                       // weight rows per workgroup

template <int MODE, int NK, int MSUB = kMSub, int BD = 2, int FMT = MOE_FMT_Q4_0>
__global__ __launch_bounds__(64 * kPWaves, 1) void k_expert_gemm_pipe(GemmArgs a) {
  static_assert(MODE == kGateUp || MODE == kDown, "expert GEMMs only");
  constexpr bool kAff = FMT == MOE_FMT_AFFINE4;
  __shared__ uint32_t cbt16[FMT == MOE_FMT_CB4 ? 256 : 1];
  static_assert(NK >= 3 && NK >= BD, "pipeline depth");
  static_assert(BD >= 2 && MSUB >= 1 && MSUB <= kMSub, "tile shape");
  constexpr int kPAPer = MSUB * 16 * (kKC / 8) / (64 * kPWaves);  // A 16-byte pieces per thread per chunk
  static_assert(kPAPer >= 1 && kPAPer * 64 * kPWaves == MSUB * 16 * (kKC / 8), "A pieces split evenly");
  __shared__ __attribute__((aligned(1024))) uint16_t As[3][MSUB * 16 * kKC];

  const int n_works = min(*a.n_items * a.n_ntiles, a.n_works);
  const int per_xcd = (n_works + 7) >> 3;
  const int local = (int)(blockIdx.x >> 3);
  const int work = (int)(blockIdx.x & 7) * per_xcd + local;
  if (local >= per_xcd || work >= n_works) return;
  const int item_id = work / a.n_ntiles;
  const int ntile = work - item_id * a.n_ntiles;
  const TileItem it = a.items[item_id];
  const uint8_t* blob = bucket_blob(a.src, it.bucket, a.E);
  if (!blob) {
    if (threadIdx.x == 0) set_error(a.ctrl, MOE_DERR_NOT_RESIDENT);
    return;
  }
  const int H = a.H, F = a.F;
  constexpr int K = NK * kKC;
  const int wrows = MODE == kDown ? H : F;
  const BlobLayout lay = blob_layout(H, F, FMT);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int ms = (it.rows + 15) >> 4;
  const DequantConsts uk = make_dequant_consts();

  // ---- weights: subtile s of this wave, row `row`, through the blob's buffer resource ----------
  const __amdgpu_buffer_rsrc_t rs = blob_rsrc(blob, lay.total);
  // subtile s = rows row0 + 16 s (down) or gate rows row0 + 16 (s & 1), up rows likewise (gate/up):
  // one per-lane offset per stream, the rest is uniform (scalar offset) or an immediate
  int row0;
  int32_t cb0, sb0, mb0 = 0, cb_up = 0, sb_up = 0;
  if constexpr (MODE == kGateUp) {
    row0 = ntile * (kPNTile / 2) + wave * 32 + n;
    cb0 = (int32_t)lay.gate_codes;
    sb0 = (int32_t)lay.gate_scales;
    cb_up = (int32_t)(lay.up_codes - lay.gate_codes);
    sb_up = (int32_t)(lay.up_scales - lay.gate_scales);  // the min planes are spaced as the scale planes
    if constexpr (kAff) mb0 = (int32_t)lay.gate_mins;
  } else {
    row0 = ntile * kPNTile + wave * 64 + n;
    cb0 = (int32_t)lay.down_codes;
    sb0 = (int32_t)lay.down_scales;
    if constexpr (kAff) mb0 = (int32_t)lay.down_mins;
  }
  // record (kc, row): codes at 64 (kc R + row), scales at 8 (kc R + row), mins likewise
  const int voff_c = row0 * kGroupBytes + 16 * g, voff_s = row0 * kGroupScaleBytes;
  u32x4 bc[BD][4];
  u32x2 bs[BD][4];
  u32x2 bm[kAff ? BD : 1][4];  // affine format: the records' mins
  // a bucket with one item: its weights are read once, with the non-temporal hint (the items of a
  // larger bucket re-read theirs through the L2)
  const bool w_once = (it.pad & kItemOnly) != 0;
  auto load_b = [&](auto slot_c, int kc) {
    constexpr int sl = decltype(slot_c)::value;
    auto go = [&](auto nt_c) {
      constexpr bool kNT = decltype(nt_c)::value;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int rsub = MODE == kGateUp ? 16 * (s & 1) : 16 * s;  // row offset of the subtile
        const bool up = MODE == kGateUp && s >= 2;
        const int vc = voff_c + rsub * kGroupBytes, vs = voff_s + rsub * kGroupScaleBytes;
        const int oc = cb0 + (up ? cb_up : 0) + kc * wrows * kGroupBytes;
        const int os = sb0 + (up ? sb_up : 0) + kc * wrows * kGroupScaleBytes;
        bc[sl][s] = kNT ? buf_load16_nt(rs, vc, oc) : buf_load16(rs, vc, oc);
        bs[sl][s] = kNT ? buf_load8_nt(rs, vs, os) : buf_load8(rs, vs, os);
        if constexpr (kAff) {
          const int om = mb0 + (up ? sb_up : 0) + kc * wrows * kGroupScaleBytes;
          bm[sl][s] = kNT ? buf_load8_nt(rs, vs, om) : buf_load8(rs, vs, om);
        }
      }
    };
    if (w_once) go(std::true_type{});
    else go(std::false_type{});
  };

  // ---- activations: piece j of this thread = row r_j, logical 16-byte chunk lc of the K chunk ----
  const int a_ld = MODE == kDown ? F : H;
  const int lc = threadIdx.x & 15;
  // element offset of each piece from a_base: gate/up reads token rows of x16 (T H elements, under
  // 2^31: checked on the host); down reads the item's own rows of h16, counted from the item's
  // first row, so the offsets stay small however many rows the call has
  const uint16_t* a_base = MODE == kGateUp ? a.a16 : a.a16 + (size_t)it.row0 * a_ld;
  int a_src[kPAPer];
  // LDS element offset of piece j: row r_j = r_0 + 32 j has the same r & 15, so only the row moves
  const int a_dst0 = (threadIdx.x >> 4) * kKC + ((lc ^ ((threadIdx.x >> 4) & 15)) * 8);
  constexpr int kRowStep = 64 * kPWaves / 16;
  static_assert(kRowStep % 16 == 0, "pieces keep their chunk swizzle");
#pragma unroll
  for (int j = 0; j < kPAPer; ++j) {
    const int r = (threadIdx.x >> 4) + kRowStep * j;
    const int rr = r < it.rows ? r : 0;  // padding rows copy row 0 (their outputs are dropped)
    const int src = MODE == kGateUp ? a.row_tok[it.row0 + rr] : rr;
    a_src[j] = src * a_ld + lc * 8;
  }
  auto load_a = [&](u32x4 (&v)[kPAPer], int kc) {
#pragma unroll
    for (int j = 0; j < kPAPer; ++j) v[j] = *(const u32x4*)(a_base + a_src[j] + kc * kKC);
  };
  auto store_a = [&](const u32x4 (&v)[kPAPer], uint16_t* buf) {
#pragma unroll
    for (int j = 0; j < kPAPer; ++j) *(u32x4*)(buf + a_dst0 + kRowStep * kKC * j) = v[j];
  };
  auto barrier = [&]() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  float4v acc[MSUB][4];
#pragma unroll
  for (int i = 0; i < MSUB; ++i)
#pragma unroll
    for (int s = 0; s < 4; ++s) acc[i][s] = (float4v){0.f, 0.f, 0.f, 0.f};

  if constexpr (FMT == MOE_FMT_CB4) fill_codebook_f16(a.src.cb, cbt16);  // visible after the prologue's barrier

  // ---- prologue: A(0), A(1) in LDS, A(2) and B(0 .. BD-2) in flight -------------------------------
  u32x4 av[kPAPer];
  {
    u32x4 a0[kPAPer];
    load_a(a0, 0);
    load_a(av, 1);
    static_for<BD - 1>([&](auto bc_c) { load_b(bc_c, decltype(bc_c)::value); });
    store_a(a0, As[0]);
    store_a(av, As[1]);
    load_a(av, 2);
    barrier();
  }

  static_for<NK>([&](auto kc_c) {
    constexpr int kc = decltype(kc_c)::value;
    constexpr int sl = kc % BD;
    if constexpr (kc + BD - 1 < NK) load_b(std::integral_constant<int, (kc + BD - 1) % BD>{}, kc + BD - 1);
    __builtin_amdgcn_sched_barrier(0);
    const uint16_t* Ab = As[kc % 3];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      // fragment read: row 16i + n, inputs 32 d + 8 g .. +7 = logical chunk 4d + g -> physical
      // chunk (4d + g) ^ n
      const int pcol = ((4 * d + g) ^ n) * 8;
      half8 bf[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint32_t sw = bs[sl][s][d >> 1];
        const uint32_t sv = (d & 1) ? (sw >> 16) : (sw & 0xFFFFu);
        const half2v s2 = __builtin_bit_cast(half2v, sv | (sv << 16));
        if constexpr (kAff) {
          const uint32_t mw = bm[sl][s][d >> 1];
          const _Float16 mv = __builtin_bit_cast(_Float16, (uint16_t)((d & 1) ? (mw >> 16) : (mw & 0xFFFFu)));
          bf[s] = dequant_word_affine(bc[sl][s][d], s2, (half2v){-mv, -mv});
        } else if constexpr (FMT == MOE_FMT_CB4) {
          bf[s] = dequant_word_cb(bc[sl][s][d], s2, cbt16);
        } else {
          bf[s] = dequant_word_k(bc[sl][s][d], s2, uk);
        }
      }
      // each subtile's MFMAs run while the next subtile's fragment is read (the read of the
      // last one is clamped and not used), so the LDS latency is not paid once per subtile: the
      // read is scheduled before the four MFMAs, and the wait for it falls before the next ones
      half8 af = *(const half8*)(Ab + n * kKC + pcol);
#pragma unroll
      for (int i = 0; i < MSUB; ++i) {
        if (i < ms) {
          const int inext = i + 1 < MSUB ? i + 1 : i;
          half8 af_next = *(const half8*)(Ab + (16 * inext + n) * kKC + pcol);
#pragma unroll
          for (int s = 0; s < 4; ++s)
            acc[i][s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[s], acc[i][s], 0, 0, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // the DS read
          __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // then the MFMAs
          af = af_next;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (kc + 2 < NK) {
      store_a(av, As[(kc + 2) % 3]);  // its stage was last read in chunk kc - 1
      if constexpr (kc + 3 < NK) load_a(av, kc + 3);
    }
    if constexpr (kc + 1 < NK) barrier();
  });

  // ---- epilogue: lane holds D[16i + 4g + r][16s + n] -----------------------------------------
  bool range_bad = false;
#pragma unroll
  for (int i = 0; i < MSUB; ++i) {
    if (i >= ms) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * i + 4 * g + r;
      if (row >= it.rows) continue;
      if constexpr (MODE == kGateUp) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const float gv = acc[i][s][r], uv = acc[i][s + 2][r];
          const int col = ntile * (kPNTile / 2) + wave * 32 + 16 * s + n;
          const float hv = silu(gv) * uv;
          range_bad |= f16_out_of_range(hv);
          a.h_out[(size_t)(it.row0 + row) * F + col] = (_Float16)hv;
        }
      } else {
        const float wv = a.row_w[it.row0 + row];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int col = ntile * kPNTile + wave * 64 + 16 * s + n;
          const float yv = acc[i][s][r] * wv;
          range_bad |= f16_out_of_range(yv);
          a.y16_out[(size_t)(it.row0 + row) * H + col] = (_Float16)yv;
        }
      }
    }
  }
  report_range(range_bad, a.ctrl);
  (void)K;
}

// x (bf16) -> fp16, exact for values inside the fp16 normal range; a value beyond the fp16 range
// is reported (MOE_DERR_RANGE).
// Eight values per thread and step (16-byte loads and stores), then a tail of single values.
__global__ __launch_bounds__(256) void k_bf16_to_f16(const uint16_t* __restrict__ x, _Float16* __restrict__ y,
                                                     size_t n, int32_t* __restrict__ ctrl) {
  typedef _Float16 half8v __attribute__((ext_vector_type(8)));
  bool bad = false;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const size_t n8 = n / 8;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n8; i += stride) {
    const uint4 w = ((const uint4*)x)[i];
    const uint32_t word[4] = {w.x, w.y, w.z, w.w};
    half8v h;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = __uint_as_float(word[j] << 16), hi = __uint_as_float(word[j] & 0xFFFF0000u);
      bad |= f16_out_of_range(lo) | f16_out_of_range(hi);
      h[2 * j] = (_Float16)lo;
      h[2 * j + 1] = (_Float16)hi;
    }
    ((half8v*)y)[i] = h;
  }
  for (size_t i = 8 * n8 + blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += stride) {
    const float v = __uint_as_float((uint32_t)x[i] << 16);
    bad |= f16_out_of_range(v);
    y[i] = (_Float16)v;
  }
  report_range(bad, ctrl);
}

// y[t] = sum_{j<k} y_rows[inv[t*k+j]] + y_rows[inv[T*k+t]] (rows already weighted, fp16), fixed
// order, fp32 sums.  Every row position and every row of a thread's outputs is loaded before any
// is added (no chain of dependent loads).
__global__ __launch_bounds__(256) void k_prefill_combine(const _Float16* __restrict__ y_rows,
                                                          const int32_t* __restrict__ inv, int T, int k,
                                                          int n_shared, int H, float* __restrict__ y) {
  typedef _Float16 half8v __attribute__((ext_vector_type(8)));
  const int H8 = H / 8;  // 8 outputs per thread and step (16-byte row loads)
  for (size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x; idx < (size_t)T * H8;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int t = (int)(idx / H8), o8 = (int)(idx - (size_t)t * H8);
    int pos[kMaxK + 1];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) pos[j] = j < k ? inv[t * k + (j < k ? j : 0)] : -1;
    pos[kMaxK] = n_shared ? inv[T * k + t] : -1;
    half8v v[kMaxK + 1];
#pragma unroll
    for (int j = 0; j <= kMaxK; ++j)
      v[j] = ((const half8v*)(y_rows + (size_t)(pos[j] < 0 ? 0 : pos[j]) * H))[o8];
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j <= kMaxK; ++j) {
      if (pos[j] >= 0) {
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] += (float)v[j][c];
      }
    }
    float4* out = (float4*)(y + (size_t)t * H) + 2 * o8;
    out[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    out[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

static int round8(int v) { return (v + 7) & ~7; }

bool prefill_kernel_fits(int kernel, int mode_down, int H, int F, int fmt, int item_rows) {
  if (kernel == kGemmGeneral) return true;
  if (kernel == kGemmPipe64Deep && item_rows > 64) return false;
  // the affine format's min records do not fit the 128-row kernel's registers beside its ring
  if (kernel == kGemmPipe128 && fmt == MOE_FMT_AFFINE4) return false;
  // built for the model's reduction widths: gate/up over H = 2048 (16 chunks), down over F = 768 (6)
  return mode_down ? (F == 6 * kKC && H % kPNTile == 0) : (H == 16 * kKC && F % (kPNTile / 2) == 0);
}

hipError_t launch_prefill_ffn(int H, int F, int k, int E, int n_shared, int T, const ExpertSource& src,
                              const void* x_bf16, const GroupBuffers& g, const PrefillBuffers& b, float* y,
                              int32_t* ctrl, const PrefillPlan& plan, hipStream_t st) {
  hipError_t err;
  const size_t nx = (size_t)T * H;
  int grid = (int)((nx + 255) / 256);
  if (grid > 4096) grid = 4096;
  k_bf16_to_f16<<<grid, 256, 0, st>>>((const uint16_t*)x_bf16, b.x16, nx, ctrl);
  if ((err = hipGetLastError()) != hipSuccess) return err;

  const int max_items = prefill_max_items(T, k, E, n_shared, plan.item_rows);
  GemmArgs a{};
  a.src = src;
  a.items = g.items;
  a.n_items = ctrl + kCtrlNTiles;
  a.ctrl = ctrl;
  a.E = E;
  a.H = H;
  a.F = F;
  a.T = T;

  // the plan's kernel for one projection: a pipelined shape where it is built for the widths and the
  // format, else the general kernel (which also runs the codebook and affine formats)
  auto run = [&](auto mode_c, int kernel) {
    constexpr int M = decltype(mode_c)::value;
    constexpr int timed = M == kGateUp ? kTimePrefillGateUp : kTimePrefillDown;
    constexpr int NK = M == kGateUp ? 16 : 6;
    const int pipe_cols = M == kGateUp ? kPNTile / 2 : kPNTile;  // output columns per pipelined workgroup
    const int gen_cols = M == kGateUp ? kNTileW / 2 : kNTileW;
    if (!prefill_kernel_fits(kernel, M == kDown, H, F, src.fmt, plan.item_rows)) kernel = kGemmGeneral;
    a.n_ntiles = (M == kGateUp ? F : H) / (kernel == kGemmGeneral ? gen_cols : pipe_cols);
    a.n_works = max_items * a.n_ntiles;
    const int blocks = round8(a.n_works);
    auto pipe = [&](auto fmt_c) -> hipError_t {
      constexpr int FMT = decltype(fmt_c)::value;
      if constexpr (FMT != MOE_FMT_AFFINE4)
        if (kernel == kGemmPipe128)
          return launch_timed(timed, k_expert_gemm_pipe<M, NK, kMSub, 2, FMT>, blocks, 64 * kPWaves, 0, st, a);
      return launch_timed(timed, k_expert_gemm_pipe<M, NK, 4, 4, FMT>, blocks, 64 * kPWaves, 0, st, a);
    };
    if (kernel == kGemmPipe128 || kernel == kGemmPipe64Deep) {
      if (src.fmt == MOE_FMT_CB4) return pipe(std::integral_constant<int, MOE_FMT_CB4>{});
      if (src.fmt == MOE_FMT_AFFINE4) return pipe(std::integral_constant<int, MOE_FMT_AFFINE4>{});
      return pipe(std::integral_constant<int, MOE_FMT_Q4_0>{});
    }
    if (src.fmt == MOE_FMT_CB4)
      return launch_timed(timed, k_expert_gemm<M, kRouterTileRows, MOE_FMT_CB4>, blocks, 256, 0, st, a);
    if (src.fmt == MOE_FMT_AFFINE4)
      return launch_timed(timed, k_expert_gemm<M, kRouterTileRows, MOE_FMT_AFFINE4>, blocks, 256, 0, st, a);
    return launch_timed(timed, k_expert_gemm<M>, blocks, 256, 0, st, a);
  };

  // gate/up + SwiGLU: h16[row][F]
  a.a16 = (const uint16_t*)b.x16;
  a.row_tok = g.row_tok;
  a.h_out = b.h16;
  if ((err = run(std::integral_constant<int, kGateUp>{}, plan.gate_up)) != hipSuccess) return err;

  // down: y_rows[row][H] = w_row * (Wd h)
  a.a16 = (const uint16_t*)b.h16;
  a.row_w = g.row_w;
  a.y16_out = b.y_rows;
  if ((err = run(std::integral_constant<int, kDown>{}, plan.down)) != hipSuccess) return err;

  const size_t nc = (size_t)T * (H / 8);
  grid = (int)((nc + 255) / 256);
  if (grid > 8192) grid = 8192;
  k_prefill_combine<<<grid, 256, 0, st>>>(b.y_rows, g.inv, T, k, n_shared, H, y);
  return hipGetLastError();
}

// ---- router logits for prefill, pipelined ------------------------------------------------------
// logits[t][e] = bias[e] + sum_k x[t][k] Wr[e][k] over a work of RM tokens x 64 NS router rows:
// four waves of 16 NS router rows each, every wave over all RM tokens.  The token tile goes through a
// 3-stage LDS ring loaded through registers 3 chunks ahead (as in the expert GEMM above); the
// router rows through a 3-slot register ring 2 chunks ahead.  Each logit takes the same sequence of
// MFMA steps (128-input chunks, then 32-input steps, in ascending order) as the general kernel's
// router mode, so both give the same bits.  XCD-aware: an XCD runs consecutive works, and the
// router-row tiles of one token tile are consecutive, so they share that tile in the XCD's L2.
template <int NK, int RM, int NS>
__global__ __launch_bounds__(256, 2) void k_router_gemm_pipe(GemmArgs a) {
  constexpr int kCols = 64 * NS;              // router rows per work: 4 waves x NS subtiles of 16
  constexpr int MS = RM / 16;                 // 16-token subtiles
  constexpr int kAPer = RM * (kKC / 8) / 256;  // A 16-byte pieces per thread per chunk
  static_assert(kAPer >= 1 && kAPer * 256 == RM * (kKC / 8), "A pieces split evenly");
  constexpr int BD = 3;                       // B slots (2 chunks ahead)
  __shared__ __attribute__((aligned(1024))) uint16_t As[3][RM * kKC];

  const int n_works = a.n_works;
  const int per_xcd = (n_works + 7) >> 3;
  const int local = (int)(blockIdx.x >> 3);
  const int work = (int)(blockIdx.x & 7) * per_xcd + local;
  if (local >= per_xcd || work >= n_works) return;
  const int mtile = work / a.n_ntiles;
  const int ntile = work - mtile * a.n_ntiles;
  const int row0 = mtile * RM;
  const int rows = min(RM, a.T - row0);
  const int H = a.H, E = a.E;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int ms = (rows + 15) >> 4;

  // B: lane (g, n) of subtile s takes router row e_s, inputs 32 d + 8 g .. +7 of each 32-input step d
  const int e0 = ntile * kCols + wave * 16 * NS + n;  // e_s = e0 + 16 s < E: E % kCols == 0
  const uint16_t* wr = a.wr + (size_t)e0 * H + 8 * g;
  u32x4 b[BD][NS][4];
  auto load_b = [&](auto slot_c, int kc) {
    constexpr int sl = decltype(slot_c)::value;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int d = 0; d < 4; ++d) b[sl][s][d] = *(const u32x4*)(wr + (size_t)16 * s * H + kc * kKC + 32 * d);
  };

  // A: piece j of this thread = token row r_j = (tid >> 4) + 16 j, logical 16-byte chunk tid & 15,
  // stored at chunk lc ^ (r & 15) of its LDS row
  const int lc = threadIdx.x & 15;
  const int a_dst0 = (threadIdx.x >> 4) * kKC + ((lc ^ ((threadIdx.x >> 4) & 15)) * 8);
  const uint16_t* a_base = a.a16 + (size_t)row0 * H;  // offsets from the work's first token row
  int a_src[kAPer];
#pragma unroll
  for (int j = 0; j < kAPer; ++j) {
    const int r = (threadIdx.x >> 4) + 16 * j;
    a_src[j] = (r < rows ? r : 0) * H + lc * 8;  // padding rows copy row 0 (outputs dropped)
  }
  auto load_a = [&](u32x4 (&v)[kAPer], int kc) {
#pragma unroll
    for (int j = 0; j < kAPer; ++j) v[j] = *(const u32x4*)(a_base + a_src[j] + kc * kKC);
  };
  auto store_a = [&](const u32x4 (&v)[kAPer], uint16_t* buf) {
#pragma unroll
    for (int j = 0; j < kAPer; ++j) *(u32x4*)(buf + a_dst0 + 16 * kKC * j) = v[j];
  };
  auto barrier = [&]() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  float4v acc[MS][NS];
#pragma unroll
  for (int i = 0; i < MS; ++i)
#pragma unroll
    for (int s = 0; s < NS; ++s) acc[i][s] = (float4v){0.f, 0.f, 0.f, 0.f};

  // prologue: A(0), A(1) in LDS, A(2) and B(0), B(1) in flight
  u32x4 av[kAPer];
  {
    u32x4 a0[kAPer];
    load_a(a0, 0);
    load_a(av, 1);
    load_b(std::integral_constant<int, 0>{}, 0);
    if constexpr (NK > 1) load_b(std::integral_constant<int, 1>{}, 1);
    store_a(a0, As[0]);
    if constexpr (NK > 1) store_a(av, As[1]);
    if constexpr (NK > 2) load_a(av, 2);
    barrier();
  }
  static_for<NK>([&](auto kc_c) {
    constexpr int kc = decltype(kc_c)::value;
    constexpr int sl = kc % BD;
    if constexpr (kc + BD - 1 < NK) load_b(std::integral_constant<int, (kc + BD - 1) % BD>{}, kc + BD - 1);
    __builtin_amdgcn_sched_barrier(0);
    const uint16_t* Ab = As[kc % 3];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int pcol = ((4 * d + g) ^ n) * 8;
#pragma unroll
      for (int i = 0; i < MS; ++i) {
        if (i < ms) {
          const bf16x8 af = *(const bf16x8*)(Ab + (16 * i + n) * kKC + pcol);
#pragma unroll
          for (int s = 0; s < NS; ++s)
            acc[i][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, __builtin_bit_cast(bf16x8, b[sl][s][d]), acc[i][s], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kc + 2 < NK) {
      store_a(av, As[(kc + 2) % 3]);  // its stage was last read in chunk kc - 1
      if constexpr (kc + 3 < NK) load_a(av, kc + 3);
    }
    if constexpr (kc + 1 < NK) barrier();
  });

  // epilogue: lane holds D[16 i + 4 g + r][16 s + n]
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int e = e0 + 16 * s;
    const float bv = a.bias ? a.bias[e] : 0.f;
#pragma unroll
    for (int i = 0; i < MS; ++i) {
      if (i >= ms) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * i + 4 * g + r;
        if (row < rows) a.y_out[(size_t)(row0 + row) * E + e] = acc[i][s][r] + bv;
      }
    }
  }
}

hipError_t launch_router_gemm(const void* x_bf16, const void* Wr_bf16, const float* bias, int T, int E, int H,
                              float* logits, int rows_per_work, hipStream_t st) {
  GemmArgs a{};
  a.E = E;
  a.H = H;
  a.T = T;
  a.a16 = (const uint16_t*)x_bf16;
  a.wr = (const uint16_t*)Wr_bf16;
  a.bias = bias;
  a.y_out = logits;
  // the pipelined kernel at the covered widths (the plan's token rows per work, 128 router rows)
  const int nk = H / kKC;
  constexpr int kRgNS = 2;  // 128 router rows per work (measured: 4K 40 -> 39 us, 32K 189 -> 168 us against 64)
  if (E % (64 * kRgNS) == 0 && H % kKC == 0 && (nk == 8 || nk == 16 || nk == 32)) {
    const int rm = rows_per_work == kRouterTallRows ? 64 : 32;
    a.n_ntiles = E / (64 * kRgNS);
    a.n_works = ((T + rm - 1) / rm) * a.n_ntiles;
    auto go = [&](auto kern) { kern<<<round8(a.n_works), 256, 0, st>>>(a); return hipGetLastError(); };
    if (rm == 64) {
      if (nk == 8) return go(k_router_gemm_pipe<8, 64, kRgNS>);
      if (nk == 16) return go(k_router_gemm_pipe<16, 64, kRgNS>);
      return go(k_router_gemm_pipe<32, 64, kRgNS>);
    }
    if (nk == 8) return go(k_router_gemm_pipe<8, 32, kRgNS>);
    if (nk == 16) return go(k_router_gemm_pipe<16, 32, kRgNS>);
    return go(k_router_gemm_pipe<32, 32, kRgNS>);
  }
  a.n_ntiles = (E + kNTileW - 1) / kNTileW;
  if (rows_per_work == kRouterTallRows) {
    a.n_works = ((T + kRouterTallRows - 1) / kRouterTallRows) * a.n_ntiles;
    k_expert_gemm<kRouter, kRouterTallRows><<<round8(a.n_works), 256, 0, st>>>(a);
  } else {
    a.n_works = ((T + kRouterTileRows - 1) / kRouterTileRows) * a.n_ntiles;
    k_expert_gemm<kRouter><<<round8(a.n_works), 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace moe
