// Device helpers and the workspace layout shared by the layer's HIP sources.
// gfx950 (CDNA4) only: 64-wide wavefronts, v_dot2c_f32_bf16, MFMA f16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "../../include/moe_route.h"

#define MOE_DEV __device__ __forceinline__

namespace moe {

constexpr int kBlock = 32;        // weights per quantization block
constexpr int kWave = 64;         // CDNA wavefront
constexpr int kMaxDecodeTok = MOE_DECODE_MAX_TOKENS;
constexpr int kMaxDecodeTokNarrow = MOE_DECODE_MAX_TOKENS_NARROW;
constexpr int kMaxDecodeF16Tok = 2048;  // largest F with 16 decode tokens (their h rows staged in LDS)
constexpr int kMaxK = 16;
constexpr int kMaxExperts = 1024;
constexpr int kCtrlBytes = 4096;  // control area at the start of the workspace

// Control words (int32 index into the control area).
enum CtrlWord {
  kCtrlError = 0,      // device error bits (moe_device_error)
  kCtrlNTasks = 1,     // decode: number of expert tasks
  kCtrlMissCount = 2,  // residency: number of misses
  kCtrlNTiles = 3,     // prefill: number of m-tiles in the work list
  kCtrlRouteDone = 4,  // decode route: router workgroups finished (zero between calls)
  kCtrlTileDone = 64,  // decode down: 64 per-row-tile counters (words 64..127), zero between calls
};


// ---------------------------------------------------------------------------------------
// Expert blob layout (see moe_route.h)
// ---------------------------------------------------------------------------------------
struct BlobLayout {
  int64_t gate_codes, up_codes, down_codes, gate_scales, up_scales, down_scales;
  int64_t gate_mins, up_mins, down_mins;  // affine format only (else equal to total)
  int64_t total;
};

__host__ __device__ inline BlobLayout blob_layout(int H, int F, int fmt = MOE_FMT_Q4_0) {
  BlobLayout L;
  const int64_t gu = (int64_t)F * H / 2, d = (int64_t)H * F / 2;
  const int64_t sgu = (int64_t)F * (H / kBlock) * 2, sd = (int64_t)H * (F / kBlock) * 2;
  L.gate_codes = 0;
  L.up_codes = gu;
  L.down_codes = 2 * gu;
  L.gate_scales = 2 * gu + d;
  L.up_scales = L.gate_scales + sgu;
  L.down_scales = L.up_scales + sgu;
  L.gate_mins = L.down_scales + sd;
  L.up_mins = L.gate_mins + sgu;
  L.down_mins = L.up_mins + sgu;
  L.total = fmt == MOE_FMT_AFFINE4 ? L.down_mins + sd : L.gate_mins;
  if (fmt != MOE_FMT_AFFINE4) L.up_mins = L.down_mins = L.gate_mins;
  return L;
}

// ---------------------------------------------------------------------------------------
// Weight formats (moe_format).  The codebook's 16 signed bytes travel to the kernels as four
// words; a workgroup expands them into a 256-entry LDS table indexed by a code pair (the two
// codes of a word's pair j: bits 4j and 16 + 4j), each entry the pair's two values as 16-bit
// floats, so one LDS read gives a ready operand register.
// ---------------------------------------------------------------------------------------
struct Codebook {
  uint32_t w[4];  // value u in byte u % 4 of word u / 4
};
MOE_DEV int codebook_value(const Codebook& cb, int u) { return (int)(int8_t)(cb.w[u >> 2] >> (8 * (u & 3))); }
// Index of pair j of a code word in the 256-entry table: code 2j in bits 0..3, code 2j+1 in 4..7.
MOE_DEV uint32_t code_pair_index(uint32_t w, int j) {
  return ((w >> (4 * j)) & 0xFu) | ((w >> (12 + 4 * j)) & 0xF0u);
}

// ---------------------------------------------------------------------------------------
// Matrix-core operand types (v_mfma_f32_16x16x32_{bf16,f16}).  For a 16x16x32 step, lane l
// supplies row (A) / column (B) l % 16 at k = 8 (l / 16) .. 8 (l / 16) + 7 as 8 packed 16-bit
// values, and receives D rows 4 (l / 16) .. 4 (l / 16) + 3 of column l % 16.
// ---------------------------------------------------------------------------------------
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// Code words of a 4-bit matrix of R rows: every row is split into groups of 128 elements (4
// blocks of 32) stored as 64-byte records, group-major: record (c, r) = group c of row r at byte
// 64 (c R + r), its four fp16 block scales at byte 8 (c R + r) of the scale section.  Word 4g + i
// of a record holds slice g (elements 8g .. 8g+7) of block i.  A lane that loads bytes 16g..16g+15
// of a record therefore holds slice g of each of the group's four blocks: exactly its share of
// four 16x16x32 matrix-core steps, one block (one scale) per step; and 16 rows x 4 lanes read
// 1 KiB of consecutive records.
constexpr int kGroupElems = 128;
constexpr int kGroupBytes = 64;
constexpr int kGroupScaleBytes = 8;

// Asynchronous global -> LDS copy of 16 bytes per active lane: lane l's bytes land at
// lds_base + 16 l (lds_base wave-uniform).  Counted by vmcnt like any vector load.
MOE_DEV void lds_dma16(const void* gsrc, uint16_t* lds_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}

// ---------------------------------------------------------------------------------------
// Small numeric helpers
// ---------------------------------------------------------------------------------------
MOE_DEV float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
MOE_DEV float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (inputs are finite).
MOE_DEV uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

MOE_DEV float fp16_bits_to_f32(uint32_t h) {
  _Float16 v = __builtin_bit_cast(_Float16, (uint16_t)h);
  return (float)v;
}

// acc + a.lo*b.lo + a.hi*b.hi for bf16 pairs (v_dot2c_f32_bf16).  bf16 x bf16 products
// are exact in fp32.
MOE_DEV float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, a), __builtin_bit_cast(v2bf, b), acc,
                                         false);
}

// Pair j (0..3) of a code word as two bf16 values (128 + u): elements 2j and 2j+1 of the
// word sit in bits 4j and 16+4j, so one mask puts both codes under the bf16 exponent of
// 128 (0x4300), whose mantissa step is 1.  128 + u = q + 136 with q = u - 8, exact.
MOE_DEV uint32_t code_pair_bf16_q136(uint32_t w, int j) {
  return ((w >> (4 * j)) & 0x000F000Fu) | 0x43004300u;
}

// ---------------------------------------------------------------------------------------
// Wave reductions (64 lanes)
// ---------------------------------------------------------------------------------------
MOE_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Sum over aligned groups of `width` lanes (power of two <= 64).
MOE_DEV float group_sum(float v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

MOE_DEV void set_error(int32_t* ctrl, int bits) {
  atomicOr(&ctrl[kCtrlError], bits);
}

MOE_DEV float silu(float g) { return g / (1.0f + expf(-g)); }

// ---------------------------------------------------------------------------------------
// DPP reductions (VALU lane moves instead of LDS-crossbar shuffles)
// ---------------------------------------------------------------------------------------
enum DppCtrl {
  kDppQuadXor1 = 0xB1,  // quad_perm [1,0,3,2]
  kDppQuadXor2 = 0x4E,  // quad_perm [2,3,0,1]
  kDppRowRor4 = 0x124,
  kDppRowRor8 = 0x128,
  kDppRowBcast15 = 0x142,
  kDppRowBcast31 = 0x143,
};

template <int CTRL, int ROW_MASK>
MOE_DEV float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}
template <int CTRL, int ROW_MASK>
MOE_DEV int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, ROW_MASK, 0xF, false);
}

// Sum over aligned groups of `width` lanes (16, 32 or 64); the total is valid in the last lane of
// each group (lane 15 of each row for 16; lanes 31 and 63 for 32; lane 63 for 64).
MOE_DEV float group_sum_dpp(float v, int width) {
  v += dpp_f<kDppQuadXor1, 0xF>(v);
  v += dpp_f<kDppQuadXor2, 0xF>(v);
  v += dpp_f<kDppRowRor4, 0xF>(v);
  v += dpp_f<kDppRowRor8, 0xF>(v);
  if (width >= 32) v += dpp_f<kDppRowBcast15, 0xA>(v);
  if (width >= 64) v += dpp_f<kDppRowBcast31, 0xC>(v);
  return v;
}

MOE_DEV bool group_last_lane(int lane, int width) { return (lane & (width - 1)) == width - 1; }

// Wave-wide maximum of a 64-bit key (DPP, no branches); returned to every lane.
MOE_DEV uint64_t wave_max_u64(uint64_t key) {
#define MOE_MAX64_STEP(C, M)                                                              \
  {                                                                                       \
    const uint32_t lo = (uint32_t)dpp_i<C, M>((int)(uint32_t)key);                        \
    const uint32_t hi = (uint32_t)dpp_i<C, M>((int)(uint32_t)(key >> 32));                \
    const uint64_t other = ((uint64_t)hi << 32) | lo;                                     \
    key = other > key ? other : key;                                                      \
  }
  MOE_MAX64_STEP(kDppQuadXor1, 0xF)
  MOE_MAX64_STEP(kDppQuadXor2, 0xF)
  MOE_MAX64_STEP(kDppRowRor4, 0xF)
  MOE_MAX64_STEP(kDppRowRor8, 0xF)
  MOE_MAX64_STEP(kDppRowBcast15, 0xA)
  MOE_MAX64_STEP(kDppRowBcast31, 0xC)
#undef MOE_MAX64_STEP
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)key, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(key >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// Wave-wide maximum of a 32-bit key (DPP, no branches); returned to every lane.  Lanes a DPP
// step does not write read 0, the identity of the unsigned maximum, so each step can fold into
// one v_max_u32 with a DPP source.
MOE_DEV uint32_t wave_max_u32(uint32_t v) {
#define MOE_MAX32_STEP(C, M)                               \
  {                                                        \
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, C, M, 0xF, false); \
    v = o > v ? o : v;                                     \
  }
  MOE_MAX32_STEP(kDppQuadXor1, 0xF)
  MOE_MAX32_STEP(kDppQuadXor2, 0xF)
  MOE_MAX32_STEP(kDppRowRor4, 0xF)
  MOE_MAX32_STEP(kDppRowRor8, 0xF)
  MOE_MAX32_STEP(kDppRowBcast15, 0xA)
  MOE_MAX32_STEP(kDppRowBcast31, 0xC)
#undef MOE_MAX32_STEP
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Order-preserving map of a float to uint32 (a > b as floats <=> map(a) > map(b); no NaN).
MOE_DEV uint32_t f32_order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
MOE_DEV float f32_from_order_key(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Wave-wide arg-max on (value desc, index asc); the result is returned to every lane.
MOE_DEV void wave_argmax(float& v, int& i) {
#define MOE_ARGMAX_STEP(C, M)                                        \
  {                                                                  \
    const float ov = dpp_f<C, M>(v);                                 \
    const int oi = dpp_i<C, M>(i);                                   \
    const bool take = ov > v || (ov == v && oi < i);                 \
    v = take ? ov : v;                                               \
    i = take ? oi : i;                                               \
  }
  MOE_ARGMAX_STEP(kDppQuadXor1, 0xF)
  MOE_ARGMAX_STEP(kDppQuadXor2, 0xF)
  MOE_ARGMAX_STEP(kDppRowRor4, 0xF)
  MOE_ARGMAX_STEP(kDppRowRor8, 0xF)
  MOE_ARGMAX_STEP(kDppRowBcast15, 0xA)
  MOE_ARGMAX_STEP(kDppRowBcast31, 0xC)
#undef MOE_ARGMAX_STEP
  v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  i = __builtin_amdgcn_readlane(i, 63);
}

// f(integral_constant<int, 0>) .. f(integral_constant<int, N - 1>): indexes into a register array
// that are constants from the start, so the array never lives in scratch memory.
template <typename Fn, int... I>
MOE_DEV void static_for_impl(Fn&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename Fn>
MOE_DEV void static_for(Fn&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// A blob as a buffer resource: loads take a per-lane 32-bit offset and a wave-uniform one, so a
// wave's addresses cost one register instead of a 64-bit pointer per load; reads past `bytes`
// return zero.  Word 3 = 0x00020000: 32-bit data format, the value raw loads need on this family.
MOE_DEV __amdgpu_buffer_rsrc_t blob_rsrc(const uint8_t* blob, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)blob, 0, (int)bytes, 0x00020000);
}
MOE_DEV u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
MOE_DEV u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
}

// Weight streams that a decode call reads exactly once: loads with the non-temporal hint (cache
// policy bit NT), so the caches keep those lines at low priority.  Measured on the 8-token decode
// of the model-shaped layer: ~4 % less time per layer call than the same loads without the hint.
constexpr int kCpolNT = 2;
MOE_DEV u32x4 buf_load16_nt(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kCpolNT);
}
MOE_DEV u32x2 buf_load8_nt(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kCpolNT);
}
MOE_DEV u32x4 ld16_nt(const uint8_t* p) { return __builtin_nontemporal_load((const u32x4*)p); }
MOE_DEV u32x2 ld8_nt(const uint8_t* p) { return __builtin_nontemporal_load((const u32x2*)p); }
MOE_DEV uint4 ld16_nt_u4(const uint8_t* p) {
  const u32x4 v = ld16_nt(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
MOE_DEV uint2 ld8_nt_u2(const uint8_t* p) {
  const u32x2 v = ld8_nt(p);
  return make_uint2(v.x, v.y);
}

}  // namespace moe
