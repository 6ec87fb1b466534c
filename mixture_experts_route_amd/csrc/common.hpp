// Device helpers and the workspace layout shared by the layer's HIP sources.
// gfx950 (CDNA4) only: 64-wide wavefronts, v_dot2c_f32_bf16, MFMA f16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_route.h"

#define MOE_DEV __device__ __forceinline__

namespace moe {

constexpr int kBlock = 32;        // weights per quantization block
constexpr int kWave = 64;         // CDNA wavefront
constexpr int kMaxDecodeTok = MOE_DECODE_MAX_TOKENS;
constexpr int kMaxK = 16;
constexpr int kMaxExperts = 1024;
constexpr int kCtrlBytes = 4096;  // control area at the start of the workspace

// Control words (int32 index into the control area).
enum CtrlWord {
  kCtrlError = 0,      // device error bits (moe_device_error)
  kCtrlNTasks = 1,     // decode: number of expert tasks
  kCtrlMissCount = 2,  // residency: number of misses
  kCtrlNTiles = 3,     // prefill: number of m-tiles in the work list
};

// ---------------------------------------------------------------------------------------
// Expert blob layout (see moe_route.h)
// ---------------------------------------------------------------------------------------
struct BlobLayout {
  int64_t gate_codes, up_codes, down_codes, gate_scales, up_scales, down_scales, total;
};

__host__ __device__ inline BlobLayout blob_layout(int H, int F) {
  BlobLayout L;
  const int64_t gu = (int64_t)F * H / 2, d = (int64_t)H * F / 2;
  const int64_t sgu = (int64_t)F * (H / kBlock) * 2, sd = (int64_t)H * (F / kBlock) * 2;
  L.gate_codes = 0;
  L.up_codes = gu;
  L.down_codes = 2 * gu;
  L.gate_scales = 2 * gu + d;
  L.up_scales = L.gate_scales + sgu;
  L.down_scales = L.up_scales + sgu;
  L.total = L.down_scales + sd;
  return L;
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

}  // namespace moe
