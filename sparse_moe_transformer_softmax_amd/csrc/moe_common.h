// Device-side building blocks shared by the MoE kernels (gfx950 / CDNA4).
//
// Operand encodings used inside the library:
//  * MXFP4 weights are consumed raw: E2M1 nibbles (low nibble = even
//    element) with one E8M0 scale byte per 32 elements, the microscaling
//    format the gpt-oss pages give for the expert weights ("OpenAI 最新开源
//    模型 gpt-oss 架构与训练解析", 权重量化 item).
//  * Activations that feed the block-scaled MFMA (the token rows x of the
//    gate/up projection and the SwiGLU output h of the down projection) are
//    stored as "MX6x3" rows: every 32-element block becomes three FP6 (E2M3)
//    terms, each with its own E8M0 scale, such that the sum of the terms
//    reproduces the value to about 2^-13 of the block maximum.  One block
//    has 80 bytes: term0 codes [0,24), term1 [24,48), term2 [48,72) (32
//    six-bit codes packed little-endian), scale bytes at 72,73,74, padding
//    to 80.  In a row, blocks are grouped four at a time (one 128-wide MFMA
//    step, 320 bytes) and the group is stored piece-interleaved: byte i of
//    block 4c + g sits at 320c + (4 * (i / 16) + g) * 16 + i % 16, so the
//    four lanes that read the same 16-byte piece of four consecutive blocks
//    read one 64-byte line.  A row of n blocks occupies ceil(n / 4) * 320
//    bytes.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v32f __attribute__((ext_vector_type(32)));
typedef unsigned int v6u __attribute__((ext_vector_type(6)));

constexpr int MX6_BLOCK_BYTES = 80;
constexpr int MX6_TERMS = 3;
constexpr int MX6_GROUP_BYTES = 4 * MX6_BLOCK_BYTES;  // four blocks, piece-interleaved

// bytes of an MX6x3 row of nblk blocks
__host__ __device__ constexpr int mx6_row_bytes(int nblk) { return ((nblk + 3) >> 2) * MX6_GROUP_BYTES; }

// offset within a row of byte i (0..79) of block b
__host__ __device__ __forceinline__ int mx6_byte_offset(int b, int i) {
  return (b >> 2) * MX6_GROUP_BYTES + (((i >> 4) << 2) + (b & 3)) * 16 + (i & 15);
}

// s_waitcnt with only the vector-memory counter (vmcnt, 6 bits: bits 3:0
// and 15:14 of the gfx9 encoding) or only the LDS/scalar counter (lgkmcnt,
// bits 11:8) waited on; the other fields are left at their maxima.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
template <int N>
__device__ __forceinline__ void wait_lgkmcnt() {
  static_assert(N >= 0 && N < 16, "lgkmcnt is 4 bits");
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (N << 8));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// float -> bf16, round to nearest even (NaN kept quiet)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// E8M0 byte k+127 of the smallest power of two 2^k with 7.5 * 2^k >= amax
// (7.5 is the largest E2M3 magnitude), so that amax / 2^k never saturates.
// amax == 0 gives 127.  Non-finite amax gives 0xFF (NaN scale).
__device__ __forceinline__ int mx6_scale_exp(float amax) {
  if (!(amax <= 3.0e38f)) return 255;
  if (amax == 0.0f) return 127;
  const uint32_t bits = __float_as_uint(amax);
  const int ex = (int)((bits >> 23) & 0xffu);
  if (ex == 0) return 0;  // subnormal amax: 2^-127 * 7.5 covers it
  // amax = 1.m * 2^(ex-127) and 7.5 = 1.875 * 2^2: k = ex - 129 when
  // 1.m <= 1.875 (mantissa field <= 0x700000), else ex - 128
  int k = ((bits & 0x7fffffu) <= 0x700000u) ? ex - 129 : ex - 128;
  k = k < -127 ? -127 : (k > 127 ? 127 : k);
  return k + 127;
}

__device__ __forceinline__ float exp2i(int k) {  // 2^k for k in [-126, 127]
  return __uint_as_float((uint32_t)(k + 127) << 23);
}

// Round v (|v| <= 7.5) to the nearest E2M3 value, ties to even; returns the
// 6-bit code and writes the rounded value.  E2M3: sign, 2 exponent bits
// (bias 1), 3 mantissa bits; exponent field 0 is subnormal.  The grid step
// is 1/8 on [0, 2), 1/4 on [2, 4), 1/2 on [4, 7.5]; with n the rounded
// multiple of the step, the code is n, n + 8 and n + 16 on the three ranges.
__device__ __forceinline__ uint32_t e2m3_round(float v, float& q) {
  const float a = fabsf(v);
  const bool lo = a < 2.0f, mid = a < 4.0f;
  const float inv = lo ? 8.0f : (mid ? 4.0f : 2.0f);
  const float step = lo ? 0.125f : (mid ? 0.25f : 0.5f);
  float n = __builtin_rintf(a * inv);  // exact scaling by a power of two
  n = fminf(n, lo ? 16.0f : (mid ? 16.0f : 15.0f));
  const float r = n * step;
  const uint32_t code = (uint32_t)n + (lo ? 0u : (mid ? 8u : 16u));
  const uint32_t s = (__float_as_uint(v) >> 31) & 1u;
  q = s ? -r : r;
  return code | (s << 5);
}

// Pack 32 six-bit codes (one per byte of `c`) little-endian into 6 dwords.
__device__ __forceinline__ void pack6x32(const uint8_t* c, uint32_t out[6]) {
#pragma unroll
  for (int w = 0; w < 6; ++w) out[w] = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int bit = 6 * i;
    const uint32_t v = c[i] & 63u;
    out[bit >> 5] |= v << (bit & 31);
    if ((bit & 31) > 26) out[(bit >> 5) + 1] |= v >> (32 - (bit & 31));
  }
}

// MX6x3 split of one 32-element block on the gfx950 scaled conversions: the lane
// holds a whole 32-element block, even elements in ve and odd elements in vo
// (the conversion packs source pair (ve[i], vo[i]) as elements 2i, 2i+1).
// v_cvt_scalef32_2xpk16_fp6_f32 divides by the power-of-two scale and rounds
// to nearest even, which for the non-saturating scale is exactly e2m3_round;
// v_cvt_scalef32_pk32_f32_fp6 gives the rounded values back, so the residual
// is exact.  Both are written as asm with early-clobber outputs: the
// compiler's builtin lets the result registers overlap the sources, which
// these instructions do not support.  On return codes[6t .. 6t+5] hold term
// t's 32 codes packed little-endian (the MX6x3 byte layout), scw the three
// scale bytes.  A block with a NaN gets scale 0xFF on every term.  The first
// term's block maximum is the integer maximum of the magnitudes' bit
// patterns, where a NaN (every pattern above infinity's) shows itself; the
// later terms' residuals are then finite, and take the float maximum.
__device__ __forceinline__ void mx6x3_split_lane(v16f& ve, v16f& vo, uint32_t (&codes)[18], uint32_t& scw) {
  uint32_t mbits = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i)
    mbits = max(mbits, max(__float_as_uint(ve[i]) & 0x7fffffffu, __float_as_uint(vo[i]) & 0x7fffffffu));
  if (mbits > 0x7f800000u) {
#pragma unroll
    for (int w = 0; w < 18; ++w) codes[w] = 0;
    scw = 0xffffffu;
    return;
  }
  scw = 0;
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    float amax = __uint_as_float(mbits);
    if (t > 0) {
      amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fmaxf(fabsf(ve[i]), fabsf(vo[i])));
    }
    int se = mx6_scale_exp(amax);
    // a subnormal maximum takes 2^-126 (one step coarser, still no
    // saturation), so the scale operand is a normal float
    se = se == 0 ? 1 : se;
    scw |= (uint32_t)se << (8 * t);
    if (se == 255) {
#pragma unroll
      for (int w = 0; w < 6; ++w) codes[6 * t + w] = 0;
      continue;
    }
    const float scale = __uint_as_float((uint32_t)se << 23);
    v6u c;
    asm volatile("v_cvt_scalef32_2xpk16_fp6_f32 %0, %1, %2, %3" : "=&v"(c) : "v"(ve), "v"(vo), "v"(scale));
#pragma unroll
    for (int w = 0; w < 6; ++w) codes[6 * t + w] = c[w];
    if (t == 2) break;
    v32f q;
    asm volatile("v_cvt_scalef32_pk32_f32_fp6 %0, %1, %2" : "=&v"(q) : "v"(c), "v"(scale));
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      ve[i] -= q[2 * i];
      vo[i] -= q[2 * i + 1];
    }
  }
}

}  // namespace moe
