// Internal helpers shared by the library's kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/smoe.h"

namespace smoe {

constexpr int kWave = 64;
constexpr int kMaxTopK = 16;
constexpr int kMaxExperts = 256;
constexpr int kMaxPrefillTokens = 64;

// Byte offsets of the sections of one SMOE-Q4 expert blob (layout in smoe.h).
struct BlobLayout {
  size_t up_codes, down_codes, gate_params, up_params, down_params, bytes;
};

inline BlobLayout blob_layout(int d, int f, int chunk) {
  BlobLayout b;
  const size_t df = (size_t)d * (size_t)f;
  b.up_codes = df / 2;
  b.down_codes = df;
  b.gate_params = df + df / 2;
  b.up_params = b.gate_params + df / chunk * 4;
  b.down_params = b.up_params + df / chunk * 4;
  b.bytes = b.down_params + df / chunk * 4;
  return b;
}

// ---------------------------------------------------------------------------
// Scalar conversions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// bf16 bit pattern of the double v, rounded to nearest, ties to even, in one
// step from the double (no float intermediate rounding).
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double v) {
  uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint64_t sign = b & 0x8000000000000000ull;
  uint64_t a = b ^ sign;
  float f;
  if ((a >> 52) >= (uint64_t)(1023 - 126)) {
    // bf16 keeps the top 7 of the 52 stored fraction bits: round at bit 45.
    const uint64_t lsb = (a >> 45) & 1ull;
    a += 0x00000FFFFFFFFFFFull + lsb;
    a &= ~0x00001FFFFFFFFFFFull;
    f = (float)__longlong_as_double((long long)a);  // exact, or +inf on overflow
  } else {
    // below the bf16 normal range the spacing is 2^-133
    double s = rint(__longlong_as_double((long long)a) * 0x1p133);
    f = (float)(s * 0x1p-133);
  }
  return (uint16_t)((__float_as_uint(f) >> 16) | (uint32_t)(sign >> 48));
}

__device__ __forceinline__ uint32_t f16_bits(float v) {
  _Float16 h = (_Float16)v;
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

// Storage order inside each group of 8 values for the nibble-pair dot
// products: stored slot i holds element kPairSlot^-1(i); element j goes to
// slot (j < 4 ? 2j : 2(j-4)+1), so dword p of the group holds (e_p, e_{p+4}).
__device__ __forceinline__ int pair_slot(int j) { return j < 4 ? 2 * j : 2 * (j - 4) + 1; }

// ---------------------------------------------------------------------------
// Wave reductions (butterfly; every lane of the group ends with the result;
// the summation tree is fixed, so results are bitwise reproducible)
// ---------------------------------------------------------------------------
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int m = 1; m < W; m <<= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

template <int W>
__device__ __forceinline__ double group_sum_f64(double v) {
#pragma unroll
  for (int m = 1; m < W; m <<= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// ---------------------------------------------------------------------------
// Nibble-pair dot products.
// A dword w of codes holds elements e0..e7 (e_j in bits 4j..4j+3).  OR-ing the
// f16 pattern of 1024.0 onto a 4-bit field placed at mantissa bits 0..3 gives
// 1024 + q exactly; at bits 4..7 it gives 1024 + 16 q exactly.  So
//   (w & 0x000F000F) | 0x64006400 = (1024 + e0, 1024 + e4)
//   (w & 0x00F000F0) | 0x64006400 = (1024 + 16 e1, 1024 + 16 e5)
// and the same on w >> 8 for (e2, e6), (e3, e7).  With the input stored in
// pair order, v_dot2_f32_f16 accumulates
//   acc_lo += sum (1024 + q) x   over the even elements
//   acc_hi += sum (1024 + 16 q) x over the odd elements
// and  sum q x = acc_lo + acc_hi / 16 - (1024 X_even + 64 X_odd).
// ---------------------------------------------------------------------------
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c,
                                false);
}

// One dword of codes against four dwords of pair-ordered f16 inputs.
__device__ __forceinline__ void nib8_dot(uint32_t w, const uint32_t* xp, float& lo, float& hi) {
  const uint32_t magic = 0x64006400u;
  const uint32_t w8 = w >> 8;
  lo = dot2((w & 0x000F000Fu) | magic, xp[0], lo);
  hi = dot2((w & 0x00F000F0u) | magic, xp[1], hi);
  lo = dot2((w8 & 0x000F000Fu) | magic, xp[2], lo);
  hi = dot2((w8 & 0x00F000F0u) | magic, xp[3], hi);
}

// Contribution of one 16-byte segment (32 codes, inside one chunk) of a row:
// scale * sum(q x) + min * sum(x).  xp: 16 pair-ordered input dwords;
// cseg = 1024 X_even + 64 X_odd and xseg = X_even + X_odd for the segment;
// params: bf16 scale (low half) and bf16 min (high half).
__device__ __forceinline__ float seg_contrib(const uint4& c, const uint32_t* xp, float cseg, float xseg,
                                             uint32_t params) {
  float lo = 0.f, hi = 0.f;
  nib8_dot(c.x, xp + 0, lo, hi);
  nib8_dot(c.y, xp + 4, lo, hi);
  nib8_dot(c.z, xp + 8, lo, hi);
  nib8_dot(c.w, xp + 12, lo, hi);
  const float sq = fmaf(hi, 0.0625f, lo) - cseg;
  const float s = __uint_as_float(params << 16);
  const float m = __uint_as_float(params & 0xFFFF0000u);
  return fmaf(s, sq, m * xseg);
}

// Builds the pair-ordered f16 dwords and the two sums of a 32-value segment
// from 32 float values v[0..31] (exact in f16 for the magnitudes used here).
__device__ __forceinline__ void pack_segment(const float* v, uint32_t* xp, float& cseg, float& xseg) {
  float se = 0.f, so = 0.f;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const float* e = v + 8 * g;
#pragma unroll
    for (int p = 0; p < 4; ++p) xp[4 * g + p] = f16_bits(e[p]) | (f16_bits(e[p + 4]) << 16);
    se += (e[0] + e[2]) + (e[4] + e[6]);
    so += (e[1] + e[3]) + (e[5] + e[7]);
  }
  cseg = fmaf(1024.f, se, 64.f * so);
  xseg = se + so;
}

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + __expf(-g)); }

}  // namespace smoe
