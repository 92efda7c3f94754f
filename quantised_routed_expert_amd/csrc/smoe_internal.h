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

// Byte offsets of the sections of one SMOE-Q4 / SMOE-Q2 expert blob (layout
// in smoe.h); `bits` is the code width.
struct BlobLayout {
  size_t up_codes, down_codes, gate_params, up_params, down_params, bytes;
};

inline BlobLayout blob_layout(int d, int f, int chunk, int bits) {
  BlobLayout b;
  const size_t df = (size_t)d * (size_t)f;
  const size_t mat = df * (size_t)bits / 8;  // code bytes of one matrix
  b.up_codes = mat;
  b.down_codes = 2 * mat;
  b.gate_params = 3 * mat;
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

// bf16 bits of fl64(r / den) for a float r.  Fast path: q = r * inv32 in
// fp32 (inv32 = fp32(1 / den)) is within about one fp32 ulp of the exact
// quotient; unless it lies within 4 fp32 ulps of a bf16 tie point (or is
// zero / below the fp32 normal range), its round-to-nearest-even bf16 equals
// that of the correctly rounded double quotient.  Otherwise divide in fp64.
__device__ __forceinline__ uint32_t bf16_of_quotient(float r, double den, float inv32) {
  const float q = r * inv32;
  const uint32_t b = __float_as_uint(q);
  const uint32_t rem = b & 0xFFFFu;
  const uint32_t dist = rem > 0x8000u ? rem - 0x8000u : 0x8000u - rem;
  if (dist <= 4u || (b & 0x7F800000u) == 0u) return f64_to_bf16_rne((double)r / den);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t f16_bits(float v) {
  _Float16 h = (_Float16)v;
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

// Storage order inside each group of 8 values for the nibble-pair dot
// products: stored slot i holds element kPairSlot^-1(i); element j goes to
// slot (j < 4 ? 2j : 2(j-4)+1), so dword p of the group holds (e_p, e_{p+4}).
__device__ __forceinline__ int pair_slot(int j) { return j < 4 ? 2 * j : 2 * (j - 4) + 1; }

// The same for SMOE-Q2's groups of 16: dword p of a group holds (e_p, e_{p+8}).
__device__ __forceinline__ int pair_slot16(int j) { return j < 8 ? 2 * j : 2 * (j - 8) + 1; }

// Pair order of code width BITS (groups of 8 for Q4, 16 for Q2): the storage
// index of element n of a vector.
template <int BITS>
__device__ __forceinline__ int pair_index(int n) {
  if (BITS == 4) return (n & ~7) + pair_slot(n & 7);
  return (n & ~15) + pair_slot16(n & 15);
}

// ---------------------------------------------------------------------------
// Wave reductions.  Within a row of 16 lanes the partial sums move with DPP
// (quad_perm xor 1 / xor 2, half-row mirror, row mirror), across rows with
// ds_bpermute.  Every lane of a W-lane group ends with a sum of the group;
// the order is fixed, so results are bitwise reproducible.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <int W>
__device__ __forceinline__ float group_sum(float v) {
  if (W >= 2) v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
  if (W >= 4) v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
  if (W >= 8) v += dpp_f32<0x141>(v);  // row_half_mirror
  if (W >= 16) v += dpp_f32<0x140>(v); // row_mirror
  if (W >= 32) v += __shfl_xor(v, 16, kWave);
  if (W >= 64) v += __shfl_xor(v, 32, kWave);
  return v;
}

// Maximum over each row of 16 lanes, valid in every lane of the row.
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f32<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f32<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp_f32<0x140>(v));  // row_mirror
  return v;
}

// Power-of-two scaling of a block of activations for fp16 storage: the shift
// sh such that mx * 2^sh lies in [2^14, 2^15) for the block's largest
// magnitude mx (so no value of the block overflows fp16, whose largest finite
// value is 65504, and the largest keep fp16's full precision); 15 for zero,
// infinity or NaN (v_frexp_exp gives 0 for them), and clamped so that 2^sh and
// 2^-sh are normal floats.
__device__ __forceinline__ int f16_block_shift(float mx) {
  const int sh = 15 - __builtin_amdgcn_frexp_expf(mx);
  return sh < -120 ? -120 : (sh > 120 ? 120 : sh);
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Sum over each W-lane group, valid in the LAST lane of the group (lane
// W-1 of it): DPP inside rows of 16, then row_bcast:15 / row_bcast:31 to
// carry row sums upward (no LDS traffic).
template <int W>
__device__ __forceinline__ float group_sum_last(float v) {
  if (W >= 2) v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
  if (W >= 4) v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
  if (W >= 8) v += dpp_f32<0x141>(v);  // row_half_mirror
  if (W >= 16) v += dpp_f32<0x140>(v); // row_mirror: every lane of a row holds its row sum
  if (W >= 32)                          // rows 1, 3 += rows 0, 2
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
  if (W >= 64)                          // rows 2, 3 += row 1 (= rows 0 + 1)
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));
  return v;
}

template <int W>
__device__ __forceinline__ double group_sum_f64(double v) {
  if (W >= 2) v += dpp_f64<0xB1>(v);
  if (W >= 4) v += dpp_f64<0x4E>(v);
  if (W >= 8) v += dpp_f64<0x141>(v);
  if (W >= 16) v += dpp_f64<0x140>(v);
  if (W >= 32) v += __shfl_xor(v, 16, kWave);
  if (W >= 64) v += __shfl_xor(v, 32, kWave);
  return v;
}

// ---------------------------------------------------------------------------
// Nibble-pair dot products.
// A dword w of codes holds elements e0..e7 (e_j in bits 4j..4j+3).  Masking a
// 4-bit field into the low mantissa bits of an fp16 half gives the fp16
// subnormal q * 2^-24 exactly; at bits 4..7 it gives 16 q * 2^-24.  So
//   w & 0x000F000F        = (e0, e4) * 2^-24
//   w & 0x00F000F0        = (e1, e5) * 16 * 2^-24
//   (w >> 8) & 0x000F000F = (e2, e6) * 2^-24
//   (w >> 8) & 0x00F000F0 = (e3, e7) * 16 * 2^-24
// and, with the input stored in pair order (dword p of a group of 8 holds
// (x_p, x_{p+4})), v_dot2_f32_f16 -- which keeps fp16 subnormal inputs on
// gfx950 -- accumulates exact products into lo (even elements) and hi (odd):
//   sum q x = 2^24 * (lo + hi / 16).
// ---------------------------------------------------------------------------
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c,
                                false);
}

// One dword of codes against four dwords of pair-ordered f16 inputs.
__device__ __forceinline__ void nib8_dot(uint32_t w, const uint32_t* xp, float& lo, float& hi) {
  const uint32_t w8 = w >> 8;
  lo = dot2(w & 0x000F000Fu, xp[0], lo);
  hi = dot2(w & 0x00F000F0u, xp[1], hi);
  lo = dot2(w8 & 0x000F000Fu, xp[2], lo);
  hi = dot2(w8 & 0x00F000F0u, xp[3], hi);
}

// Contribution of one 16-byte segment (32 codes, inside one chunk) of a row:
// scale * sum(q x) + min * sum(x).  xp: 16 pair-ordered input dwords; xseg =
// sum of the segment's inputs; params: bf16 scale (low half), bf16 min (high).
__device__ __forceinline__ float seg_contrib(const uint4& c, const uint32_t* xp, float xseg, uint32_t params) {
  float lo = 0.f, hi = 0.f;
  nib8_dot(c.x, xp + 0, lo, hi);
  nib8_dot(c.y, xp + 4, lo, hi);
  nib8_dot(c.z, xp + 8, lo, hi);
  nib8_dot(c.w, xp + 12, lo, hi);
  const float sq = fmaf(hi, 0.0625f, lo) * 16777216.0f;  // sum q x
  const float s = __uint_as_float(params << 16);
  const float m = __uint_as_float(params & 0xFFFF0000u);
  return fmaf(s, sq, m * xseg);
}

// 2-bit pairs.  A dword w of SMOE-Q2 codes holds elements e0..e15 (e_j in
// bits 2j..2j+1).  Masking a 2-bit field at bit 2i of each half gives the fp16
// subnormals (e_i, e_{i+8}) * 4^i * 2^-24 exactly, and w >> 8 brings
// (e_{i+4}, e_{i+12}) to the same positions.  With the input in 16-group pair
// order (dword p holds (x_p, x_{p+8})), four accumulators a_i collect the
// products of field i, and sum q x = 2^24 * (a0 + a1/4 + a2/16 + a3/64).
__device__ __forceinline__ void crumb16_dot(uint32_t w, const uint32_t* xp, float* acc) {
  const uint32_t w8 = w >> 8;
  acc[0] = dot2(w & 0x00030003u, xp[0], acc[0]);
  acc[1] = dot2(w & 0x000C000Cu, xp[1], acc[1]);
  acc[2] = dot2(w & 0x00300030u, xp[2], acc[2]);
  acc[3] = dot2(w & 0x00C000C0u, xp[3], acc[3]);
  acc[0] = dot2(w8 & 0x00030003u, xp[4], acc[0]);
  acc[1] = dot2(w8 & 0x000C000Cu, xp[5], acc[1]);
  acc[2] = dot2(w8 & 0x00300030u, xp[6], acc[2]);
  acc[3] = dot2(w8 & 0x00C000C0u, xp[7], acc[3]);
}

// Contribution of one 16-byte SMOE-Q2 segment (64 codes = one chunk of 64):
// scale * sum(q x) + min * sum(x); xp: 32 pair-ordered input dwords.
__device__ __forceinline__ float seg_contrib_q2(const uint4& c, const uint32_t* xp, float xseg, uint32_t params) {
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  crumb16_dot(c.x, xp + 0, acc);
  crumb16_dot(c.y, xp + 8, acc);
  crumb16_dot(c.z, xp + 16, acc);
  crumb16_dot(c.w, xp + 24, acc);
  const float sq = fmaf(fmaf(acc[3], 0.25f, acc[2]), 0.0625f, fmaf(acc[1], 0.25f, acc[0])) * 16777216.0f;
  const float s = __uint_as_float(params << 16);
  const float m = __uint_as_float(params & 0xFFFF0000u);
  return fmaf(s, sq, m * xseg);
}

// Sum of the 2 * NDW values of NDW pair-ordered f16 dwords (dot2 against ones).
template <int NDW = 16>
__device__ __forceinline__ float seg_sum(const uint32_t* xp) {
  float a = 0.f, b = 0.f;
#pragma unroll
  for (int i = 0; i < NDW; i += 2) {
    a = dot2(xp[i], 0x3C003C00u, a);
    b = dot2(xp[i + 1], 0x3C003C00u, b);
  }
  return a + b;
}

// Pair-ordered f16 dwords of a 32-value segment from 32 float values v[0..31]
// (exact in f16 for the magnitudes used here).
__device__ __forceinline__ void pack_segment(const float* v, uint32_t* xp) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const float* e = v + 8 * g;
#pragma unroll
    for (int p = 0; p < 4; ++p) xp[4 * g + p] = f16_bits(e[p]) | (f16_bits(e[p + 4]) << 16);
  }
}

// The same for a 64-value SMOE-Q2 segment in 16-group pair order.
__device__ __forceinline__ void pack_segment_q2(const float* v, uint32_t* xp) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const float* e = v + 16 * g;
#pragma unroll
    for (int p = 0; p < 8; ++p) xp[8 * g + p] = f16_bits(e[p]) | (f16_bits(e[p + 8]) << 16);
  }
}

// Loads through the global address space (pointers read from LDS or kernel
// arguments are otherwise generic, and would become flat loads).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4_t g_u32x4;
typedef __attribute__((address_space(1))) const uint32_t g_uint32;
__device__ __forceinline__ uint4 gload16(const void* p) {
  const u32x4_t v = *(g_u32x4*)(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t gload4(const void* p) { return *(g_uint32*)(p); }

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + __expf(-g)); }

}  // namespace smoe
