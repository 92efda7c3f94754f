// Device twin of synth/gen.py's expert streams: fills SMOE-Q4 or SMOE-Q2 blobs with the
// seeded codes and per-chunk (scale, min) pairs, bit for bit as the numpy
// generator draws them, so that a whole vault can be drawn in HBM.
//
// SplitMix64 (Steele, Lea and Flood, OOPSLA 2014): word i of the stream with
// key K is mix64(K + (i + 1) * GAMMA).  Keys: mix64(mix64(seed + GAMMA) ^ tag),
// tag = kind << 56 | mat << 48 | layer << 24 | expert.
// Codes: the little-endian bytes of the words of stream (kind 1 for Q4, kind 6
// for Q2, mat).
// Scales: s = bf16(0.002 + 0.008 * U), U = (word >> 11) * 2^-53, two separately
// rounded double operations (this file is built with -ffp-contract=off);
// min = -8 * s (Q4) or -2 * s (Q2).  Holds no arithmetic of the MoE layer.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__host__ __device__ inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__host__ __device__ inline uint64_t stream_key(uint64_t seed, uint64_t kind, uint64_t layer, uint64_t expert,
                                               uint64_t mat) {
  const uint64_t tag = (kind << 56) | (mat << 48) | (layer << 24) | expert;
  return mix64(mix64(seed + kGamma) ^ tag);
}

__device__ inline uint64_t stream_word(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * kGamma); }

// bf16 pattern of v: round to nearest even at 8 significant bits, directly from
// the double (spacing 2^-133 below the normal range).
__device__ inline uint16_t bf16_bits(double v) {
  const double ax = fabs(v);
  int e = 0;
  frexp(ax, &e);
  int ue = e - 8;
  if (ue < -133) ue = -133;
  double r = ldexp(rint(ldexp(ax, -ue)), ue);
  if (ax == 0.0) r = 0.0;
  const float f = (float)r;
  uint32_t b = __float_as_uint(f) >> 16;
  if (v < 0) b |= 0x8000u;
  return (uint16_t)b;
}

struct Geo {
  int64_t rows[3], cols[3];
  int64_t code_off[3], par_off[3];
  int64_t code_words[3], par_count[3];
  int64_t bytes, stride;
};

// One thread per 8-byte unit of a blob: code words first, then 8-byte pairs of
// (scale, min) records (two chunks), then zero padding.
__global__ void fill_kernel(uint64_t seed, int layer, int e_begin, int bits, Geo g, uint8_t* dst) {
  const int eo = blockIdx.y;
  const int expert = e_begin + eo;
  uint8_t* blob = dst + (size_t)eo * g.stride;
  const int64_t units = g.stride / 8;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < units;
       u += (int64_t)gridDim.x * blockDim.x) {
    const int64_t byte = u * 8;
    uint64_t out = 0;
    bool done = false;
    for (int m = 0; m < 3 && !done; ++m) {
      if (byte >= g.code_off[m] && byte < g.code_off[m] + g.code_words[m] * 8) {
        const uint64_t key = stream_key(seed, bits == 4 ? 1 : 6, layer, expert, m);
        out = stream_word(key, (byte - g.code_off[m]) / 8);
        done = true;
      } else if (byte >= g.par_off[m] && byte < g.par_off[m] + g.par_count[m] * 4) {
        const uint64_t key = stream_key(seed, 2, layer, expert, m);
        const int64_t first = (byte - g.par_off[m]) / 4;
        for (int h = 0; h < 2; ++h) {
          const int64_t idx = first + h;
          if (idx >= g.par_count[m]) break;
          const double U = (double)(stream_word(key, idx) >> 11) * 0x1p-53;
          const double t = 0.008 * U;
          const double s = 0.002 + t;
          const uint16_t sb = bf16_bits(s);
          const float sv = __uint_as_float((uint32_t)sb << 16);
          const float mul = bits == 4 ? -8.0f : -2.0f;
          const uint16_t mb = (uint16_t)(__float_as_uint(mul * sv) >> 16);
          out |= ((uint64_t)sb | ((uint64_t)mb << 16)) << (32 * h);
        }
        done = true;
      }
    }
    *reinterpret_cast<uint64_t*>(blob + byte) = out;
  }
}

}  // namespace

extern "C" {

// Fills n_exp blobs of `layer`, experts e_begin.., at dst + i * stride, with
// codes of `bits` (4 or 2) bits.
// Returns 0, or -1 for bad arguments, -2 for a HIP launch error.
int synth_fill_experts(uint64_t seed, int d_model, int d_ff, int chunk, int bits, int layer, int e_begin,
                       int n_exp, void* dst, size_t stride, void* stream) {
  if (d_model <= 0 || d_ff <= 0 || (chunk != 32 && chunk != 64) || n_exp < 0 || !dst) return -1;
  if (bits != 4 && bits != 2) return -1;
  if ((int64_t)d_model * d_ff % 64 != 0 || d_model % chunk || d_ff % chunk) return -1;
  if (n_exp == 0) return 0;
  Geo g;
  const int64_t d = d_model, f = d_ff;
  g.rows[0] = f; g.cols[0] = d;
  g.rows[1] = f; g.cols[1] = d;
  g.rows[2] = d; g.cols[2] = f;
  int64_t pos = 0;
  for (int m = 0; m < 3; ++m) {
    g.code_off[m] = pos;
    g.code_words[m] = g.rows[m] * g.cols[m] * bits / 64;
    pos += g.rows[m] * g.cols[m] * bits / 8;
  }
  for (int m = 0; m < 3; ++m) {
    g.par_off[m] = pos;
    g.par_count[m] = g.rows[m] * (g.cols[m] / chunk);
    pos += g.par_count[m] * 4;
  }
  g.bytes = pos;
  g.stride = (int64_t)stride;
  if (g.stride < g.bytes || g.stride % 8) return -1;
  // every section boundary is 8-byte aligned, so no 8-byte unit straddles two
  for (int m = 0; m < 3; ++m)
    if (g.code_off[m] % 8 || g.par_off[m] % 8 || g.par_count[m] % 2) return -1;
  const int64_t units = g.stride / 8;
  int bx = (int)((units + 255) / 256);
  if (bx > 4096) bx = 4096;
  hipLaunchKernelGGL(fill_kernel, dim3(bx, n_exp), dim3(256), 0, (hipStream_t)stream, (uint64_t)seed, layer,
                     e_begin, bits, g, reinterpret_cast<uint8_t*>(dst));
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
