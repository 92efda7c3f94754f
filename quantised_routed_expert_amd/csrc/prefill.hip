// Layer-major batched prefill of one chunk (at most 64 tokens) through one MoE
// layer ("Prefill Reads Each Expert Once, Not Once Per Token", Optimizations
// page): the distinct experts the chunk routes to form its union, each union
// expert's blob is streamed once, and its tokens are processed together.
//
// Kernels (one launch each, in stream order):
//   1. union:   first-touch order of the routed experts (t ascending, then
//               rank), per-expert token counts and offsets, and the token
//               permutation (t ascending within an expert) -- integers only,
//               deterministic (LDS min/add/or atomics on integers).
//   2. gate_up: grouped GEMM per union expert on MFMA (v_mfma_f32_16x16x32_f16):
//               Q4 codes dequantised to fp16 in registers (exact when
//               min = -8 * scale), the chunk's token rows staged in LDS as
//               fp16, SwiGLU in the epilogue -> H [T*k][d_ff] fp16.
//   3. down:    grouped GEMM H x D^T per union expert -> Y [T*k][d_model] fp32.
//   4. combine: residual[t] += sum_r w[t][r] * Y[position of (t, r)], in rank
//               order (no atomics).
// The pages' own prefill FFN kernels keep a thread-per-row layout (Optimizations,
// "The Dense Ceiling"); here the dense contraction runs on the matrix cores.
#include "prefill.h"

namespace smoe {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// 1. Union and permutation.  One workgroup of 1024 threads (thread i <-> entry
// i = t * k + r of the routing).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void prefill_union_kernel(PrefillArgs a) {
  __shared__ int first[kMaxExperts];
  __shared__ int cnt[kMaxExperts];
  __shared__ unsigned long long tmask[kMaxExperts];
  __shared__ int rank_of[kMaxExperts];
  __shared__ int uid[kMaxExperts];
  __shared__ int scan[2][kMaxExperts + 1];
  __shared__ int s_nu;
  const int tid = threadIdx.x;
  const int n = a.T * a.k;
  if (tid < a.E) {
    first[tid] = 0x7FFFFFFF;
    cnt[tid] = 0;
    tmask[tid] = 0ull;
  }
  __syncthreads();
  int e = -1;
  if (tid < n) {
    e = a.idx[tid];
    if (e >= 0 && e < a.E) {
      atomicMin(&first[e], tid);
      atomicAdd(&cnt[e], 1);
      atomicOr(&tmask[e], 1ull << (tid / a.k));
    } else {
      e = -1;
    }
  }
  __syncthreads();
  // rank of each touched expert in first-touch order
  if (tid < a.E) {
    const int f0 = first[tid];
    int rank = -1;
    if (f0 != 0x7FFFFFFF) {
      rank = 0;
      for (int j = 0; j < a.E; ++j) rank += first[j] < f0;
      uid[rank] = tid;
    }
    rank_of[tid] = rank;
  }
  if (tid == 0) {
    int c = 0;
    for (int j = 0; j < a.E; ++j) c += first[j] != 0x7FFFFFFF;
    s_nu = c;
  }
  __syncthreads();
  const int nu = s_nu;
  // inclusive scan of the counts in union order (Hillis-Steele, ping-pong)
  if (tid < nu) scan[0][tid] = cnt[uid[tid]];
  __syncthreads();
  int src = 0;
  for (int off = 1; off < nu; off <<= 1) {
    if (tid < nu) scan[src ^ 1][tid] = scan[src][tid] + (tid >= off ? scan[src][tid - off] : 0);
    __syncthreads();
    src ^= 1;
  }
  if (tid < nu) {
    a.union_ids[tid] = uid[tid];
    a.offsets[tid + 1] = scan[src][tid];
  }
  if (tid == 0) {
    a.offsets[0] = 0;
    *a.union_count = nu;
  }
  if (tid < n) {
    int pos = -1;
    if (e >= 0) {
      const int u = rank_of[e];
      const int base = u == 0 ? 0 : scan[src][u - 1];
      const int t = tid / a.k;
      pos = base + __popcll(tmask[e] & ((1ull << t) - 1ull));
      a.perm[pos] = tid;
    }
    a.invperm[tid] = pos;
  }
}

// ---------------------------------------------------------------------------
// Dequantisation of one dword of codes (elements e0..e7 of one row) to the
// fp16 B fragment of one MFMA step, in pair order (e0,e4,e1,e5,e2,e6,e3,e7):
// 1024 + q (or 1024 + 16 q) via the fp16 exponent of 1024, minus 1024 exactly,
// then scale * q + min with one packed fp16 FMA (single rounding; exact when
// the result is representable, as for min = -8 * scale).
// ---------------------------------------------------------------------------
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ h2_t as_h2(uint32_t v) { return __builtin_bit_cast(h2_t, v); }

__device__ __forceinline__ half8_t dequant8(uint32_t w, h2_t s, h2_t s16, h2_t m) {
  const uint32_t magic = 0x64006400u;
  const h2_t k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
  const uint32_t w8 = w >> 8;
  const h2_t q0 = as_h2((w & 0x000F000Fu) | magic) - k1024;   // (e0, e4)
  const h2_t q1 = as_h2((w & 0x00F000F0u) | magic) - k1024;   // 16 (e1, e5)
  const h2_t q2 = as_h2((w8 & 0x000F000Fu) | magic) - k1024;  // (e2, e6)
  const h2_t q3 = as_h2((w8 & 0x00F000F0u) | magic) - k1024;  // 16 (e3, e7)
  const h2_t w0 = __builtin_elementwise_fma(q0, s, m);
  const h2_t w1 = __builtin_elementwise_fma(q1, s16, m);
  const h2_t w2 = __builtin_elementwise_fma(q2, s, m);
  const h2_t w3 = __builtin_elementwise_fma(q3, s16, m);
  half8_t r;
  r[0] = w0[0]; r[1] = w0[1]; r[2] = w1[0]; r[3] = w1[1];
  r[4] = w2[0]; r[5] = w2[1]; r[6] = w3[0]; r[7] = w3[1];
  return r;
}

// (scale, min) bf16 pair -> fp16 pairs (s, s), (s/16, s/16), (m, m)
__device__ __forceinline__ void params_f16(uint32_t p, h2_t& s, h2_t& s16, h2_t& m) {
  const _Float16 sv = (_Float16)__uint_as_float(p << 16);
  const _Float16 mv = (_Float16)__uint_as_float(p & 0xFFFF0000u);
  const _Float16 sv16 = (_Float16)(__uint_as_float(p << 16) * 0.0625f);
  s = h2_t{sv, sv};
  s16 = h2_t{sv16, sv16};
  m = h2_t{mv, mv};
}

constexpr int kPfKT = 128;      // K per iteration (4 MFMA steps)
constexpr int kPfMaxMT = 4;     // up to 64 tokens per expert = 4 M tiles of 16

// Rows of the union expert's tokens in LDS, fp16 pair order within groups of 8,
// for one K block: xs[mt][row][kPfKT].
template <bool FROM_BF16>
__device__ __forceinline__ void stage_rows(_Float16 (*xs)[16][kPfKT], const void* src, size_t row_elems,
                                           const int* rows, int n_rows, int mt_count, int kb) {
  const int tid = threadIdx.x;  // 256 threads: 16 rows x 16 groups of 8 per M tile
  const int r = tid >> 4, c8 = (tid & 15) * 8;
  for (int mt = 0; mt < mt_count; ++mt) {
    const int m = mt * 16 + r;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (m < n_rows) {
      const size_t off = (size_t)rows[m] * row_elems + kb + c8;
      v = gload16(reinterpret_cast<const uint16_t*>(src) + off);
    }
    uint4 o;
    if (FROM_BF16) {
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
      float f[8];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        f[2 * p] = bf16_to_f32(w4[p] & 0xFFFF);
        f[2 * p + 1] = bf16_to_f32(w4[p] >> 16);
      }
      o.x = f16_bits(f[0]) | (f16_bits(f[4]) << 16);
      o.y = f16_bits(f[1]) | (f16_bits(f[5]) << 16);
      o.z = f16_bits(f[2]) | (f16_bits(f[6]) << 16);
      o.w = f16_bits(f[3]) | (f16_bits(f[7]) << 16);
    } else {
      o = v;  // already fp16 in pair order
    }
    *reinterpret_cast<uint4*>(&xs[mt][r][c8]) = o;
  }
}

// One wave: 16 output features (rows n0..n0+15 of a matrix) x all M tiles,
// one K block.  Lane (nl = l % 16, g = l / 16) dequantises 32 codes of row
// n0 + nl at K [kb + 32 g, kb + 32 g + 32): dword t feeds MFMA step t.
template <int CHUNK, int MT>
__device__ __forceinline__ void mma_block(float4_t (*acc)[1], const uint8_t* codes_row, const uint8_t* par_row,
                                          _Float16 (*xs)[16][kPfKT], int kb, int lane) {
  const int g = lane >> 4, ml = lane & 15;
  const uint4 c = gload16(codes_row + kb / 2 + 16 * g);
  const uint32_t p = gload4(par_row + ((kb + 32 * g) / CHUNK) * 4);
  h2_t s, s16, m;
  params_f16(p, s, s16, m);
  const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const half8_t b = dequant8(cw[t], s, s16, m);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const half8_t av = *reinterpret_cast<const half8_t*>(&xs[mt][ml][32 * g + 8 * t]);
      acc[mt][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, b, acc[mt][0], 0, 0, 0);
    }
  }
}

// ---------------------------------------------------------------------------
// 2. Grouped gate/up GEMM + SwiGLU.  grid = (d_ff / 64, min(E, T*k)),
// 256 threads (4 waves x 16 features).  Workgroup (nt, u) handles union expert
// u (exits when u >= |union|) and features [64 nt, 64 nt + 64).
// ---------------------------------------------------------------------------
template <int CHUNK, int MT>
__device__ void gate_up_body(const PrefillArgs& a, const uint8_t* blob, int o, int n_u, const int* rows,
                             _Float16 (*xs)[kPfMaxMT][16][kPfKT]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * 64 + wave * 16;
  const size_t row_bytes = (size_t)a.d / 2, prow = (size_t)(a.d / CHUNK) * 4;
  const uint8_t* gc = blob + (size_t)(n0 + (lane & 15)) * row_bytes;
  const uint8_t* uc = blob + a.lay.up_codes + (size_t)(n0 + (lane & 15)) * row_bytes;
  const uint8_t* gp = blob + a.lay.gate_params + (size_t)(n0 + (lane & 15)) * prow;
  const uint8_t* up = blob + a.lay.up_params + (size_t)(n0 + (lane & 15)) * prow;
  float4_t accg[MT][1], accu[MT][1];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    accg[mt][0] = float4_t{0.f, 0.f, 0.f, 0.f};
    accu[mt][0] = float4_t{0.f, 0.f, 0.f, 0.f};
  }
  int buf = 0;
  stage_rows<true>(xs[0], a.x, (size_t)a.d, rows, n_u, MT, 0);
  __syncthreads();
  for (int kb = 0; kb < a.d; kb += kPfKT) {
    if (kb + kPfKT < a.d) stage_rows<true>(xs[buf ^ 1], a.x, (size_t)a.d, rows, n_u, MT, kb + kPfKT);
    mma_block<CHUNK, MT>(accg, gc, gp, xs[buf], kb, lane);
    mma_block<CHUNK, MT>(accu, uc, up, xs[buf], kb, lane);
    __syncthreads();
    buf ^= 1;
  }
  // epilogue: lane holds rows 4 (l / 16) + i of each M tile, feature n0 + l % 16
  const int n = n0 + (lane & 15);
  const int hcol = (n & ~7) + pair_slot(n & 7);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = mt * 16 + 4 * (lane >> 4) + i;
      if (row < n_u) {
        const float gv = accg[mt][0][i], uv = accu[mt][0][i];
        a.H[(size_t)(o + row) * a.f + hcol] = (_Float16)(silu_f32(gv) * uv);
      }
    }
  }
}

template <int CHUNK>
__global__ __launch_bounds__(256) void prefill_gate_up_kernel(PrefillArgs a) {
  __shared__ _Float16 xs[2][kPfMaxMT][16][kPfKT];
  __shared__ int rows[kMaxPrefillTokens];
  const int u = blockIdx.y;
  if (u >= *a.union_count) return;
  const int e = a.union_ids[u];
  const int o = a.offsets[u], n_u = a.offsets[u + 1] - o;
  if (e < 0 || e >= a.E || n_u <= 0) return;
  const uint8_t* blob = reinterpret_cast<const uint8_t*>(a.table[e]);
  if (threadIdx.x < n_u) rows[threadIdx.x] = a.perm[o + threadIdx.x] / a.k;  // token of each entry
  __syncthreads();
  const int mt = (n_u + 15) / 16;
  switch (mt) {
    case 1: gate_up_body<CHUNK, 1>(a, blob, o, n_u, rows, xs); break;
    case 2: gate_up_body<CHUNK, 2>(a, blob, o, n_u, rows, xs); break;
    case 3: gate_up_body<CHUNK, 3>(a, blob, o, n_u, rows, xs); break;
    default: gate_up_body<CHUNK, 4>(a, blob, o, n_u, rows, xs); break;
  }
}

// ---------------------------------------------------------------------------
// 3. Grouped down GEMM.  grid = (d_model / 64, min(E, T*k)), 256 threads.
// A = H rows o..o+n_u-1 (fp16, pair order), B = D rows (output features).
// ---------------------------------------------------------------------------
template <int CHUNK, int MT>
__device__ void down_body(const PrefillArgs& a, const uint8_t* blob, int o, int n_u, const int* rows,
                          _Float16 (*xs)[kPfMaxMT][16][kPfKT]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * 64 + wave * 16;
  const size_t row_bytes = (size_t)a.f / 2, prow = (size_t)(a.f / CHUNK) * 4;
  const uint8_t* dc = blob + a.lay.down_codes + (size_t)(n0 + (lane & 15)) * row_bytes;
  const uint8_t* dp = blob + a.lay.down_params + (size_t)(n0 + (lane & 15)) * prow;
  float4_t acc[MT][1];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt][0] = float4_t{0.f, 0.f, 0.f, 0.f};
  int buf = 0;
  stage_rows<false>(xs[0], a.H, (size_t)a.f, rows, n_u, MT, 0);
  __syncthreads();
  for (int kb = 0; kb < a.f; kb += kPfKT) {
    if (kb + kPfKT < a.f) stage_rows<false>(xs[buf ^ 1], a.H, (size_t)a.f, rows, n_u, MT, kb + kPfKT);
    mma_block<CHUNK, MT>(acc, dc, dp, xs[buf], kb, lane);
    __syncthreads();
    buf ^= 1;
  }
  const int n = n0 + (lane & 15);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = mt * 16 + 4 * (lane >> 4) + i;
      if (row < n_u) a.Y[(size_t)(o + row) * a.d + n] = acc[mt][0][i];
    }
  }
}

template <int CHUNK>
__global__ __launch_bounds__(256) void prefill_down_kernel(PrefillArgs a) {
  __shared__ _Float16 xs[2][kPfMaxMT][16][kPfKT];
  __shared__ int rows[kMaxPrefillTokens];
  const int u = blockIdx.y;
  if (u >= *a.union_count) return;
  const int e = a.union_ids[u];
  const int o = a.offsets[u], n_u = a.offsets[u + 1] - o;
  if (e < 0 || e >= a.E || n_u <= 0) return;
  const uint8_t* blob = reinterpret_cast<const uint8_t*>(a.table[e]);
  if (threadIdx.x < n_u) rows[threadIdx.x] = o + threadIdx.x;  // H rows of this expert
  __syncthreads();
  const int mt = (n_u + 15) / 16;
  switch (mt) {
    case 1: down_body<CHUNK, 1>(a, blob, o, n_u, rows, xs); break;
    case 2: down_body<CHUNK, 2>(a, blob, o, n_u, rows, xs); break;
    case 3: down_body<CHUNK, 3>(a, blob, o, n_u, rows, xs); break;
    default: down_body<CHUNK, 4>(a, blob, o, n_u, rows, xs); break;
  }
}

// ---------------------------------------------------------------------------
// 4. Combine.  grid = (ceil(d / 256), T), 256 threads: residual[t][n] +=
// sum_r w[t][r] * Y[invperm[t*k + r]][n], r ascending.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prefill_combine_kernel(PrefillArgs a) {
  const int t = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= a.d) return;
  float acc = 0.f;
  for (int r = 0; r < a.k; ++r) {
    const int pos = a.invperm[t * a.k + r];
    if (pos >= 0) acc = fmaf(a.w[t * a.k + r], a.Y[(size_t)pos * a.d + n], acc);
  }
  a.residual[(size_t)t * a.d + n] += acc;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
  const int max_union = a.E < a.T * a.k ? a.E : a.T * a.k;
  hipLaunchKernelGGL(prefill_union_kernel, dim3(1), dim3(1024), 0, s, a);
  if (a.chunk == 64) {
    hipLaunchKernelGGL(prefill_gate_up_kernel<64>, dim3(a.f / 64, max_union), dim3(256), 0, s, a);
    hipLaunchKernelGGL(prefill_down_kernel<64>, dim3(a.d / 64, max_union), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL(prefill_gate_up_kernel<32>, dim3(a.f / 64, max_union), dim3(256), 0, s, a);
    hipLaunchKernelGGL(prefill_down_kernel<32>, dim3(a.d / 64, max_union), dim3(256), 0, s, a);
  }
  hipLaunchKernelGGL(prefill_combine_kernel, dim3((a.d + 255) / 256, a.T), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace smoe
