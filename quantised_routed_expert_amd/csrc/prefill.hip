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
//   2. gate_up: grouped GEMM per union expert on MFMA (v_mfma_f32_16x16x32_f16),
//               the chunk's token rows staged in LDS as fp16, SwiGLU in the
//               epilogue -> H [T*k][d_ff] fp16.  Chunk 64 (d_model, d_ff
//               multiples of 256): the raw codes enter MFMA and the affine
//               step is folded per chunk (the *_fold kernels; for SMOE-Q2
//               blobs the *_fold_q2 kernels), after a small kernel has put
//               the chunk's x rows in the fold's A layout once per call
//               (prefill_stage_x*); otherwise the codes are dequantised to
//               fp16 in registers (exact when min = -8 * scale, or -2 * scale
//               for SMOE-Q2, whose down GEMM takes this form when d_ff is not
//               a multiple of 512).
//   3. down:    grouped GEMM H x D^T per union expert -> Y [T*k][d_model] fp32,
//               in the same two forms (the SMOE-Q4 fold with two 64-column
//               tiles per workgroup).
//   4. combine: residual[t] += sum_r w[t][r] * Y[position of (t, r)], in rank
//               order (no atomics).
// The pages' own prefill FFN kernels keep a thread-per-row layout (Optimizations,
// "The Dense Ceiling"); here the dense contraction runs on the matrix cores.
#include <hip/hip_ext.h>

#include "prefill.h"

namespace smoe {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// 1. Union and permutation.  One workgroup of 1024 threads (thread i <-> entry
// i = t * k + r of the routing).  An entry whose expert is outside [0, E) or
// has a NULL table entry takes no part (its invperm is -1, so it contributes
// nothing, as a null blob does in decode).  Entries are listed per expert in
// (t, r) order; a token that lists an expert more than once gets one slot per
// entry (the router never does this; such chunks take a slower serial path).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void prefill_union_kernel(PrefillArgs a) {
  __shared__ int first[kMaxExperts];
  __shared__ int cnt[kMaxExperts];
  __shared__ unsigned long long tmask[kMaxExperts];
  __shared__ int rank_of[kMaxExperts];
  __shared__ int uid[kMaxExperts];
  __shared__ int usable[kMaxExperts];
  __shared__ int eidx[kMaxPrefillTokens * kMaxTopK];
  __shared__ int pos_of[kMaxPrefillTokens * kMaxTopK];
  __shared__ int scan[2][kMaxExperts + 1];
  __shared__ int sscan[2][kMaxExperts + 1];
  __shared__ int s_nu, s_dup;
  const int tid = threadIdx.x;
  const int n = a.T * a.k;
  if (tid < a.E) {
    first[tid] = 0x7FFFFFFF;
    cnt[tid] = 0;
    tmask[tid] = 0ull;
    usable[tid] = a.table[tid] != nullptr;
  }
  if (tid == 0) s_dup = 0;
  __syncthreads();
  int e = -1;
  if (tid < n) {
    e = a.idx[tid];
    if (!(e >= 0 && e < a.E && usable[e])) e = -1;
    eidx[tid] = e;
  }
  __syncthreads();
  if (e >= 0) {
    atomicMin(&first[e], tid);
    atomicAdd(&cnt[e], 1);
    atomicOr(&tmask[e], 1ull << (tid / a.k));
    const int t0 = tid - tid % a.k;  // the token's first entry
    for (int j = t0; j < tid; ++j)
      if (eidx[j] == e) s_dup = 1;   // (benign race: every writer stores 1)
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
  // slices of 16 entries per union expert, in union order (inclusive scan)
  if (tid < nu) sscan[0][tid] = (cnt[uid[tid]] + 15) / 16;
  __syncthreads();
  int ssrc = 0;
  for (int off = 1; off < nu; off <<= 1) {
    if (tid < nu) sscan[ssrc ^ 1][tid] = sscan[ssrc][tid] + (tid >= off ? sscan[ssrc][tid - off] : 0);
    __syncthreads();
    ssrc ^= 1;
  }
  if (tid < nu) {
    const int e = uid[tid], n_u = cnt[e];
    const int end = sscan[ssrc][tid], ns = (n_u + 15) / 16;
    const int base = tid == 0 ? 0 : scan[src][tid - 1];
    const void* blob = a.table[e];
    for (int q = 0; q < ns; ++q) {
      a.slices[end - ns + q] = (tid << 8) | q;
      PrefillArgs::SliceRec r;
      r.blob = blob;
      r.o = base + 16 * q;
      r.n_rows = n_u - 16 * q < 16 ? n_u - 16 * q : 16;
      a.recs[end - ns + q] = r;
    }
    if (tid == nu - 1) *a.n_slices = end;
  }
  if (tid == 0 && nu == 0) *a.n_slices = 0;
  if (!s_dup) {  // uniform: one entry per (token, expert), placed by its token's rank
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
  } else {  // some token lists an expert twice: each expert walks the entries in order
    if (tid < n) pos_of[tid] = -1;
    __syncthreads();
    if (tid < a.E && rank_of[tid] >= 0) {
      const int u = rank_of[tid];
      int pos = u == 0 ? 0 : scan[src][u - 1];
      for (int j = 0; j < n; ++j) {
        if (eidx[j] == tid) {
          a.perm[pos] = j;
          pos_of[j] = pos++;
        }
      }
    }
    __syncthreads();
    if (tid < n) a.invperm[tid] = pos_of[tid];
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

// SMOE-Q2: one dword holds 16 two-bit codes, element 4j + i in bits 2i..2i+1
// of byte j.  Its low half (bytes 0 and 2 after the shifts below) gives the
// pairs (e_p, e_{p+8}) for p = 0..3 in this order; the caller passes w >> 8
// for p = 4..7.  A code at bits 2..3 of a byte reads as 4 q, so those pairs
// take s/4; every (scale, min) of the format keeps s/4 a normal fp16.
__device__ __forceinline__ half8_t dequant8_q2(uint32_t w, h2_t s, h2_t s4, h2_t m) {
  const uint32_t magic = 0x64006400u;
  const h2_t k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
  const uint32_t w4 = w >> 4;
  const h2_t q0 = as_h2((w & 0x00030003u) | magic) - k1024;   // (e0, e8)
  const h2_t q1 = as_h2((w & 0x000C000Cu) | magic) - k1024;   // 4 (e1, e9)
  const h2_t q2 = as_h2((w4 & 0x00030003u) | magic) - k1024;  // (e2, e10)
  const h2_t q3 = as_h2((w4 & 0x000C000Cu) | magic) - k1024;  // 4 (e3, e11)
  const h2_t w0 = __builtin_elementwise_fma(q0, s, m);
  const h2_t w1 = __builtin_elementwise_fma(q1, s4, m);
  const h2_t w2 = __builtin_elementwise_fma(q2, s, m);
  const h2_t w3 = __builtin_elementwise_fma(q3, s4, m);
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


// ---------------------------------------------------------------------------
// SwiGLU epilogue of a gate/up tile: up to 16 entries x the 64 features of
// workgroup column blockIdx.x.  The lane computes h = silu(g) * u for its
// feature (stored at column hcol of H) and its rows 4 (lane / 16) + i.  Each
// row of the tile is scaled by one power of two (f16_block_shift of the row's
// largest |h| over the tile) before it is rounded to fp16, and the inverse
// scale goes to Hs[row][tile]: H stays fp16 without overflow, and the down
// GEMM multiplies each tile's contribution back (a tile is one chunk of 64 of
// the down projection's reduction).  red: [4][16] floats of LDS.  Every thread
// of the workgroup calls it (it holds a barrier).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void store_h_tile(const PrefillArgs& a, const float4_t& ag, const float4_t& au, int o,
                                             int n_rows, int hcol, float (*red)[16]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float h[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = silu_f32(ag[i]) * au[i];
    const float m = row_max16(fabsf(h[i]));  // over the wave's 16 features
    if ((lane & 15) == 0) red[wave][4 * (lane >> 4) + i] = m;
  }
  __syncthreads();
  const int tiles = a.f / 64;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * (lane >> 4) + i;
    const float mx = fmaxf(fmaxf(red[0][row], red[1][row]), fmaxf(red[2][row], red[3][row]));
    const int sh = f16_block_shift(mx);
    if (row < n_rows) {
      a.H[(size_t)(o + row) * a.f + hcol] = (_Float16)(h[i] * __builtin_ldexpf(1.0f, sh));
      if (wave == 0 && (lane & 15) == 0)
        a.Hs[(size_t)(o + row) * tiles + blockIdx.x] = __builtin_ldexpf(1.0f, -sh);
    }
  }
}

// ---------------------------------------------------------------------------
// 2-3. Grouped GEMMs over slices: a slice is up to 16 consecutive entries of
// one union expert (one MFMA M tile).  grid = (N / 64, max slices), 256
// threads; workgroup (nt, s) computes features [64 nt, 64 nt + 64) of slice s,
// wave w the 16 features 64 nt + 16 w .. + 15.  An expert with more than 16
// entries has several slices whose workgroups run side by side, so its
// weights come from HBM once and from cache for the others.
//
// K advances in blocks of KT.  In a block, lane (nl = l % 16, g = l / 16)
// holds the KT / 4 consecutive codes of row nl starting at kb + g KT / 4
// (KT / 64 16-byte loads, so a row is read in runs of KT / 2 bytes), and MFMA
// step t (0 .. KT / 32 - 1) takes k = kb + g KT / 4 + 8 t + i (i < 8) from
// lane group g; the A fragments in LDS use the same k order.  Token rows and
// weights of block i + 1 are requested before block i is computed.
// ---------------------------------------------------------------------------
template <int KT>
struct KBlock {
  static constexpr int KPL = KT / 4;      // codes per lane per block
  static constexpr int NC = KPL / 32;     // 16-byte code loads per lane
  static constexpr int STEPS = KT / 32;   // MFMA steps per block
};

// A slice's token rows for one K block (16 rows x KT fp16) staged in LDS.
// Thread (r = tid / 16, c = tid % 16) moves KT / 16 consecutive values of row
// r; load() and store() are separate so the loads run a block ahead.  From
// bf16, the values are stored in the pair order of groups of 8; fp16 rows (H)
// are copied as they are (in the pair order of their code width).
// For H rows (FROM_BF16 false) the stage also brings the rows' tile scales:
// the values of a K block are put on one common scale per row (the block's
// largest tile scale F, a power of two; a tile's values are multiplied by its
// scale / F <= 1, exactly unless they fall below the fp16 normal range), and
// F goes to fblk[row] for the caller to multiply the block's result by.  A
// thread's KT / 16 values lie in one tile, and the 16 threads of a row are
// one row of lanes, so F is a 16-lane maximum.
template <bool FROM_BF16, int KT>
struct RowStage {
  static constexpr int V = KT / 16 / 8;  // uint4 (8 values) per thread
  uint4 v[V];
  float fs;                              // tile scale of this thread's values (H rows)

  __device__ __forceinline__ void load(const void* src, size_t row_elems, const int* rows, int n_rows, int kb,
                                       const float* hs = nullptr, int tiles = 0) {
    const int tid = threadIdx.x, r = tid >> 4, c = (tid & 15) * (KT / 16);
#pragma unroll
    for (int j = 0; j < V; ++j) {
      v[j] = make_uint4(0, 0, 0, 0);
      if (r < n_rows) v[j] = gload16(reinterpret_cast<const uint16_t*>(src) + (size_t)rows[r] * row_elems + kb + c + 8 * j);
    }
    fs = 1.0f;
    if (!FROM_BF16 && r < n_rows) fs = hs[(size_t)rows[r] * tiles + (kb + c) / 64];
  }

  __device__ __forceinline__ void store(_Float16 (*xs)[KT + 8], float* fblk = nullptr) const {
    const int tid = threadIdx.x, r = tid >> 4, c = (tid & 15) * (KT / 16);
    h2_t ratio = {(_Float16)1.0f, (_Float16)1.0f};
    if (!FROM_BF16) {
      const float fb = row_max16(fs);
      const _Float16 rh = (_Float16)(fs / fb);  // a power of two <= 1 (0 below fp16's range)
      ratio = h2_t{rh, rh};
      if ((tid & 15) == 0) fblk[r] = fb;
    }
#pragma unroll
    for (int j = 0; j < V; ++j) {
      uint4 o;
      if (FROM_BF16) {
        const uint32_t w4[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
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
      } else {  // already fp16 in pair order: onto the block's common scale
        o.x = __builtin_bit_cast(uint32_t, as_h2(v[j].x) * ratio);
        o.y = __builtin_bit_cast(uint32_t, as_h2(v[j].y) * ratio);
        o.z = __builtin_bit_cast(uint32_t, as_h2(v[j].z) * ratio);
        o.w = __builtin_bit_cast(uint32_t, as_h2(v[j].w) * ratio);
      }
      *reinterpret_cast<uint4*>(&xs[r][c + 8 * j]) = o;
    }
  }
};

// One K block of one weight row per lane (codes and the (scale, min) words of
// the chunks they fall in).
template <int CHUNK, int KT>
struct WBlock {
  static constexpr int NC = KBlock<KT>::NC;
  static constexpr int NP = (KBlock<KT>::KPL + CHUNK - 1) / CHUNK;  // chunks per lane run
  uint4 c[NC];
  uint32_t p[NP];

  __device__ __forceinline__ void load(const uint8_t* codes_row, const uint8_t* par_row, int kb, int lane) {
    const int k0 = kb + (lane >> 4) * KBlock<KT>::KPL;
#pragma unroll
    for (int j = 0; j < NC; ++j) c[j] = gload16(codes_row + k0 / 2 + 16 * j);
#pragma unroll
    for (int j = 0; j < NP; ++j) p[j] = gload4(par_row + (k0 / CHUNK + j) * 4);
  }
};

// acc += A (16 rows in xs, k order as above) x B (one N tile), one K block.
template <int CHUNK, int KT>
__device__ __forceinline__ void mma_kblock(float4_t& acc, const WBlock<CHUNK, KT>& w, _Float16 (*xs)[KT + 8],
                                           int lane) {
  const int g = lane >> 4, ml = lane & 15;
#pragma unroll
  for (int j = 0; j < KBlock<KT>::NC; ++j) {
    // 32 codes (4 MFMA steps) of this lane; their chunk
    const int pj = (32 * j) / CHUNK;
    h2_t sc, sc16, mn;
    params_f16(w.p[pj], sc, sc16, mn);
    const uint32_t cw[4] = {w.c[j].x, w.c[j].y, w.c[j].z, w.c[j].w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const half8_t av =
          *reinterpret_cast<const half8_t*>(&xs[ml][g * KBlock<KT>::KPL + 32 * j + 8 * t]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, dequant8(cw[t], sc, sc16, mn), acc, 0, 0, 0);
    }
  }
}

// SMOE-Q2: one K block of one weight row per lane, KT / 4 codes (KT / 16
// bytes: one 8-byte load at KT = 128, 16-byte loads above).
template <int CHUNK, int KT>
struct WBlockQ2 {
  static constexpr int KPL = KBlock<KT>::KPL;
  static constexpr int NDW = KPL / 16;                   // code dwords per lane
  static constexpr int NP = (KPL + CHUNK - 1) / CHUNK;   // chunks per lane run
  static_assert(NDW == 2 || NDW % 4 == 0, "K block of 128, 256 or 512 codes");
  uint32_t c[NDW];
  uint32_t p[NP];

  __device__ __forceinline__ void load(const uint8_t* codes_row, const uint8_t* par_row, int kb, int lane) {
    const int k0 = kb + (lane >> 4) * KPL;
    const uint8_t* src = codes_row + k0 / 4;
    if constexpr (NDW == 2) {
      const uint2 v = *reinterpret_cast<const uint2*>(src);
      c[0] = v.x;
      c[1] = v.y;
    } else {
#pragma unroll
      for (int j = 0; j < NDW / 4; ++j) {
        const uint4 v = gload16(src + 16 * j);
        c[4 * j] = v.x;
        c[4 * j + 1] = v.y;
        c[4 * j + 2] = v.z;
        c[4 * j + 3] = v.w;
      }
    }
#pragma unroll
    for (int j = 0; j < NP; ++j) p[j] = gload4(par_row + (k0 / CHUNK + j) * 4);
  }
};

// acc += A x B for an SMOE-Q2 block: code dword t of the lane covers its k
// run's elements 16 t .. 16 t + 15, and the A rows in LDS hold each group of
// 16 in the pair order (e_p, e_{p+8}), so the dword's low and high halves
// meet the 8 A values at 16 t and at 16 t + 8.
template <int CHUNK, int KT>
__device__ __forceinline__ void mma_kblock_q2(float4_t& acc, const WBlockQ2<CHUNK, KT>& w,
                                              _Float16 (*xs)[KT + 8], int lane) {
  const int g = lane >> 4, ml = lane & 15;
#pragma unroll
  for (int t = 0; t < WBlockQ2<CHUNK, KT>::NDW; ++t) {
    const uint32_t p = w.p[(16 * t) / CHUNK];
    const _Float16 sv = (_Float16)__uint_as_float(p << 16);
    const _Float16 sv4 = (_Float16)(__uint_as_float(p << 16) * 0.25f);
    const _Float16 mv = (_Float16)__uint_as_float(p & 0xFFFF0000u);
    const h2_t sc = {sv, sv}, sc4 = {sv4, sv4}, mn = {mv, mv};
    const _Float16* xr = &xs[ml][g * KBlock<KT>::KPL + 16 * t];
    const half8_t a0 = *reinterpret_cast<const half8_t*>(xr);
    const half8_t a1 = *reinterpret_cast<const half8_t*>(xr + 8);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, dequant8_q2(w.c[t], sc, sc4, mn), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, dequant8_q2(w.c[t] >> 8, sc, sc4, mn), acc, 0, 0, 0);
  }
}

// The weight block and MFMA step of code width BITS.
template <int CHUNK, int KT, int BITS>
struct WFormat;
template <int CHUNK, int KT>
struct WFormat<CHUNK, KT, 4> {
  using Block = WBlock<CHUNK, KT>;
  static __device__ __forceinline__ void mma(float4_t& acc, const Block& w, _Float16 (*xs)[KT + 8], int lane) {
    mma_kblock<CHUNK, KT>(acc, w, xs, lane);
  }
};
template <int CHUNK, int KT>
struct WFormat<CHUNK, KT, 2> {
  using Block = WBlockQ2<CHUNK, KT>;
  static __device__ __forceinline__ void mma(float4_t& acc, const Block& w, _Float16 (*xs)[KT + 8], int lane) {
    mma_kblock_q2<CHUNK, KT>(acc, w, xs, lane);
  }
};

struct SliceInfo {
  int u, o, n_rows;
};

__device__ __forceinline__ bool slice_info(const PrefillArgs& a, SliceInfo& si) {
  const int sidx = blockIdx.y;
  if (sidx >= *a.n_slices) return false;
  const int packed = a.slices[sidx];
  si.u = packed >> 8;
  const int q = packed & 255;
  const int o = a.offsets[si.u], n_u = a.offsets[si.u + 1] - o;
  si.o = o + 16 * q;
  si.n_rows = n_u - 16 * q < 16 ? n_u - 16 * q : 16;
  return si.n_rows > 0;
}

template <int CHUNK, int KT>
__global__ __launch_bounds__(256) void prefill_gate_up_kernel(PrefillArgs a) {
  using F = WFormat<CHUNK, KT, 4>;
  __shared__ _Float16 xs[2][16][KT + 8];  // padded rows: conflict-free A reads
  __shared__ int rows[16];
  __shared__ float red[4][16];
  SliceInfo si;
  if (!slice_info(a, si)) return;
  const int e = a.union_ids[si.u];
  if (e < 0 || e >= a.E) return;
  const uint8_t* blob = reinterpret_cast<const uint8_t*>(a.table[e]);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < si.n_rows) rows[tid] = a.perm[si.o + tid] / a.k;  // token of each entry
  __syncthreads();
  const int n0 = blockIdx.x * 64 + wave * 16 + (lane & 15);
  const size_t row_bytes = (size_t)a.d / 2, prow = (size_t)(a.d / CHUNK) * 4;
  const uint8_t* gc = blob + (size_t)n0 * row_bytes;
  const uint8_t* uc = blob + a.lay.up_codes + (size_t)n0 * row_bytes;
  const uint8_t* gp = blob + a.lay.gate_params + (size_t)n0 * prow;
  const uint8_t* up = blob + a.lay.up_params + (size_t)n0 * prow;
  float4_t ag = {0.f, 0.f, 0.f, 0.f}, au = ag;
  const int nk = a.d / KT;
  RowStage<true, KT> xr;
  typename F::Block g0, u0, g1, u1;
  xr.load(a.x, (size_t)a.d, rows, si.n_rows, 0);
  g0.load(gc, gp, 0, lane);
  u0.load(uc, up, 0, lane);
  xr.store(xs[0]);
  __syncthreads();
  for (int i = 0; i < nk; ++i) {
    if (i + 1 < nk) {  // rows first, then weights, of block i + 1
      xr.load(a.x, (size_t)a.d, rows, si.n_rows, (i + 1) * KT);
      g1.load(gc, gp, (i + 1) * KT, lane);
      u1.load(uc, up, (i + 1) * KT, lane);
    }
    F::mma(ag, g0, xs[i & 1], lane);
    F::mma(au, u0, xs[i & 1], lane);
    if (i + 1 < nk) xr.store(xs[(i + 1) & 1]);
    g0 = g1;
    u0 = u1;
    __syncthreads();
  }
  // epilogue: lane holds rows 4 (l / 16) + i of the tile, feature n0
  store_h_tile(a, ag, au, si.o, si.n_rows, pair_index<4>(n0), red);
}

template <int CHUNK, int KT, int BITS = 4>
__global__ __launch_bounds__(256) void prefill_down_kernel(PrefillArgs a) {
  using F = WFormat<CHUNK, KT, BITS>;
  __shared__ _Float16 xs[2][16][KT + 8];
  __shared__ __attribute__((aligned(16))) float fblk[2][16];  // the H rows' scale per K block
  __shared__ int rows[16];
  SliceInfo si;
  if (!slice_info(a, si)) return;
  const int e = a.union_ids[si.u];
  if (e < 0 || e >= a.E) return;
  const uint8_t* blob = reinterpret_cast<const uint8_t*>(a.table[e]);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < si.n_rows) rows[tid] = si.o + tid;  // H rows of this slice
  __syncthreads();
  const int n0 = blockIdx.x * 64 + wave * 16 + (lane & 15);
  const size_t row_bytes = (size_t)a.f * BITS / 8, prow = (size_t)(a.f / CHUNK) * 4;
  const uint8_t* dc = blob + a.lay.down_codes + (size_t)n0 * row_bytes;
  const uint8_t* dp = blob + a.lay.down_params + (size_t)n0 * prow;
  const float4_t zero = {0.f, 0.f, 0.f, 0.f};
  float4_t acc = zero;
  const int nk = a.f / KT, tiles = a.f / 64;
  RowStage<false, KT> hr;
  typename F::Block w0, w1;
  hr.load(a.H, (size_t)a.f, rows, si.n_rows, 0, a.Hs, tiles);
  w0.load(dc, dp, 0, lane);
  hr.store(xs[0], fblk[0]);
  __syncthreads();
  for (int i = 0; i < nk; ++i) {
    if (i + 1 < nk) {
      hr.load(a.H, (size_t)a.f, rows, si.n_rows, (i + 1) * KT, a.Hs, tiles);
      w1.load(dc, dp, (i + 1) * KT, lane);
    }
    float4_t P = zero;  // this block on the rows' common scale, then scaled back
    F::mma(P, w0, xs[i & 1], lane);
    const float4 fb = *reinterpret_cast<const float4*>(&fblk[i & 1][4 * (lane >> 4)]);
    acc[0] = fmaf(fb.x, P[0], acc[0]);
    acc[1] = fmaf(fb.y, P[1], acc[1]);
    acc[2] = fmaf(fb.z, P[2], acc[2]);
    acc[3] = fmaf(fb.w, P[3], acc[3]);
    if (i + 1 < nk) hr.store(xs[(i + 1) & 1], fblk[(i + 1) & 1]);
    w0 = w1;
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * (lane >> 4) + i;
    if (row < si.n_rows) a.Y[(size_t)(si.o + row) * a.d + n0] = acc[i];
  }
}

// ---------------------------------------------------------------------------
// 2-3 (chunk 64).  The same grouped GEMMs with the affine dequant folded per
// chunk instead of applied to every weight: sum_k W x = sum_c (s_c P_c +
// m_c X_c), P_c = sum_{k in c} q x on MFMA over the raw codes, X_c = sum_{k in
// c} x.  A weight then costs two VALU ops per pair of codes less than the
// dequant above (a profile of the kernels above showed them VALU-bound: taking
// the affine step out of their dequant alone cut the prompt time by a fifth).
//
// Raw codes as MFMA inputs: masking a nibble into the low mantissa bits of an
// fp16 half gives the subnormal q * 2^-24 exactly, a nibble at bits 4..7 gives
// 16 q * 2^-24; the odd elements' inputs are staged divided by 16, so every
// product is q x 2^-24 exactly (subnormal fp16 MFMA inputs are kept), and
// s_c 2^24 scales the chunk's fp32 result.
//
// K order: MFMA step t of a K block takes the block's codes 32 t .. 32 t + 31,
// lane group g the eight at 32 t + 8 g, so that two consecutive steps cover one
// chunk.  Lane group g loads 16-byte pieces 4 q + g of its row (whole pieces,
// as before), and a 4x4 dword transpose across the four lane groups hands each
// group its dword of every piece.
// ---------------------------------------------------------------------------

// 4x4 transpose of dwords across the wave's four 16-lane rows: lane n of row
// g holds v[j] = T[g][j] on entry and v[j] = T[j][g] on return.  Rows g = 2a +
// b: v_permlane32_swap exchanges the row pairs (a) on the high bit of j, then
// v_permlane16_swap exchanges odd and even rows (b) on its low bit.
__device__ __forceinline__ void xpose4(uint32_t (&v)[4]) {
  const auto s0 = __builtin_amdgcn_permlane32_swap(v[0], v[2], false, false);
  const auto s1 = __builtin_amdgcn_permlane32_swap(v[1], v[3], false, false);
  v[0] = s0[0]; v[2] = s0[1]; v[1] = s1[0]; v[3] = s1[1];
  const auto t0 = __builtin_amdgcn_permlane16_swap(v[0], v[1], false, false);
  const auto t1 = __builtin_amdgcn_permlane16_swap(v[2], v[3], false, false);
  v[0] = t0[0]; v[1] = t0[1]; v[2] = t1[0]; v[3] = t1[1];
}

// Eight codes (one dword, e_j in bits 4j..4j+3) as the B fragment of one MFMA
// step, pair order (e0, e4, 16 e1, 16 e5, e2, e6, 16 e3, 16 e7) * 2^-24.
__device__ __forceinline__ half8_t codes8(uint32_t w) {
  const uint32_t w8 = w >> 8;
  const uint4 r = make_uint4(w & 0x000F000Fu, w & 0x00F000F0u, w8 & 0x000F000Fu, w8 & 0x00F000F0u);
  return __builtin_bit_cast(half8_t, r);
}

// A slice's 16 H rows (the down GEMM's A operand) for one K block, as fp16
// in pair order with the odd elements divided by 16, and the sum of each
// row's fp16 values over each chunk of 64 (xsum[chunk of the block][row]).
// Thread (r = tid / 16, k = tid % 16) moves pieces 16 j + k of row r (the
// 16 threads of a row read 256 contiguous bytes per load instruction);
// load() and store() are separate so that the loads run a block ahead.  H
// comes with one scale per 64-value tile: the block's tiles are put on one
// common scale per row (the largest tile scale F of the block, a power of
// two; a tile's values are multiplied by its scale / F <= 1, exactly unless
// they fall below the fp16 normal range, where they are at most 2^-24 of the
// block's largest), and F goes to fblk[row], by which the caller multiplies
// the block's result.
template <int KT>
struct FoldStage {
  static constexpr int V = KT / 128;  // 16-byte pieces (8 values) per thread
  uint4 v[V];
  float fs[V];                        // the tile scale of each piece

  __device__ __forceinline__ void load(const _Float16* src, size_t row_elems, const int* rows, int n_rows, int kb,
                                       const float* hs, int tiles) {
    const int tid = threadIdx.x, r = tid >> 4, k = tid & 15;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      v[j] = make_uint4(0, 0, 0, 0);
      fs[j] = 1.0f;
      if (r < n_rows) {
        v[j] = gload16(src + (size_t)rows[r] * row_elems + kb + 8 * (16 * j + k));
        fs[j] = hs[(size_t)rows[r] * tiles + kb / 64 + 2 * j + (k >> 3)];
      }
    }
  }

  __device__ __forceinline__ void store(_Float16 (*xs)[KT + 8], float (*xsum)[16], float* fblk) const {
    const int tid = threadIdx.x, r = tid >> 4, k = tid & 15;
    const uint32_t k16 = 0x2C002C00u;  // (1/16, 1/16) in fp16
    float m = fs[0];
#pragma unroll
    for (int j = 1; j < V; ++j) m = fmaxf(m, fs[j]);
    const float fb = row_max16(m);
    if (k == 0) fblk[r] = fb;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const _Float16 rh = (_Float16)(fs[j] / fb);  // a power of two <= 1 (0 below fp16's range)
      const h2_t ratio = {rh, rh};
      const uint32_t w4[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
      h2_t hv[4];
      float part = 0.f;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        hv[p] = as_h2(w4[p]) * ratio;
        part += (float)hv[p][0] + (float)hv[p][1];
      }
      uint4 o;
      o.x = __builtin_bit_cast(uint32_t, hv[0]);
      o.y = __builtin_bit_cast(uint32_t, hv[1] * as_h2(k16));
      o.z = __builtin_bit_cast(uint32_t, hv[2]);
      o.w = __builtin_bit_cast(uint32_t, hv[3] * as_h2(k16));
      *reinterpret_cast<uint4*>(&xs[r][8 * (16 * j + k)]) = o;
      // a chunk is 8 pieces: threads 8h .. 8h + 7 of the row (adjacent lanes)
      part = group_sum<8>(part);
      if ((k & 7) == 0) xsum[2 * j + (k >> 3)][r] = part;
    }
  }
};

// The chunk's x in the folded gate/up GEMM's A layout, once per call
// (rather than once per slice and feature block): x_a[t][j] as fp16 in pair
// order (dword p of each group of 8 holds e_p, e_{p+4}), the odd dwords
// divided by 16, and x_as[t][c] the sum of chunk c's 64 fp16 values, in the
// order the H stage sums its rows.  grid = (ceil(d / 2048), T), 256 threads;
// thread i owns the 8 values 8 i .. 8 i + 7 of its 2048 (threads past d read
// the row's first piece and store nothing; d is a multiple of 256, so they
// make up whole chunks).
__global__ __launch_bounds__(256) void prefill_stage_x_kernel(PrefillArgs a) {
  const int t = blockIdx.y, piece = blockIdx.x * 256 + threadIdx.x;
  const bool in = 8 * piece < a.d;
  const uint4 v = gload16(a.x + (size_t)t * a.d + (in ? 8 * piece : 0));
  const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
  float f[8];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    f[2 * p] = (float)(_Float16)bf16_to_f32(w4[p] & 0xFFFF);
    f[2 * p + 1] = (float)(_Float16)bf16_to_f32(w4[p] >> 16);
  }
  float part = 0.f;
#pragma unroll
  for (int p = 0; p < 8; ++p) part += f[p];
  uint4 o;
  o.x = f16_bits(f[0]) | (f16_bits(f[4]) << 16);
  o.y = f16_bits(f[1] * 0.0625f) | (f16_bits(f[5] * 0.0625f) << 16);
  o.z = f16_bits(f[2]) | (f16_bits(f[6]) << 16);
  o.w = f16_bits(f[3] * 0.0625f) | (f16_bits(f[7] * 0.0625f) << 16);
  if (in) *reinterpret_cast<uint4*>(a.xa + (size_t)t * a.d + 8 * piece) = o;
  part = group_sum<8>(part);  // a chunk is 8 pieces: 8 adjacent lanes
  if (in && (piece & 7) == 0) a.xas[(size_t)t * (a.d / 64) + piece / 8] = part;
}

// The token rows of a slice for one K block, copied from x_a / x_as (already
// in the A layout) into the workgroup's stage: thread (r, k) moves pieces
// 16 j + k of row r, and the first thread of each chunk its chunk sum.
template <int KT>
struct XCopyStage {
  static constexpr int V = KT / 128;
  uint4 v[V];
  float sum[V];
  __device__ __forceinline__ void load(const PrefillArgs& a, const int* rows, int n_rows, int kb) {
    const int tid = threadIdx.x, r = tid >> 4, k = tid & 15;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      v[j] = make_uint4(0, 0, 0, 0);
      sum[j] = 0.f;
      if (r < n_rows) {
        v[j] = gload16(a.xa + (size_t)rows[r] * a.d + kb + 8 * (16 * j + k));
        if ((k & 7) == 0) sum[j] = a.xas[(size_t)rows[r] * (a.d / 64) + kb / 64 + 2 * j + (k >> 3)];
      }
    }
  }
  __device__ __forceinline__ void store(_Float16 (*xs)[KT + 8], float (*xsum)[16]) const {
    const int tid = threadIdx.x, r = tid >> 4, k = tid & 15;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      *reinterpret_cast<uint4*>(&xs[r][8 * (16 * j + k)]) = v[j];
      if ((k & 7) == 0) xsum[2 * j + (k >> 3)][r] = sum[j];
    }
  }
};

// One K block of one weight row per lane: pieces 4 q + g of the row's codes in
// the block and the (scale, min) words of the block's KT / 64 chunks.
template <int KT>
struct FoldW {
  static constexpr int NL = KT / 128;  // 16-byte code loads per lane
  static constexpr int NPW = KT / 64;  // chunks per block
  static_assert(NPW % 4 == 0, "K blocks of a multiple of 256 codes");
  uint4 c[NL];
  uint4 p[NPW / 4];

  __device__ __forceinline__ void load(const uint8_t* codes_row, const uint8_t* par_row, int kb, int g) {
#pragma unroll
    for (int q = 0; q < NL; ++q) c[q] = gload16(codes_row + kb / 2 + 16 * (4 * q + g));
#pragma unroll
    for (int q = 0; q < NPW / 4; ++q) p[q] = gload16(par_row + (kb / 64) * 4 + 16 * q);
  }
};

// Line-wise loads of one K block of 256 codes for the 16 weight rows of a
// wave: 8 lanes cover one row's 128-byte line, so an instruction reads 8
// whole lines (lane l: row 8 q + l / 8, bytes 16 (l % 8) of the block) rather
// than half lines of 16 rows; relayout() then moves the pieces through the
// wave's LDS stage into the FoldW register layout (lane (n, g): pieces
// 4 q + g of row n).  Rows are 144 bytes apart in the stage (2-way read
// conflicts at most).
constexpr int kLineStageRow = 144;
__device__ __forceinline__ void load_lines256(FoldW<256>& w, const uint8_t* codes_row0, size_t row_bytes,
                                              const uint8_t* par_row, int kb, int lane) {
#pragma unroll
  for (int q = 0; q < 2; ++q)
    w.c[q] = gload16(codes_row0 + (size_t)(8 * q + (lane >> 3)) * row_bytes + kb / 2 + 16 * (lane & 7));
  w.p[0] = gload16(par_row + (kb / 64) * 4);
}
template <class W>
__device__ __forceinline__ void relayout256(W& w, uint8_t* stage, int lane) {
#pragma unroll
  for (int q = 0; q < 2; ++q)
    *reinterpret_cast<uint4*>(stage + (8 * q + (lane >> 3)) * kLineStageRow + 16 * (lane & 7)) = w.c[q];
#pragma unroll
  for (int q = 0; q < 2; ++q)
    w.c[q] = *reinterpret_cast<const uint4*>(stage + (lane & 15) * kLineStageRow + 16 * (4 * q + (lane >> 4)));
}

// acc += sum over the block's chunks of s_c P_c + m_c X_c for this lane's
// column (feature) and its four rows 4 (lane / 16) + i.  All of the block's
// MFMA chains are issued before the first result is folded, so the VALU
// epilogue of one chunk overlaps the MFMAs of the next.  The m_c X_c terms of
// four chunks are one fp32 MFMA (v_mfma_f32_16x16x4f32: X[rows][chunks] times
// m[chunks][columns], accumulated onto the sum), which leaves the VALU one
// FMA per element and chunk, s_c P_c.
// With SCALED, the A rows are H rows on one power-of-two scale per row for
// the block, and the block's sum is multiplied by that scale fblk[row].
template <int KT, bool SCALED = false>
__device__ __forceinline__ void fold_kblock(float4_t& acc, const FoldW<KT>& w, _Float16 (*xs)[KT + 8],
                                            float (*xsum)[16], int lane, const float* fblk = nullptr) {
  constexpr int NC = FoldW<KT>::NPW;
  const int g = lane >> 4, ml = lane & 15, r4 = 4 * (lane >> 4);
  const float4_t zero = {0.f, 0.f, 0.f, 0.f};
  float4_t P[NC];
#pragma unroll
  for (int q = 0; q < FoldW<KT>::NL; ++q) {
    uint32_t u[4] = {w.c[q].x, w.c[q].y, w.c[q].z, w.c[q].w};
    xpose4(u);  // u[j] = dword g of piece 4 q + j: the codes of step 4 q + j
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t0 = 4 * q + 2 * h, cl = 2 * q + h;  // steps t0, t0 + 1 = chunk cl of the block
      const half8_t a0 = *reinterpret_cast<const half8_t*>(&xs[ml][32 * t0 + 8 * g]);
      const half8_t a1 = *reinterpret_cast<const half8_t*>(&xs[ml][32 * t0 + 32 + 8 * g]);
      P[cl] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, codes8(u[2 * h]), zero, 0, 0, 0);
      P[cl] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, codes8(u[2 * h + 1]), P[cl], 0, 0, 0);
    }
  }
  float4_t blk = zero;
  float4_t& sum = SCALED ? blk : acc;  // the block's sum, scaled once at the end
  // the min terms of four chunks at a time as one fp32 MFMA: lane (g, ml)
  // gives X[chunk g][row ml] and m[chunk g][its column]
#pragma unroll
  for (int c4 = 0; c4 < NC / 4; ++c4) {
    const uint4 pw = w.p[c4];
    const uint32_t pm = g == 0 ? pw.x : g == 1 ? pw.y : g == 2 ? pw.z : pw.w;
    sum = __builtin_amdgcn_mfma_f32_16x16x4f32(xsum[4 * c4 + g][ml], __uint_as_float(pm & 0xFFFF0000u), sum, 0, 0, 0);
  }
#pragma unroll
  for (int cl = 0; cl < NC; ++cl) {
    const uint4 pw = w.p[cl >> 2];
    const uint32_t prm = (cl & 3) == 0 ? pw.x : (cl & 3) == 1 ? pw.y : (cl & 3) == 2 ? pw.z : pw.w;
    const float S = __uint_as_float(prm << 16) * 16777216.0f;  // scale * 2^24
    sum[0] = fmaf(S, P[cl][0], sum[0]);
    sum[1] = fmaf(S, P[cl][1], sum[1]);
    sum[2] = fmaf(S, P[cl][2], sum[2]);
    sum[3] = fmaf(S, P[cl][3], sum[3]);
  }
  if constexpr (SCALED) {
    const float4 F = *reinterpret_cast<const float4*>(&fblk[r4]);
    acc[0] = fmaf(F.x, blk[0], acc[0]);
    acc[1] = fmaf(F.y, blk[1], acc[1]);
    acc[2] = fmaf(F.z, blk[2], acc[2]);
    acc[3] = fmaf(F.w, blk[3], acc[3]);
  }
}

template <int KT>
__global__ __launch_bounds__(256, 3) void prefill_gate_up_fold_kernel(PrefillArgs a) {
  __shared__ _Float16 xs[2][16][KT + 8];  // padded rows: conflict-free A reads
  __shared__ __attribute__((aligned(16))) float xsum[2][KT / 64][16];
  __shared__ int rows[16];
  __shared__ float red[4][16];
  __shared__ __attribute__((aligned(16))) uint8_t wst[4][2][16 * kLineStageRow];
  // the slice's record (written by the union kernel) and the slice count are
  // independent loads: one round trip before the weights stream
  const int n_slices = *a.n_slices;
  const PrefillArgs::SliceRec rec = a.recs[blockIdx.y];
  if ((int)blockIdx.y >= n_slices || !rec.blob) return;
  SliceInfo si;
  si.o = rec.o;
  si.n_rows = rec.n_rows;
  const uint8_t* blob = reinterpret_cast<const uint8_t*>(rec.blob);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4;
  const int n0 = blockIdx.x * 64 + wave * 16 + (lane & 15);
  const size_t row_bytes = (size_t)a.d / 2, prow = (size_t)(a.d / 64) * 4;
  const uint8_t* gp = blob + a.lay.gate_params + (size_t)n0 * prow;
  const uint8_t* up = blob + a.lay.up_params + (size_t)n0 * prow;
  float4_t ag = {0.f, 0.f, 0.f, 0.f}, au = ag;
  const int nk = a.d / KT;
  XCopyStage<KT> xr;  // the token rows, staged once per call by prefill_stage_x_kernel
  FoldW<KT> g0, u0, g1, u1;
  const size_t nw0 = (size_t)(blockIdx.x * 64 + wave * 16) * row_bytes;  // the wave's first row
  const uint8_t* gc0 = blob + nw0;
  const uint8_t* uc0 = blob + a.lay.up_codes + nw0;
  uint8_t* gst = wst[wave][0];
  uint8_t* ust = wst[wave][1];
  load_lines256(g0, gc0, row_bytes, gp, 0, lane);  // the first weights go out before the token lookup
  load_lines256(u0, uc0, row_bytes, up, 0, lane);
  if (tid < si.n_rows) rows[tid] = a.perm[si.o + tid] / a.k;  // token of each entry
  __syncthreads();
  xr.load(a, rows, si.n_rows, 0);
  xr.store(xs[0], xsum[0]);
  __syncthreads();
  for (int i = 0; i < nk; ++i) {
    if (i + 1 < nk) {  // rows first, then weights, of block i + 1
      xr.load(a, rows, si.n_rows, (i + 1) * KT);
      load_lines256(g1, gc0, row_bytes, gp, (i + 1) * KT, lane);
      load_lines256(u1, uc0, row_bytes, up, (i + 1) * KT, lane);
    }
    // block i's weights were loaded one iteration ago: re-laid only now, so
    // that their loads have a whole iteration to land
    relayout256(g0, gst, lane);
    relayout256(u0, ust, lane);
    fold_kblock<KT>(ag, g0, xs[i & 1], xsum[i & 1], lane);
    fold_kblock<KT>(au, u0, xs[i & 1], xsum[i & 1], lane);
    if (i + 1 < nk) xr.store(xs[(i + 1) & 1], xsum[(i + 1) & 1]);
    g0 = g1;
    u0 = u1;
    __syncthreads();
  }
  store_h_tile(a, ag, au, si.o, si.n_rows, pair_index<4>(n0), red);
}

// Y = H x D^T for one slice, folded per chunk like the gate/up GEMM.  A
// workgroup computes two 64-column tiles of the slice's 16 rows (each wave 16
// columns of each), so the H rows it stages in LDS per K block serve 128
// output columns: half the H gathers, conversions, barriers and workgroup
// prologues of one tile per workgroup.  Grid (d_model / 128, max slices);
// occupancy 3 is held by a launch bound (one tile: 102 registers, occupancy
// 4, and slower).
template <int KT>
__global__ __launch_bounds__(256, 3) void prefill_down_fold_kernel(PrefillArgs a) {
  constexpr int NT = 2;  // 64-column tiles per workgroup
  __shared__ _Float16 xs[2][16][KT + 8];
  __shared__ __attribute__((aligned(16))) float xsum[2][KT / 64][16];
  __shared__ __attribute__((aligned(16))) float fblk[2][16];  // the blocks' common H scales
  __shared__ int rows[16];
  __shared__ __attribute__((aligned(16))) uint8_t wst[4][NT][16 * kLineStageRow];
  const int n_slices = *a.n_slices;
  const PrefillArgs::SliceRec rec = a.recs[blockIdx.y];
  if ((int)blockIdx.y >= n_slices || !rec.blob) return;
  SliceInfo si;
  si.o = rec.o;
  si.n_rows = rec.n_rows;
  const uint8_t* blob = reinterpret_cast<const uint8_t*>(rec.blob);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t row_bytes = (size_t)a.f / 2, prow = (size_t)(a.f / 64) * 4;
  int n0[NT];
  const uint8_t* dp[NT];
  const uint8_t* dc0[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int c0 = blockIdx.x * 64 * NT + t * 64 + wave * 16;
    n0[t] = c0 + (lane & 15);
    dp[t] = blob + a.lay.down_params + (size_t)n0[t] * prow;
    dc0[t] = blob + a.lay.down_codes + (size_t)c0 * row_bytes;
  }
  float4_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = float4_t{0.f, 0.f, 0.f, 0.f};
  const int nk = a.f / KT;
  FoldStage<KT> hr;
  FoldW<KT> w0[NT], w1[NT];
  const int tiles = a.f / 64;
#pragma unroll
  for (int t = 0; t < NT; ++t) load_lines256(w0[t], dc0[t], row_bytes, dp[t], 0, lane);
  if (tid < si.n_rows) rows[tid] = si.o + tid;  // H rows of this slice
  __syncthreads();
  hr.load(a.H, (size_t)a.f, rows, si.n_rows, 0, a.Hs, tiles);
  hr.store(xs[0], xsum[0], fblk[0]);
  __syncthreads();
  for (int i = 0; i < nk; ++i) {
    if (i + 1 < nk) {
      hr.load(a.H, (size_t)a.f, rows, si.n_rows, (i + 1) * KT, a.Hs, tiles);
#pragma unroll
      for (int t = 0; t < NT; ++t) load_lines256(w1[t], dc0[t], row_bytes, dp[t], (i + 1) * KT, lane);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) relayout256(w0[t], wst[wave][t], lane);  // block i, loaded one iteration ago
#pragma unroll
    for (int t = 0; t < NT; ++t) fold_kblock<KT, true>(acc[t], w0[t], xs[i & 1], xsum[i & 1], lane, fblk[i & 1]);
    if (i + 1 < nk) hr.store(xs[(i + 1) & 1], xsum[(i + 1) & 1], fblk[(i + 1) & 1]);
#pragma unroll
    for (int t = 0; t < NT; ++t) w0[t] = w1[t];
    __syncthreads();
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * (lane >> 4) + i;
      if (row < si.n_rows) a.Y[(size_t)(si.o + row) * a.d + n0[t]] = acc[t][i];
    }
}

// ---------------------------------------------------------------------------
// 2-3 for SMOE-Q2 blobs: the chunk fold above on 2-bit codes.  A K block is
// 512 codes, one 128-byte line per row and eight chunks: each 16-byte piece
// of the line is one chunk, so the line-wise loads, the LDS relayout and the
// 4x4 transpose above serve unchanged, and after the transpose lane group g
// holds dword g (the chunk's elements 16 g .. 16 g + 15) of every chunk.
// Masking a code at bits 2..3 of a byte gives 4 q 2^-24, so the odd elements'
// inputs are staged divided by 4.  Token rows and H are in the pair order of
// groups of 16 (dword p of a group = (e_p, e_{p+8})): MFMA step (chunk c, half
// h) takes from lane group g the A values at 64 c + 16 g + 8 h and the codes
// of the low (h = 0) or high half of its dword.
// ---------------------------------------------------------------------------

// Codes (e0, e8, 4 e1, 4 e9, e2, e10, 4 e3, 4 e11) * 2^-24 of a code dword
// (the caller passes the dword shifted right by 8 for e4..e7, e12..e15).
__device__ __forceinline__ half8_t codes8_q2(uint32_t w) {
  const uint32_t w4 = w >> 4;
  const uint4 r = make_uint4(w & 0x00030003u, w & 0x000C000Cu, w4 & 0x00030003u, w4 & 0x000C000Cu);
  return __builtin_bit_cast(half8_t, r);
}

// A slice's 16 H rows (the down GEMM's A operand) for one K block of 512 as
// fp16 in the 16-group pair order, the odd elements divided by 4, and each
// row's sum over each chunk of 64 (xsum[chunk of the block][row]).  Thread
// (r = tid / 16, k = tid % 16) takes the groups 16 j + k (two adjacent
// 16-byte pieces each) of row r; a chunk's four groups sit in four adjacent
// lanes.  The block's tiles are put on one common scale per row, as for the
// SMOE-Q4 H stage, and that scale goes to fblk[row].
struct FoldStageQ2 {
  uint4 v[4];
  float fs[2];  // the tile scale of each group pair's chunk

  __device__ __forceinline__ void load(const _Float16* src, size_t row_elems, const int* rows, int n_rows, int kb,
                                       const float* hs, int tiles) {
    const int tid = threadIdx.x, r = tid >> 4, k = tid & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = make_uint4(0, 0, 0, 0);
      if (r < n_rows) v[i] = gload16(src + (size_t)rows[r] * row_elems + kb + 16 * (16 * (i >> 1) + k) + 8 * (i & 1));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      fs[j] = 1.0f;
      if (r < n_rows) fs[j] = hs[(size_t)rows[r] * tiles + kb / 64 + 4 * j + (k >> 2)];
    }
  }

  __device__ __forceinline__ void store(_Float16 (*xs)[512 + 8], float (*xsum)[16], float* fblk) const {
    const int tid = threadIdx.x, r = tid >> 4, k = tid & 15;
    const uint32_t k4 = 0x34003400u;  // (1/4, 1/4) in fp16
    const float fb = row_max16(fmaxf(fs[0], fs[1]));
    if (k == 0) fblk[r] = fb;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      // onto the common scale, the odd dwords divided by 4
      const _Float16 rh = (_Float16)(fs[j] / fb);  // a power of two <= 1 (0 below fp16's range)
      const h2_t ratio = {rh, rh};
      const uint32_t w8[8] = {v[2 * j].x, v[2 * j].y, v[2 * j].z, v[2 * j].w,
                              v[2 * j + 1].x, v[2 * j + 1].y, v[2 * j + 1].z, v[2 * j + 1].w};
      uint32_t q[8];
      float part = 0.f;
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const h2_t hv = as_h2(w8[p]) * ratio;
        part += (float)hv[0] + (float)hv[1];
        q[p] = __builtin_bit_cast(uint32_t, (p & 1) ? hv * as_h2(k4) : hv);
      }
      *reinterpret_cast<uint4*>(&xs[r][16 * (16 * j + k)]) = make_uint4(q[0], q[1], q[2], q[3]);
      *reinterpret_cast<uint4*>(&xs[r][16 * (16 * j + k) + 8]) = make_uint4(q[4], q[5], q[6], q[7]);
      part = group_sum<4>(part);
      if ((k & 3) == 0) xsum[4 * j + (k >> 2)][r] = part;
    }
  }
};

// One K block (512 codes) of one weight row per lane after the relayout:
// pieces (= chunks) 4 q + g, and the (scale, min) words of the block's eight
// chunks.
// SMOE-Q2's A layout of the chunk's x, once per call: groups of 16 in pair
// order (dword p holds e_p, e_{p+8}), the odd dwords divided by 4, and the
// chunk sums, in the order the H stage forms them.  grid = (ceil(d / 4096), T), 256
// threads; thread i owns the 16 values 16 i .. 16 i + 15 of its 4096 (d is a
// multiple of 512 for SMOE-Q2, so the threads past d make up whole chunks).
__global__ __launch_bounds__(256) void prefill_stage_x_q2_kernel(PrefillArgs a) {
  const int t = blockIdx.y, piece = blockIdx.x * 256 + threadIdx.x;
  const bool in = 16 * piece < a.d;
  const uint16_t* src = a.x + (size_t)t * a.d + (in ? 16 * piece : 0);
  const uint4 v0 = gload16(src), v1 = gload16(src + 8);
  const uint32_t w8[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  float f[16];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    f[2 * p] = (float)(_Float16)bf16_to_f32(w8[p] & 0xFFFF);
    f[2 * p + 1] = (float)(_Float16)bf16_to_f32(w8[p] >> 16);
  }
  float part = 0.f;
#pragma unroll
  for (int p = 0; p < 16; ++p) part += f[p];
  uint4 o0, o1;
  o0.x = f16_bits(f[0]) | (f16_bits(f[8]) << 16);
  o0.y = f16_bits(f[1] * 0.25f) | (f16_bits(f[9] * 0.25f) << 16);
  o0.z = f16_bits(f[2]) | (f16_bits(f[10]) << 16);
  o0.w = f16_bits(f[3] * 0.25f) | (f16_bits(f[11] * 0.25f) << 16);
  o1.x = f16_bits(f[4]) | (f16_bits(f[12]) << 16);
  o1.y = f16_bits(f[5] * 0.25f) | (f16_bits(f[13] * 0.25f) << 16);
  o1.z = f16_bits(f[6]) | (f16_bits(f[14]) << 16);
  o1.w = f16_bits(f[7] * 0.25f) | (f16_bits(f[15] * 0.25f) << 16);
  if (in) {
    _Float16* dst = a.xa + (size_t)t * a.d + 16 * piece;
    *reinterpret_cast<uint4*>(dst) = o0;
    *reinterpret_cast<uint4*>(dst + 8) = o1;
  }
  part = group_sum<4>(part);  // a chunk is 4 groups of 16: 4 adjacent lanes
  if (in && (piece & 3) == 0) a.xas[(size_t)t * (a.d / 64) + piece / 4] = part;
}

// The slice's token rows for one K block of 512, copied from x_a / x_as.
struct XCopyStageQ2 {
  uint4 v[4];
  float sum[2];
  __device__ __forceinline__ void load(const PrefillArgs& a, const int* rows, int n_rows, int kb) {
    const int tid = threadIdx.x, r = tid >> 4, k = tid & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = make_uint4(0, 0, 0, 0);
      if (r < n_rows) v[i] = gload16(a.xa + (size_t)rows[r] * a.d + kb + 16 * (16 * (i >> 1) + k) + 8 * (i & 1));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      sum[j] = 0.f;
      if (r < n_rows && (k & 3) == 0) sum[j] = a.xas[(size_t)rows[r] * (a.d / 64) + kb / 64 + 4 * j + (k >> 2)];
    }
  }
  __device__ __forceinline__ void store(_Float16 (*xs)[512 + 8], float (*xsum)[16]) const {
    const int tid = threadIdx.x, r = tid >> 4, k = tid & 15;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      *reinterpret_cast<uint4*>(&xs[r][16 * (16 * j + k)]) = v[2 * j];
      *reinterpret_cast<uint4*>(&xs[r][16 * (16 * j + k) + 8]) = v[2 * j + 1];
      if ((k & 3) == 0) xsum[4 * j + (k >> 2)][r] = sum[j];
    }
  }
};

struct FoldWQ2 {
  uint4 c[2];
  uint4 p[2];
};

// Line-wise loads of one K block for the 16 rows of a wave (as load_lines256).
__device__ __forceinline__ void load_lines_q2(FoldWQ2& w, const uint8_t* codes_row0, size_t row_bytes,
                                              const uint8_t* par_row, int kb, int lane) {
#pragma unroll
  for (int q = 0; q < 2; ++q)
    w.c[q] = gload16(codes_row0 + (size_t)(8 * q + (lane >> 3)) * row_bytes + kb / 4 + 16 * (lane & 7));
#pragma unroll
  for (int q = 0; q < 2; ++q) w.p[q] = gload16(par_row + (kb / 64) * 4 + 16 * q);
}

// acc += sum over the block's eight chunks of s_c P_c + m_c X_c, four chunks
// (one transposed piece row) at a time: their MFMA chains first, then the
// folds.
template <bool SCALED = false>
__device__ __forceinline__ void fold_kblock_q2(float4_t& acc, const FoldWQ2& w, _Float16 (*xs)[512 + 8],
                                               float (*xsum)[16], int lane, const float* fblk = nullptr) {
  const int g = lane >> 4, ml = lane & 15, r4 = 4 * (lane >> 4);
  const float4_t zero = {0.f, 0.f, 0.f, 0.f};
  float4_t blk = zero;
  float4_t& sum = SCALED ? blk : acc;  // the block's sum, scaled once at the end
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    uint32_t u[4] = {w.c[q].x, w.c[q].y, w.c[q].z, w.c[q].w};
    xpose4(u);  // u[j] = dword g of chunk 4 q + j
    float4_t P[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const _Float16* xr = &xs[ml][64 * (4 * q + j) + 16 * g];
      const half8_t a0 = *reinterpret_cast<const half8_t*>(xr);
      const half8_t a1 = *reinterpret_cast<const half8_t*>(xr + 8);
      P[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, codes8_q2(u[j]), zero, 0, 0, 0);
      P[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, codes8_q2(u[j] >> 8), P[j], 0, 0, 0);
    }
    const uint32_t pw[4] = {w.p[q].x, w.p[q].y, w.p[q].z, w.p[q].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float S = __uint_as_float(pw[j] << 16) * 16777216.0f;  // scale * 2^24
      const float M = __uint_as_float(pw[j] & 0xFFFF0000u);
      const float4 X = *reinterpret_cast<const float4*>(&xsum[4 * q + j][r4]);
      sum[0] = fmaf(S, P[j][0], fmaf(M, X.x, sum[0]));
      sum[1] = fmaf(S, P[j][1], fmaf(M, X.y, sum[1]));
      sum[2] = fmaf(S, P[j][2], fmaf(M, X.z, sum[2]));
      sum[3] = fmaf(S, P[j][3], fmaf(M, X.w, sum[3]));
    }
  }
  if constexpr (SCALED) {
    const float4 F = *reinterpret_cast<const float4*>(&fblk[r4]);
    acc[0] = fmaf(F.x, blk[0], acc[0]);
    acc[1] = fmaf(F.y, blk[1], acc[1]);
    acc[2] = fmaf(F.z, blk[2], acc[2]);
    acc[3] = fmaf(F.w, blk[3], acc[3]);
  }
}

__global__ __launch_bounds__(256, 2) void prefill_gate_up_fold_q2_kernel(PrefillArgs a) {
  constexpr int KT = 512;
  __shared__ _Float16 xs[2][16][KT + 8];
  __shared__ __attribute__((aligned(16))) float xsum[2][KT / 64][16];
  __shared__ int rows[16];
  __shared__ float red[4][16];
  __shared__ __attribute__((aligned(16))) uint8_t wst[4][2][16 * kLineStageRow];
  const int n_slices = *a.n_slices;
  const PrefillArgs::SliceRec rec = a.recs[blockIdx.y];
  if ((int)blockIdx.y >= n_slices || !rec.blob) return;
  const int o = rec.o, n_rows = rec.n_rows;
  const uint8_t* blob = reinterpret_cast<const uint8_t*>(rec.blob);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * 64 + wave * 16 + (lane & 15);
  const size_t row_bytes = (size_t)a.d / 4, prow = (size_t)(a.d / 64) * 4;
  const uint8_t* gp = blob + a.lay.gate_params + (size_t)n0 * prow;
  const uint8_t* up = blob + a.lay.up_params + (size_t)n0 * prow;
  float4_t ag = {0.f, 0.f, 0.f, 0.f}, au = ag;
  const int nk = a.d / KT;
  XCopyStageQ2 xr;  // the token rows, staged once per call by prefill_stage_x_q2_kernel
  FoldWQ2 g0, u0, g1, u1;
  const size_t nw0 = (size_t)(blockIdx.x * 64 + wave * 16) * row_bytes;  // the wave's first row
  const uint8_t* gc0 = blob + nw0;  // gate codes start the blob
  const uint8_t* uc0 = blob + a.lay.up_codes + nw0;
  uint8_t* gst = wst[wave][0];
  uint8_t* ust = wst[wave][1];
  load_lines_q2(g0, gc0, row_bytes, gp, 0, lane);
  load_lines_q2(u0, uc0, row_bytes, up, 0, lane);
  if (tid < n_rows) rows[tid] = a.perm[o + tid] / a.k;  // token of each entry
  __syncthreads();
  xr.load(a, rows, n_rows, 0);
  xr.store(xs[0], xsum[0]);
  __syncthreads();
  for (int i = 0; i < nk; ++i) {
    if (i + 1 < nk) {
      xr.load(a, rows, n_rows, (i + 1) * KT);
      load_lines_q2(g1, gc0, row_bytes, gp, (i + 1) * KT, lane);
      load_lines_q2(u1, uc0, row_bytes, up, (i + 1) * KT, lane);
    }
    relayout256(g0, gst, lane);  // block i, loaded one iteration ago
    relayout256(u0, ust, lane);
    fold_kblock_q2(ag, g0, xs[i & 1], xsum[i & 1], lane);
    fold_kblock_q2(au, u0, xs[i & 1], xsum[i & 1], lane);
    if (i + 1 < nk) xr.store(xs[(i + 1) & 1], xsum[(i + 1) & 1]);
    g0 = g1;
    u0 = u1;
    __syncthreads();
  }
  store_h_tile(a, ag, au, o, n_rows, pair_index<2>(n0), red);
}

__global__ __launch_bounds__(256) void prefill_down_fold_q2_kernel(PrefillArgs a) {
  constexpr int KT = 512;
  __shared__ _Float16 xs[2][16][KT + 8];
  __shared__ __attribute__((aligned(16))) float xsum[2][KT / 64][16];
  __shared__ __attribute__((aligned(16))) float fblk[2][16];  // the blocks' common H scales
  __shared__ int rows[16];
  __shared__ __attribute__((aligned(16))) uint8_t wst[4][16 * kLineStageRow];
  const int n_slices = *a.n_slices;
  const PrefillArgs::SliceRec rec = a.recs[blockIdx.y];
  if ((int)blockIdx.y >= n_slices || !rec.blob) return;
  const int o = rec.o, n_rows = rec.n_rows;
  const uint8_t* blob = reinterpret_cast<const uint8_t*>(rec.blob);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * 64 + wave * 16 + (lane & 15);
  const size_t row_bytes = (size_t)a.f / 4, prow = (size_t)(a.f / 64) * 4;
  const uint8_t* dp = blob + a.lay.down_params + (size_t)n0 * prow;
  const uint8_t* dc0 = blob + a.lay.down_codes + (size_t)(blockIdx.x * 64 + wave * 16) * row_bytes;
  uint8_t* dst = wst[wave];
  float4_t acc = {0.f, 0.f, 0.f, 0.f};
  const int nk = a.f / KT;
  FoldStageQ2 hr;
  FoldWQ2 w0, w1;
  const int tiles = a.f / 64;
  load_lines_q2(w0, dc0, row_bytes, dp, 0, lane);
  if (tid < n_rows) rows[tid] = o + tid;  // H rows of this slice
  __syncthreads();
  hr.load(a.H, (size_t)a.f, rows, n_rows, 0, a.Hs, tiles);
  hr.store(xs[0], xsum[0], fblk[0]);
  __syncthreads();
  for (int i = 0; i < nk; ++i) {
    if (i + 1 < nk) {
      hr.load(a.H, (size_t)a.f, rows, n_rows, (i + 1) * KT, a.Hs, tiles);
      load_lines_q2(w1, dc0, row_bytes, dp, (i + 1) * KT, lane);
    }
    relayout256(w0, dst, lane);  // block i, loaded one iteration ago
    fold_kblock_q2<true>(acc, w0, xs[i & 1], xsum[i & 1], lane, fblk[i & 1]);
    if (i + 1 < nk) hr.store(xs[(i + 1) & 1], xsum[(i + 1) & 1], fblk[(i + 1) & 1]);
    w0 = w1;
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * (lane >> 4) + i;
    if (row < n_rows) a.Y[(size_t)(o + row) * a.d + n0] = acc[i];
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

#ifndef SMOE_PF_GU_KT
#define SMOE_PF_GU_KT 256  // K block of the gate/up GEMM (codes per row per block)
#endif
#ifndef SMOE_PF_DN_KT
#define SMOE_PF_DN_KT 512  // K block of the down GEMM
#endif

// Launch on s, bracketed by start/stop events when ev0 is not null.
#define SMOE_PF_LAUNCH(K, GRID, BLOCK, S, EV0, EV1, ...)                                      \
  do {                                                                                     \
    if (EV0) hipExtLaunchKernelGGL(K, GRID, BLOCK, 0, S, EV0, EV1, 0, __VA_ARGS__);           \
    else hipLaunchKernelGGL(K, GRID, BLOCK, 0, S, __VA_ARGS__);                              \
  } while (0)

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s, const hipEvent_t* ev) {
  // events 0/1 bracket the gate/up GEMM, 2/3 the down GEMM
  const hipEvent_t g0 = ev ? ev[0] : nullptr, g1 = ev ? ev[1] : nullptr;
  const hipEvent_t d0 = ev ? ev[2] : nullptr, d1 = ev ? ev[3] : nullptr;
  hipLaunchKernelGGL(prefill_union_kernel, dim3(1), dim3(1024), 0, s, a);
  const int ms = prefill_max_slices(a.T, a.k, a.E);
  const dim3 gu(a.f / 64, ms), dn(a.d / 64, ms);
  // K blocks of 256 codes for gate/up (two matrices in registers), 512 for
  // down, when K allows (runs of 128 / 256 bytes per row); else 128
  constexpr int GKT = SMOE_PF_GU_KT, DKT = SMOE_PF_DN_KT;
  if (a.bits == 2) {  // SMOE-Q2 (chunk 64, d_model a multiple of 512): folded per chunk in K
    // blocks of 512; a d_ff that is not a multiple of 512 takes the fp16-dequant down GEMM
    hipLaunchKernelGGL(prefill_stage_x_q2_kernel, dim3((a.d + 4095) / 4096, a.T), dim3(256), 0, s, a);
    SMOE_PF_LAUNCH(prefill_gate_up_fold_q2_kernel, gu, dim3(256), s, g0, g1, a);
    if (a.f % 512 == 0) SMOE_PF_LAUNCH(prefill_down_fold_q2_kernel, dn, dim3(256), s, d0, d1, a);
    else if (a.f % 256 == 0) SMOE_PF_LAUNCH((prefill_down_kernel<64, 256, 2>), dn, dim3(256), s, d0, d1, a);
    else SMOE_PF_LAUNCH((prefill_down_kernel<64, 128, 2>), dn, dim3(256), s, d0, d1, a);
  } else if (a.chunk == 64 && a.d % 256 == 0 && a.f % 256 == 0) {  // affine folded per chunk
    hipLaunchKernelGGL(prefill_stage_x_kernel, dim3((a.d + 2047) / 2048, a.T), dim3(256), 0, s, a);
    SMOE_PF_LAUNCH((prefill_gate_up_fold_kernel<256>), gu, dim3(256), s, g0, g1, a);
    // K blocks of 256 for the down GEMM too (512 measured slower)
    SMOE_PF_LAUNCH((prefill_down_fold_kernel<256>), dim3(a.d / 128, ms), dim3(256), s, d0, d1, a);
  } else if (a.chunk == 64) {
    if (a.d % GKT == 0) SMOE_PF_LAUNCH((prefill_gate_up_kernel<64, GKT>), gu, dim3(256), s, g0, g1, a);
    else SMOE_PF_LAUNCH((prefill_gate_up_kernel<64, 128>), gu, dim3(256), s, g0, g1, a);
    if (a.f % DKT == 0) SMOE_PF_LAUNCH((prefill_down_kernel<64, DKT>), dn, dim3(256), s, d0, d1, a);
    else SMOE_PF_LAUNCH((prefill_down_kernel<64, 128>), dn, dim3(256), s, d0, d1, a);
  } else {
    if (a.d % GKT == 0) SMOE_PF_LAUNCH((prefill_gate_up_kernel<32, GKT>), gu, dim3(256), s, g0, g1, a);
    else SMOE_PF_LAUNCH((prefill_gate_up_kernel<32, 128>), gu, dim3(256), s, g0, g1, a);
    if (a.f % DKT == 0) SMOE_PF_LAUNCH((prefill_down_kernel<32, DKT>), dn, dim3(256), s, d0, d1, a);
    else SMOE_PF_LAUNCH((prefill_down_kernel<32, 128>), dn, dim3(256), s, d0, d1, a);
  }
  hipLaunchKernelGGL(prefill_combine_kernel, dim3((a.d + 255) / 256, a.T), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace smoe
