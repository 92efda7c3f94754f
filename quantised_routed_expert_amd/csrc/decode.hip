// Decode-time fused SMOE-Q4 expert FFN (one token, k routed experts).
//
// "Coalesced GPU Kernels -- Expert FFN and Dense Matvec" (Optimizations page):
// the expert FFN dequantises 4-bit codes with a per-chunk affine epilogue and
// computes gate and up in one pass, then the down projection; the System
// Overview step table adds the gate-weighted sum into the residual.  The pages'
// Metal design (one 32-lane simdgroup per output row, input staged per 8-row
// threadgroup) is prior art; on gfx950 a row is split over LR lanes of a
// wave64, each lane loading NSEG 16-byte segments of packed nibbles
// (global_load_dwordx4), the input held in registers as f16 pairs for
// v_dot2_f32_f16, and rows reduced with DPP.  Segment s of lane li sits at
// byte s * LR * 16 + li * 16 of the row, so the LR lanes of one load
// instruction read LR * 16 contiguous bytes (whole cache lines); a lane-major
// run (each lane NSEG adjacent segments) makes every instruction touch each
// line of the row at half width, which measured markedly slower.
//
// Affine folding: a 16-byte segment (32 Q4 or 64 Q2 codes) lies inside one
// chunk, so its contribution is scale * sum(q x) + min * sum(x); sum(x) over
// the segment is computed once per wave because every row of a wave uses the
// same columns.  The code width BITS (4: SMOE-Q4, 2: SMOE-Q2, the halved blobs
// of the Optimizations page's "Q2 Vaults") is a template parameter: a Q2
// segment holds twice the values, read in 16-value pair groups.
#include <hip/hip_ext.h>

#include "kernels.h"

#ifndef SMOE_GU_WAVES
#define SMOE_GU_WAVES 4        // waves per gate/up workgroup (a multiple of 2)
#endif
// every gate/up thread stages one logit and one blob pointer of the layer
static_assert(64 * SMOE_GU_WAVES == smoe::kMaxExperts, "a gate/up workgroup has one thread per expert slot");
#ifndef SMOE_GU_ROWS_MAX
#define SMOE_GU_ROWS_MAX 4     // rows per wave of the gate/up kernel (upper bound)
#endif
#ifndef SMOE_GU_MIN_WAVES
#define SMOE_GU_MIN_WAVES 2048 // keep at least this many waves per gate/up launch
#endif
#ifndef SMOE_DN_PASSES_MAX
#define SMOE_DN_PASSES_MAX 8   // row passes per wave of the down kernel (upper bound)
#endif
#ifndef SMOE_DN_MIN_WG
#define SMOE_DN_MIN_WG 256     // keep at least this many down workgroups
#endif

namespace smoe {

// Per-lane layout of one row: lane li owns the NSEG 16-byte code segments at
// row bytes s * STRIDE + li * 16 (s < NSEG) and the (scale, min) record of the
// chunk each falls in.  A segment (SEGV codes) never straddles a chunk (a chunk
// holds >= 16 code bytes), and two segments of a lane are STRIDE >= 32 bytes
// apart, so each has its own record.
template <int LR, int CHUNK, int BITS>
struct LaneRun {
  static constexpr int STRIDE = LR * 16;      // bytes between a lane's segments
  static constexpr int CB = CHUNK * BITS / 8; // code bytes per chunk
  static constexpr int SEGV = 128 / BITS;     // values per segment
  static constexpr int NQ = SEGV / 8;         // 16-byte pieces of a segment's 16-bit inputs
  static constexpr int NDW = SEGV / 2;        // f16-pair dwords per segment
  static_assert(CB >= 16 && CB % 16 == 0, "a segment must lie inside one chunk");
  __device__ static int chunk_of(int li, int s) { return (s * STRIDE + li * 16) / CB; }
};

// Pair-ordered f16 input of a lane's NSEG segments (SEGV values each, the
// columns of its code segments: SEGV * (s * LR + li) onwards) and the
// per-segment sums, from bf16 or pair-ordered f16 storage (x), or fp32 (h,
// below).  The raw loads are separate from the conversion so that the weight
// loads can be issued in between.  `base` points at the lane's first segment;
// segments are LR * NQ * 16 bytes apart (NQ 16-byte pieces per segment).
template <int LR, int NSEG, int NQ>
__device__ __forceinline__ void load_raw(const void* base, uint4 (*raw)[NQ]) {
#pragma unroll
  for (int s = 0; s < NSEG; ++s)
#pragma unroll
    for (int q = 0; q < NQ; ++q)
      raw[s][q] = gload16(reinterpret_cast<const uint8_t*>(base) + (size_t)s * LR * NQ * 16 + q * 16);
}

template <int NSEG, int NQ>
__device__ __forceinline__ void pack_bf16_run(const uint4 (*raw)[NQ], uint32_t (*xp)[NQ * 4], float* xseg) {
#pragma unroll
  for (int s = 0; s < NSEG; ++s) {
    float v[NQ * 8];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const uint32_t w4[4] = {raw[s][q].x, raw[s][q].y, raw[s][q].z, raw[s][q].w};
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        v[8 * q + 2 * p] = bf16_to_f32(w4[p] & 0xFFFF);
        v[8 * q + 2 * p + 1] = bf16_to_f32(w4[p] >> 16);
      }
    }
    if constexpr (NQ == 4) pack_segment(v, xp[s]);
    else pack_segment_q2(v, xp[s]);
    xseg[s] = seg_sum<NQ * 4>(xp[s]);
  }
}

// Pair-ordered f16 storage (the router's prepared x) is used as is.
template <int NSEG, int NQ>
__device__ __forceinline__ void pack_f16_run(const uint4 (*raw)[NQ], uint32_t (*hp)[NQ * 4], float* xseg) {
#pragma unroll
  for (int s = 0; s < NSEG; ++s) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      hp[s][4 * q + 0] = raw[s][q].x; hp[s][4 * q + 1] = raw[s][q].y;
      hp[s][4 * q + 2] = raw[s][q].z; hp[s][4 * q + 3] = raw[s][q].w;
    }
    xseg[s] = seg_sum<NQ * 4>(hp[s]);
  }
}

// fp32 activations (h) of a lane's NSEG segments as pair-ordered f16, each
// segment with its own power-of-two scale: the segment's largest magnitude is
// brought into [2^14, 2^15), so no value overflows fp16 (whose largest finite
// value is 65504) and the largest values keep fp16's full precision; fac[s] is
// the inverse scale, by which the segment's contribution is multiplied back.
// Scaling by a power of two is exact; only the f16 rounding is new.  v: the
// raw fp32 values, NQ4 16-byte pieces (4 floats each) per segment.
template <int NSEG, int NQ4, int BITS>
__device__ __forceinline__ void pack_scaled_run(const uint4 (*raw)[NQ4], uint32_t (*hp)[NQ4 * 2], float* xseg,
                                                float* fac) {
#pragma unroll
  for (int s = 0; s < NSEG; ++s) {
    float v[NQ4 * 4];
#pragma unroll
    for (int q = 0; q < NQ4; ++q) {
      v[4 * q + 0] = __uint_as_float(raw[s][q].x);
      v[4 * q + 1] = __uint_as_float(raw[s][q].y);
      v[4 * q + 2] = __uint_as_float(raw[s][q].z);
      v[4 * q + 3] = __uint_as_float(raw[s][q].w);
    }
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < NQ4 * 4; ++i) mx = fmaxf(mx, fabsf(v[i]));
    const int sh = f16_block_shift(mx);
    const float up = __builtin_ldexpf(1.0f, sh);
    fac[s] = __builtin_ldexpf(1.0f, -sh);
#pragma unroll
    for (int i = 0; i < NQ4 * 4; ++i) v[i] *= up;
    if constexpr (BITS == 4) pack_segment(v, hp[s]);
    else pack_segment_q2(v, hp[s]);
    xseg[s] = seg_sum<NQ4 * 2>(hp[s]);
  }
}

// One 32-value piece of a segment of fp32 activations as 16 pair-ordered f16
// dwords at the segment's power-of-two scale, with the segment's sum and
// inverse scale.  A SMOE-Q4 segment (32 values) is one piece; a SMOE-Q2
// segment (64 values) is two, held by lanes 2i and 2i + 1, which combine
// their maxima and sums with one DPP swap (every lane must call this).
template <int BITS>
__device__ __forceinline__ void pack_scaled_piece(const uint4 (&raw)[8], uint32_t (&hp)[16], float& xsum,
                                                  float& fac) {
  float v[32];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    v[4 * q + 0] = __uint_as_float(raw[q].x);
    v[4 * q + 1] = __uint_as_float(raw[q].y);
    v[4 * q + 2] = __uint_as_float(raw[q].z);
    v[4 * q + 3] = __uint_as_float(raw[q].w);
  }
  float mx = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) mx = fmaxf(mx, fabsf(v[i]));
  if constexpr (BITS == 2) mx = fmaxf(mx, dpp_f32<0xB1>(mx));  // the segment's other half
  const int sh = f16_block_shift(mx);
  const float up = __builtin_ldexpf(1.0f, sh);
  fac = __builtin_ldexpf(1.0f, -sh);
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] *= up;
  if constexpr (BITS == 4) {
    pack_segment(v, hp);
  } else {  // two groups of 16 in pair order: dword p of a group holds (e_p, e_{p+8})
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int p = 0; p < 8; ++p) hp[8 * g + p] = f16_bits(v[16 * g + p]) | (f16_bits(v[16 * g + p + 8]) << 16);
  }
  xsum = seg_sum<16>(hp);
  if constexpr (BITS == 2) xsum += dpp_f32<0xB1>(xsum);
}

// One 16-byte code segment's contribution for code width BITS.
template <int BITS>
__device__ __forceinline__ float seg_contrib_b(const uint4& c, const uint32_t* xp, float xseg, uint32_t params) {
  if constexpr (BITS == 4) return seg_contrib(c, xp, xseg, params);
  else return seg_contrib_q2(c, xp, xseg, params);
}

// Blob of rank r: passed by value, published by the router, or looked up in the
// layer's table; null when the index is outside [0, E) (the rank then
// contributes nothing -- the router itself never produces such an index).
__device__ __forceinline__ const void* expert_pointer(const DecodeArgs& a, int r) {
  if (a.src.direct[0]) return a.src.direct[r];
  if (a.ptrs) return a.ptrs[r];
  const int e = a.src.idx[r];
  return (e >= 0 && e < a.E) ? a.src.table[e] : nullptr;
}

// The NP * (64 / LR) rows of one wave (all in expert r, starting at row
// n_begin): every weight load is issued before any is consumed.
template <int LR, int NSEG, int NP, int CHUNK, int BITS, bool PX>
__device__ __forceinline__ void gate_up_rows(const DecodeArgs& a, const uint8_t* blob, int r, int n_begin, int li,
                                             int grp, const uint4 (*xraw)[LaneRun<LR, CHUNK, BITS>::NQ]) {
  using Run = LaneRun<LR, CHUNK, BITS>;
  constexpr int P = kWave / LR;
  const size_t row_bytes = (size_t)a.d * BITS / 8;
  const size_t prow_bytes = (size_t)(a.d / CHUNK) * 4;
  const size_t first = (size_t)(n_begin + grp);
  const uint8_t* gcodes = blob + first * row_bytes + li * 16;
  const uint8_t* ucodes = blob + a.lay.up_codes + first * row_bytes + li * 16;
  const uint8_t* gpar = blob + a.lay.gate_params + first * prow_bytes;
  const uint8_t* upar = blob + a.lay.up_params + first * prow_bytes;

  uint4 cg[NP][NSEG], cu[NP][NSEG];
  uint32_t pg[NP][NSEG], pu[NP][NSEG];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
#pragma unroll
    for (int s = 0; s < NSEG; ++s) {
      cg[p][s] = gload16(gcodes + (size_t)p * P * row_bytes + s * Run::STRIDE);
      cu[p][s] = gload16(ucodes + (size_t)p * P * row_bytes + s * Run::STRIDE);
    }
#pragma unroll
    for (int s = 0; s < NSEG; ++s) {
      const size_t po = (size_t)p * P * prow_bytes + Run::chunk_of(li, s) * 4;
      pg[p][s] = gload4(gpar + po);
      pu[p][s] = gload4(upar + po);
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // all weight loads are in flight before any math

  // this lane's input columns as f16 pairs, converted while the weights stream
  uint32_t xp[NSEG][Run::NDW];
  float xseg[NSEG];
  if constexpr (PX) pack_f16_run<NSEG, Run::NQ>(xraw, xp, xseg);
  else pack_bf16_run<NSEG, Run::NQ>(xraw, xp, xseg);

#pragma unroll
  for (int p = 0; p < NP; ++p) {
    float g = 0.f, u = 0.f;
#pragma unroll
    for (int s = 0; s < NSEG; ++s) {
      g += seg_contrib_b<BITS>(cg[p][s], xp[s], xseg[s], pg[p][s]);
      u += seg_contrib_b<BITS>(cu[p][s], xp[s], xseg[s], pu[p][s]);
    }
    g = group_sum<LR>(g);
    u = group_sum<LR>(u);
    if (li == 0) a.h[(size_t)r * a.f + n_begin + p * P + grp] = silu_f32(g) * u;
  }
}

// ---------------------------------------------------------------------------
// Gate + up + SwiGLU.  One wave owns NP * (64 / LR) consecutive rows of the
// flattened (rank, row) space, all inside one expert; LR lanes share a row.
// FUSED (the chained decode): the workgroup first selects the top k itself
// from the layer's logits (every workgroup reaches the same, deterministic
// selection), finds the blobs in src.table and reads the router's
// pair-ordered f16 x; workgroup 0 also publishes ids, weights and pointers.
// Otherwise the k experts come from src (or ptrs) and x is bf16.  The
// prologue's loads are unconditional (clamped indices), so the kernel
// arguments they need are fetched together rather than one dependent scalar
// load after another.  grid = ceil(k * d_ff / (4 * rows per wave)) workgroups
// of 4 waves.
// ---------------------------------------------------------------------------
template <int LR, int NSEG, int NP, int CHUNK, int BITS, bool FUSED>
__global__ __launch_bounds__(64 * SMOE_GU_WAVES) void decode_gate_up_kernel(const double* logits,
                                                                             const void* const* table,
                                                                             const uint16_t* xin, int E,
                                                                             DecodeArgs a) {
  using Run = LaneRun<LR, CHUNK, BITS>;
  constexpr int P = kWave / LR;  // rows per pass
  constexpr int RPW = NP * P;    // rows per wave
  __shared__ const void* s_ptr[kMaxTopK];
  __shared__ TopkShared tk;
  __shared__ const void* s_tab[kMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane % LR, grp = lane / LR;

  double lv = 0.0;
  const void* tv = nullptr;
  if constexpr (FUSED) {  // the layer's logits and blob table (clamped: no branch)
    const int te = tid < E ? tid : E - 1;
    lv = logits[te];
    tv = table[te];
    __builtin_amdgcn_sched_barrier(0);  // these first: the selection waits on them, not on x
  } else {
    if (tid < a.k) s_ptr[tid] = expert_pointer(a, tid);
  }
  // (the router writes its pair-ordered f16 copy of x in the order of BITS)
  uint4 xraw[NSEG][Run::NQ];
  load_raw<LR, NSEG, Run::NQ>(xin + li * Run::SEGV, xraw);
  if constexpr (FUSED) {  // stored after the input loads are issued (one thread per expert slot)
    // padding, and a NaN logit (from a non-finite residual), rank as -inf
    const double l = (tid < E && lv == lv) ? lv : -__builtin_inf();
    tk.log[tid] = l;
    tk.logf[tid] = (float)l;
    if (tid < E) s_tab[tid] = tv;
    if (tid < kMaxTopK) tk.idx[tid] = -1;
  }
  __syncthreads();
  if constexpr (FUSED) {
    if (E <= 128) topk_select_fast128<64 * SMOE_GU_WAVES>(tk, E, a.k, s_tab, s_ptr);
    else topk_select_fast(tk, E, a.k, s_tab, s_ptr);
  }

  const int gw = blockIdx.x * (blockDim.x >> 6) + wave;
  const int row0 = gw * RPW;
  if (row0 < a.k * a.f) {
    const int r = row0 / a.f;
    const int n_begin = row0 - r * a.f;
    const uint8_t* blob = reinterpret_cast<const uint8_t*>(s_ptr[r]);
    if (blob) {
      gate_up_rows<LR, NSEG, NP, CHUNK, BITS, FUSED>(a, blob, r, n_begin, li, grp, xraw);
    } else {  // an index outside [0, E) or a null table entry: the rank contributes nothing
      for (int it = lane; it < RPW; it += kWave) a.h[(size_t)r * a.f + n_begin + it] = 0.f;
    }
  }

  // Workgroup 0 publishes the selection for the down kernel after its own rows
  // (uniform branch: every wave of the workgroup reaches the barriers inside).
  if (FUSED && blockIdx.x == 0) {
    topk_weights(tk, E, a.k, a.norm);
    if (tid < a.k) {
      const int e = tk.idx[tid];
      a.sel.idx_out[tid] = e;
      a.sel.w_out[tid] = tk.w[tid];
      a.sel.ptr_out[tid] = s_tab[e];
      if (a.sel.idx_rec) a.sel.idx_rec[tid] = e;
      if (a.sel.w_rec) a.sel.w_rec[tid] = tk.w[tid];
    }
  }
}

// ---------------------------------------------------------------------------
// Down projection + weighted combine into the residual.  A workgroup owns
// NPASS * (64 / LR) output rows; its wave w handles ranks w, w + nw, ... so
// that each wave keeps one expert's h in registers; per-row partial results
// meet in LDS and are mixed in rank order (no atomics).  Each wave issues all
// weight loads of its rows before it computes.  Only the first LA lanes of
// each LR-lane group hold segments (LA < LR when a row's segment count is not
// a power of two: one segment per active lane, so that the LR-lane groups
// share one expert's h as few times as possible); the others contribute 0.
// grid = ceil(d / rows per workgroup), block = 64 * min(k, 8).
// ---------------------------------------------------------------------------
template <int LR, int NSEG, int NPASS, int CHUNK, int BITS, int LA, bool FROM_PTRS>
__global__ __launch_bounds__(512) void decode_down_kernel(const float* w_mix, const void* const* ptrs,
                                                          const float* h, float* residual, int k, int f,
                                                          DecodeArgs a) {
  using Run = LaneRun<LR, CHUNK, BITS>;
  constexpr int P = kWave / LR;
  constexpr int ROWS = NPASS * P;
  // With a row over LR < 64 lanes, the P row groups of a wave need the same
  // activation segments: the wave converts each segment once, 32 values per
  // lane (lane l takes piece l, l + 64, ...; a SMOE-Q2 segment is two pieces),
  // into its own LDS stage, with the segment's sum and inverse scale, and
  // every lane reads back the segments it multiplies.  The stage is private
  // to the wave, so no workgroup barrier is involved.
  constexpr int NQ4 = Run::SEGV / 4;   // 16-byte pieces of a segment's fp32 activations
  constexpr int SSEG = NSEG * LR;      // segments of a row (those with s % LR < LA are used)
  constexpr int LPS = Run::SEGV / 32;  // 32-value pieces (lanes) per segment
  constexpr bool STAGE = P > 1 && SSEG * Run::NDW * 4 <= 8192;
  constexpr int PER = (SSEG * LPS + kWave - 1) / kWave;  // pieces each lane converts
  __shared__ uint4 hst[STAGE ? 8 : 1][STAGE ? SSEG : 1][Run::NDW / 4];
  __shared__ float2 hsx[STAGE ? 8 : 1][STAGE ? SSEG : 1];
  __shared__ float ylds[kMaxTopK][ROWS];
  __shared__ const void* s_ptr[kMaxTopK];
  __shared__ float s_w[kMaxTopK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nw = blockDim.x >> 6;
  {
    // the mixing weights and blob pointers (FROM_PTRS: the ones the chained
    // gate/up kernel published), both loads in flight before either is
    // stored; clamped indices keep branches out of the loads' way
    const int tk = tid < k ? tid : 0;
    const float w = w_mix[tk];
    const void* p = FROM_PTRS ? ptrs[tk] : expert_pointer(a, tk);
    if (tid < k) {
      s_w[tid] = w;
      s_ptr[tid] = p;
    }
  }
  // the residual entries this workgroup updates at the end, loaded now so
  // that the final read-modify-write does not wait on memory (no other
  // workgroup touches these rows)
  const float res_pre = residual[(size_t)blockIdx.x * ROWS + (tid < ROWS ? tid : 0)];
  // Pull the next layer's router rows into cache while this kernel streams:
  // the router workgroup w (rows [2w, 2w + 2)) runs on XCD w % 8, so the down
  // workgroups of that XCD each fetch one slice of those rows.  Each thread
  // takes at most kPrefetchPerThread 16-byte pieces (out-of-range pieces read
  // the first 16 bytes instead, harmlessly); the loads are issued after the
  // weight loads and their values are only folded at the very end.
  constexpr int kPrefetchPerThread = 2;
  const uint8_t* pf_addr[kPrefetchPerThread];
  if (a.pf_base) {
    const size_t row_bytes = (size_t)a.d * 2, blk = (size_t)kRouteDecRowsPerWG * row_bytes;
    const size_t total = (size_t)a.E * row_bytes;
    const int x = blockIdx.x % kXcds, q = blockIdx.x / kXcds, Q = (gridDim.x + kXcds - 1) / kXcds;
    const int rw = (a.E + kRouteDecRowsPerWG - 1) / kRouteDecRowsPerWG;
    const int cx = x < rw ? (rw - x + kXcds - 1) / kXcds : 0;
    const size_t bx = (size_t)cx * blk, share = ((bx + Q - 1) / Q + 15) & ~(size_t)15;
    const size_t lo = (size_t)q * share, hi = lo + share < bx ? lo + share : bx;
#pragma unroll
    for (int i = 0; i < kPrefetchPerThread; ++i) {
      const size_t o = lo + ((size_t)i * blockDim.x + tid) * 16;
      const size_t addr = (size_t)(x + kXcds * (int)(o / blk)) * blk + o % blk;
      pf_addr[i] = a.pf_base + ((o < hi && addr + 16 <= total) ? addr : 0);
    }
  }
  uint4 pf[kPrefetchPerThread];
#pragma unroll
  for (int i = 0; i < kPrefetchPerThread; ++i) pf[i] = make_uint4(0, 0, 0, 0);

  const int li = lane % LR, grp = lane / LR;
  const bool act = LA == LR || li < LA;
  const int n0 = blockIdx.x * ROWS;
  const size_t row_bytes = (size_t)f * BITS / 8;
  const size_t prow_bytes = (size_t)(f / CHUNK) * 4;

  // h_r for this lane's columns as scaled pair-ordered f16, its segment sums
  // and the segments' inverse scales.  An idle lane (li >= LA) keeps zero
  // inputs (and below zero codes and parameters), so its contribution is 0.
  uint32_t hp[NSEG][Run::NDW];
  float xseg[NSEG], fac[NSEG];
  constexpr int NRAW = STAGE ? PER : NSEG;
  constexpr int NQR = STAGE ? 8 : NQ4;  // 16-byte pieces per raw entry
  uint4 hraw[NRAW][NQR];
  bool conv[NRAW];  // (staging) this lane converts its m-th piece
  auto load_h = [&](int r) {
    if constexpr (STAGE) {
#pragma unroll
      for (int m = 0; m < PER; ++m) {
        const int u = lane + kWave * m, j = u / LPS;
        conv[m] = j < SSEG && (j % LR) < LA;
#pragma unroll
        for (int q = 0; q < 8; ++q)
          hraw[m][q] = conv[m] ? gload16(h + (size_t)r * f + (size_t)u * 32 + 4 * q) : make_uint4(0, 0, 0, 0);
      }
    } else if (act) {
      load_raw<LR, NSEG, NQ4>(h + (size_t)r * f + li * Run::SEGV, hraw);
    } else {
#pragma unroll
      for (int s = 0; s < NSEG; ++s)
#pragma unroll
        for (int q = 0; q < NQ4; ++q) hraw[s][q] = make_uint4(0, 0, 0, 0);
    }
  };
  auto convert_h = [&]() {
    if constexpr (STAGE) {
#pragma unroll
      for (int m = 0; m < PER; ++m) {
        uint32_t cp[16];
        float cx, cf;
        pack_scaled_piece<BITS>(hraw[m], cp, cx, cf);
        if (conv[m]) {
          const int u = lane + kWave * m, j = u / LPS, part = u % LPS;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            hst[wave][j][4 * part + q] = make_uint4(cp[4 * q], cp[4 * q + 1], cp[4 * q + 2], cp[4 * q + 3]);
          if (part == 0) hsx[wave][j] = make_float2(cx, cf);
        }
      }
      // the stage is read by other lanes of this wave: LDS operations of a
      // wave complete in order; keep the compiler from reordering them
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int s = 0; s < NSEG; ++s) {
        const int j = s * LR + li;
        if (act) {
#pragma unroll
          for (int q = 0; q < Run::NDW / 4; ++q) {
            const uint4 v = hst[wave][j][q];
            hp[s][4 * q] = v.x; hp[s][4 * q + 1] = v.y; hp[s][4 * q + 2] = v.z; hp[s][4 * q + 3] = v.w;
          }
          const float2 sx = hsx[wave][j];
          xseg[s] = sx.x;
          fac[s] = sx.y;
        } else {
#pragma unroll
          for (int q = 0; q < Run::NDW; ++q) hp[s][q] = 0u;
          xseg[s] = 0.f;
          fac[s] = 0.f;
        }
      }
      // before the stage is written again (next rank of this wave)
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    } else {
      pack_scaled_run<NSEG, NQ4, BITS>(hraw, hp, xseg, fac);
    }
  };
  // The first rank's activations do not depend on the expert pointers: their
  // loads go out with the pointers' (the conversion waits until the weight
  // loads are in flight).
  if (wave < k) load_h(wave);
  __syncthreads();

  for (int r = wave, it = 0; r < k; r += nw, ++it) {
    const uint8_t* blob = reinterpret_cast<const uint8_t*>(s_ptr[r]);
    if (!blob) {
      for (int row = lane; row < ROWS; row += kWave) ylds[r][row] = 0.f;
      continue;
    }
    const uint8_t* codes = blob + a.lay.down_codes + li * 16;
    const uint8_t* par = blob + a.lay.down_params;
    if (it > 0) load_h(r);
    __builtin_amdgcn_sched_barrier(0);  // h first: the math can start when it lands
    uint4 c[NPASS][NSEG];
    uint32_t pr[NPASS][NSEG];
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      const int n = n0 + p * P + grp;  // < d: the launcher checks d % ROWS == 0
#pragma unroll
      for (int s = 0; s < NSEG; ++s)
        c[p][s] = act ? gload16(codes + (size_t)n * row_bytes + s * Run::STRIDE) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int s = 0; s < NSEG; ++s)
        pr[p][s] = act ? gload4(par + (size_t)n * prow_bytes + Run::chunk_of(li, s) * 4) : 0u;
    }
    if (it == 0 && a.pf_base) {
#pragma unroll
      for (int i = 0; i < kPrefetchPerThread; ++i) pf[i] = gload16(pf_addr[i]);
    }
    __builtin_amdgcn_sched_barrier(0);  // all weight loads are in flight before any math
    convert_h();
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      float y = 0.f;
#pragma unroll
      for (int s = 0; s < NSEG; ++s)
        y = fmaf(fac[s], seg_contrib_b<BITS>(c[p][s], hp[s], xseg[s], pr[p][s]), y);
      y = group_sum<LR>(y);
      if (li == 0) ylds[r][p * P + grp] = y;
    }
  }
  __syncthreads();
  for (int row = tid; row < ROWS; row += blockDim.x) {
    const int n = n0 + row;
    float acc = 0.f;
    for (int r = 0; r < k; ++r) acc = fmaf(s_w[r], ylds[r][row], acc);
    residual[n] = (row == tid ? res_pre : residual[n]) + acc;
  }
  // keeps the prefetch loads alive (all four words, so that no register of a
  // pending load is reused early, which would force a wait for it)
#pragma unroll
  for (int i = 0; i < kPrefetchPerThread; ++i) asm volatile("" ::"v"(pf[i].x), "v"(pf[i].y), "v"(pf[i].z), "v"(pf[i].w));
}

// ---------------------------------------------------------------------------
// Shape dispatch
// ---------------------------------------------------------------------------
static int pow2_part(int v) { return v & (-v); }

struct RowSplit {
  int lr, nseg;
};

// LR = the largest power of two <= 64 dividing the row's segment count.
static RowSplit split_row(int cols, int bits) {
  const int segs = cols * bits / 128;  // 16-byte segments per row
  int lr = pow2_part(segs);
  if (lr > 64) lr = 64;
  return {lr, segs / lr};
}

bool decode_shape_supported(int d, int f, int chunk, int bits) {
  if (bits == 4) {
    if (chunk != 32 && chunk != 64) return false;
    if (d % 256 || f % 64) return false;
  } else if (bits == 2) {
    if (chunk != 64) return false;  // a Q2 segment (64 codes) is one chunk of 64
    if (d % 512 || f % 128) return false;
  } else {
    return false;
  }
  const RowSplit g = split_row(d, bits), dn = split_row(f, bits);
  return g.lr >= 8 && g.nseg <= 4 && dn.lr >= 2 && dn.nseg <= 4;
}

#define SMOE_CASE(N, NAME, ...) case N: { constexpr int NAME = N; __VA_ARGS__; } break;
#define SMOE_NSEG_SWITCH(V, ...)                                                            \
  switch (V) { SMOE_CASE(1, NSEG, __VA_ARGS__) SMOE_CASE(2, NSEG, __VA_ARGS__)             \
               SMOE_CASE(3, NSEG, __VA_ARGS__) SMOE_CASE(4, NSEG, __VA_ARGS__)             \
               default: return hipErrorInvalidValue; }
#define SMOE_LR_SWITCH(V, ...)                                                              \
  switch (V) { SMOE_CASE(2, LR, __VA_ARGS__) SMOE_CASE(4, LR, __VA_ARGS__)                 \
               SMOE_CASE(8, LR, __VA_ARGS__) SMOE_CASE(16, LR, __VA_ARGS__)                \
               SMOE_CASE(32, LR, __VA_ARGS__) SMOE_CASE(64, LR, __VA_ARGS__)               \
               default: return hipErrorInvalidValue; }
#define SMOE_NP_SWITCH(V, NAME, ...)                                                        \
  switch (V) { SMOE_CASE(1, NAME, __VA_ARGS__) SMOE_CASE(2, NAME, __VA_ARGS__)             \
               SMOE_CASE(4, NAME, __VA_ARGS__)                                             \
               default: return hipErrorInvalidValue; }
#define SMOE_NP8_SWITCH(V, NAME, ...)                                                       \
  switch (V) { SMOE_CASE(1, NAME, __VA_ARGS__) SMOE_CASE(2, NAME, __VA_ARGS__)             \
               SMOE_CASE(4, NAME, __VA_ARGS__) SMOE_CASE(8, NAME, __VA_ARGS__)             \
               default: return hipErrorInvalidValue; }
// (code width, chunk): SMOE-Q4 with chunks of 32 or 64, SMOE-Q2 with chunks of 64
#define SMOE_FORMAT_SWITCH(B, C, ...)                                                      \
  if ((B) == 4 && (C) == 32) { constexpr int BITS = 4, CHUNK = 32; __VA_ARGS__; }          \
  else if ((B) == 4 && (C) == 64) { constexpr int BITS = 4, CHUNK = 64; __VA_ARGS__; }     \
  else if ((B) == 2 && (C) == 64) { constexpr int BITS = 2, CHUNK = 64; __VA_ARGS__; }     \
  else return hipErrorInvalidValue;

// Rows per wave of the gate/up kernel: NP passes of 64/LR rows, the largest
// NP <= SMOE_GU_ROWS_MAX that divides d_ff and leaves >= SMOE_GU_MIN_WAVES waves.
static int gate_up_np(int lr, int total, int f) {
  const int P = 64 / lr;
  int np = 1;
  while (np * 2 <= SMOE_GU_ROWS_MAX && f % (P * np * 2) == 0 && total / (P * np * 2) >= SMOE_GU_MIN_WAVES)
    np *= 2;
  return np;
}

hipError_t launch_decode_gate_up(const DecodeArgs& a, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
  const RowSplit sp = split_row(a.d, a.bits);
  const int total = a.k * a.f;
  const int np = gate_up_np(sp.lr, total, a.f);
  const int waves = total / (np * (64 / sp.lr));
  // the launch bounds and the selection's thread count are SMOE_GU_WAVES waves
  constexpr int nw = SMOE_GU_WAVES;
  const dim3 grid((waves + nw - 1) / nw);
  // the chained decode selects inside the kernel and reads the router's
  // pair-ordered x; the per-layer calls give experts and bf16 x
  const bool fused = a.sel.logits != nullptr;
  if (fused != (a.px != nullptr)) return hipErrorInvalidValue;
  const uint16_t* px = reinterpret_cast<const uint16_t*>(a.px);
  if (fused) {
    SMOE_FORMAT_SWITCH(a.bits, a.chunk, SMOE_LR_SWITCH(sp.lr, SMOE_NSEG_SWITCH(sp.nseg, SMOE_NP_SWITCH(np, NP,
        if (start || stop) {
          hipExtLaunchKernelGGL((decode_gate_up_kernel<LR, NSEG, NP, CHUNK, BITS, true>), grid, dim3(64 * nw), 0, s,
                                start, stop, 0, a.sel.logits, a.src.table, px, a.E, a);
        } else {
          hipLaunchKernelGGL((decode_gate_up_kernel<LR, NSEG, NP, CHUNK, BITS, true>), grid, dim3(64 * nw), 0, s,
                             a.sel.logits, a.src.table, px, a.E, a);
        }))));
  } else {
    SMOE_FORMAT_SWITCH(a.bits, a.chunk, SMOE_LR_SWITCH(sp.lr, SMOE_NSEG_SWITCH(sp.nseg, SMOE_NP_SWITCH(np, NP,
        if (start || stop) {
          hipExtLaunchKernelGGL((decode_gate_up_kernel<LR, NSEG, NP, CHUNK, BITS, false>), grid, dim3(64 * nw), 0, s,
                                start, stop, 0, a.sel.logits, a.src.table, a.x, a.E, a);
        } else {
          hipLaunchKernelGGL((decode_gate_up_kernel<LR, NSEG, NP, CHUNK, BITS, false>), grid, dim3(64 * nw), 0, s,
                             a.sel.logits, a.src.table, a.x, a.E, a);
        }))));
  }
  return hipGetLastError();
}

// The down rows' split.  SMOE-Q2 rows of 3 * 2^m segments (3 <= segs <= 48)
// take one segment per lane over the next power of two (LR lanes, LA = segs
// active): with split_row's LR = segs / 3 lanes, each lane would hold three
// 64-value h segments and the 64 / LR row groups of a wave would each re-read
// h (235B shape: 24 KB of h per wave against 6 KB of codes), which measured
// slower than the idle quarter of lanes.  For SMOE-Q4 (32-value segments) the
// power-of-two split measured faster.  Otherwise split_row's split.
struct DownSplit {
  int lr, nseg, la;
};
static DownSplit split_down(int f, int bits) {
  const int segs = f * bits / 128;
  if (bits == 2 && segs >= 3 && segs <= 48 && segs % 3 == 0 && pow2_part(segs / 3) == segs / 3)
    return {segs / 3 * 4, 1, segs};
  const RowSplit sp = split_row(f, bits);
  return {sp.lr, sp.nseg, sp.lr};
}

// the down kernel's leading scalar arguments (preloaded into registers at
// dispatch) and the argument block
#define SMOE_DOWN_HOT_ARGS(a) (a).w, (a).ptrs, (a).h, (a).residual, (a).k, (a).f, (a)

hipError_t launch_decode_down(const DecodeArgs& a, hipStream_t s) {
  const DownSplit sp = split_down(a.f, a.bits);
  const int P = 64 / sp.lr;
  int np = 1;
  while (np * 2 <= SMOE_DN_PASSES_MAX && a.d / (P * np * 2) >= SMOE_DN_MIN_WG) np *= 2;
  // register budget: a lane holding more than 128 fp32 activations takes one
  // row pass, three or more segments at most four (more would spill)
  if (sp.nseg * (128 / a.bits) > 128) np = 1;
  if (sp.nseg >= 3 && np > 4) np = 4;
  const int rows = np * P;
  if (a.d % rows) return hipErrorInvalidValue;  // every workgroup owns full rows
  const int nw = a.k < 8 ? a.k : 8;
  const dim3 grid(a.d / rows);
  // the chained decode's pointers, published by its gate/up kernel
  const bool from_ptrs = a.ptrs != nullptr && !a.src.direct[0];
  if (sp.la != sp.lr) {  // one segment per active lane: LA = 3 LR / 4
    if (a.bits != 2 || a.chunk != 64) return hipErrorInvalidValue;
    constexpr int BITS = 2, CHUNK = 64;
    if (from_ptrs) {
      SMOE_LR_SWITCH(sp.lr, SMOE_NP8_SWITCH(np, NPASS,
          hipLaunchKernelGGL((decode_down_kernel<LR, 1, NPASS, CHUNK, BITS, LR * 3 / 4, true>), grid, dim3(64 * nw),
                             0, s, SMOE_DOWN_HOT_ARGS(a))));
    } else {
      SMOE_LR_SWITCH(sp.lr, SMOE_NP8_SWITCH(np, NPASS,
          hipLaunchKernelGGL((decode_down_kernel<LR, 1, NPASS, CHUNK, BITS, LR * 3 / 4, false>), grid, dim3(64 * nw),
                             0, s, SMOE_DOWN_HOT_ARGS(a))));
    }
    return hipGetLastError();
  }
  if (from_ptrs) {
    SMOE_FORMAT_SWITCH(a.bits, a.chunk, SMOE_LR_SWITCH(sp.lr, SMOE_NSEG_SWITCH(sp.nseg, SMOE_NP8_SWITCH(np, NPASS,
        hipLaunchKernelGGL((decode_down_kernel<LR, NSEG, NPASS, CHUNK, BITS, LR, true>), grid, dim3(64 * nw), 0, s,
                           SMOE_DOWN_HOT_ARGS(a))))));
  } else {
    SMOE_FORMAT_SWITCH(a.bits, a.chunk, SMOE_LR_SWITCH(sp.lr, SMOE_NSEG_SWITCH(sp.nseg, SMOE_NP8_SWITCH(np, NPASS,
        hipLaunchKernelGGL((decode_down_kernel<LR, NSEG, NPASS, CHUNK, BITS, LR, false>), grid, dim3(64 * nw), 0, s,
                           SMOE_DOWN_HOT_ARGS(a))))));
  }
  return hipGetLastError();
}

}  // namespace smoe
