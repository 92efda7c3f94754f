// Decode-time fused SMOE-Q4 expert FFN (one token, k routed experts).
//
// "Coalesced GPU Kernels -- Expert FFN and Dense Matvec" (Optimizations page):
// the expert FFN dequantises 4-bit codes with a per-chunk affine epilogue and
// computes gate and up in one pass, then the down projection; the System
// Overview step table adds the gate-weighted sum into the residual.  The pages'
// Metal design (one 32-lane simdgroup per output row, input staged per 8-row
// threadgroup) is prior art; on gfx950 the row is split over LR lanes of a
// wave64 (LR = 64 for the 235B/30B gate-up rows), each lane streaming 16-byte
// segments of packed nibbles with global_load_dwordx4, the input held in
// registers as f16 pairs for v_dot2_f32_f16, and rows reduced with butterflies.
//
// Affine folding: a 16-byte segment (32 codes) lies inside one chunk, so its
// contribution is scale * sum(q x) + min * sum(x); sum(x) over the segment is
// computed once per wave because every row of a wave uses the same columns.
#include <hip/hip_ext.h>

#include "kernels.h"

namespace smoe {

// Blob of rank r, or null when the routed index is outside [0, E) (such a
// rank contributes nothing; it cannot come from the router itself).
__device__ __forceinline__ const uint8_t* expert_blob(const DecodeArgs& a, const int* s_idx, int r) {
  if (a.src.direct[0]) return reinterpret_cast<const uint8_t*>(a.src.direct[r]);
  const int e = s_idx[r];
  if (e < 0 || e >= a.E) return nullptr;
  return reinterpret_cast<const uint8_t*>(a.src.table[e]);
}

// ---------------------------------------------------------------------------
// Gate + up + SwiGLU.  One wave owns rows_per_wave consecutive rows of the
// flattened (rank, row) space, all inside one expert; LR lanes share a row.
// grid = ceil(k * d_ff / (4 * rows_per_wave)), 256 threads.
// ---------------------------------------------------------------------------
template <int LR, int NLD>
__global__ __launch_bounds__(256) void decode_gate_up_kernel(DecodeArgs a, int rows_per_wave) {
  __shared__ int s_idx[kMaxTopK];
  __shared__ float s_w[kMaxTopK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  if (a.logits) {
    // fused routing: every workgroup selects the experts itself
    if (wave == 0) topk_wave(a.logits, a.E, a.k, a.norm, s_idx, s_w);
    __syncthreads();
    if (blockIdx.x == 0 && tid < a.k) {
      a.idx_ws[tid] = s_idx[tid];
      a.w_ws[tid] = s_w[tid];
      if (a.idx_rec) a.idx_rec[tid] = s_idx[tid];
      if (a.w_rec) a.w_rec[tid] = s_w[tid];
    }
  } else if (!a.src.direct[0]) {
    if (tid < a.k) s_idx[tid] = a.src.idx[tid];
    __syncthreads();
  }

  constexpr int P = kWave / LR;  // rows per pass
  const int li = lane % LR, grp = lane / LR;
  const int gw = blockIdx.x * 4 + wave;
  const int total = a.k * a.f;
  const int row0 = gw * rows_per_wave;
  if (row0 >= total) return;
  const int r = row0 / a.f;
  const uint8_t* blob = expert_blob(a, s_idx, r);
  const int n_begin = row0 - r * a.f;
  if (!blob) {
    for (int it = lane; it < rows_per_wave; it += kWave) {
      const int n = n_begin + it;
      a.h[(size_t)r * a.f + (n & ~7) + pair_slot(n & 7)] = (_Float16)0.0f;
    }
    return;
  }

  // the wave's input columns, as f16 pairs, and their per-segment sums
  uint32_t xp[NLD][16];
  float cseg[NLD], xseg[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int seg = li + LR * i;
    const uint4* xv = reinterpret_cast<const uint4*>(a.x + seg * 32);
    float v[32];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 u = xv[q];
      const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        v[8 * q + 2 * p] = bf16_to_f32(w4[p] & 0xFFFF);
        v[8 * q + 2 * p + 1] = bf16_to_f32(w4[p] >> 16);
      }
    }
    pack_segment(v, xp[i], cseg[i], xseg[i]);
  }

  const size_t row_bytes = (size_t)a.d / 2;
  const size_t prow_bytes = (size_t)(a.d / a.chunk) * 4;
  const uint8_t* gcodes = blob;
  const uint8_t* ucodes = blob + a.lay.up_codes;
  const uint8_t* gpar = blob + a.lay.gate_params;
  const uint8_t* upar = blob + a.lay.up_params;
  int poff[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) poff[i] = ((li + LR * i) * 32 / a.chunk) * 4;

  for (int it = 0; it < rows_per_wave; it += P) {
    const int n = n_begin + it + grp;
    uint4 cg[NLD], cu[NLD];
    uint32_t pg[NLD], pu[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const size_t co = (size_t)n * row_bytes + (size_t)(li + LR * i) * 16;
      cg[i] = *reinterpret_cast<const uint4*>(gcodes + co);
      cu[i] = *reinterpret_cast<const uint4*>(ucodes + co);
      const size_t po = (size_t)n * prow_bytes + poff[i];
      pg[i] = *reinterpret_cast<const uint32_t*>(gpar + po);
      pu[i] = *reinterpret_cast<const uint32_t*>(upar + po);
    }
    float g = 0.f, u = 0.f;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      g += seg_contrib(cg[i], xp[i], cseg[i], xseg[i], pg[i]);
      u += seg_contrib(cu[i], xp[i], cseg[i], xseg[i], pu[i]);
    }
    g = group_sum<LR>(g);
    u = group_sum<LR>(u);
    if (li == 0) {
      const float h = silu_f32(g) * u;
      a.h[(size_t)r * a.f + (n & ~7) + pair_slot(n & 7)] = (_Float16)h;
    }
  }
}

// ---------------------------------------------------------------------------
// Down projection + weighted combine into the residual.  A workgroup owns
// rows_per_wg output rows; its wave w handles ranks w, w + nw, ... so that each
// wave keeps one expert's h in registers; per-row partial results meet in LDS
// and are mixed in rank order (no atomics).  grid = ceil(d / rows_per_wg),
// block = 64 * min(k, 8).
// ---------------------------------------------------------------------------
constexpr int kDownMaxRows = 64;

template <int LR, int NLD>
__global__ __launch_bounds__(512) void decode_down_kernel(DecodeArgs a, int rows_per_wg) {
  __shared__ float ylds[kMaxTopK][kDownMaxRows];
  __shared__ int s_idx[kMaxTopK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nw = blockDim.x >> 6;
  if (!a.src.direct[0] && tid < a.k) s_idx[tid] = a.src.idx[tid];
  __syncthreads();

  constexpr int P = kWave / LR;
  const int li = lane % LR, grp = lane / LR;
  const int n0 = blockIdx.x * rows_per_wg;
  const size_t row_bytes = (size_t)a.f / 2;
  const size_t prow_bytes = (size_t)(a.f / a.chunk) * 4;
  int poff[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) poff[i] = ((li + LR * i) * 32 / a.chunk) * 4;

  for (int r = wave; r < a.k; r += nw) {
    const uint8_t* blob = expert_blob(a, s_idx, r);
    if (!blob) {
      for (int row = lane; row < rows_per_wg; row += kWave) ylds[r][row] = 0.f;
      continue;
    }
    const uint8_t* codes = blob + a.lay.down_codes;
    const uint8_t* par = blob + a.lay.down_params;
    // h_r for this lane's columns (already pair-ordered) and its segment sums
    uint32_t hp[NLD][16];
    float cseg[NLD], xseg[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const uint4* hv = reinterpret_cast<const uint4*>(a.h + (size_t)r * a.f + (li + LR * i) * 32);
      float se = 0.f, so = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 u = hv[q];
        hp[i][4 * q + 0] = u.x; hp[i][4 * q + 1] = u.y; hp[i][4 * q + 2] = u.z; hp[i][4 * q + 3] = u.w;
        const half2_t h0 = __builtin_bit_cast(half2_t, u.x), h1 = __builtin_bit_cast(half2_t, u.y);
        const half2_t h2 = __builtin_bit_cast(half2_t, u.z), h3 = __builtin_bit_cast(half2_t, u.w);
        // dwords 0 and 2 hold the even elements, 1 and 3 the odd ones
        se += ((float)h0.x + (float)h0.y) + ((float)h2.x + (float)h2.y);
        so += ((float)h1.x + (float)h1.y) + ((float)h3.x + (float)h3.y);
      }
      cseg[i] = fmaf(1024.f, se, 64.f * so);
      xseg[i] = se + so;
    }
    for (int pass = 0; pass < rows_per_wg; pass += P) {
      const int n = n0 + pass + grp;
      const bool ok = n < a.d;
      uint4 c[NLD];
      uint32_t pr[NLD];
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        if (ok) {
          c[i] = *reinterpret_cast<const uint4*>(codes + (size_t)n * row_bytes + (size_t)(li + LR * i) * 16);
          pr[i] = *reinterpret_cast<const uint32_t*>(par + (size_t)n * prow_bytes + poff[i]);
        } else {
          c[i] = make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
          pr[i] = 0;
        }
      }
      float y = 0.f;
#pragma unroll
      for (int i = 0; i < NLD; ++i) y += seg_contrib(c[i], hp[i], cseg[i], xseg[i], pr[i]);
      y = group_sum<LR>(y);
      if (li == 0) ylds[r][pass + grp] = y;
    }
  }
  __syncthreads();
  for (int row = tid; row < rows_per_wg; row += blockDim.x) {
    const int n = n0 + row;
    if (n >= a.d) break;
    float acc = 0.f;
    for (int r = 0; r < a.k; ++r) acc = fmaf(a.w[r], ylds[r][row], acc);
    a.residual[n] += acc;
  }
}

// ---------------------------------------------------------------------------
// Shape dispatch
// ---------------------------------------------------------------------------
static int pow2_part(int v) { return v & (-v); }

struct RowSplit {
  int lr, nld;
};

static RowSplit split_row(int cols) {
  const int segs = cols / 32;  // 16-byte segments per row
  int lr = pow2_part(segs);
  if (lr > 64) lr = 64;
  return {lr, segs / lr};
}

bool decode_shape_supported(int d, int f, int chunk) {
  if (chunk != 32 && chunk != 64) return false;
  if (d % 256 || f % 64) return false;
  const RowSplit g = split_row(d), dn = split_row(f);
  return g.lr >= 8 && g.nld <= 4 && dn.lr >= 2 && dn.nld <= 4;
}

#define SMOE_NLD_SWITCH(NLD_VAL, ...)          \
  switch (NLD_VAL) {                           \
    case 1: { constexpr int NLD = 1; __VA_ARGS__; } break; \
    case 2: { constexpr int NLD = 2; __VA_ARGS__; } break; \
    case 3: { constexpr int NLD = 3; __VA_ARGS__; } break; \
    case 4: { constexpr int NLD = 4; __VA_ARGS__; } break; \
    default: return hipErrorInvalidValue;      \
  }

#define SMOE_LR_SWITCH(LR_VAL, ...)            \
  switch (LR_VAL) {                            \
    case 2: { constexpr int LR = 2; __VA_ARGS__; } break;  \
    case 4: { constexpr int LR = 4; __VA_ARGS__; } break;  \
    case 8: { constexpr int LR = 8; __VA_ARGS__; } break;  \
    case 16: { constexpr int LR = 16; __VA_ARGS__; } break; \
    case 32: { constexpr int LR = 32; __VA_ARGS__; } break; \
    case 64: { constexpr int LR = 64; __VA_ARGS__; } break; \
    default: return hipErrorInvalidValue;      \
  }

hipError_t launch_decode_gate_up(const DecodeArgs& a, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
  const RowSplit sp = split_row(a.d);
  const int P = 64 / sp.lr;
  const int total = a.k * a.f;
  // about 2048 waves per launch; rows per wave a power of two dividing d_ff
  int rpw = P;
  while (rpw * 2 <= 64 && a.f % (rpw * 2) == 0 && total / (rpw * 2) >= 2048) rpw *= 2;
  const int waves = total / rpw;
  const dim3 grid((waves + 3) / 4);
  if (start || stop) {
    SMOE_LR_SWITCH(sp.lr, SMOE_NLD_SWITCH(sp.nld,
        hipExtLaunchKernelGGL((decode_gate_up_kernel<LR, NLD>), grid, dim3(256), 0, s, start, stop, 0, a, rpw)));
  } else {
    SMOE_LR_SWITCH(sp.lr, SMOE_NLD_SWITCH(sp.nld,
        hipLaunchKernelGGL((decode_gate_up_kernel<LR, NLD>), grid, dim3(256), 0, s, a, rpw)));
  }
  return hipGetLastError();
}

hipError_t launch_decode_down(const DecodeArgs& a, hipStream_t s) {
  const RowSplit sp = split_row(a.f);
  const int P = 64 / sp.lr;
  int rows = P;
  while (rows * 2 <= kDownMaxRows && a.d / (rows * 2) >= 256) rows *= 2;
  const int nw = a.k < 8 ? a.k : 8;
  const dim3 grid((a.d + rows - 1) / rows);
  SMOE_LR_SWITCH(sp.lr, SMOE_NLD_SWITCH(sp.nld,
      hipLaunchKernelGGL((decode_down_kernel<LR, NLD>), grid, dim3(64 * nw), 0, s, a, rows)));
  return hipGetLastError();
}

}  // namespace smoe
