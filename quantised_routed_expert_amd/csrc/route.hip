// Exact router: RMSNorm -> bf16 x, float64 gate matvec, top-k, mixing weights.
//
// "Routing Is Exact" (Optimizations page) and the per-token step table of the
// System Overview page: each MoE layer runs its own E x d_model router gate on
// the actual hidden state (no predictor), then selects the top k with Qwen3's
// weighting (softmax over all E, keep the k largest, renormalise).
// The pages run this gate on the CPU; here the norm and the gate run on the
// GPU, as the pages' own "GPU-Resident Epilogue" plan (Optimizations, "The
// Dense Ceiling") proposes.
#include "kernels.h"

namespace smoe {

constexpr int kRouteMaxR = 8;   // float4 of residual per thread: d <= 8192

// ---------------------------------------------------------------------------
// RMSNorm + logits for one token (decode).  grid = E workgroups, one router
// row each, of 64 * ceil(d / 512) threads; thread t owns the 8 consecutive
// columns [8t, 8t + 8) (threads at or past d / 8 own none), normalises exactly
// the columns it multiplies, and x never goes through LDS.  The sum of squares
// is complete in every workgroup: float64, in a fixed order (thread, wave DPP
// tree, waves in order), as is the row's dot product of exact bf16 products.
// Few columns per lane keep each wave's chain of dependent float64 work short
// (the token's latency is the kernel's cost).  Workgroup 0 writes x (bf16) and
// its pair-ordered f16 copy with 16-byte stores.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void route_logits_decode_kernel(const uint16_t* w_router, const float* residual,
                                                                   int d, RouteArgs a) {
  __shared__ double red[16];
  __shared__ double part[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  const int e = blockIdx.x;
  const int j = tid * 8;
  const bool has = j < d;
  // loads at clamped columns, zeroed when the thread owns none (no branch
  // before the loads; the arguments they need come preloaded in registers)
  const int jc = has ? j : 0;
  uint4 wv = gload16(w_router + (size_t)e * d + jc);
  float4 r0 = *reinterpret_cast<const float4*>(residual + jc);
  float4 r1 = *reinterpret_cast<const float4*>(residual + jc + 4);
  if (!has) {
    wv = make_uint4(0, 0, 0, 0);
    r0 = r1 = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  double ss = (((double)r0.x * r0.x + (double)r0.y * r0.y) + ((double)r0.z * r0.z + (double)r0.w * r0.w)) +
              (((double)r1.x * r1.x + (double)r1.y * r1.y) + ((double)r1.z * r1.z + (double)r1.w * r1.w));
  ss = group_sum_f64<64>(ss);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  double tot = 0.0;
  for (int w = 0; w < nw; ++w) tot += red[w];
  const double den = sqrt(tot / (double)d + (double)a.eps);
  const float inv = (float)(1.0 / den);

  // x (bf16 pairs) for this thread's 8 columns
  const float v[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
  uint32_t xb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    xb[i] = bf16_of_quotient(v[2 * i], den, inv) | (bf16_of_quotient(v[2 * i + 1], den, inv) << 16);
  if (blockIdx.x == 0 && has) {
    if (a.x_out) *reinterpret_cast<uint4*>(a.x_out + j) = make_uint4(xb[0], xb[1], xb[2], xb[3]);
    if (a.px_out && !a.px16) {
      // dword p of the group of 8 holds (e_p, e_{p+4}) as f16
      uint32_t pw[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t lo = (xb[p >> 1] >> (16 * (p & 1))) & 0xFFFFu;
        const uint32_t hi = (xb[2 + (p >> 1)] >> (16 * (p & 1))) & 0xFFFFu;
        pw[p] = f16_bits(bf16_to_f32(lo)) | (f16_bits(bf16_to_f32(hi)) << 16);
      }
      *reinterpret_cast<uint4*>(a.px_out + j) = make_uint4(pw[0], pw[1], pw[2], pw[3]);
    }
  }
  if (blockIdx.x == 0 && a.px_out && a.px16) {
    // groups of 16 (SMOE-Q2): dword p holds (e_p, e_{p+8}).  A group spans
    // threads 2i (e_0..e_7) and 2i+1 (e_8..e_15): the even thread writes
    // dwords 0..3 and needs e_8..e_11, the odd thread dwords 4..7 and needs
    // e_4..e_7, so each hands its partner two of its four bf16 pairs (d is a
    // multiple of 512 for SMOE-Q2, so both partners own columns).
    const bool odd = lane & 1;
    const uint32_t s0 = __shfl_xor(odd ? xb[0] : xb[2], 1, kWave);
    const uint32_t s1 = __shfl_xor(odd ? xb[1] : xb[3], 1, kWave);
    const uint32_t A[2] = {odd ? s0 : xb[0], odd ? s1 : xb[1]};  // e_p
    const uint32_t B[2] = {odd ? xb[2] : s0, odd ? xb[3] : s1};  // e_{p+8}
    uint32_t pw[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t lo = (A[p >> 1] >> (16 * (p & 1))) & 0xFFFFu;
      const uint32_t hi = (B[p >> 1] >> (16 * (p & 1))) & 0xFFFFu;
      pw[p] = f16_bits(bf16_to_f32(lo)) | (f16_bits(bf16_to_f32(hi)) << 16);
    }
    // the even thread's dwords start the group, the odd thread's follow: px + j
    if (has) *reinterpret_cast<uint4*>(a.px_out + j) = make_uint4(pw[0], pw[1], pw[2], pw[3]);
  }

  // this row's dot product over the thread's columns: float64 pair sums
  const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
  double acc = 0.0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // products of two bf16 values are exact in fp32
    const float p0 = bf16_to_f32(ww[i] & 0xFFFF) * bf16_to_f32(xb[i] & 0xFFFF);
    const float p1 = bf16_to_f32(ww[i] >> 16) * bf16_to_f32(xb[i] >> 16);
    acc += (double)p0 + (double)p1;
  }
  acc = group_sum_f64<64>(acc);
  if (lane == 0) part[wave] = acc;
  __syncthreads();
  if (tid == 0) {
    double l = 0.0;
    for (int w = 0; w < nw; ++w) l += part[w];
    a.logits[e] = l + (a.bias ? (double)a.bias[e] : 0.0);
  }
}

// ---------------------------------------------------------------------------
// RMSNorm for 2..64 tokens: one workgroup of 256 threads per token.  The sum of
// squares is float64 in a fixed order (per thread, then per wave, then waves
// 0..3); x = bf16(r / den) is written to x_out for the logits kernel below and
// for the expert FFN.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void route_norm_kernel(RouteArgs a) {
  __shared__ double red[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int d = a.d;
  const float* r = a.residual + (size_t)blockIdx.x * d;
  float4 rv[kRouteMaxR];
#pragma unroll
  for (int q = 0; q < kRouteMaxR; ++q) {
    const int j = tid * 4 + 1024 * q;
    rv[q] = j < d ? *reinterpret_cast<const float4*>(r + j) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  double s = 0.0;
#pragma unroll
  for (int q = 0; q < kRouteMaxR; ++q)
    s += ((double)rv[q].x * rv[q].x + (double)rv[q].y * rv[q].y) + ((double)rv[q].z * rv[q].z + (double)rv[q].w * rv[q].w);
  s = group_sum_f64<64>(s);
  if (lane == 0) red[wave] = s;
  __syncthreads();
  const double den = sqrt(((red[0] + red[1]) + (red[2] + red[3])) / (double)d + (double)a.eps);
  const float inv = (float)(1.0 / den);
  uint16_t* xo = a.x_out + (size_t)blockIdx.x * d;
#pragma unroll
  for (int q = 0; q < kRouteMaxR; ++q) {
    const int j = tid * 4 + 1024 * q;
    if (j < d) {
      const uint32_t b0 = bf16_of_quotient(rv[q].x, den, inv), b1 = bf16_of_quotient(rv[q].y, den, inv);
      const uint32_t b2 = bf16_of_quotient(rv[q].z, den, inv), b3 = bf16_of_quotient(rv[q].w, den, inv);
      *reinterpret_cast<uint2*>(xo + j) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
    }
  }
}

// ---------------------------------------------------------------------------
// Logits for 2..64 tokens on float64 MFMA (v_mfma_f64_16x16x4f64), from the
// bf16 x that route_norm_kernel wrote.  grid = (ceil(n_tok / 16), d / 128),
// block = 64 * ceil(E / 16) threads.  Workgroup (m, g) owns tokens 16m.. and
// columns 128g..; lane l of wave w feeds 32 columns of token 16m + (l & 15)
// (columns 128g + 32 (l >> 4) + [0, 32)) as the A operand and the same
// columns of router row 16w + (l & 15) as the B operand.  MFMA step s takes
// offset s of every lane's run, so the four k of a step are 32 columns apart.
// The bf16 products are exact and the 128 of them are summed in float64; the
// partial logits of the column group go to partial[g][t][e], and the top-k
// kernel adds the d / 128 partials in order, then the bias.
// ---------------------------------------------------------------------------
typedef double f64x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(1024) void route_logits_mfma_kernel(RouteArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int d = a.d, t0 = blockIdx.x * 16, k0 = blockIdx.y * kRouteGroupCols;
  const int nt = min(16, a.n_tok - t0);
  const int j = lane & 15, kq = lane >> 4;
  const int e = wave * 16 + j;
  const bool tok_ok = j < nt;
  uint4 wv[4], xv[4];
  const uint16_t* wrow = a.w_router + (size_t)(e < a.E ? e : 0) * d + k0 + 32 * kq;
  const uint16_t* xrow = a.x_out + (size_t)(t0 + (tok_ok ? j : 0)) * d + k0 + 32 * kq;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    wv[q] = e < a.E ? *reinterpret_cast<const uint4*>(wrow + 8 * q) : make_uint4(0, 0, 0, 0);
    xv[q] = tok_ok ? *reinterpret_cast<const uint4*>(xrow + 8 * q) : make_uint4(0, 0, 0, 0);
  }
  const uint32_t xb[16] = {xv[0].x, xv[0].y, xv[0].z, xv[0].w, xv[1].x, xv[1].y, xv[1].z, xv[1].w,
                           xv[2].x, xv[2].y, xv[2].z, xv[2].w, xv[3].x, xv[3].y, xv[3].z, xv[3].w};
  const uint32_t wb[16] = {wv[0].x, wv[0].y, wv[0].z, wv[0].w, wv[1].x, wv[1].y, wv[1].z, wv[1].w,
                           wv[2].x, wv[2].y, wv[2].z, wv[2].w, wv[3].x, wv[3].y, wv[3].z, wv[3].w};
  f64x4_t acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int s = 0; s < 32; ++s) {
    const double xa = (double)bf16_to_f32((xb[s >> 1] >> (16 * (s & 1))) & 0xFFFFu);
    const double wbv = (double)bf16_to_f32((wb[s >> 1] >> (16 * (s & 1))) & 0xFFFFu);
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(xa, wbv, acc, 0, 0, 0);
  }
  // D layout (measured): lane l, register r holds row 4 r + (l >> 4) (token),
  // column l & 15 (expert)
  double* out = a.partial + (size_t)blockIdx.y * a.n_tok * a.E;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int tt = 4 * r + kq;
    if (tt < nt && e < a.E) out[(size_t)(t0 + tt) * a.E + e] = acc[r];
  }
}

// Top-k for each token: one workgroup of 1024 threads per token (the rank
// count is spread over 8 slices of the experts).  Optionally also publishes the
// selected blob pointers from the layer's table and copies of the routing.
__global__ __launch_bounds__(1024) void route_topk_kernel(TopkArgs a) {
  __shared__ TopkShared tk;
  const int t = blockIdx.x, tid = threadIdx.x;
  if (tid < a.E) {  // a NaN logit (from a non-finite residual) ranks as -inf
    double l;
    if (a.groups > 0) {  // the partials in order, eight loads in flight at a time
      const double* p = a.partial + (size_t)t * a.E + tid;
      const size_t step = (size_t)a.n_tok * a.E;
      l = 0.0;
      for (int g0 = 0; g0 < a.groups; g0 += 8) {
        double v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = g0 + u < a.groups ? p[(size_t)(g0 + u) * step] : 0.0;
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (g0 + u < a.groups) l = (g0 + u == 0) ? v[u] : l + v[u];
      }
      if (a.bias) l += (double)a.bias[tid];
    } else {
      l = a.logits[(size_t)t * a.E + tid];
    }
    tk.log[tid] = l == l ? l : -__builtin_inf();
  }
  __syncthreads();
  topk_block(tk, a.E, a.k, a.norm);
  if (tid < a.k) {
    const size_t o = (size_t)t * a.k + tid;
    const int e = tk.idx[tid];
    a.idx[o] = e;
    a.w[o] = tk.w[tid];
    if (a.ptr_out) a.ptr_out[o] = a.table[e];
    if (a.idx_rec) a.idx_rec[o] = e;
    if (a.w_rec) a.w_rec[o] = tk.w[tid];
  }
  if (a.next_idx && tid < a.E) {  // the ranking past k, from the same exact ranks
    const int rk = tk.rank[tid] - a.k;
    if (rk >= 0 && rk < a.n_next) a.next_idx[(size_t)t * a.n_next + rk] = tid;
  }
}

hipError_t launch_route_logits(const RouteArgs& a, hipStream_t s, int* groups) {
  *groups = 0;
  if (a.n_tok >= 2) {  // d % 128 == 0 and E <= 256 are checked with the dims
    if (!a.partial || !a.x_out || a.d % kRouteGroupCols || a.d > 1024 * kRouteMaxR || a.E > 256 ||
        a.n_tok > 64)
      return hipErrorInvalidValue;
    *groups = a.d / kRouteGroupCols;
    hipLaunchKernelGGL(route_norm_kernel, dim3(a.n_tok), dim3(256), 0, s, a);
    hipLaunchKernelGGL(route_logits_mfma_kernel, dim3((a.n_tok + 15) / 16, *groups), dim3(64 * ((a.E + 15) / 16)),
                       0, s, a);
  } else if (a.n_tok == 1 && a.d % 256 == 0 && a.d <= 8192) {
    hipLaunchKernelGGL(route_logits_decode_kernel, dim3(a.E), dim3(64 * ((a.d + 511) / 512)), 0, s, a.w_router,
                       a.residual, a.d, a);
  } else {
    return hipErrorInvalidValue;  // (the dims checks admit no other shape)
  }
  return hipGetLastError();
}

hipError_t launch_route_topk(const TopkArgs& a, int n_tok, hipStream_t s) {
  hipLaunchKernelGGL(route_topk_kernel, dim3(n_tok), dim3(1024), 0, s, a);
  return hipGetLastError();
}

}  // namespace smoe
