// Exact router: RMSNorm -> bf16 x, float64 gate matvec, top-k, mixing weights.
//
// "Routing Is Exact" (Optimizations page) and the per-token step table of the
// System Overview page: every MoE layer evaluates the real E x d_model router
// gate on the true hidden state, then top-k and norm_topk_prob weights as
// Qwen3 defines them (softmax over all E, keep the k largest, renormalise).
// The pages run this gate on the CPU; here the norm and the gate run on the
// GPU, as the pages' own "GPU-Resident Epilogue" plan (Optimizations, "The
// Dense Ceiling") proposes.
#include "kernels.h"

namespace smoe {

// ---------------------------------------------------------------------------
// RMSNorm + logits.  grid = (ceil(E / 4), ceil(n_tok / TB)); 256 threads.
// Each workgroup normalises its TB tokens into LDS (redundantly across the
// expert blocks: the residual is tiny and L2-resident), then each wave computes
// one expert row's dot products for all TB tokens.  Every bf16*bf16 product is
// exact in fp32; partial sums are float64.
// ---------------------------------------------------------------------------
template <int TB>
__global__ __launch_bounds__(256) void route_logits_kernel(RouteArgs a) {
  extern __shared__ uint16_t xs[];  // [TB][d]
  __shared__ double red[TB][4];
  __shared__ double rms_den[TB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.y * TB;
  const int nt = min(TB, a.n_tok - t0);
  const int d = a.d;

  // --- RMSNorm: sum of squares in float64, fixed reduction tree
  for (int t = 0; t < nt; ++t) {
    const float* r = a.residual + (size_t)(t0 + t) * d;
    double s = 0.0;
    for (int j = tid * 4; j < d; j += 256 * 4) {
      const float4 v = *reinterpret_cast<const float4*>(r + j);
      s += (double)v.x * v.x + (double)v.y * v.y + (double)v.z * v.z + (double)v.w * v.w;
    }
    s = group_sum_f64<64>(s);
    if (lane == 0) red[t][wave] = s;
  }
  __syncthreads();
  if (tid < nt) {
    const double ss = (red[tid][0] + red[tid][1]) + (red[tid][2] + red[tid][3]);
    rms_den[tid] = sqrt(ss / (double)d + (double)a.eps);
  }
  __syncthreads();
  for (int t = 0; t < nt; ++t) {
    const float* r = a.residual + (size_t)(t0 + t) * d;
    const double den = rms_den[t];
    for (int j = tid * 4; j < d; j += 256 * 4) {
      const float4 v = *reinterpret_cast<const float4*>(r + j);
      const uint32_t b0 = f64_to_bf16_rne((double)v.x / den), b1 = f64_to_bf16_rne((double)v.y / den);
      const uint32_t b2 = f64_to_bf16_rne((double)v.z / den), b3 = f64_to_bf16_rne((double)v.w / den);
      const uint2 packed = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
      *reinterpret_cast<uint2*>(xs + (size_t)t * d + j) = packed;
      if (blockIdx.x == 0 && a.x_out) *reinterpret_cast<uint2*>(a.x_out + (size_t)(t0 + t) * d + j) = packed;
    }
  }
  __syncthreads();

  // --- logits: one expert row per wave, 8 bf16 per lane per step
  const int e = blockIdx.x * 4 + wave;
  if (e >= a.E) return;
  const uint16_t* w = a.w_router + (size_t)e * d;
  double acc[TB];
#pragma unroll
  for (int t = 0; t < TB; ++t) acc[t] = 0.0;
  for (int j = lane * 8; j < d; j += 64 * 8) {
    const uint4 wv = *reinterpret_cast<const uint4*>(w + j);
    float wf[8];
    wf[0] = bf16_to_f32(wv.x & 0xFFFF); wf[1] = bf16_to_f32(wv.x >> 16);
    wf[2] = bf16_to_f32(wv.y & 0xFFFF); wf[3] = bf16_to_f32(wv.y >> 16);
    wf[4] = bf16_to_f32(wv.z & 0xFFFF); wf[5] = bf16_to_f32(wv.z >> 16);
    wf[6] = bf16_to_f32(wv.w & 0xFFFF); wf[7] = bf16_to_f32(wv.w >> 16);
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      if (t < nt) {
        const uint4 xv = *reinterpret_cast<const uint4*>(xs + (size_t)t * d + j);
        const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
        double s = 0.0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // products of two bf16 values are exact in fp32
          s += (double)(wf[2 * i] * bf16_to_f32(xw[i] & 0xFFFF));
          s += (double)(wf[2 * i + 1] * bf16_to_f32(xw[i] >> 16));
        }
        acc[t] += s;
      }
    }
  }
  const double b = a.bias ? (double)a.bias[e] : 0.0;
#pragma unroll
  for (int t = 0; t < TB; ++t) {
    if (t < nt) {
      const double v = group_sum_f64<64>(acc[t]);
      if (lane == 0) a.logits[(size_t)(t0 + t) * a.E + e] = v + b;
    }
  }
}

// One wave per token.  grid = ceil(n_tok / 4), 256 threads.
__global__ __launch_bounds__(256) void route_topk_kernel(const double* logits, int n_tok, int E, int k,
                                                         int norm, int32_t* idx, float* w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= n_tok) return;
  topk_wave(logits + (size_t)t * E, E, k, norm, idx + (size_t)t * k, w + (size_t)t * k);
}

hipError_t launch_route_logits(const RouteArgs& a, hipStream_t s) {
  const int eb = (a.E + 3) / 4;
  // tokens per workgroup: the normalised inputs of TB tokens live in LDS
  if (a.n_tok <= 1) {
    hipLaunchKernelGGL(route_logits_kernel<1>, dim3(eb, a.n_tok), dim3(256), (size_t)a.d * 2, s, a);
  } else if (a.d > 4096) {
    hipLaunchKernelGGL(route_logits_kernel<2>, dim3(eb, (a.n_tok + 1) / 2), dim3(256), (size_t)a.d * 2 * 2,
                       s, a);
  } else {
    hipLaunchKernelGGL(route_logits_kernel<4>, dim3(eb, (a.n_tok + 3) / 4), dim3(256), (size_t)a.d * 2 * 4,
                       s, a);
  }
  return hipGetLastError();
}

hipError_t launch_route_topk(const double* logits, int n_tok, int E, int k, int norm, int32_t* idx,
                             float* w, hipStream_t s) {
  hipLaunchKernelGGL(route_topk_kernel, dim3((n_tok + 3) / 4), dim3(256), 0, s, logits, n_tok, E, k,
                     norm, idx, w);
  return hipGetLastError();
}

}  // namespace smoe
