// Kernel argument blocks and launchers (internal to the library).
#pragma once

#include "smoe_internal.h"

namespace smoe {

// ---------------------------------------------------------------------------
// top-k of one token's E float64 logits by one wave: k rounds of a wave-wide
// argmax on (logit, -index).  Results in rank order.  Weights in float64.
// ---------------------------------------------------------------------------
__device__ inline void topk_wave(const double* logits, int E, int k, int norm, int* idx_out, float* w_out) {
  const int lane = threadIdx.x & 63;
  double v[4];
  int id[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    id[i] = lane + 64 * i;
    v[i] = id[i] < E ? logits[id[i]] : -INFINITY;
  }
  bool taken[4] = {id[0] >= E, id[1] >= E, id[2] >= E, id[3] >= E};
  double sel_v[kMaxTopK];
  int sel_i[kMaxTopK];
  for (int r = 0; r < k; ++r) {
    double bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (!taken[i] && (v[i] > bv || (v[i] == bv && id[i] < bi))) { bv = v[i]; bi = id[i]; }
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const double ov = __shfl_xor(bv, m, 64);
      const int oi = __shfl_xor(bi, m, 64);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) if (id[i] == bi) taken[i] = true;
    sel_v[r] = bv;
    sel_i[r] = bi;
  }
  // softmax over all E at the selected logits; renormalise over the k if asked
  const double lmax = sel_v[0];
  double den;
  if (norm) {
    den = 0.0;
    for (int r = 0; r < k; ++r) den += exp(sel_v[r] - lmax);
  } else {
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) if (id[i] < E) s += exp(v[i] - lmax);
    den = group_sum_f64<64>(s);
  }
  if (lane == 0) {
    for (int r = 0; r < k; ++r) {
      idx_out[r] = sel_i[r];
      w_out[r] = (float)(exp(sel_v[r] - lmax) / den);
    }
  }
}

struct RouteArgs {
  const float* residual;    // [n_tok][d]
  uint16_t* x_out;          // [n_tok][d] bf16, or null
  const uint16_t* w_router; // [E][d] bf16
  const float* bias;        // [E] or null
  double* logits;           // [n_tok][E]
  int n_tok, d, E;
  float eps;
};

hipError_t launch_route_logits(const RouteArgs& a, hipStream_t s);
hipError_t launch_route_topk(const double* logits, int n_tok, int E, int k, int norm, int32_t* idx,
                             float* w, hipStream_t s);

// Where the k experts of a decode step come from.
struct ExpertSource {
  const int32_t* idx;               // [k] device (rank order), used when direct[0] == null
  const void* const* table;         // [E] device blob pointers
  const void* direct[kMaxTopK];     // blob pointers passed by value (ring slots)
};

struct DecodeArgs {
  const uint16_t* x;        // [d] bf16
  ExpertSource src;
  const float* w;           // [k] mixing weights (device), read by the down kernel
  // fused routing (gate/up kernel computes top-k from logits when non-null)
  const double* logits;     // [E]
  int32_t* idx_ws;          // [k] written by block 0 when routing is fused
  float* w_ws;              // [k]
  int32_t* idx_rec;         // optional copies of the routing
  float* w_rec;
  _Float16* h;              // [k][d_ff], pair-ordered within groups of 8
  float* residual;          // [d]
  int d, f, E, k, chunk, norm;
  BlobLayout lay;
};

hipError_t launch_decode_gate_up(const DecodeArgs& a, hipStream_t s, hipEvent_t start = nullptr,
                                 hipEvent_t stop = nullptr);
hipError_t launch_decode_down(const DecodeArgs& a, hipStream_t s);
bool decode_shape_supported(int d, int f, int chunk);

}  // namespace smoe
