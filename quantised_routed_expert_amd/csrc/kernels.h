// Kernel argument blocks, the block-wide top-k, and launchers (internal).
#pragma once

#include "smoe_internal.h"

namespace smoe {

// ---------------------------------------------------------------------------
// Exact top-k of E <= 256 float64 logits by one workgroup of NT threads
// (NT a multiple of 128 when E <= 128, of 256 otherwise).
// Order: logit descending, equal logits -> lower expert index first.  The rank
// of expert i is the number of experts that beat it; thread t counts the
// beaters of expert t % EP over one slice of the others (broadcast LDS reads,
// no cross-lane shuffles), the slices are summed, and the experts of rank < k
// land in rank order.  Weights: softmax over all E at the selected logits,
// renormalised over the k when `norm` (Qwen3's norm_topk_prob), in float64.
// `s.log` must hold the E logits before the call; every thread must call it.
// ---------------------------------------------------------------------------
constexpr int kTopkMaxSlices = 8;

struct alignas(16) TopkShared {
  double log[kMaxExperts];
  alignas(16) float logf[kMaxExperts];  // the logits rounded to float (topk_select_fast*)
  int part[kTopkMaxSlices][kMaxExperts];
  int idx[kMaxTopK];
  int rank[kMaxExperts];     // exact rank of every expert (topk_select)
  double val[kMaxTopK];
  double ex[kMaxExperts];
  float w[kMaxTopK];
};

// Selection only: s.idx / s.val in rank order (ends with a barrier).
__device__ inline void topk_select(TopkShared& s, int E, int k) {
  const int t = threadIdx.x, nt = blockDim.x;
  const int ep = E <= 128 ? 128 : 256;  // experts per slice row
  int slices = nt / ep;
  if (slices > kTopkMaxSlices) slices = kTopkMaxSlices;
  const int i = t % ep, h = t / ep;
  if (h < slices && i < E) {
    const int span = (E + slices - 1) / slices;
    const int j0 = h * span, j1 = min(E, j0 + span);
    const double li = s.log[i];
    int cnt = 0;
#pragma unroll 4
    for (int j = j0; j < j1; ++j) {
      const double lj = s.log[j];
      cnt += (lj > li) | ((lj == li) & (j < i));
    }
    s.part[h][i] = cnt;
  }
  __syncthreads();
  if (t < E) {
    int rank = 0;
    for (int q = 0; q < slices; ++q) rank += s.part[q][t];
    s.rank[t] = rank;
    if (rank < k) {
      s.idx[rank] = t;
      s.val[rank] = s.log[t];
    }
  }
  __syncthreads();
}

// The same selection, fast path, for a workgroup of NW >= ceil(E / 64) waves.
// Experts are split into G = ceil(E / 64) groups of 64 (one per lane) and the
// logits into S = NW / G slices (multiples of 16); wave w takes group w % G
// and slice w / G and counts, per expert i, c_i = #{j : f_j >= f_i} over its
// slice, where f = the logits rounded to float (monotone, so f_j > f_i implies
// l_j > l_i and f_j < f_i implies l_j < l_i).  Slices are read from LDS at
// wave-uniform addresses (broadcast reads, 16 in flight).  Without float ties
// touching the top k, rank_i = c_i - 1 exactly, and each expert of rank < k
// writes its id, logit and table entry to its rank's slot.  Any tie that
// touches the top k (float or exact) leaves some slot unclaimed, since every
// member of a tied group claims the group's last rank; the workgroup then
// falls back to the exact float64 rank counting of topk_select.
// Before the call: s.log / s.logf hold the E logits followed by -inf up to
// kMaxExperts, s.idx[0..k) = -1, and a barrier has made them visible.  `tab`
// (E entries, may be null) is looked up into `slot_ptr` (k entries, shared
// memory).  Ends with a barrier.
__device__ inline void topk_select_fast(TopkShared& s, int E, int k, const void* const* tab,
                                        const void** slot_ptr) {
  const int t = threadIdx.x, lane = t & 63;
  const int nw = blockDim.x >> 6;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int G = (E + 63) >> 6;
  int S = nw / G < kTopkMaxSlices ? nw / G : kTopkMaxSlices;
  int span = (((E + S - 1) / S) + 15) & ~15;
  while (S > 1 && S * span > kMaxExperts) {
    --S;
    span = (((E + S - 1) / S) + 15) & ~15;
  }
  const int g = w % G, sl = w / G;
  if (sl < S) {
    const int i = 64 * g + lane;
    const float x = i < E ? s.logf[i] : __builtin_inff();
    const int j0 = sl * span;
    int c = 0;
    for (int j = j0; j < j0 + span; j += 16) {
      float v[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) v[q] = s.logf[j + q];
#pragma unroll
      for (int q = 0; q < 16; ++q) c += (v[q] >= x) ? 1 : 0;
    }
    s.part[sl][i] = c;
  }
  __syncthreads();
  if (t < E) {
    int c = 0;
    for (int q = 0; q < S; ++q) c += s.part[q][t];
    if (c >= 1 && c <= k) {
      s.idx[c - 1] = t;
      s.val[c - 1] = s.log[t];
      if (tab) slot_ptr[c - 1] = tab[t];
    }
  }
  __syncthreads();
  bool ok = true;
  for (int r = 0; r < k; ++r) ok &= s.idx[r] >= 0;
  if (!ok) {  // uniform: every thread read the same slots
    topk_select(s, E, k);
    if (tab && t < k) slot_ptr[t] = tab[s.idx[t]];
    __syncthreads();
  }
}

// The same fast path for E <= 128 on a workgroup of exactly NT threads (a
// multiple of 128), with every bound fixed at compile time: thread t counts
// for expert t % 128 over slice t / 128 of the (padded) float logits, read
// from LDS four at a time at wave-uniform addresses; the slices' counts are
// added once.  Preconditions as for topk_select_fast, with s.logf padded with
// -inf up to S * SPAN.
template <int NT>
__device__ inline void topk_select_fast128(TopkShared& s, int E, int k, const void* const* tab,
                                           const void** slot_ptr) {
  constexpr int S = NT / 128;                          // slices
  constexpr int SPAN = ((128 + S - 1) / S + 3) & ~3;   // logits per slice, a multiple of 4
  static_assert(NT % 128 == 0 && S <= kTopkMaxSlices && S * SPAN <= kMaxExperts, "slice layout");
  const int t = threadIdx.x;
  const int i = t & 127, h = t >> 7;
  const float x = s.logf[i];
  const float4* v4 = reinterpret_cast<const float4*>(s.logf + SPAN * h);
  int c = 0;
#pragma unroll
  for (int q = 0; q < SPAN / 4; ++q) {
    const float4 v = v4[q];
    c += (v.x >= x ? 1 : 0) + (v.y >= x ? 1 : 0) + (v.z >= x ? 1 : 0) + (v.w >= x ? 1 : 0);
  }
  s.part[h][i] = c;
  __syncthreads();
  if (t < E) {
    c = 0;
#pragma unroll
    for (int q = 0; q < S; ++q) c += s.part[q][t];
    if (c >= 1 && c <= k) {
      s.idx[c - 1] = t;
      s.val[c - 1] = s.log[t];
      if (tab) slot_ptr[c - 1] = tab[t];
    }
  }
  __syncthreads();
  bool ok = true;
#pragma unroll
  for (int r = 0; r < kMaxTopK; ++r) ok &= (r >= k) || (s.idx[r] >= 0);
  if (!ok) {  // uniform: every thread read the same slots
    topk_select(s, E, k);
    if (tab && t < k) slot_ptr[t] = tab[s.idx[t]];
    __syncthreads();
  }
}

// Mixing weights of the selected experts: s.w (ends with a barrier).
__device__ inline void topk_weights(TopkShared& s, int E, int k, int norm) {
  const int t = threadIdx.x;
  const double lmax = s.val[0];
  if (norm) {
    if (t < k) s.ex[t] = exp(s.val[t] - lmax);
  } else {
    if (t < E) s.ex[t] = exp(s.log[t] - lmax);
  }
  __syncthreads();
  if (t < k) {
    const int n = norm ? k : E;
    double den = 0.0;
    for (int j = 0; j < n; ++j) den += s.ex[j];
    const double num = norm ? s.ex[t] : exp(s.val[t] - lmax);
    s.w[t] = (float)(num / den);
  }
  __syncthreads();
}

__device__ inline void topk_block(TopkShared& s, int E, int k, int norm) {
  topk_select(s, E, k);
  topk_weights(s, E, k, norm);
}

struct RouteArgs {
  const float* residual;    // [n_tok][d]
  uint16_t* x_out;          // [n_tok][d] bf16, or null
  _Float16* px_out;         // [d] the same values as f16 in pair order (one token), or null
  const uint16_t* w_router; // [E][d] bf16
  const float* bias;        // [E] or null
  double* logits;           // [n_tok][E]
  int n_tok, d, E;
  float eps;
  double* partial;          // [d / kRouteGroupCols][n_tok][E] workspace for the MFMA path, or null
  int px16;                 // px_out pair order: 0 = groups of 8 (SMOE-Q4), 1 = groups of 16 (SMOE-Q2)
};

// Columns per workgroup of the multi-token MFMA router: its partial logits
// are added (bias last) by the top-k kernel.
constexpr int kRouteGroupCols = 128;

// Launches the logits kernel for a.n_tok tokens.  *groups = 0 when the logits
// were written to a.logits (bias included), else the number of column-group
// partials written to a.partial (no bias) that the top-k kernel must add.
hipError_t launch_route_logits(const RouteArgs& a, hipStream_t s, int* groups);

struct TopkArgs {
  const double* logits;      // [n_tok][E] (groups == 0)
  const double* partial;     // [groups][n_tok][E] partial logits, added in order (groups > 0)
  const float* bias;         // [E] added to the partial sums, or null
  int groups, n_tok;
  int32_t* idx;              // [n_tok][k]
  float* w;                  // [n_tok][k]
  const void* const* table;  // [E] blob pointers of the layer (with ptr_out)
  const void** ptr_out;      // [n_tok][k] selected blob pointers, or null
  int32_t* idx_rec;          // optional copies
  float* w_rec;
  int32_t* next_idx;         // [n_tok][n_next] experts at ranks k .. k + n_next - 1, or null
  int n_next;
  int E, k, norm;
};
hipError_t launch_route_topk(const TopkArgs& a, int n_tok, hipStream_t s);

// A layer's expert table, passed by value (2 KiB of kernel arguments).
struct RingTable {
  const void* ptr[kMaxExperts];
};
hipError_t launch_ring_table(const RingTable& t, const void** table, int E, hipStream_t s);

// Where the k experts of a decode step come from.
struct ExpertSource {
  const int32_t* idx;               // [k] device (rank order), used when direct[0] == null
  const void* const* table;         // [E] device blob pointers
  const void* direct[kMaxTopK];     // blob pointers passed by value (ring slots)
};

// Router rows per workgroup of the one-token logits kernel; the down kernel
// uses it to prefetch the next layer's router rows per XCD.
constexpr int kRouteDecRowsPerWG = 1;
constexpr int kXcds = 8;  // MI355X: workgroup i is dispatched to XCD i % 8

// Selection inside the gate/up kernel: every workgroup ranks the layer's E
// logits itself (the selection is deterministic, so all agree) and looks its
// experts up in src.table; workgroup 0 publishes ids, weights and pointers for
// the down kernel and the optional records.
struct FusedTopk {
  const double* logits;     // [E], or null: the experts come from src / ptrs
  int32_t* idx_out;         // [k]
  float* w_out;             // [k]
  const void** ptr_out;     // [k]
  int32_t* idx_rec;         // [k] or null
  float* w_rec;             // [k] or null
};

struct DecodeArgs {
  const uint16_t* x;        // [d] bf16
  const _Float16* px;       // [d] x as f16 in pair order, or null (then x is converted)
  ExpertSource src;
  FusedTopk sel;
  const float* w;           // [k] mixing weights (device), read by the down kernel
  const void* const* ptrs;   // [k] device blob pointers from the router, or null
  float* h;                 // [k][d_ff] SwiGLU activations, fp32 in natural order
  float* residual;          // [d]
  const uint8_t* pf_base;   // next layer's router [E][d] bf16 to pull into cache, or null
  int d, f, E, k, chunk, norm;
  int bits;                 // code width: 4 (SMOE-Q4) or 2 (SMOE-Q2)
  BlobLayout lay;
};

hipError_t launch_decode_gate_up(const DecodeArgs& a, hipStream_t s, hipEvent_t start = nullptr,
                                 hipEvent_t stop = nullptr);
hipError_t launch_decode_down(const DecodeArgs& a, hipStream_t s);
bool decode_shape_supported(int d, int f, int chunk, int bits);

}  // namespace smoe
