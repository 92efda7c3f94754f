// Prefill (layer-major, one chunk of at most 64 tokens) argument block (internal).
#pragma once

#include "kernels.h"

namespace smoe {

struct PrefillArgs {
  const uint16_t* x;          // [T][d] bf16 (the router's RMSNorm output)
  const int32_t* idx;         // [T][k]
  const float* w;             // [T][k]
  const void* const* table;   // [E] blob pointers of the layer
  float* residual;            // [T][d]
  int32_t* union_ids;         // [min(E, T*k)]
  int32_t* union_count;       // [1]
  int32_t* offsets;           // [min(E, T*k) + 1]
  int32_t* perm;              // [T*k]
  int32_t* invperm;           // [T*k] position of entry t*k+r in perm (workspace)
  int32_t* slices;            // [T*k/16 + min(E, T*k)] (u << 8 | s): slice s = entries
                              // 16 s .. 16 s + 15 of union expert u (workspace)
  int32_t* n_slices;          // [1] (workspace)
  struct SliceRec {           // one slice, ready for a GEMM workgroup: its blob,
    const void* blob;         // first entry (in perm order) and entry count
    int32_t o, n_rows;
  }* recs;                    // [prefill max slices] (workspace, 16-byte aligned)
  _Float16* H;                // [T*k][f] SwiGLU activations, fp16 in the pair order of
                              // the code width (groups of 8 for Q4, 16 for SMOE-Q2), each
                              // row's 64-feature tile scaled by a power of two
  float* Hs;                  // [T*k][f / 64] inverse scale of each tile: H = fp16 * Hs
  float* Y;                   // [T*k][d] per-entry expert outputs
  _Float16* xa;               // [T][d] the chunk's x as the folded gate/up GEMM's A operand: fp16
                              // in pair order (groups of 8: e_p, e_{p+4}), odd dwords divided by 16
  float* xas;                 // [T][d / 64] sum of each chunk of 64 x values (before the division)
  int T, d, f, E, k, chunk;
  int bits;                   // code width: 4 (SMOE-Q4) or 2 (SMOE-Q2)
  BlobLayout lay;
};

// ev: null, or 4 events recorded around the gate/up GEMM (0, 1) and the down GEMM (2, 3)
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s, const hipEvent_t* ev = nullptr);

// Upper bound on the number of 16-entry slices of a chunk's union experts.
inline int prefill_max_slices(int T, int k, int E) { return (T * k + 15) / 16 + (E < T * k ? E : T * k); }

}  // namespace smoe
