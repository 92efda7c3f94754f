// C ABI entry points: argument validation, workspace carving, kernel launches.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>

#include "kernels.h"
#include "prefill.h"


namespace smoe {

static thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

static int hip_fail(hipError_t e, const char* what) {
  return fail(SMOE_EHIP, "%s: %s", what, hipGetErrorString(e));
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Code width of the dims' blobs (0 is read as 4).
static int quant_bits(const smoe_dims* d) { return d->quant_bits == 0 ? 4 : d->quant_bits; }

int check_dims(const smoe_dims* d) {
  if (!d) return fail(SMOE_EINVAL, "dims is NULL");
  if (d->d_model <= 0 || d->d_model > 8192 || d->d_model % 256)
    return fail(SMOE_EINVAL, "d_model=%d must be a multiple of 256 in [256, 8192]", d->d_model);
  if (d->d_ff <= 0 || d->d_ff > 8192 || d->d_ff % 128)
    return fail(SMOE_EINVAL, "d_ff=%d must be a multiple of 128 in [128, 8192]", d->d_ff);
  if (d->n_experts < 1 || d->n_experts > kMaxExperts)
    return fail(SMOE_EINVAL, "n_experts=%d must be in [1, %d]", d->n_experts, kMaxExperts);
  if (d->top_k < 1 || d->top_k > d->n_experts || d->top_k > kMaxTopK)
    return fail(SMOE_EINVAL, "top_k=%d must be in [1, min(n_experts, %d)]", d->top_k, kMaxTopK);
  if (d->chunk != 32 && d->chunk != 64) return fail(SMOE_EINVAL, "chunk=%d must be 32 or 64", d->chunk);
  if (!(d->rms_eps >= 0.0f) || d->rms_eps > 1.0f) return fail(SMOE_EINVAL, "rms_eps out of range");
  const int bits = quant_bits(d);
  if (bits != 4 && bits != 2) return fail(SMOE_EINVAL, "quant_bits=%d must be 4 (or 0) or 2", d->quant_bits);
  if (bits == 2 && (d->chunk != 64 || d->d_model % 512))
    return fail(SMOE_EINVAL, "SMOE-Q2 needs chunk 64 and d_model a multiple of 512 (chunk=%d d_model=%d)",
                d->chunk, d->d_model);
  if (!decode_shape_supported(d->d_model, d->d_ff, d->chunk, bits))
    return fail(SMOE_EINVAL, "unsupported row split for d_model=%d d_ff=%d", d->d_model, d->d_ff);
  return SMOE_OK;
}

// Workspace carve-up (offsets from the workspace base, 256-byte aligned).
struct Workspace {
  size_t logits, plog, idx, w, ptr, x, px, h, ph, phs, py, pxa, pxas, pinv, slices, recs, end;
};

Workspace ws_layout(const smoe_dims* d, int max_tokens) {
  Workspace w;
  const size_t T = (size_t)(max_tokens < 1 ? 1 : max_tokens);
  const size_t E = d->n_experts, k = d->top_k, D = d->d_model, F = d->d_ff;
  size_t o = 0;
  w.logits = o; o = align_up(o + T * E * 8, 256);
  w.plog = o;   o = align_up(o + (size_t)(d->d_model / kRouteGroupCols) * T * E * 8, 256);
  w.idx = o;    o = align_up(o + k * 4, 256);
  w.w = o;      o = align_up(o + k * 4, 256);
  w.ptr = o;    o = align_up(o + k * 8, 256);
  w.x = o;      o = align_up(o + T * D * 2, 256);
  w.px = o;     o = align_up(o + D * 2, 256);
  w.h = o;      o = align_up(o + k * F * 4, 256);
  w.ph = o;     o = align_up(o + T * k * F * 2, 256);
  w.phs = o;    o = align_up(o + T * k * (F / 64) * 4, 256);
  w.py = o;     o = align_up(o + T * k * D * 4, 256);
  w.pxa = o;    o = align_up(o + T * D * 2, 256);
  w.pxas = o;   o = align_up(o + T * (D / 64) * 4, 256);
  w.pinv = o;   o = align_up(o + T * k * 4, 256);
  w.slices = o; o = align_up(o + ((T * k + 15) / 16 + (E < T * k ? E : T * k) + 1) * 4, 256);
  w.recs = o;   o = align_up(o + ((T * k + 15) / 16 + (E < T * k ? E : T * k)) * 16, 256);
  w.end = o;
  return w;
}

static int check_ws(const smoe_dims* d, int tokens, const void* ws, size_t bytes, Workspace* out) {
  *out = ws_layout(d, tokens);
  if (!ws) return fail(SMOE_EINVAL, "workspace is NULL");
  if (((uintptr_t)ws & 255u) != 0) return fail(SMOE_EINVAL, "workspace must be 256-byte aligned");
  if (bytes < out->end)
    return fail(SMOE_EINVAL, "workspace too small: %zu < %zu bytes", bytes, out->end);
  return SMOE_OK;
}

static DecodeArgs decode_args(const smoe_dims* d, char* ws, const Workspace& L) {
  DecodeArgs a;
  memset(&a, 0, sizeof(a));
  a.d = d->d_model;
  a.f = d->d_ff;
  a.E = d->n_experts;
  a.k = d->top_k;
  a.chunk = d->chunk;
  a.norm = d->norm_topk_prob ? 1 : 0;
  a.bits = quant_bits(d);
  a.lay = blob_layout(d->d_model, d->d_ff, d->chunk, a.bits);
  a.h = reinterpret_cast<float*>(ws + L.h);
  return a;
}

// The chained decode of smoe_decode_layers on a carved workspace.
static int decode_layers_on(const smoe_dims* d, int32_t n_layers, float* residual, const uint16_t* w_router,
                            const float* bias, const void* const* expert_tables, uint16_t* x_rec, int32_t* idx_rec,
                            float* w_rec, void* const* events, char* base, const Workspace& L, hipStream_t s) {
  double* logits = reinterpret_cast<double*>(base + L.logits);
  uint16_t* xbuf = reinterpret_cast<uint16_t*>(base + L.x);
  const size_t D = d->d_model, E = d->n_experts, K = d->top_k;
  for (int layer = 0; layer < n_layers; ++layer) {
    uint16_t* xl = x_rec ? x_rec + (size_t)layer * D : xbuf;
    _Float16* px = reinterpret_cast<_Float16*>(base + L.px);
    const RouteArgs ra{residual, xl, px, w_router + (size_t)layer * E * D, bias ? bias + (size_t)layer * E : nullptr,
                       logits, 1, d->d_model, d->n_experts, d->rms_eps, nullptr, quant_bits(d) == 2 ? 1 : 0};
    int groups = 0;  // one token: the logits are written directly
    hipError_t he = launch_route_logits(ra, s, &groups);
    if (he != hipSuccess) return hip_fail(he, "route_logits launch");
    // the top-k selection runs inside the gate/up kernel, which publishes ids,
    // weights and blob pointers for the down kernel
    DecodeArgs a = decode_args(d, base, L);
    a.x = xl;
    a.px = px;
    a.src.table = expert_tables + (size_t)layer * E;
    a.sel.logits = logits;
    a.sel.idx_out = reinterpret_cast<int32_t*>(base + L.idx);
    a.sel.w_out = reinterpret_cast<float*>(base + L.w);
    a.sel.ptr_out = reinterpret_cast<const void**>(base + L.ptr);
    a.sel.idx_rec = idx_rec ? idx_rec + (size_t)layer * K : nullptr;
    a.sel.w_rec = w_rec ? w_rec + (size_t)layer * K : nullptr;
    a.ptrs = a.sel.ptr_out;
    a.w = a.sel.w_out;
    a.residual = residual;
    if (layer + 1 < n_layers) a.pf_base = reinterpret_cast<const uint8_t*>(w_router + (size_t)(layer + 1) * E * D);
    he = events ? launch_decode_gate_up(a, s, (hipEvent_t)events[2 * layer], (hipEvent_t)events[2 * layer + 1])
                : launch_decode_gate_up(a, s);
    if (he != hipSuccess) return hip_fail(he, "decode gate/up launch");
    he = launch_decode_down(a, s);
    if (he != hipSuccess) return hip_fail(he, "decode down launch");
  }
  return SMOE_OK;
}

static int check_decode_layers_args(const smoe_dims* d, int32_t n_layers, const float* residual,
                                    const uint16_t* w_router, const void* const* expert_tables,
                                    const uint16_t* x_rec) {
  if (!residual || !w_router || !expert_tables) return fail(SMOE_EINVAL, "NULL tensor argument");
  if (!aligned16(residual) || !aligned16(w_router) || (x_rec && !aligned16(x_rec)))
    return fail(SMOE_EINVAL, "residual, w_router and x_rec must be 16-byte aligned");
  (void)d;
  (void)n_layers;
  return SMOE_OK;
}

// ---------------------------------------------------------------------------
// Library-owned scratch for smoe_decode_layers_static (callers that cannot
// allocate).  Each GPU the library runs on holds its own copy of this array
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory: its device address is looked up once per device with
// hipGetSymbolAddress and only that address is handed to kernels.
// ---------------------------------------------------------------------------
constexpr size_t kStaticScratchBytes = (size_t)2 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
static std::atomic<void*> g_scratch_dev[kMaxDevices];

// The current device's address of `scratch`: looked up on the first call on
// that device (with it current), then read from g_scratch_dev.  Concurrent
// first calls may both look it up; they store the same address.
static int static_scratch(void** out) {
  int dev = -1;
  hipError_t he = hipGetDevice(&dev);
  if (he != hipSuccess) return hip_fail(he, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(SMOE_EINVAL, "device %d beyond the %d the library tracks", dev,
                                                 kMaxDevices);
  void* p = g_scratch_dev[dev].load(std::memory_order_acquire);
  if (!p) {
    he = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (he != hipSuccess || !p) return hip_fail(he, "hipGetSymbolAddress(scratch)");
    g_scratch_dev[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return SMOE_OK;
}

}  // namespace smoe

using namespace smoe;

extern "C" {

const char* smoe_last_error(void) { return g_err; }

int32_t smoe_version(void) { return 2; }

size_t smoe_blob_bytes(const smoe_dims* d) {
  if (check_dims(d) != SMOE_OK) return 0;
  return blob_layout(d->d_model, d->d_ff, d->chunk, quant_bits(d)).bytes;
}

size_t smoe_blob_stride(const smoe_dims* d) {
  const size_t b = smoe_blob_bytes(d);
  return (b + 16383) / 16384 * 16384;
}

size_t smoe_q4_blob_bytes(const smoe_dims* d) { return smoe_blob_bytes(d); }

size_t smoe_q4_blob_stride(const smoe_dims* d) { return smoe_blob_stride(d); }

int smoe_workspace_bytes(const smoe_dims* d, int32_t max_tokens, size_t* bytes) {
  g_err[0] = 0;
  if (int e = check_dims(d)) return e;
  if (!bytes) return fail(SMOE_EINVAL, "bytes is NULL");
  if (max_tokens < 0 || max_tokens > kMaxPrefillTokens)
    return fail(SMOE_EINVAL, "max_tokens=%d must be in [0, %d]", max_tokens, kMaxPrefillTokens);
  *bytes = ws_layout(d, max_tokens).end;
  return SMOE_OK;
}

int smoe_route(const smoe_dims* d, int32_t n_tok, const float* residual, uint16_t* x_out,
               const uint16_t* w_router, const float* bias, int32_t* topk_idx, float* topk_w, void* ws,
               size_t ws_bytes, void* stream) {
  return smoe_route_ext(d, n_tok, residual, x_out, w_router, bias, topk_idx, topk_w, 0, nullptr, ws, ws_bytes,
                        stream);
}

int smoe_route_ext(const smoe_dims* d, int32_t n_tok, const float* residual, uint16_t* x_out,
                   const uint16_t* w_router, const float* bias, int32_t* topk_idx, float* topk_w, int32_t n_next,
                   int32_t* next_idx, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (int e = check_dims(d)) return e;
  if (n_tok < 0 || n_tok > kMaxPrefillTokens)
    return fail(SMOE_EINVAL, "n_tok=%d must be in [0, %d]", n_tok, kMaxPrefillTokens);
  if (n_tok == 0) return SMOE_OK;  // nothing to route; the buffers may be NULL
  if (n_next < 0 || n_next > d->n_experts - d->top_k || (n_next > 0 && !next_idx))
    return fail(SMOE_EINVAL, "n_next=%d must be in [0, E - k] with next_idx given", n_next);
  if (!residual || !x_out || !w_router || !topk_idx || !topk_w)
    return fail(SMOE_EINVAL, "NULL tensor argument");
  if (!aligned16(residual) || !aligned16(x_out) || !aligned16(w_router))
    return fail(SMOE_EINVAL, "residual, x_out and w_router must be 16-byte aligned");
  Workspace L;
  if (int e = check_ws(d, n_tok, ws, ws_bytes, &L)) return e;
  hipStream_t s = (hipStream_t)stream;
  double* logits = reinterpret_cast<double*>((char*)ws + L.logits);
  double* partial = reinterpret_cast<double*>((char*)ws + L.plog);
  RouteArgs ra{residual, x_out, nullptr, w_router, bias, logits, n_tok, d->d_model, d->n_experts, d->rms_eps,
               partial};
  int groups = 0;
  hipError_t he = launch_route_logits(ra, s, &groups);
  if (he != hipSuccess) return hip_fail(he, "route_logits launch");
  TopkArgs ta;
  memset(&ta, 0, sizeof(ta));
  ta.logits = logits;
  ta.partial = partial;
  ta.groups = groups;
  ta.bias = bias;
  ta.n_tok = n_tok;
  ta.next_idx = n_next > 0 ? next_idx : nullptr;
  ta.n_next = n_next;
  ta.idx = topk_idx;
  ta.w = topk_w;
  ta.E = d->n_experts;
  ta.k = d->top_k;
  ta.norm = d->norm_topk_prob ? 1 : 0;
  he = launch_route_topk(ta, n_tok, s);
  if (he != hipSuccess) return hip_fail(he, "route_topk launch");
  return SMOE_OK;
}

int smoe_moe_decode(const smoe_dims* d, const uint16_t* x, const int32_t* topk_idx, const float* topk_w,
                    const void* const* expert_table, float* residual, void* ws, size_t ws_bytes,
                    void* stream) {
  g_err[0] = 0;
  if (int e = check_dims(d)) return e;
  if (!x || !topk_idx || !topk_w || !expert_table || !residual)
    return fail(SMOE_EINVAL, "NULL tensor argument");
  if (!aligned16(x) || !aligned16(residual)) return fail(SMOE_EINVAL, "x and residual must be 16-byte aligned");
  Workspace L;
  if (int e = check_ws(d, 1, ws, ws_bytes, &L)) return e;
  DecodeArgs a = decode_args(d, (char*)ws, L);
  a.x = x;
  a.src.idx = topk_idx;
  a.src.table = expert_table;
  a.w = topk_w;
  a.residual = residual;
  hipStream_t s = (hipStream_t)stream;
  hipError_t he = launch_decode_gate_up(a, s);
  if (he != hipSuccess) return hip_fail(he, "decode gate/up launch");
  he = launch_decode_down(a, s);
  if (he != hipSuccess) return hip_fail(he, "decode down launch");
  return SMOE_OK;
}

int smoe_moe_decode_slots(const smoe_dims* d, const uint16_t* x, const float* topk_w,
                          const void* const* blobs_host, float* residual, void* ws, size_t ws_bytes,
                          void* stream) {
  g_err[0] = 0;
  if (int e = check_dims(d)) return e;
  if (!x || !topk_w || !blobs_host || !residual) return fail(SMOE_EINVAL, "NULL argument");
  if (!aligned16(x) || !aligned16(residual)) return fail(SMOE_EINVAL, "x and residual must be 16-byte aligned");
  for (int r = 0; r < d->top_k; ++r)
    if (!blobs_host[r] || !aligned16(blobs_host[r]))
      return fail(SMOE_EINVAL, "blob pointer %d is NULL or not 16-byte aligned", r);
  Workspace L;
  if (int e = check_ws(d, 1, ws, ws_bytes, &L)) return e;
  DecodeArgs a = decode_args(d, (char*)ws, L);
  a.x = x;
  for (int r = 0; r < d->top_k; ++r) a.src.direct[r] = blobs_host[r];
  a.w = topk_w;
  a.residual = residual;
  hipStream_t s = (hipStream_t)stream;
  hipError_t he = launch_decode_gate_up(a, s);
  if (he != hipSuccess) return hip_fail(he, "decode gate/up launch");
  he = launch_decode_down(a, s);
  if (he != hipSuccess) return hip_fail(he, "decode down launch");
  return SMOE_OK;
}

int smoe_decode_layers(const smoe_dims* d, int32_t n_layers, float* residual, const uint16_t* w_router,
                       const float* bias, const void* const* expert_tables, uint16_t* x_rec,
                       int32_t* idx_rec, float* w_rec, void* const* events, void* ws, size_t ws_bytes,
                       void* stream) {
  g_err[0] = 0;
  if (int e = check_dims(d)) return e;
  if (n_layers < 0) return fail(SMOE_EINVAL, "n_layers=%d < 0", n_layers);
  if (n_layers == 0) return SMOE_OK;  // nothing to run; the buffers may be NULL
  if (int e = check_decode_layers_args(d, n_layers, residual, w_router, expert_tables, x_rec)) return e;
  Workspace L;
  if (int e = check_ws(d, 1, ws, ws_bytes, &L)) return e;
  return decode_layers_on(d, n_layers, residual, w_router, bias, expert_tables, x_rec, idx_rec, w_rec, events,
                          (char*)ws, L, (hipStream_t)stream);
}

int smoe_decode_layers_static(const smoe_dims* d, int32_t n_layers, float* residual, const uint16_t* w_router,
                              const float* bias, const void* const* expert_tables, uint16_t* x_rec,
                              int32_t* idx_rec, float* w_rec, void* stream) {
  g_err[0] = 0;
  if (int e = check_dims(d)) return e;
  if (n_layers < 0) return fail(SMOE_EINVAL, "n_layers=%d < 0", n_layers);
  if (n_layers == 0) return SMOE_OK;  // nothing to run; the buffers may be NULL
  if (int e = check_decode_layers_args(d, n_layers, residual, w_router, expert_tables, x_rec)) return e;
  const Workspace L = ws_layout(d, 1);
  if (L.end > kStaticScratchBytes)
    return fail(SMOE_EINVAL, "these dims need %zu bytes of scratch; the library's static scratch holds %zu",
                L.end, kStaticScratchBytes);
  void* base = nullptr;
  if (int e = static_scratch(&base)) return e;
  return decode_layers_on(d, n_layers, residual, w_router, bias, expert_tables, x_rec, idx_rec, w_rec, nullptr,
                          (char*)base, L, (hipStream_t)stream);
}

int smoe_moe_prefill_chunk(const smoe_dims* d, int32_t n_tok, const uint16_t* x, const int32_t* topk_idx,
                           const float* topk_w, const void* const* expert_table, float* residual,
                           int32_t* union_ids, int32_t* union_count, int32_t* offsets, int32_t* perm, void* ws,
                           size_t ws_bytes, void* const* events, void* stream) {
  g_err[0] = 0;
  if (int e = check_dims(d)) return e;
  if (n_tok < 1 || n_tok > kMaxPrefillTokens)
    return fail(SMOE_EINVAL, "n_tok=%d must be in [1, %d]", n_tok, kMaxPrefillTokens);
  if (!x || !topk_idx || !topk_w || !expert_table || !residual || !union_ids || !union_count || !offsets || !perm)
    return fail(SMOE_EINVAL, "NULL argument");
  if (!aligned16(x) || !aligned16(residual)) return fail(SMOE_EINVAL, "x and residual must be 16-byte aligned");
  Workspace L;
  if (int e = check_ws(d, n_tok, ws, ws_bytes, &L)) return e;
  char* base = (char*)ws;
  PrefillArgs a;
  memset(&a, 0, sizeof(a));
  a.x = x;
  a.idx = topk_idx;
  a.w = topk_w;
  a.table = expert_table;
  a.residual = residual;
  a.union_ids = union_ids;
  a.union_count = union_count;
  a.offsets = offsets;
  a.perm = perm;
  a.invperm = reinterpret_cast<int32_t*>(base + L.pinv);
  a.slices = reinterpret_cast<int32_t*>(base + L.slices);
  a.n_slices = a.slices + prefill_max_slices(n_tok, d->top_k, d->n_experts);
  a.recs = reinterpret_cast<PrefillArgs::SliceRec*>(base + L.recs);
  a.H = reinterpret_cast<_Float16*>(base + L.ph);
  a.Hs = reinterpret_cast<float*>(base + L.phs);
  a.Y = reinterpret_cast<float*>(base + L.py);
  a.xa = reinterpret_cast<_Float16*>(base + L.pxa);
  a.xas = reinterpret_cast<float*>(base + L.pxas);
  a.T = n_tok;
  a.d = d->d_model;
  a.f = d->d_ff;
  a.E = d->n_experts;
  a.k = d->top_k;
  a.chunk = d->chunk;
  a.bits = quant_bits(d);
  a.lay = blob_layout(d->d_model, d->d_ff, d->chunk, a.bits);
  hipError_t he = launch_prefill(a, (hipStream_t)stream, reinterpret_cast<const hipEvent_t*>(events));
  if (he != hipSuccess) return hip_fail(he, "prefill launch");
  return SMOE_OK;
}

}  // extern "C"
