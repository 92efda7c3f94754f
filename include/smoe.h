/*
 * smoe.h -- C ABI of the MI355X (gfx950) routed-expert MoE library.
 *
 * The library computes one routed Mixture-of-Experts FFN layer of an S-MoE
 * style engine, as the S-MoE documentation pages describe it:
 *   - the exact router: RMSNorm of the residual, an E x d_model bf16 gate
 *     matvec on the actual (not predicted) hidden state, top-k selection and
 *     Qwen3's norm_topk_prob weighting ("Optimizations", section "Routing Is
 *     Exact"; "System Overview", per-token step table);
 *   - the fused SMOE-Q4 expert FFN: per-chunk affine dequant, gate and up in
 *     one pass, SwiGLU, down projection, and the gate-weighted sum of the
 *     experts' outputs into the residual ("Optimizations", section "Coalesced
 *     GPU Kernels"; "System Overview", step table, Metal-kernel row);
 *   - layer-major prefill: a chunk holds at most 64 tokens, and the set of
 *     distinct experts its tokens route to is streamed once per chunk rather
 *     than once per token ("Optimizations", section "Prefill Reads Each Expert
 *     Once");
 *   - an LRU ring of expert slots in HBM, refilled from a vault in host memory
 *     ("Optimizations", section "The Ring Is an LRU Cache"; "System Overview",
 *     memory-budget paragraph on the [64, 4096] slot clamp).
 *
 * Conventions (all entry points):
 *   - Every call returns an smoe_status.  Arguments are checked before any
 *     work is enqueued: a call that fails validation has no side effects and
 *     smoe_last_error() describes the problem.  A failed HIP launch returns
 *     SMOE_EHIP; faults inside a kernel surface at the caller's next
 *     synchronisation, as with any asynchronous HIP work.
 *   - "device" pointers are HIP device memory (or memory the GPU can read
 *     directly); "host" pointers are ordinary host memory.  The caller owns
 *     every buffer; the library never allocates or frees device memory and
 *     keeps no pointer after the call returns (the ring keeps the pointers
 *     given in its descriptor until smoe_ring_destroy).
 *   - `stream` is a hipStream_t (NULL = the null stream).  The layer calls only
 *     enqueue kernels on it; they never synchronise and never allocate, so they
 *     can be captured into a HIP graph (no memset nodes are recorded).
 *   - Scalars are passed by value in kernel arguments.
 *   - bf16 tensors are arrays of uint16_t bit patterns.
 *   - Calls on one stream are ordered; concurrent calls that share a workspace
 *     race.  A ring handle is single-threaded.
 *
 * SMOE-Q4 expert blob (the pages fix only "4-bit codes, per-chunk affine
 * dequant, 16 KB-aligned blobs"; this byte layout is the library's):
 *   matrices G (gate) [d_ff][d_model], U (up) [d_ff][d_model],
 *            D (down) [d_model][d_ff];
 *   W[n][k] = scale[n][k / chunk] * q[n][k] + min[n][k / chunk], q in 0..15;
 *   sections, in order: G codes, U codes, D codes (row-major, two codes per
 *   byte, the even element in the low nibble), then G params, U params,
 *   D params (per row and chunk: bf16 scale, then bf16 min);
 *   blob bytes = 1.5*d_model*d_ff + 12*d_model*d_ff/chunk; blobs sit at a
 *   stride rounded up to 16384 bytes; a blob must be 16-byte aligned.
 *
 * SMOE-Q2 expert blob (the 2-bit vault the Optimizations page announces in
 * "Q2 Vaults -- the Next 2x, Twice Over": same affine dequant, every blob
 * about half the size; the layout is again the library's): as SMOE-Q4 with
 * q in 0..3 and four codes per byte, element 4j + i of a row in bits
 * [2i, 2i + 2) of the row's byte j; parameters unchanged.  Chunk 64 only.
 *   blob bytes = 0.75*d_model*d_ff + 12*d_model*d_ff/chunk.
 * SMOE-Q2 is supported by the decode calls (smoe_moe_decode,
 * smoe_moe_decode_slots, smoe_decode_layers), by smoe_moe_prefill_chunk and
 * by the ring, which moves blobs of any size.
 */
#ifndef SMOE_H
#define SMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SMOE_OK = 0,
  SMOE_EINVAL = -1,  /* bad argument; nothing was enqueued                    */
  SMOE_EHIP = -2,    /* a HIP runtime call or launch failed                   */
  SMOE_ENOSLOT = -3, /* ring: every slot is held by the current layer         */
  SMOE_EBUSY = -4,   /* ring: destroy while slots are held or fills pending   */
  SMOE_ENOMEM = -5   /* ring: host metadata allocation failed                 */
} smoe_status;

/* Geometry of one MoE layer. */
typedef struct {
  int32_t d_model;        /* hidden size; multiple of 256, <= 8192           */
  int32_t d_ff;           /* expert FFN size; multiple of 128, <= 8192       */
  int32_t n_experts;      /* E, 1..256                                       */
  int32_t top_k;          /* k, 1..min(E, 16)                                */
  int32_t chunk;          /* Q4 affine chunk along the reduction dim: 32, 64 */
  int32_t norm_topk_prob; /* 1: divide the k weights by their sum (Qwen3)    */
  float rms_eps;          /* RMSNorm epsilon (1e-6 for the Qwen3 shapes)     */
  int32_t quant_bits;     /* code width of the expert blobs: 4 (SMOE-Q4; 0 is
                             read as 4) or 2 (SMOE-Q2, chunk 64, d_model a
                             multiple of 512)                                */
} smoe_dims;

/* Message describing the last failed call on this thread ("" if none). */
const char* smoe_last_error(void);

/* Library ABI version (this header: 2; 2 added smoe_dims.quant_bits). */
int32_t smoe_version(void);

/* Exact byte size of one expert blob (in the format dims->quant_bits
 * selects) and its 16 KiB-aligned stride; 0 for invalid dims. */
size_t smoe_blob_bytes(const smoe_dims* dims);
size_t smoe_blob_stride(const smoe_dims* dims);
/* The same two functions under their SMOE-Q4-era names. */
size_t smoe_q4_blob_bytes(const smoe_dims* dims);
size_t smoe_q4_blob_stride(const smoe_dims* dims);

/* Workspace bytes needed by smoe_route / smoe_moe_decode /
 * smoe_decode_layers / smoe_moe_prefill_chunk for up to `max_tokens` tokens
 * per call (1 for decode, up to 64 for prefill).  Writes *bytes.  The
 * workspace must be 256-byte aligned; its contents need no initialisation. */
int smoe_workspace_bytes(const smoe_dims* dims, int32_t max_tokens, size_t* bytes);

/* Exact router for n_tok tokens ("Routing Is Exact"; step table, heavy-pass
 * row).
 *   residual  device fp32 [n_tok][d_model]            (read)
 *   x_out     device bf16 [n_tok][d_model]            (written) the RMSNorm
 *             output x = bf16(r / sqrt(mean(r^2) + eps)), round to nearest
 *             even; gain 1
 *   w_router  device bf16 [E][d_model]                 (read)
 *   bias      device fp32 [E] or NULL                   added to every logit
 *             before selection and softmax
 *   topk_idx  device int32 [n_tok][k]                   (written) rank order:
 *             logits descending, equal logits -> lower expert index first
 *   topk_w    device fp32 [n_tok][k]                    (written) softmax over
 *             all E logits at the selected experts, renormalised over the k
 *             when dims->norm_topk_prob
 * Logits are accumulated in float64 (each bf16*bf16 product is exact); for
 * 2..64 tokens on float64 MFMA, as d_model / 128 partial sums added in a fixed
 * order.  A NaN logit (from a non-finite residual) ranks as -inf.
 * 0 <= n_tok <= 64; n_tok == 0 does nothing (and accepts NULL buffers).
 * Pointers 16-byte aligned. */
int smoe_route(const smoe_dims* dims, int32_t n_tok, const float* residual, uint16_t* x_out,
               const uint16_t* w_router, const float* bias, int32_t* topk_idx, float* topk_w,
               void* workspace, size_t workspace_bytes, void* stream);

/* smoe_route, plus the gate ranking past the top k (the speculative-prefetch
 * bets of the Optimizations page, "ranks 9-16"):
 *   next_idx  device int32 [n_tok][n_next] (written) the experts at exact ranks
 *             k .. k + n_next - 1, from the same ranking as topk_idx
 * 0 <= n_next <= E - k; n_next == 0 is smoe_route. */
int smoe_route_ext(const smoe_dims* dims, int32_t n_tok, const float* residual, uint16_t* x_out,
                   const uint16_t* w_router, const float* bias, int32_t* topk_idx, float* topk_w,
                   int32_t n_next, int32_t* next_idx, void* workspace, size_t workspace_bytes,
                   void* stream);

/* Decode MoE FFN for one token ("Coalesced GPU Kernels"; step table,
 * Metal-kernel row): for r = 0..k-1, expert e = topk_idx[r]:
 *   h_r = silu(G_e x) * (U_e x),   y = sum_r topk_w[r] * (D_e h_r)  (rank order)
 *   residual += y
 *   x             device bf16 [d_model]   (from smoe_route)
 *   topk_idx      device int32 [k], topk_w device fp32 [k]
 *   expert_table  device array [E] of device blob pointers (this layer)
 *   residual      device fp32 [d_model], updated in place
 * The activations h_r are kept in fp32 and reach the down projection as fp16
 * with one power-of-two scale per 32 (SMOE-Q4) or 64 (SMOE-Q2) values, so
 * they cannot overflow fp16.  An index outside [0, E) or a NULL table entry
 * contributes nothing.  Deterministic: no atomics, fixed reduction order. */
int smoe_moe_decode(const smoe_dims* dims, const uint16_t* x, const int32_t* topk_idx,
                    const float* topk_w, const void* const* expert_table, float* residual,
                    void* workspace, size_t workspace_bytes, void* stream);

/* As smoe_moe_decode, but the k blob pointers come from the host, in rank
 * order, and travel as kernel arguments (the pages pass dispatch parameters by
 * value, "Zero Allocations, Zero Locks in the Token Loop").  Used with the
 * ring, which returns slot pointers on the host.
 *   blobs_host  host array [k] of device blob pointers */
int smoe_moe_decode_slots(const smoe_dims* dims, const uint16_t* x, const float* topk_w,
                          const void* const* blobs_host, float* residual, void* workspace,
                          size_t workspace_bytes, void* stream);

/* n_layers chained decode layers for one token, all experts resident
 * ("What Happens at Each Generated Token Step"): for L = 0..n_layers-1,
 * smoe_route then smoe_moe_decode with layer L's weights, the residual carried
 * from layer to layer.  Three kernels per layer (router logits; top-k +
 * gate/up + SwiGLU; down + combine), no host synchronisation; capturable into
 * a HIP graph.  Results are bitwise equal to the per-layer calls.
 * n_layers == 0 does nothing (and accepts NULL buffers).
 *   residual       device fp32 [d_model], updated in place
 *   w_router       device bf16 [n_layers][E][d_model]
 *   bias           device fp32 [n_layers][E] or NULL
 *   expert_tables  device array [n_layers][E] of device blob pointers
 *   x_rec          device bf16 [n_layers][d_model] or NULL: x used per layer
 *   idx_rec        device int32 [n_layers][k] or NULL: routing per layer
 *   w_rec          device fp32 [n_layers][k] or NULL: weights per layer
 *   events         host array [n_layers][2] of hipEvent_t, or NULL: when
 *                  given, layer L's gate/up kernel is launched with
 *                  hipExtLaunchKernel, which records events[2L] at the
 *                  kernel's start and events[2L+1] at its end (per-kernel
 *                  timing, in the spirit of the pages' instrument panel; not
 *                  for use under stream capture) */
int smoe_decode_layers(const smoe_dims* dims, int32_t n_layers, float* residual,
                       const uint16_t* w_router, const float* bias,
                       const void* const* expert_tables, uint16_t* x_rec, int32_t* idx_rec,
                       float* w_rec, void* const* events, void* workspace, size_t workspace_bytes,
                       void* stream);

/* smoe_decode_layers without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the scratch lives in a 2 MiB array that
 * the library holds in each GPU's memory until the process ends (every valid
 * smoe_dims needs at most about 1.5 MiB of it; larger needs are rejected with
 * SMOE_EINVAL).  Arguments and results as smoe_decode_layers (no per-kernel
 * events).  The call allocates nothing: the array's device address is looked
 * up once per device, on the first call with that device current.  Every
 * call on one GPU uses that GPU's one array, whose contents carry over from
 * call to call (nothing in it needs to start at zero): calls that overlap on
 * one GPU (other streams, other threads) race; serialise them. */
int smoe_decode_layers_static(const smoe_dims* dims, int32_t n_layers, float* residual,
                              const uint16_t* w_router, const float* bias,
                              const void* const* expert_tables, uint16_t* x_rec, int32_t* idx_rec,
                              float* w_rec, void* stream);

/* Layer-major prefill of one chunk through one layer ("Prefill Reads Each
 * Expert Once, Not Once Per Token").  Inputs x/topk_idx/topk_w come from
 * smoe_route over the chunk's n_tok tokens (1..64).
 *   union_ids    device int32 [min(E, n_tok*k)] (written) experts the chunk
 *                routes to, in first-touch order (t ascending, then rank)
 *   union_count  device int32 [1] (written) |union|
 *   offsets      device int32 [min(E, n_tok*k) + 1] (written) exclusive scan of
 *                the per-expert token counts, in union order
 *   perm         device int32 [n_tok*k] (written) for union member u, entries
 *                offsets[u]..offsets[u+1]-1 list t*k + r of its tokens, t ascending
 *   residual     device fp32 [n_tok][d_model], += the MoE output per token
 * Each union expert's blob is streamed once per chunk; the grouped FFN runs on
 * MFMA with fp16 inputs: at chunk 64 the raw codes, with the affine step
 * applied per chunk to the fp32 sums; otherwise (chunk 32, and SMOE-Q2 down
 * projections whose d_ff is not a multiple of 512) the weights dequantised to
 * fp16 (exact for min = -8*scale, and -2*scale for SMOE-Q2).  The SwiGLU
 * activations go to the down GEMM as fp16 with one power-of-two scale per
 * token and 64 features (the tile's largest |h| mapped into [2^14, 2^15)), so
 * they cannot overflow fp16.  The per-token mix is summed in rank order; no
 * atomics.  An entry whose expert is outside [0, E) or whose table entry is
 * NULL (e.g. a ring table that holds only an acquired union) takes no part:
 * it is left out of the union and contributes nothing.  A token that lists
 * an expert more than once gets one row per entry (each weight applies).
 *   events       host array [4] of hipEvent_t, or NULL: when given, 0 and 1
 *                are recorded at the start and end of the grouped gate/up
 *                GEMM and 2 and 3 around the down GEMM (kernel timing) */
int smoe_moe_prefill_chunk(const smoe_dims* dims, int32_t n_tok, const uint16_t* x,
                           const int32_t* topk_idx, const float* topk_w,
                           const void* const* expert_table, float* residual, int32_t* union_ids,
                           int32_t* union_count, int32_t* offsets, int32_t* perm, void* workspace,
                           size_t workspace_bytes, void* const* events, void* stream);

/* ---------------------------------------------------------------------------
 * Expert ring ("The Ring Is an LRU Cache"): HBM slots caching (layer, expert)
 * blobs from a vault in pinned host memory.  Released slots keep their data
 * and identity; a re-request is a hit that moves zero bytes; eviction is lazy
 * least-recently-used and never touches a slot held by the current layer.
 * Every request (hit or load) stamps the slot with a fresh tick.  Empty slots
 * are used first, lowest index first.  Misses are copied with hipMemcpyAsync
 * on copy_stream, after all work already enqueued on the compute stream (so
 * no slot is overwritten while a kernel may still read it); the compute
 * stream then waits on the completion events of the slots it is handed.
 * ------------------------------------------------------------------------- */
typedef struct smoe_ring smoe_ring;

typedef struct {
  int32_t n_slots;        /* 64..4096 (the pages' clamp), >= top_k          */
  int32_t n_layers;       /* >= 1                                          */
  int32_t n_experts;      /* E                                             */
  int32_t top_k;          /* k of a decode step (validated; an acquisition
                             may hold up to min(E, n_slots) experts)       */
  size_t slot_bytes;      /* bytes copied per fill (the blob size)         */
  size_t slot_stride;     /* distance between slots in slab_dev (>= bytes) */
  const void* const* vault_layers; /* host array [n_layers] of host pointers:
                             blob (L, e) at vault_layers[L] + e*vault_stride.
                             Pinned (hipHostMalloc) memory gives asynchronous
                             full-rate copies; one allocation per layer keeps
                             each under the driver's pinned-allocation limit.
                             A pageable layer is detected at create and filled
                             through the ring's own pipeline (host threads copy
                             each blob into one of 4 page-locked staging
                             buffers of slot_bytes, allocated by the ring,
                             while the previous blob's DMA runs); acquire then
                             blocks for those host copies.
                             The array is copied at create; the memory it
                             points to must outlive the ring. */
  size_t vault_stride;
  void* slab_dev;         /* device: n_slots * slot_stride bytes            */
  void* copy_stream;      /* hipStream_t used for fills                     */
  size_t log_capacity;    /* events kept for smoe_ring_log (0 = none)       */
} smoe_ring_desc;

/* One ring decision. */
typedef struct {
  int32_t layer, rank, expert;
  int32_t kind;           /* 0 = hit, 1 = miss, 2 = speculative load       */
  int32_t slot;
  int32_t evicted_layer;  /* -1 if no eviction                              */
  int32_t evicted_expert;
  int32_t pad;
} smoe_ring_event;

int smoe_ring_create(const smoe_ring_desc* desc, smoe_ring** out);

/* Acquire k experts of `layer` (host array, in request order): a decode
 * step's k routed experts in rank order, or a prefill chunk's expert union in
 * first-touch order (1 <= k <= min(E, n_slots)).  Drops the previous
 * acquisition's holds first (an implicit release).  Fills are issued in
 * request order.  On return slot_ptrs_host[r] is the device blob pointer of
 * request r, and compute_stream will not run later work until the fills are
 * complete.  Errors: SMOE_EINVAL (layer, k or an expert out of range, an
 * expert twice), SMOE_ENOSLOT (every slot held), SMOE_EHIP (a copy or event
 * call failed). */
int smoe_ring_acquire(smoe_ring* ring, int32_t layer, const int32_t* experts_host, int32_t k,
                      const void** slot_ptrs_host, void* compute_stream);

/* smoe_ring_acquire, then the layer's expert table for the kernels that find
 * blobs through one ("Prefill Reads Each Expert Once"; ring-backed prefill):
 * table_dev (device, [E] blob pointers, caller-owned) gets the slot pointer of
 * every requested expert and NULL for every other one, written by a kernel on
 * compute_stream after the fills' waits (stream-ordered; the pointers travel
 * as kernel arguments, so no host buffer must outlive the call).  Errors as
 * smoe_ring_acquire, plus SMOE_EINVAL for a NULL or unaligned table_dev. */
int smoe_ring_acquire_table(smoe_ring* ring, int32_t layer, const int32_t* experts_host, int32_t k,
                            void* table_dev, void* compute_stream);

/* Ring-backed layer-major prefill of one chunk ("Prefill Reads Each Expert
 * Once, Not Once Per Token"): reads the chunk's routing back from the device
 * (waiting for the work on compute_stream that writes it), forms the chunk's
 * expert union in first-touch order (t ascending, then rank -- the order in
 * which the section has each expert sent to the streamer), acquires it (as
 * smoe_ring_acquire: hits, fills in union order, holds) and writes the
 * layer's expert table as smoe_ring_acquire_table does, for
 * smoe_moe_prefill_chunk.
 *   n_tok, k        the routing's shape: 1..64 tokens, 1..16 ranks
 *   topk_idx_dev    device int32 [n_tok][k] (smoe_route's topk_idx); ids
 *                   outside [0, E) take no part
 *   table_dev       device [E] blob pointers (caller-owned, 8-byte aligned)
 *   union_host      host int32 [min(E, n_tok*k)] or NULL: the union, in
 *                   first-touch order
 *   n_union         host int32 or NULL: |union|
 * Blocks the calling thread until the routing is on the host (one read of at
 * most 4 KiB into page-locked memory the ring owns); allocates nothing.
 * Errors: as smoe_ring_acquire_table (SMOE_EINVAL also when the union exceeds
 * min(E, n_slots) or holds no valid expert). */
int smoe_ring_acquire_routed(smoe_ring* ring, int32_t layer, int32_t n_tok, int32_t k,
                             const int32_t* topk_idx_dev, void* table_dev, int32_t* union_host,
                             int32_t* n_union, void* compute_stream);

/* Speculative loads ("Speculative prefetch"; "Idle-time popularity
 * prewarm"): each of the n experts of `layer` (host array) that is not
 * resident is loaded into the slot a miss would take (the lowest empty slot,
 * else the unpinned slot with the oldest tick), with a fresh tick and no hold;
 * a resident expert is left as it is.  Stops at the first expert for which
 * every slot is held: a bet never displaces the current acquisition.  Fills
 * go on copy_stream after the work already enqueued on compute_stream (the
 * same FIFO as demand fills, at the default priority).  Each load is logged
 * with kind 2.  *n_loaded (may be NULL) = loads issued. */
int smoe_ring_prefetch(smoe_ring* ring, int32_t layer, const int32_t* experts_host, int32_t n,
                       int32_t* n_loaded, void* compute_stream);

/* The claim histogram the ring keeps: every demand request of
 * smoe_ring_acquire(_table) counts one claim of its (layer, expert).  Writes
 * the n most claimed pairs (most claims first, ties to the lower layer, then
 * the lower expert) to host arrays; counts_out may be NULL; *n_out = pairs
 * written (only pairs with at least one claim). */
int smoe_ring_hottest(const smoe_ring* ring, int32_t n, int32_t* layers_out, int32_t* experts_out,
                      uint64_t* counts_out, int32_t* n_out);

/* Drop the current holds (the slots stay resident for later hits). */
int smoe_ring_release(smoe_ring* ring);

int smoe_ring_stats(const smoe_ring* ring, uint64_t* hits, uint64_t* misses, uint64_t* evictions,
                    uint64_t* h2d_bytes);

/* Copy up to `cap` logged events (oldest first) to events_host; *n_out = count. */
int smoe_ring_log(const smoe_ring* ring, smoe_ring_event* events_host, size_t cap, size_t* n_out);

/* Returns SMOE_EBUSY (and keeps the ring) if slots are still held. */
int smoe_ring_destroy(smoe_ring* ring);

#ifdef __cplusplus
}
#endif

#endif /* SMOE_H */
