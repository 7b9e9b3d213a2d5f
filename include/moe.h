/*
 * moe.h -- C ABI of the MI355X (gfx950) sparse mixture-of-experts FFN library.
 *
 * The operation (Strata pages: "single RTX 5090 runs a 125B model", section on
 * on-demand expert scheduling; "How Strata works", section on the three storage
 * tiers): hidden states x [T, d] pass a router that picks the top-k of E
 * experts per token; each picked expert is a SwiGLU FFN; the layer output is
 * the gate-weighted sum of the picked experts' outputs plus an ungated,
 * always-resident shared expert.  The model these pages describe has 24,576
 * experts (512 per layer over 48 layers) with 10 picked per token.
 *
 *   out[t] = residual[t] + shared(x_t) + sum_{j<k} g[t,j] * FFN_{ids[t,j]}(x_t)
 *   FFN(x) = Wd (silu(Wg x) * (Wu x)),   silu(z) = z / (1 + exp(-z))
 *
 * Call sequence for one layer (all enqueued on the caller's stream):
 *   moe_route -> moe_permute -> [moe_quantize_act] -> moe_expert_ffn -> moe_combine
 * or, fused: moe_route_permute -> [moe_quantize_act] -> moe_expert_ffn_combine;
 * for decode batches (float mode, int4, T <= 8) with no grouping at all:
 *   moe_route -> moe_expert_ffn_combine_slots, or moe_route_ffn_combine_slots
 *
 * Conventions
 *  - Every tensor argument is a DEVICE pointer owned by the caller unless the
 *    argument says "host".  The library never frees caller memory and never
 *    allocates in the per-layer calls; scratch comes from a caller-provided
 *    workspace sized by moe_workspace_size.
 *  - Calls enqueue work on `stream` (a hipStream_t; NULL = the null stream)
 *    and return without synchronising; no call reads device data back to the
 *    host.  Asynchronous kernel faults surface at the caller's next sync.
 *  - Arguments are validated before any HIP call.  Return value: MOE_OK or an
 *    MOE_ERR_* status; on MOE_ERR_HIP, moe_last_hip_error() gives the
 *    hipError_t of the failing runtime call.  No C++ exception crosses the ABI.
 *  - Row-major layouts; int32 indices; T == 0 is a valid no-op.
 *  - Shape limits: d % 128 == 0, f % 128 == 0, 1 <= k <= 64, k <= E <= 1024.
 *  - Not thread-safe for concurrent calls that share a workspace or a cache
 *    handle; otherwise reentrant.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_VERSION 10100

typedef void* moe_stream_t; /* hipStream_t */
typedef void* moe_event_t;  /* hipEvent_t  */

/* status codes */
#define MOE_OK 0
#define MOE_ERR_INVALID_ARG 1    /* null pointer, bad shape, k > E, unsupported dtype value */
#define MOE_ERR_UNSUPPORTED 2    /* valid request no kernel of the library covers */
#define MOE_ERR_HIP 3            /* a HIP runtime call failed; see moe_last_hip_error */
#define MOE_ERR_NO_MEMORY 4      /* workspace too small, or host bookkeeping allocation failed */
#define MOE_ERR_CACHE_CAPACITY 5 /* slot pool or staging buffer too small for the request */

/* element types of activations */
#define MOE_DT_F32 0
#define MOE_DT_BF16 1
#define MOE_DT_F16 2

/* expert weight formats: block-32 quantisation along each row (the reduction
 * axis), one IEEE fp16 scale per 32 weights; int4 values are offset-binary
 * nibbles u = q + 8 (element 2i in the low nibble), int8 values are
 * two's complement. */
#define MOE_WFMT_I4B32 4
#define MOE_WFMT_I8B32 8

/* activation modes of the expert FFN */
#define MOE_ACT_FLOAT 0 /* fp32 accumulation of dequantised weights x activations */
#define MOE_ACT_Q8 1    /* int8 activations per 32-feature block, int8 matrix cores */

int moe_version(void);
/* hipError_t of the most recent failing HIP call made by this thread (0 = none). */
int moe_last_hip_error(void);
/* Static string naming a status code. */
const char* moe_status_string(int status);

/*
 * Size in bytes of one expert blob (canonical or packed; both have the same
 * size): three matrices Wg [f,d], Wu [f,d], Wd [d,f] of block-32 quants
 * followed by their fp16 scales.  Canonical blob layout, all row-major:
 *   [qg][qu][qd][sg : f x d/32][su : f x d/32][sd : d x f/32]
 * Returns 0 for an invalid format or shape.
 */
size_t moe_expert_bytes(int wfmt, int d, int f);

/*
 * Repack n canonical expert blobs (device, contiguous [n, expert_bytes]) into
 * the kernel-native tiled layout consumed by moe_expert_ffn (device `dst`,
 * same size, must not alias `src`).  One-time, untimed preparation step.
 * The packed layout is private to this library version.
 */
int moe_pack_experts(const void* src, void* dst, int n, int wfmt, int d, int f, moe_stream_t stream);
/* Inverse of moe_pack_experts (for verification): packed -> canonical. */
int moe_unpack_experts(const void* src, void* dst, int n, int wfmt, int d, int f, moe_stream_t stream);

/*
 * Workspace bytes needed by route, permute and expert_ffn for a layer with
 * these shapes (the same workspace may be passed to all three calls of one
 * layer; calls on one stream are ordered).  Writes *bytes.  The workspace is
 * scratch: its contents need no initialisation and are not preserved.  No
 * passage defines this; it is the library's sizing convention (a workspace
 * sized for T tokens serves every smaller batch of the same layer).
 * Errors: MOE_ERR_INVALID_ARG for shapes outside the limits above.
 */
int moe_workspace_size(int T, int d, int f, int E, int k, int act_mode, size_t* bytes);

/*
 * Router: logits z[t,e] = sum_i x[t,i] * Wr[e,i] (+ bias[e]) and top-k
 * selection, as described on "single RTX 5090 runs a 125B model" (on-demand
 * expert scheduling: a light gating network picks the top-K experts).
 *   x     [T, d]   x_dtype MOE_DT_F32 or MOE_DT_BF16
 *   Wr    [E, d]   fp32
 *   bias  [E]      fp32 or NULL (added to the logits before selection)
 *   ids   [T, k]   int32 out: experts in descending-logit order; equal logits
 *                  are ordered by ascending expert index.  The ranking is that
 *                  of the exact real-valued logits (products of the fp32/bf16
 *                  inputs are exact in double; sums are double).
 *   gates [T, k]   fp32 out: softmax over the k selected logits (equal to the
 *                  full softmax renormalised over the top k).
 * Batches of more than 256 bf16 tokens (k <= 32, d <= 4096) first bound every
 * logit with a bf16 matrix-core filter and take exact double logits only for
 * the experts that can still rank in the top k; the outputs are the same.
 */
int moe_route(const void* x, int x_dtype, int T, int d, const float* Wr, const float* bias, int E, int k,
              int32_t* ids, float* gates, void* ws, size_t ws_bytes, moe_stream_t stream);

/*
 * moe_route followed by moe_permute.  For small batches (T <= 16 and
 * T*k <= 512: decode, MTP verify) this is two launches: the router logits,
 * then one workgroup that selects the top-k of every token and groups the
 * slots; larger batches run the two calls' kernels in sequence.  Outputs and
 * numerics are those of the two calls.
 */
int moe_route_permute(const void* x, int x_dtype, int T, int d, const float* Wr, const float* bias, int E, int k,
                      int32_t* ids, float* gates, int32_t* counts, int32_t* offsets, int32_t* sorted_idx,
                      int32_t* dest, int32_t* active, void* ws, size_t ws_bytes, moe_stream_t stream);

/*
 * Stable grouping of the T*k routing slots by expert (flat slot f = t*k + j).
 * No passage defines this step; it is the dispatch that on-demand expert
 * scheduling implies ("single RTX 5090 runs a 125B model": only the picked
 * experts compute), grouping each picked expert's rows so that its weights
 * are read once per call.
 *   counts     [E]      number of slots routed to each expert
 *   offsets    [E+1]    exclusive prefix sum of counts (offsets[E] = T*k)
 *   sorted_idx [T*k]    slots in (expert, slot) order: expert-major, ascending
 *                       slot (hence ascending token) within an expert
 *   dest       [T*k]    position of slot f in sorted_idx (inverse permutation)
 *   active     [E+1]    work list: active[0] = number of experts with
 *                       count > 0, active[1..] = those experts, ascending
 * Integer outputs; bit-exact and deterministic.  Ids outside [0, E) are
 * ignored (not counted, not placed).
 */
int moe_permute(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets, int32_t* sorted_idx,
                int32_t* dest, int32_t* active, void* ws, size_t ws_bytes, moe_stream_t stream);

/*
 * int8 activation quantisation (MOE_ACT_Q8 input), for the int8 matrix-core
 * prefill that "Strata benchmarks" names (bottleneck analysis 1, prefill
 * optimisation table: int8 tensor-core products without dequantisation; the
 * block of 32 and the scale rule are this library's reading): per token, per 32
 * consecutive features, s = amax / 127 (fp32, IEEE division),
 * q = clamp(rint(x / s), -127, 127) with ties to even; an all-zero block gives
 * s = 0 and q = 0.  x [T, d] (F32 or BF16) -> xq [T, d] int8, sx [T, d/32] fp32.
 */
int moe_quantize_act(const void* x, int x_dtype, int T, int d, int8_t* xq, float* sx, moe_stream_t stream);

/*
 * Pre-norm of a stacked layer's input: out[t] = x[t] / sqrt(mean_i x[t,i]^2 + eps)
 * (no learned gain), sums and scale in double, rounded once to fp32.
 * x, out [T, d] fp32 (may alias).  The pages do not describe the block around
 * the MoE layer; a stack of layers joined by a residual add, h + MoE(norm(h)),
 * needs this normalisation to stay finite.
 */
int moe_rmsnorm(const float* x, int T, int d, float eps, float* out, moe_stream_t stream);

/* Arguments of moe_expert_ffn. */
typedef struct moe_ffn_args {
    int T, d, f, E, k;
    int wfmt;     /* MOE_WFMT_* of every expert blob */
    int act_mode; /* MOE_ACT_FLOAT or MOE_ACT_Q8 */
    /* MOE_ACT_FLOAT input */
    const void* x; /* [T, d] */
    int x_dtype;   /* MOE_DT_F32 or MOE_DT_BF16 */
    /* MOE_ACT_Q8 input, from moe_quantize_act */
    const int8_t* xq; /* [T, d] */
    const float* sx;  /* [T, d/32] */
    /* experts: DEVICE array [E] of device pointers to PACKED blobs (pool
       slots and staging buffers are interchangeable) */
    const void* const* expert_ptrs;
    /* from moe_permute */
    const int32_t* counts;
    const int32_t* offsets;
    const int32_t* sorted_idx;
    const int32_t* active;
    /* routed expert outputs, row p = position p of sorted_idx, ungated */
    void* y_perm; /* [T*k, d] */
    int y_dtype;  /* MOE_DT_F32 or MOE_DT_F16 */
    /* shared expert (NULL = none): packed blob, output [T, d] fp32 */
    const void* shared_blob;
    float* y_shared;
    void* ws;
    size_t ws_bytes;
    /* 0 = whole FFN; 1 = gate/up + SwiGLU only (h left in the workspace);
       2 = down projection only (reads h from the same workspace) */
    int phase;
} moe_ffn_args;

/*
 * Grouped SwiGLU expert FFN over the rows grouped by moe_permute, plus the
 * shared expert over all T tokens ("How Strata works", three-tier division:
 * 10 of 24,576 small experts per token plus a resident shared expert).
 * Block-32 weights are dequantised in registers.  MOE_ACT_FLOAT: fp16
 * matrix-core products with fp32 accumulation; activations and the SwiGLU
 * intermediate h are rounded to fp16 once.  The weight block scale is applied
 * in fp32 to each exact block sum by the int4 gate/up kernel for T <= 16 and
 * by the general kernels (T > 64); the other small-batch kernels fold it into
 * the weights, rounding each (q - 8) * s to fp16 once (relative error at most
 * 2^-11 per weight).  MOE_ACT_Q8 (the pages' int8 prefill step, "Strata
 * benchmarks", prefill optimisation table): gate/up on int8 x int8 matrix
 * cores with exact per-block integer sums, both block scales applied in fp32;
 * the SwiGLU intermediate is requantised to int8 per 32 features.  The down
 * projection with int8 weights is exact in the same way; with int4 weights it
 * multiplies fp16 operands holding the dequantised values (h codes times their
 * scale, weights times theirs, each rounded once to fp16) with fp32
 * accumulation, which adds about 3.5e-4 relative error to the expert output
 * and no quantisation decision.
 * Errors: MOE_ERR_INVALID_ARG (null pointers, shapes not multiples of the
 * quantisation block, a workspace smaller than moe_workspace_size);
 * MOE_ERR_UNSUPPORTED for float-mode shapes no kernel covers: more than 64
 * tokens with d or f above 2048 (16 rows of either, in fp16, must fit the
 * 64 KiB of LDS the general kernels use), or, for T <= 64, a width the
 * token-dense kernels have no instance for (d / 128 or f / 128 outside their
 * sets) together with that same limit.
 */
int moe_expert_ffn(const moe_ffn_args* args, moe_stream_t stream);

/*
 * Expert FFN and combine in one call: out[t] = residual[t] + shared(x_t) +
 * sum_{j<k} gates[t,j] * FFN_{ids[t,j]}(x_t), the whole layer output after the
 * routing ("How Strata works", three-tier division: routed small experts plus
 * the resident shared expert; the weighted sum is the mixture's output).
 *   args: as for moe_expert_ffn, phase must be 0 (args->y_perm and
 *         args->y_shared must still be valid buffers: the shapes without a
 *         fused kernel go through them);
 *   ids [T, k] (from moe_route), dest [T*k] (from moe_permute), gates [T, k],
 *   residual [T, d] fp32 or NULL, out [T, d] fp32 (may alias residual).
 * For float mode, int4 weights, T <= 8 and f / 128 in {2, 4, 6, 8} the down
 * projection and the weighted sum run in one kernel: every workgroup owns one
 * token's 16 output rows, the expert outputs stay in fp32 and are summed in a
 * fixed order (deterministic; neither y_perm nor y_shared is written).  Other
 * shapes run moe_expert_ffn then moe_combine.  Ids outside [0, E) contribute
 * nothing.  Errors: those of moe_expert_ffn; MOE_ERR_INVALID_ARG for a phase
 * other than 0 or a null ids, dest, gates or out.
 */
int moe_expert_ffn_combine(const moe_ffn_args* args, const int32_t* ids, const int32_t* dest, const float* gates,
                           const float* residual, float* out, moe_stream_t stream);

/*
 * Decode batches without the grouping step: the same output as
 * moe_route_permute + moe_expert_ffn_combine, bit for bit, from moe_route's
 * ids and gates alone.  Every routed slot (t, j) is its own gate/up work item
 * reading expert ids[t, j] (only the picked experts compute: "single RTX 5090
 * runs a 125B model", on-demand expert scheduling); an expert picked by
 * several tokens is read once per slot, which at a few tokens over hundreds
 * of experts is rare.  The down projection and the weighted sum are the
 * fused kernel of moe_expert_ffn_combine; slot (t, j) keeps h row t*k + j.
 *   args: as for moe_expert_ffn; counts, offsets, sorted_idx, active, y_perm
 *         and y_shared are not read (may be NULL); phase 0 = the whole call,
 *         1 = the gate/up launch alone (h left in the workspace; gates,
 *         residual and out unused);
 *   ids [T, k], gates [T, k] (moe_route), residual [T, d] fp32 or NULL,
 *   out [T, d] fp32 (may alias residual).  Ids outside [0, E) contribute nothing.
 * Supported: float mode, int4 weights, T <= 8, d a power of two with
 * T * d * 2 <= 64 KiB, f / 128 in {2, 4, 6, 8} and (k + 1) * f <= 16384
 * (32768 for T <= 2); otherwise MOE_ERR_UNSUPPORTED before any launch.
 * Errors: MOE_ERR_INVALID_ARG (phase other than 0 or 1, bad shapes, null x,
 * expert_ptrs, ws, ids, gates or out), MOE_ERR_NO_MEMORY (workspace smaller
 * than moe_workspace_size).
 */
int moe_expert_ffn_combine_slots(const moe_ffn_args* args, const int32_t* ids, const float* gates,
                                 const float* residual, float* out, moe_stream_t stream);

/*
 * A whole decode layer after the router weights, in three launches: router
 * logits, then the by-slot gate/up whose first wavefront per workgroup selects
 * the slot's expert itself (the router's top-k of that token, as moe_route),
 * then the down projection and the weighted sum as in
 * moe_expert_ffn_combine_slots.  ids, gates and out equal, bit for bit, those
 * of moe_route + moe_expert_ffn_combine_slots (and of the grouped path); the
 * separate selection launch and its kernel boundary are saved, at the price
 * of the top-k latency inside the gate/up launch.
 *   args: as for moe_expert_ffn_combine_slots (x is also the router input);
 *         phase 0 = the whole call, 1 = the gate/up launch alone with the
 *         router logits left in the workspace by an earlier phase-0 call of
 *         the same shape (ids and gates are written, residual and out unused);
 *   Wr [E, d] fp32, bias [E] fp32 or NULL (as moe_route);
 *   ids [T, k], gates [T, k]: outputs; residual [T, d] fp32 or NULL;
 *   out [T, d] fp32 (may alias residual).
 * Supported: the shapes of moe_expert_ffn_combine_slots (E <= 1024);
 * otherwise MOE_ERR_UNSUPPORTED before any launch.  Errors as for
 * moe_expert_ffn_combine_slots, plus MOE_ERR_INVALID_ARG for a null Wr.
 */
int moe_route_ffn_combine_slots(const moe_ffn_args* args, const float* Wr, const float* bias, int32_t* ids,
                                float* gates, const float* residual, float* out, moe_stream_t stream);

/*
 * moe_route_ffn_combine_slots for callers that cannot allocate device memory
 * (code under HIP graph capture that may not call hipMalloc, tight serving
 * loops, harnesses that forbid allocation): the same launches and results, bit
 * for bit, with the workspace taken from a scratch array the library keeps in
 * device memory (MOE_NOALLOC_SCRATCH_BYTES on every GPU it runs on, held until
 * the process ends; its device address is looked up once per device).  The
 * call allocates nothing.  args->ws and args->ws_bytes are ignored; phase must
 * be 0.  Every call on one GPU shares that GPU's scratch, and the scratch
 * needs no clearing (every byte a call reads it first writes): calls that
 * overlap on one GPU (two streams, or two threads) race and must be ordered by
 * the caller.
 * Errors: those of moe_route_ffn_combine_slots; MOE_ERR_INVALID_ARG for a
 * phase other than 0; MOE_ERR_NO_MEMORY when the shape's workspace
 * (moe_workspace_size) exceeds MOE_NOALLOC_SCRATCH_BYTES; MOE_ERR_HIP when the
 * scratch address cannot be obtained.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (2u << 20)
int moe_route_ffn_combine_slots_noalloc(const moe_ffn_args* args, const float* Wr, const float* bias, int32_t* ids,
                                        float* gates, const float* residual, float* out, moe_stream_t stream);

/*
 * Host-core execution of missed experts ("How Strata works", three-tier
 * division and adaptive expert cache: experts the GPU has not cached are
 * computed by the CPU from system memory while the GPU computes the cached
 * ones; "Strata benchmarks", calibration: the share of misses copied to the
 * GPU and the number of CPU expert threads are the knobs).  HOST memory and
 * host cores only; no HIP call.
 *
 * moe_host_pool_create(n_threads, &pool): a persistent pool of n_threads
 * (1..256, the calling thread counts as one) that moe_host_expert_ffn uses.
 * moe_host_pool_destroy(pool): joins and frees it (NULL is a no-op).
 *
 * moe_host_expert_ffn: for each item i, in the given order,
 *   out[item_token[i], :] += item_gate[i] * FFN_{item_blob[i]}(x[item_token[i], :])
 * with FFN(x) = Wd (silu(Wg x) * (Wu x)) over a CANONICAL expert blob
 * (item_blob[i], host pointer; wfmt I4B32 or I8B32).  x [T, d] and out [T, d]
 * are fp32 host arrays.  Arithmetic in fp32 (block sums times the fp16 block
 * scale); the result does not depend on the pool size.
 * Errors: MOE_ERR_INVALID_ARG (null pool or pointers, shapes not multiples of
 * 32, a token outside [0, T), a null blob), MOE_ERR_NO_MEMORY.
 */
typedef struct moe_host_pool moe_host_pool;
int moe_host_pool_create(int n_threads, moe_host_pool** pool);
int moe_host_pool_destroy(moe_host_pool* pool);
int moe_host_expert_ffn(moe_host_pool* pool, int n_items, const int32_t* item_token, const float* item_gate,
                        const void* const* item_blob, int wfmt, int T, int d, int f, const float* x, float* out);

/*
 * Combine: out[t] = residual[t] + y_shared[t] + sum_{j<k} gates[t,j] * y_perm[dest[t*k+j]],
 * summed in j order (deterministic): the picked experts' outputs weighted by
 * the gating network's weights ("single RTX 5090 runs a 125B model",
 * on-demand expert scheduling) plus the always-resident shared expert ("How
 * Strata works", three-tier division), ungated.
 *   y_perm [T*k, d] (y_dtype F32 or F16), dest [T*k], gates [T, k],
 *   y_shared [T, d] fp32 or NULL, residual [T, d] fp32 or NULL, out [T, d] fp32.
 * out may alias residual.
 */
int moe_combine(const void* y_perm, int y_dtype, const int32_t* dest, const float* gates, const float* y_shared,
                const float* residual, int T, int k, int d, float* out, moe_stream_t stream);

/* ---------------------------------------------------------------------------
 * Expert slot cache ("How Strata works", section on the adaptive expert cache:
 * the most-used ~4,500 experts by a usage ranking are loaded into GPU memory;
 * "Strata benchmarks", prefill optimisation table: next-layer experts stream
 * over PCIe while the current layer computes).
 *
 * A handle holds host bookkeeping only: which global expert id (layer*E + e)
 * occupies which slot of a caller-owned device pool, and pinned host staging
 * of per-layer pointer tables.  Misses of a layer are copied from caller-owned
 * pinned host blobs into a caller-owned device staging buffer on a side
 * stream, after which the layer's device pointer table [E] is rewritten so
 * that moe_expert_ffn reads hits from the pool and misses from staging.
 * ------------------------------------------------------------------------- */
typedef struct moe_cache moe_cache;

/*
 *   dev_pool     device memory of n_slots * expert_bytes (caller-owned)
 *   dev_staging  device memory of n_staging_bufs * staging_slots * expert_bytes
 *   n_staging_bufs  number of staging buffers used in rotation (>= 1)
 */
int moe_cache_create(moe_cache** cache, int n_layers, int E, int n_slots, size_t expert_bytes, void* dev_pool,
                     void* dev_staging, int n_staging_bufs, int staging_slots);
int moe_cache_destroy(moe_cache* cache);

/*
 * Make the given global ids resident: slot i receives global_ids[i] (host
 * array, n <= n_slots, ids distinct and in [0, n_layers*E)), copied from the
 * host blob host_src[i] (host array of host pointers; pinned memory gives
 * asynchronous copies).  Enqueued on `stream`.
 */
int moe_cache_set_resident(moe_cache* cache, const int32_t* global_ids, int n, const void* const* host_src,
                           moe_stream_t stream);

/*
 * Host-side lookup for one layer: the experts of `layer` that are not
 * resident, ascending (miss_ids host array with room for E), their count in
 * *n_miss, and the resident ones (hit_ids, may be NULL) with *n_hit.
 */
int moe_cache_lookup(const moe_cache* cache, int layer, int32_t* hit_ids, int* n_hit, int32_t* miss_ids,
                     int* n_miss);

/*
 * How moe_cache_stage copies a layer's missed experts into its staging slots
 * ("Strata benchmarks", prefill optimisation table: the next layer's experts
 * are streamed over PCIe while the current layer computes):
 *   MOE_STAGE_MEMCPY (default): one hipMemcpyAsync per missed expert;
 *   MOE_STAGE_KERNEL: one copy kernel of n_workgroups workgroups (1..1024)
 *     that reads the missed blobs from mapped pinned host memory, so the host
 *     enqueues one launch per layer instead of one copy per expert.  The
 *     (source, destination) list lives in pinned memory the handle owns.
 *     Needs expert_bytes % 16 == 0.
 * Errors: MOE_ERR_INVALID_ARG.
 */
#define MOE_STAGE_MEMCPY 0
#define MOE_STAGE_KERNEL 1
int moe_cache_set_stage_mode(moe_cache* cache, int mode, int n_workgroups);

/*
 * Fault injection into staging, for tests of a caller's error handling (no
 * passage defines it; production code installs no hook).  With a hook set,
 * moe_cache_stage calls hook(user, layer, index, expert) on the host before
 * it enqueues the copy of the index-th missed expert (local id `expert`) of
 * `layer`.  A nonzero return value v stops that call: it returns MOE_ERR_HIP
 * and moe_last_hip_error() reports v.  Copies enqueued before the failure may
 * still land in staging buffer `buf`, and the device table of the layer is
 * not uploaded, so until a later moe_cache_stage of the same layer into the
 * same buffer succeeds, neither that table nor that buffer may be read.
 * Residency and the other layers' tables are unaffected.  hook NULL removes
 * the hook.  Errors: MOE_ERR_INVALID_ARG (cache NULL).
 */
typedef int (*moe_stage_fault_fn)(void* user, int layer, int index, int expert);
int moe_cache_set_stage_fault_hook(moe_cache* cache, moe_stage_fault_fn hook, void* user);

/*
 * Stage one layer: copy each missing expert of `layer` (ascending id) from its
 * host blob host_src[e] (host array [E] of pinned host pointers; only the
 * misses are read) into consecutive slots of staging buffer `buf`, then write
 * the layer's device pointer table dev_table [E] (hits -> pool slots, misses ->
 * staging slots), all on `stream`, and record `done` (may be NULL) on it.
 * Returns MOE_ERR_CACHE_CAPACITY if the misses exceed staging_slots.  The
 * caller must not reuse staging buffer `buf` before the compute that reads it
 * has finished (order with events).
 */
int moe_cache_stage(moe_cache* cache, int layer, int buf, const void* const* host_src, void** dev_table,
                    moe_stream_t stream, moe_event_t done);

/*
 * Map one layer for reading misses in place ("single RTX 5090 runs a 125B
 * model", on-demand MoE expert scheduling: only the experts the gating network
 * picks are computed, so only those need their weights): write the layer's
 * device pointer table dev_table [E] with hits -> pool slots and misses -> the
 * device address of their host blob host_src[e] (host array [E] of pointers
 * into pinned host memory from hipHostMalloc or torch's pin_memory, which is
 * mapped into the device's address space), on `stream`, then record `done`
 * (may be NULL).  moe_expert_ffn then reads a missed expert's weights over the
 * host link, and only when the routing selects it: no copy and no host round
 * trip between routing and the FFN, so a whole decode stack can be one graph.
 * The table stays valid until the residency changes (moe_cache_set_resident).
 * Errors: MOE_ERR_INVALID_ARG (null handle, host_src or dev_table, layer out
 * of range, a null host pointer for a miss); MOE_ERR_HIP when a host blob is
 * not mapped for the current device (hipHostGetDevicePointer fails).
 */
int moe_cache_map_host(moe_cache* cache, int layer, const void* const* host_src, void** dev_table,
                       moe_stream_t stream, moe_event_t done);

/* ---------------------------------------------------------------------------
 * Adaptive residency ("How Strata works", adaptive expert cache section: the
 * cache keeps learning which experts the session uses most and adjusts its
 * contents).  Usage is counted on the device from the per-layer expert counts
 * of moe_permute / moe_route_permute; the caller ages the counts into scores
 * on the host; moe_cache_plan picks which resident experts to swap for which
 * missing ones; moe_cache_replace carries the swaps out on a stream.
 * ------------------------------------------------------------------------- */

/*
 * usage[e] += counts[e] for e < E (device int32 arrays; counts as written by
 * moe_permute for one layer).  Stream-ordered; wraps modulo 2^32 like any
 * int32 counter.  Errors: MOE_ERR_INVALID_ARG (null pointer, E < 1).
 */
int moe_usage_accumulate(int32_t* usage, const int32_t* counts, int E, moe_stream_t stream);

/*
 * Replacement plan (host only, no HIP call): over n_total global ids with
 * resident[g] in {0, 1} and non-negative scores score[g], pair the missing ids
 * by descending score (ties: lower id first) with the resident ids by
 * ascending score (ties: lower id first) and keep pair i while
 * score[admit] > (1 + margin) * score[evict], at most max_swaps pairs.
 * Writes evict_ids[i], admit_ids[i] (room for max_swaps each) and *n_swaps.
 * Errors: MOE_ERR_INVALID_ARG (null pointer, n_total < 1, max_swaps < 0,
 * margin < 0 or not finite, a resident flag other than 0/1, a negative or
 * non-finite score).
 */
int moe_cache_plan(int n_total, const uint8_t* resident, const float* score, int max_swaps, float margin,
                   int32_t* evict_ids, int32_t* admit_ids, int* n_swaps);

/*
 * Carry out n swaps on `stream`: admitted expert admit_ids[i] takes the pool
 * slot of evict_ids[i] (a resident id; admit ids not resident; all 2n ids
 * distinct), its blob is copied there from host_src[admit] (host array
 * [n_layers * E] of pinned host pointers, indexed by global id), and the
 * device pointer tables dev_tables ([n_layers][E] device array of pointers)
 * of every layer that moe_cache_map_host or moe_cache_stage has written are
 * rewritten: the admitted expert -> its slot, the evicted one -> the device
 * address of its host blob (read in place).  Work already enqueued on
 * `stream` sees the old contents; work enqueued after sees the new ones, so
 * the call belongs on the stream that runs the layers.
 * Errors: MOE_ERR_INVALID_ARG (as above, or a null host pointer for an
 * involved id); MOE_ERR_HIP (a host blob not mapped for the device, a copy
 * that cannot be enqueued).
 */
int moe_cache_replace(moe_cache* cache, int n, const int32_t* evict_ids, const int32_t* admit_ids,
                      const void* const* host_src, void** dev_tables, moe_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
