/*
 * libmoe: the MoE layer forward (Gate -> Scatter -> Expert Compute -> Gather)
 * on one AMD Instinct MI355X (gfx950).
 *
 * What the layer computes. Pages are named by address: [0539edu]
 * www.0539edu.com/news/4774449, [mhpq] www.mhpq.cn/news/563172, [hotelren]
 * www.hotelren.com/news/4731937, [trdm] www.trdm.cn/news/555962, [pptc]
 * www.pptc.cn/news/100465.
 *
 *   Gate     logits = x W_router (+ b_router)           [hotelren §3.2]
 *            idx[t, 0..k-1]: the k largest logits of token t, slot 0 the
 *            largest; equal logits go to the lower expert id ([mhpq §3.2],
 *            the routing kernel's strict greater-than test);
 *            w[t, j] = softmax of the k chosen logits    [0539edu §2.1]
 *            or, as an option, the chosen logits themselves ([hotelren §3.2]
 *            top-k on raw logits without a softmax)
 *   Scatter  assignments a = t*k + j grouped by expert, stable in a, with an
 *            (E+1)-entry row-offset table                [0539edu §2.2],
 *            [hotelren §2.3] dispatch_kernel, [pptc §3.3] expert_offsets
 *   Experts  per expert e: h = silu(X_e W_gate[e]) * (X_e W_up[e]),
 *            o = h W_down[e]                              [hotelren §2.1 steps 4-5]
 *   Gather   y[t] = sum_j w[t, j] * o(t, j)              [hotelren §2.3]
 *            combine_kernel, [pptc §2.1] fused output aggregation
 *   Shared   optional always-on expert, y[t] += sigmoid(x[t] . w_s) * S(x[t])
 *            ([0539edu §2.2] shared-expert-augmented MoE, [trdm §8])
 *
 * Conventions for every entry point:
 *   - All tensor pointers are HIP device pointers, row-major, densely packed.
 *   - The caller owns every buffer it passes. moe_layer_create copies what it
 *     needs; the caller may free the weight buffers once it returns.
 *   - Argument checks run before any HIP call or launch; a failed check writes
 *     nothing and returns a negative status. moe_last_error() then holds a
 *     message (thread-local).
 *   - Inputs holding NaN or Inf are not supported (results unspecified).
 *
 * Status codes are the moe_status values below.
 */
#ifndef LIBMOE_MOE_H
#define LIBMOE_MOE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

typedef enum moe_status {
    MOE_OK = 0,
    MOE_EINVAL = -1,        /* bad argument: NULL, out of range, misaligned */
    MOE_EUNSUPPORTED = -2,  /* valid but not implemented: dtype pair, shape */
    MOE_ENOMEM = -3,        /* device allocation failed (create only) */
    MOE_EHIP = -4           /* a HIP runtime call or launch failed */
} moe_status;

typedef enum moe_dtype {
    MOE_F32 = 0,   /* IEEE binary32 */
    MOE_BF16 = 1,  /* bfloat16, stored as 16-bit patterns */
    MOE_I8 = 2,    /* int8 with one fp32 scale per output channel */
    MOE_I4 = 3     /* int4 with one fp32 scale per 128 input rows of each output
                      channel ([mhpq §4.2] group-wise int4, group size 128); two
                      values per byte along the input axis ([trdm §6.1]), low
                      nibble = even row, 4-bit two's complement */
} moe_dtype;

/* Routing weights of the Gate ([0539edu §2.1] softmax over the gate logits;
 * [hotelren §3.2] the router variant that takes the top-k of the raw logits and
 * skips the softmax, its combine weighting each expert by that gating score). */
typedef enum moe_gate_weighting {
    MOE_WEIGHT_SOFTMAX = 0,  /* w[t, j] = softmax over the k chosen logits (sums to 1) */
    MOE_WEIGHT_RAW = 1       /* w[t, j] = the chosen logit itself (bias included, after
                                the clamp when gate_clamp is on), not normalised */
} moe_gate_weighting;

/* Layer shape ([0539edu §2.2]: an MoE layer of E experts with top-k routing, the
 * shared-expert variant, and the weights stored expert-major). Supported
 * (act_dtype, expert_dtype) pairs: (F32, F32), (BF16, BF16), (BF16, I8),
 * (BF16, I4). Limits: 1 <= top_k <= n_experts <= 128, top_k <= 64; for BF16/I8
 * experts d_model % 128 == 0 and d_ff % 64 == 0; for I4 experts d_model % 128
 * == 0 and d_ff % 128 == 0; for F32 experts d_model % 64 == 0 and d_ff % 64 ==
 * 0. shared_d_ff > 0 adds a shared expert (BF16 experts only) and must be a
 * multiple of d_ff. Which kernels run is chosen per call from T: BF16 weights
 * stream from HBM for T <= 64; above it they run on the tile-stream GEMMs (token rows
 * staged in LDS, weights streamed into registers) while the experts average at most
 * 128 rows and T*top_k <= 4096 (no shared expert), else on the LDS-tiled MFMA GEMMs;
 * I8 and I4 weights stream for T <= 32 and above it run on the tile-stream GEMMs.
 * The tile-stream GEMMs need 2*d_ff and d_model to be multiples of 256; otherwise
 * the LDS-tiled GEMMs run (F32 experts always run on the fp32 kernels). */
typedef struct moe_desc {
    int32_t d_model;
    int32_t n_experts;
    int32_t d_ff;
    int32_t top_k;
    int32_t max_tokens;     /* largest T any moe_forward call will pass */
    int32_t act_dtype;      /* moe_dtype of x and y */
    int32_t expert_dtype;   /* moe_dtype of the expert weights */
    int32_t shared_d_ff;    /* 0: no shared expert */
    int32_t profile;        /* 1: start with per-stage HIP events on (moe_set_profiling) */
    int32_t gate_clamp;     /* 1: clamp the routed logits to [-50, 50] before the top-k and
                               the softmax ([0539edu §5.2], the gate's clip option against
                               overflow); 0: use them as computed */
    int32_t gate_weighting; /* moe_gate_weighting: MOE_WEIGHT_SOFTMAX (0) or MOE_WEIGHT_RAW (1) */
} moe_desc;

/* Layer weights (device pointers, read only during moe_layer_create).
 * Expert matrices are stacked over experts and multiply from the right:
 *   w_gate, w_up  [E][d_model][d_ff]     element type = expert_dtype
 *   w_down        [E][d_ff][d_model]     (I4: [E][d_model/2][d_ff] and
 *                                        [E][d_ff/2][d_model] bytes, two rows a byte)
 *   s_gate, s_up  [E][d_ff]   fp32, I8 only: scale of each output column
 *   s_down        [E][d_model] fp32, I8 only
 *   (I4: s_gate, s_up [E][d_model/128][d_ff] and s_down [E][d_ff/128][d_model]
 *   fp32, the scale of each group of 128 input rows of each output column;
 *   weight = q * scale)
 *   w_router      [d_model][E] fp32 (required)
 *   b_router      [E] fp32 or NULL (no bias)
 *   w_shared_gate [d_model] fp32; ws_gate, ws_up [d_model][shared_d_ff] and
 *   ws_down [shared_d_ff][d_model] bf16 (only when shared_d_ff > 0). */
typedef struct moe_weights {
    const float* w_router;
    const float* b_router;
    const void* w_gate;
    const void* w_up;
    const void* w_down;
    const float* s_gate;
    const float* s_up;
    const float* s_down;
    const float* w_shared_gate;
    const void* ws_gate;
    const void* ws_up;
    const void* ws_down;
} moe_weights;

/* Routing results written by moe_forward (device pointers, 4-byte aligned).
 *   topk_idx        [T][k] int32, required: expert of slot j, slot 0 largest
 *   topk_w          [T][k] fp32, required: the routing weights (moe_desc.gate_weighting)
 *   expert_counts   [E] int32 or NULL: assignments per expert
 *   expert_offsets  [E+1] int32 or NULL: exclusive prefix sum, [E] = T*k
 *   sorted_assign   [T*k] int32 or NULL: assignment ids a = t*k + j grouped
 *                   by expert, ascending a within each expert
 *   shared_gate     [T] fp32 or NULL: sigmoid(x . w_s) (shared expert only) */
typedef struct moe_route_out {
    int32_t* topk_idx;
    float* topk_w;
    int32_t* expert_counts;
    int32_t* expert_offsets;
    int32_t* sorted_assign;
    float* shared_gate;
} moe_route_out;

typedef struct moe_layer moe_layer; /* opaque */

/* Create a layer on the current HIP device: checks desc and weights, allocates
 * the packed weights and a workspace sized for desc->max_tokens, repacks the
 * caller's weights into the kernels' tile order, and waits for that to finish.
 * ([0539edu §3.1] and [hotelren §3.1]: weights are converted once, before
 * inference, into the layout the kernels read -- reordered, transposed and
 * expert-major -- so the forward never touches the original layout; [mhpq §4.3]:
 * a failed initialisation hands back NULL and leaves a message to query.)
 * On success *out holds the layer; on failure *out is set to NULL (when out is
 * not NULL) and nothing is leaked. Statuses: EINVAL (NULL desc/weights/out or a
 * required weight pointer, non-positive sizes, top_k > n_experts), EUNSUPPORTED
 * (dtype pair, shape limits), ENOMEM, EHIP. */
MOE_API int moe_layer_create(const moe_desc* desc, const moe_weights* weights, moe_layer** out);

/* Enqueue one forward pass of T tokens on `stream` (a hipStream_t; NULL is the
 * default stream) and return without waiting. ([hotelren §2.1]: the six steps
 * Gate, top-k, Scatter, expert GEMMs and the weighted combine; [hotelren §2.2]:
 * the host works out the launch shapes from the batch and top-k and hands them
 * to the kernels; [pptc §3.4]: routing results are token-major [T][k]; [0539edu
 * §2.2]: the four stages Gate -> Scatter -> Expert Compute -> Gather.) x [T][d_model] and y
 * [T][d_model] are in act_dtype and 16-byte aligned; y is fully overwritten.
 * Allocates nothing. T == 0 enqueues nothing and returns MOE_OK (x, y and
 * route may then be NULL). Statuses: EINVAL (NULL layer, T < 0,
 * T > max_tokens, and for T > 0: NULL x/y/route/topk_idx/topk_w, misaligned
 * pointer, current device differs from the layer's), EHIP.
 * One layer must not be used by two overlapping calls: its workspace is shared. */
MOE_API int moe_forward(moe_layer* layer, const void* x, int32_t T, void* y,
                const moe_route_out* route, void* stream);

/* The same forward with the routing given by the caller instead of the Gate
 * ([pptc §3.4]: the engine consumes routing results produced elsewhere, on the
 * host or by another kernel, token-major [T][k]). Reads
 *   topk_idx     [T][k] int32, required: the expert of slot j of token t. Ids
 *                need not be distinct (a repeated expert processes the token
 *                once per slot); an id outside [0, n_experts) is read as expert
 *                0 with weight 0, so it adds nothing to y (and is counted under
 *                expert 0 in expert_counts).
 *   topk_w       [T][k] fp32, required: the weight of each slot, used as given
 *                (no normalisation).
 *   shared_gate  [T] fp32: the shared expert's scale, required exactly when the
 *                layer has a shared expert, else NULL.
 * and computes y[t] = sum_j topk_w[t, j] * expert(topk_idx[t, j], x[t])
 * (+ shared_gate[t] * S(x[t])), with the Scatter, Expert and Gather stages of
 * moe_forward (bit-identical to it when given moe_forward's own routing).
 * route may be NULL; of it only expert_counts, expert_offsets and
 * sorted_assign are written (when not NULL), its other fields are ignored.
 * x, y: as moe_forward; all routing pointers 4-byte aligned. Allocates nothing.
 * Statuses: EINVAL (as moe_forward, and NULL topk_idx/topk_w, shared_gate
 * missing or given against the layer's shape), EHIP. Stage times: the gate
 * entry times the reading of the given routing. */
MOE_API int moe_forward_routed(moe_layer* layer, const void* x, int32_t T, const int32_t* topk_idx,
                               const float* topk_w, const float* shared_gate, void* y,
                               const moe_route_out* route, void* stream);

/* Size of the static device scratch that moe_forward_noalloc works in: 64 MiB on every
 * device the library runs on, held from the library's first use of that device until
 * the process ends. */
#define MOE_STATIC_SCRATCH_BYTES (64u << 20)

/* moe_forward for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. The same computation,
 * launch plan and results as moe_forward (bit for bit), but the per-call workspace (the
 * routing tables, the gathered GEMM operand, H and the combine rows) lives in one static
 * device array of MOE_STATIC_SCRATCH_BYTES instead of the layer's own workspace; the call
 * allocates nothing and launches kernels only (no memset, copy or host wait). Arguments,
 * statuses and ownership as moe_forward, plus: EINVAL when the batch needs more scratch
 * than the array holds (decode batches fit: T <= 64 for BF16 and I4 experts, T <= 32 for I8,
 * on layers up to d_model 8192 and d_ff 16384; large prefill batches do not -- use
 * moe_forward), with the needed size in moe_last_error(). Every layer and every call on
 * one device shares that device's array, whatever the stream: calls that overlap in time
 * on one device race and give wrong results, so serialise them (one stream, or events).
 * The array keeps the last call's contents; every byte a call reads from it is written
 * earlier in the same call, so nothing is cleared between calls. */
MOE_API int moe_forward_noalloc(moe_layer* layer, const void* x, int32_t T, void* y,
                                const moe_route_out* route, void* stream);

/* Turn per-stage HIP event timing on (1) or off (0) for the following
 * moe_forward calls on this layer ([0539edu §3.3]: profiling is a per-call
 * switch of the inference config). The initial state is desc->profile. Events
 * are recorded on the call's stream between the stages, so timing adds a few
 * microseconds per stage. Statuses: EINVAL (NULL layer, enable not 0 or 1),
 * EHIP (event creation failed). */
MOE_API int moe_set_profiling(moe_layer* layer, int enable);

/* Per-stage times in milliseconds of the last moe_forward that ran with
 * profiling on ([0539edu §3.3]: the profiling trace reports Gate, Scatter,
 * ExpertCompute and Gather times of each call): ms[0] gate, ms[1] scatter (with the gathering of token rows
 * for the large-batch GEMMs), ms[2] expert up (gate/up GEMM and SiLU), ms[3]
 * expert down, ms[4] gather/combine. Where the gate's launches also run the
 * scatter (batches of up to four tokens with at most 16 router columns; with
 * more than 16 router columns -- experts plus the shared gate -- batches of up
 * to 24 bf16 tokens or 64 fp32 tokens with top_k <= 8), its time is booked on
 * the gate and the scatter reads as the event overhead alone. Waits for that call's
 * last event. EINVAL if no forward has run with profiling on. */
MOE_API int moe_stage_times(moe_layer* layer, float ms[5]);

/* Release a layer and everything it allocated ([mhpq §4.3]: the engine's
 * context is freed by one call that owns every buffer it made). NULL-safe.
 * Waits for the device work of the layer to finish. */
MOE_API void moe_destroy(moe_layer* layer);

/* Static text of a status code ([0539edu §3.3]: the inference call returns an
 * int status; [hotelren §5.2]: a failed call returns -1 instead of crashing). */
MOE_API const char* moe_status_str(int status);

/* Message of the last failed call on this thread ("" if none) ([mhpq §4.3]: a
 * failed call is explained by an error-string query rather than an exception). */
MOE_API const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBMOE_MOE_H */
