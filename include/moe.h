/*
 * moe.h -- C ABI of libmoe: one GPU's share of a routed-expert MoE layer forward
 * on AMD Instinct MI355X (gfx950).
 *
 * The calls follow the pipeline of the WideEP explainer page (Kimi K3), section
 * "The router writes a network schedule": the source scores each token against the
 * experts and picks its top-k; a dispatcher tallies the rows bound for each
 * destination, reserves their places, copies the token rows there in destination
 * order and attaches routing metadata; the receiver groups rows by expert and runs
 * the expert matrix multiplies; the combine sends results back and the source puts
 * rows back in token order and
 * applies the routing weights.  On one GPU every assignment is local, so the
 * "transfer" is the permutation itself (same page, table of communication
 * paths, row "Same GPU": nothing crosses a link, but the rows are still permuted and
 * still cost HBM traffic).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every tensor pointer is a DEVICE pointer owned by the caller, dense and
 *   row-major, 16-byte aligned.  The library allocates nothing and keeps no
 *   state between calls beyond a process-wide counter that tags each
 *   decode-scale routing call (moe_layer_forward) so it never mistakes another
 *   call's hand-over word for its own; all scratch comes from the caller's
 *   workspace `ws` of `ws_bytes` bytes (size it with moe_workspace_bytes; NULL
 *   allowed when that size is 0), and nothing in it has to start at zero.
 * - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *   stream).  They never read device memory on the host and never
 *   synchronise: static grids, GPU-resident counts and offsets (same page,
 *   table row "CPU control path": fixed shapes, metadata that stays on the device).
 *   Calls are re-entrant across distinct workspaces; two calls that share a
 *   workspace or outputs must be ordered by the caller.
 * - Element types: activations, expert weights, projections and the permuted
 *   rows are MOE_BF16 or MOE_F32 as `moe_shape.dtype` says.  Router weights,
 *   bias, logits and routing weights are always fp32; ids, counts, offsets
 *   and metadata are int32.  bf16 math accumulates in fp32.
 * - Weight orientation (output-major, like a linear layer's weight, so every
 *   contraction reads both operands along contiguous K):
 *     gate_w [E x H]   logits = X gate_w^T
 *     w1, w3 [E x I x D], w2 [E x D x I]
 *                      expert e: Y = (SiLU(X w1[e]^T) * (X w3[e]^T)) w2[e]^T
 *     wd [L x H], wu [H x L]   Z = X wd^T,  out = out_L wu^T
 *   D is the dispatched width: L for latent layers (L > 0), else H.
 * - Errors: every call validates its arguments on the host before touching
 *   the GPU and returns MOE_ERR_INVALID_ARG (bad shape, NULL or misaligned
 *   pointer), MOE_ERR_UNSUPPORTED (shape outside the kernels' limits, listed
 *   per call), MOE_ERR_WORKSPACE (ws_bytes too small) or MOE_ERR_HIP (a kernel
 *   launch failed; no device status is read).  Nothing throws or aborts.
 * - Preconditions not checked (they would need a device read): logits are
 *   finite or -inf; caller-supplied topk_ids are in [0, E) and distinct per
 *   token; offsets are the exclusive prefix sum of the per-expert counts.
 *
 * Limits: 1 <= k <= E, E <= 1024, k <= 64; T*k < 2^31; bf16 layers need D % 64 == 0,
 * I % 64 == 0, (latent layers) H % 64 == 0 and (shared expert) shared_I % 64 == 0;
 * fp32 layers need D % 4 == 0 and H % 4 == 0.  A shared expert needs L == 0.
 * MXFP8 dispatch needs a bf16 layer and D % 128 == 0.
 *
 * MXFP8 dispatch (moe_shape.dispatch = MOE_DISPATCH_MXFP8; value-changing)
 * -------------------------------------------------------------------------
 * "Top-k multiplies traffic. Locality subtracts it." (WideEP explainer): the rows a
 * device sends may travel in a narrower number format with their scale factors
 * alongside, the expert math may run in that format, and results come back wide;
 * an honest comparison includes the format-conversion work, the bytes of the
 * scales and the change in the numbers.  Quantisation is a
 * value-changing optimisation ("Three Parameter Counts...", table of "Which
 * optimizations need a task-level gate").  The format is OCP MX "MXFP8-E4M3", the
 * one gfx950's scaled matrix instructions take: E4M3 codes (1 sign, 4 exponent
 * bits with bias 7, 3 mantissa bits, largest magnitude 448) with one E8M0 scale
 * byte 2^(s-127) per 32 consecutive elements of a row along the contraction axis.
 * A block with largest magnitude m gets s = 127 + floor(log2 m) - 8 (clamped to
 * 0..254; an all-zero block gets 0), and each element is divided by the scale,
 * clamped to +-448 and rounded to the nearest E4M3 value, ties to even
 * (moe_quantize_mxfp8).  Then the dispatched rows x_perm are [T*k x D] codes plus
 * x_perm_scale [T*k x D/32] scales (one byte per element plus one per 32: the
 * dispatch bytes become T*k*D*33/32), W1 / W3 are codes [E x I x D] with scales
 * [E x I x D/32], the gate/up products run on the fp8 matrix cores with fp32
 * accumulation, and everything after them (SwiGLU intermediate, W2, Y, combine)
 * stays bf16.  Routing does not change.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 5

#ifndef MOE_API
#define MOE_API __attribute__((visibility("default")))
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_WORKSPACE = 3,
  MOE_ERR_HIP = 4
} moe_status;

typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Element format of the dispatched rows (moe_shape.dispatch). */
typedef enum moe_dispatch_fmt {
  MOE_DISPATCH_DTYPE = 0,  /* the layer dtype */
  MOE_DISPATCH_MXFP8 = 1   /* MXFP8-E4M3 codes + E8M0 scales per 32 (bf16 layers, value-changing) */
} moe_dispatch_fmt;

/* Which call a workspace size is asked for. */
typedef enum moe_call {
  MOE_CALL_ROUTE = 0,
  MOE_CALL_DISPATCH = 1,
  MOE_CALL_FFN = 2,
  MOE_CALL_COMBINE = 3,
  MOE_CALL_LAYER = 4
} moe_call;

/* moe_combine flags. */
#define MOE_COMBINE_FUSED 0   /* one kernel: gather k rows, weight, sum (production) */
#define MOE_COMBINE_UNFUSED 1 /* two kernels: unpermute to token order, then weighted reduce */

/* Stage events recorded by moe_layer_forward when `stage_events` is non-NULL. */
#define MOE_NUM_STAGE_EVENTS 10
/* [0] start  [1] after latent down-projection  [2] after gate  [3] after top-k+count+scan
 * [4] after permute  [5] after expert gate/up GEMM  [6] after expert down GEMM
 * [7] after the shared expert  [8] after combine  [9] after latent up-projection.
 * Stages that do not run leave two consecutive events back to back.  When the down
 * GEMM's kernel is the fused down GEMM + combine (moe_plan.down_kernel
 * "k_down_combine<...>": bf16 steps on the 16-row decode tiles, no shared expert) the
 * combine runs inside the down GEMM's launch, so its time shows in [5]..[6] and
 * [7]..[8] is empty. */

typedef struct moe_shape {
  int64_t T;      /* tokens */
  int64_t H;      /* model width */
  int64_t E;      /* routed experts */
  int64_t k;      /* experts per token */
  int64_t I;      /* expert intermediate width */
  int64_t L;      /* latent dispatch width, 0 = none */
  int32_t dtype;  /* moe_dtype */
  int32_t shared_I;  /* intermediate width of the shared expert, 0 = no shared expert */
  int64_t capacity;  /* rows kept per expert, 0 = no limit.  With C > 0 each expert keeps
                      * its first C assignments in ascending token order and drops the rest
                      * (their token_row is -1 and they add nothing to the combine; the kept
                      * routing weights are not renormalised).  Dropping changes the layer's
                      * output: WideEP explainer, "An imbalanced router creates a network
                      * hotspot".  C >= T can drop nothing and behaves as 0. */
  int32_t dispatch;  /* moe_dispatch_fmt */
  int32_t reserved;  /* 0 */
} moe_shape;

/* Workspace bytes `call` needs for shape `s` (0 if the shape is invalid). Host only. */
MOE_API size_t moe_workspace_bytes(const moe_shape* s, int call);

/* moe_layer_plan flags: which optional inputs the planned moe_layer_forward call gets. */
#define MOE_PLAN_GATE 1    /* a router weight (gate_w) is given: the gate scores are computed */
#define MOE_PLAN_X_PERM 2  /* the caller asks for the permuted rows (aux.x_perm, and with MXFP8
                            * dispatch aux.x_perm_scale) */

/* The kernels moe_layer_forward runs for a shape: the same decision the call itself
 * takes (one function makes it for both), reported so that measurements can name and
 * price the kernels that actually ran. */
typedef struct moe_plan {
  int32_t launches;            /* kernel launches of one moe_layer_forward (stage events aside) */
  int32_t decode_path;         /* 1: decode-scale step, routing + counts + offsets + row metadata
                                * in one launch */
  int32_t rows_gathered;       /* 1: no permuted copy is written; the expert gate/up GEMM reads
                                * the token rows through row_token */
  int32_t gate_up_tile_m, gate_up_tile_n, gate_up_persistent;  /* expert gate/up GEMM */
  int32_t down_tile_m, down_tile_n, down_persistent;           /* expert down GEMM */
  int32_t route_workgroups;    /* decode path: workgroups of the routing launch (1, or
                                * ceil(T / 4) when one workgroup would take longer); else 0 */
  const char* gate_up_kernel;  /* static: kernel name up to its tile arguments, as a trace shows it */
  const char* down_kernel;     /* static, likewise */
} moe_plan;

/* Fill *plan for a moe_layer_forward call on shape s with flags MOE_PLAN_*.  Host only:
 * no GPU work.  Returns MOE_ERR_INVALID_ARG / MOE_ERR_UNSUPPORTED for a shape that
 * moe_layer_forward would reject the same way, or for a NULL plan or unknown flags. */
MOE_API moe_status moe_layer_plan(const moe_shape* s, int flags, moe_plan* plan);

/* Static string for a status code. */
MOE_API const char* moe_status_string(int status);

/* MOE_ABI_VERSION of the loaded library. */
MOE_API int moe_abi_version(void);

/*
 * Gate scores + top-k selection + per-expert counts and offsets (steps a1-a3).
 *
 * Passage: WideEP explainer, "The router writes a network schedule" (the source
 * scores tokens against experts and picks each token's top-k; the dispatcher
 * tallies rows per destination and reserves their places) and "Sparse compute. Dense availability."
 * (k of E experts per token).
 *
 * x        [T x H] activations (dtype); read only when gate_w != NULL.
 * gate_w   [E x H] fp32 router weight, or NULL when `logits` is given.
 * gate_bias[E] fp32 per-expert bias, nullable.  With gate_w the bias is added
 *          into the written logits; without it the score is the fp32 sum
 *          logits + bias, formed on the fly (logits are not modified).
 * logits   [T x E] fp32: output when gate_w != NULL, input otherwise.
 * topk_ids [T x k] int32 out: per token the k experts with the largest scores,
 *          listed by descending score; equal scores go to the lower expert
 *          index; -0.0 ranks equal to +0.0.
 * topk_w   [T x k] fp32 out: softmax over all E scores gathered at topk_ids and
 *          renormalised over the k (equal to exp(s_j - s_max) / sum_i exp(s_i - s_max)
 *          over the selected i).  A token whose scores are all -inf gets NaN.
 * counts   [E] int32 out: assignments per expert (sum = T*k), or with an expert
 *          capacity C the rows kept, min(assignments, C).
 * offsets  [E+1] int32 out: exclusive prefix sum of counts, offsets[E] = T*k (the kept
 *          rows with a capacity).
 */
MOE_API moe_status moe_route_topk(const void* x, const float* gate_w, const float* gate_bias,
                          float* logits, int32_t* topk_ids, float* topk_w, int32_t* counts,
                          int32_t* offsets, const moe_shape* s, void* ws, size_t ws_bytes,
                          void* stream);

/*
 * Permutation into expert-contiguous rows + routing metadata (step a4).
 *
 * Passage: WideEP explainer, "The router writes a network schedule" (permute
 * activations into destination-contiguous buffers and attach routing
 * metadata; the receiver groups tokens by expert).  The buffer holds exactly
 * T*k*D*elem bytes, the dispatch payload of "Top-k multiplies traffic.
 * Locality subtracts it." (no padding, every assignment local).
 *
 * x         [T x D] rows to dispatch (dtype): the activations, or Z for latent layers.
 * topk_ids  [T x k] int32, offsets [E+1] int32 (as written by moe_route_topk).
 * x_perm    [T*k x D] out: expert e's rows occupy [offsets[e], offsets[e+1]),
 *           holding, in ascending token order, a bitwise copy of every token
 *           that picked e (with a capacity C: the first C of them; rows from
 *           offsets[E] on are left untouched).  With MXFP8 dispatch: the E4M3 codes
 *           of each token's row (quantised once per token, then copied).
 * x_perm_scale [T*k x D/32] uint8 out: the rows' E8M0 scales (MXFP8 dispatch only;
 *           must be NULL otherwise).
 * row_token [T*k] int32 out: source token of each row (the first offsets[E] entries).
 * token_row [T x k] int32 out: row holding token t's j-th assignment, -1 if dropped.
 */
MOE_API moe_status moe_dispatch_permute(const void* x, const int32_t* topk_ids, const int32_t* offsets,
                                void* x_perm, uint8_t* x_perm_scale, int32_t* row_token,
                                int32_t* token_row, const moe_shape* s, void* ws, size_t ws_bytes,
                                void* stream);

/*
 * Grouped SwiGLU expert FFN over ragged row counts (step a5).
 *
 * Passage: WideEP explainer, "The router writes a network schedule" (expert
 * matrix multiplies on the grouped rows) and "Sparse compute. Dense
 * availability." (fewer, fatter grouped GEMMs); "Three Parameter Counts...",
 * table of "Which optimizations need a task-level gate" (one grouped launch covers
 * many experts' matrices whatever their row counts, and an expert without rows
 * gets no work).
 *
 * x_perm [T*k x D] (dtype), offsets [E+1] int32.
 * w1, w3 [E x I x D], w2 [E x D x I] (dtype).  Weights of experts with no rows
 *        are never read.
 * y_perm [T*k x D] out (dtype): row r of expert e holds
 *        (SiLU(x w1[e]^T) * (x w3[e]^T)) w2[e]^T, with the intermediate rounded
 *        to dtype; unweighted (weights apply in the combine).
 * MXFP8 dispatch: x_perm holds E4M3 codes with x_perm_scale [T*k x D/32], w1 / w3
 *        hold codes with w1_scale / w3_scale [E x I x D/32] (as moe_quantize_mxfp8
 *        writes them); x w1^T and x w3^T are products of the dequantised values with
 *        fp32 accumulation.  The scale pointers must be NULL otherwise.
 */
MOE_API moe_status moe_grouped_ffn(const void* x_perm, const uint8_t* x_perm_scale, const int32_t* offsets,
                           const void* w1, const uint8_t* w1_scale, const void* w3,
                           const uint8_t* w3_scale, const void* w2, void* y_perm, const moe_shape* s,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * MXFP8 conversion kernel (the conversion and scale metadata of a low-precision
 * dispatch: "Top-k multiplies traffic. Locality subtracts it.", WideEP explainer).
 *
 * src   [rows x cols] bf16 (src_dtype MOE_BF16) or fp32 (MOE_F32) values, finite.
 * q     [rows x cols] uint8 out: E4M3 codes.
 * scale [rows x cols/32] uint8 out: E8M0 scales, one per 32 consecutive elements of
 *       a row (the rule is in the MXFP8 section at the top of this file).
 * Used for the expert weights W1 / W3 (once, offline) and inside the dispatch for the
 * activations.  cols % 32 != 0 -> MOE_ERR_UNSUPPORTED; rows == 0 does nothing.
 */
MOE_API moe_status moe_quantize_mxfp8(const void* src, int src_dtype, int64_t rows, int64_t cols,
                                      uint8_t* q, uint8_t* scale, void* stream);

/*
 * Combine: unpermute and apply routing weights (step a6).
 *
 * Passage: WideEP explainer, "The router writes a network schedule" (the
 * combine reverses the route; the source unpermutes and applies routing
 * weights) and "Top-k multiplies traffic..." (combine moves about the same
 * volume as dispatch).
 *
 * y_perm    [T*k x D] (dtype), token_row [T x k] int32 (-1: dropped assignment, no
 *           term), topk_w [T x k] fp32.
 * shared_out[T x D] (dtype), nullable: the shared expert's output, added with
 *           weight 1 (a shared expert runs for every token whatever the router
 *           picks: "Three Parameter Counts...", "What the utilization dashboard
 *           smooths away").
 * out       [T x D] out, element type out_dtype (MOE_F32 or MOE_BF16):
 *           out[t] = sum_{j=0..k-1} topk_w[t,j] * y_perm[token_row[t,j]]
 *           (+ shared_out[t]), fp32 accumulation in ascending j, the shared term
 *           added last, one rounding to out_dtype.  The bf16 result is the
 *           round-to-nearest-even of the fp32 result.
 * flags     MOE_COMBINE_FUSED (one kernel) or MOE_COMBINE_UNFUSED (unpermute to
 *           token order in the workspace, then the weighted reduce: the separate
 *           "unpermutation" and "combine" timers of "Three Parameter Counts...",
 *           "What the utilization dashboard smooths away").  Same result bits.
 */
MOE_API moe_status moe_combine(const void* y_perm, const int32_t* token_row, const float* topk_w,
                       const void* shared_out, void* out, int out_dtype, int flags,
                       const moe_shape* s, void* ws, size_t ws_bytes, void* stream);

/* Weights of one layer for moe_layer_forward (device pointers, layouts as above). */
typedef struct moe_layer_weights {
  const float* gate_w;     /* [E x H] fp32, or NULL: router logits are given */
  const float* gate_bias;  /* [E] fp32, nullable */
  const void* w1;          /* [E x I x D] */
  const void* w3;          /* [E x I x D] */
  const void* w2;          /* [E x D x I] */
  const void* wd;          /* [L x H], latent layers only */
  const void* wu;          /* [H x L], latent layers only */
  const void* ws1;         /* [shared_I x H] shared expert gate branch, when shared_I > 0 */
  const void* ws3;         /* [shared_I x H] shared expert up branch */
  const void* ws2;         /* [H x shared_I] shared expert down projection */
  const uint8_t* w1_scale; /* [E x I x D/32] E8M0 scales of w1 (MXFP8 dispatch only, else NULL) */
  const uint8_t* w3_scale; /* [E x I x D/32] E8M0 scales of w3 (MXFP8 dispatch only, else NULL) */
} moe_layer_weights;

/* Optional caller buffers that expose the intermediate results (each nullable;
 * NULL fields live in the workspace). */
typedef struct moe_layer_aux {
  int32_t* topk_ids;   /* [T x k] */
  float* topk_w;       /* [T x k] */
  int32_t* counts;     /* [E] */
  int32_t* offsets;    /* [E+1] */
  int32_t* row_token;  /* [T*k] */
  int32_t* token_row;  /* [T x k] */
  void* x_perm;        /* [T*k x D] dtype */
  void* y_perm;        /* [T*k x D] dtype */
  void* z;             /* [T x L] dtype, latent layers */
  void* out_latent;    /* [T x L] dtype, latent layers: combine output before up-projection */
  uint8_t* x_perm_scale;  /* [T*k x D/32] E8M0 scales of x_perm (MXFP8 dispatch only) */
} moe_layer_aux;

/*
 * The whole layer forward in one call (steps a1-a7), the execution-only fusion
 * of "Three Parameter Counts...", table of "Which optimizations need a
 * task-level gate": routing ids, counts, offsets and the permutation are
 * bit-identical to the separate calls on the same logits.
 *
 * Decode-scale steps (fewer than 48 rows per expert on average, T <= 128) take a
 * low-latency path of three launches ("Three Parameter Counts...", "Halving top-k is a
 * network change first": at decode-scale token counts the layer is bound by launch
 * latency): routing, counts, offsets and row metadata in one launch; the gate/up GEMM
 * reading the token rows through row_token; the down GEMM with the combine, each
 * workgroup owning 16 output columns of every row.  The output bits are those of the
 * separate calls.  Latent projections, MXFP8 conversion of the token rows, a requested
 * permuted copy and a shared expert add their own launches.  The routing launch is one
 * workgroup while ceil(T / 16) * k * ceil(E / 64) <= 640, else ceil(T / 4) workgroups
 * (e.g. 896 experts, top-16, T = 128) of which the last to finish writes the metadata,
 * handing over through 8 bytes of the workspace (moe_plan.route_workgroups says which).
 * Such calls read and clear that word; calls that overlap on one workspace race on it,
 * as on the rest of the workspace.
 *
 * Latent layers (s->L > 0) follow "Latent MoE" (Definition; Current Synthesis):
 * the router scores the full-width X, the rows dispatched are Z = X wd^T, and the
 * combined latent output (rounded to dtype) is projected back: out = out_L wu^T.
 *
 * Shared expert (s->shared_I > 0, non-latent layers): a SwiGLU FFN that every
 * token passes through regardless of the router ("Three Parameter Counts...",
 * "What the utilization dashboard smooths away"; it is replicated with the
 * non-expert weights, research-vault claim IX2-0406):
 * Ys = (SiLU(X ws1^T) * (X ws3^T)) ws2^T with the intermediate and Ys rounded to
 * dtype, added in the combine as its shared_out term.
 *
 * MXFP8 dispatch (s->dispatch): w->w1 / w->w3 are E4M3 codes with w1_scale /
 * w3_scale; the dispatched rows are quantised in the dispatch (see the section at
 * the top of this file); aux->x_perm then receives codes and aux->x_perm_scale
 * their scales.
 *
 * x       [T x H] (dtype).
 * logits  [T x E] fp32: input when w->gate_w == NULL, else output (nullable: then
 *         kept in the workspace).
 * out     [T x H] out, element type out_dtype (MOE_F32 or MOE_BF16).
 * aux     nullable, see moe_layer_aux.
 * stage_events  NULL or an array of MOE_NUM_STAGE_EVENTS hipEvent_t created by
 *         the caller; each non-NULL entry is recorded on `stream` at its stage
 *         boundary (a NULL entry is skipped: every record puts a few microseconds
 *         between the kernels either side of it).
 */
MOE_API moe_status moe_layer_forward(const moe_layer_weights* w, const void* x, float* logits, void* out,
                             int out_dtype, const moe_shape* s, moe_layer_aux* aux,
                             void** stage_events, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_layer_forward without a caller workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, and harnesses that forbid
 * hipMalloc.  The same computation, kernels and results as moe_layer_forward (same
 * arguments minus ws / ws_bytes); the workspace is a device array inside the library,
 * MOE_NOALLOC_SCRATCH_BYTES long, one per GPU, set up on the first call on each device
 * (a symbol lookup, no allocation) and held until the process ends.  The call itself
 * allocates nothing.
 *
 * Limit: shapes whose layer workspace, moe_workspace_bytes(s, MOE_CALL_LAYER), exceeds
 * MOE_NOALLOC_SCRATCH_BYTES return MOE_ERR_WORKSPACE (64 MiB holds decode-scale steps, e.g.
 * the 896-expert top-16 layer up to T = 340 tokens, or a 256-expert top-8 layer of width
 * 7168 up to T = 128).  Other errors as moe_layer_forward.
 *
 * Every call on one GPU shares that GPU's array and finds the last call's contents in
 * it (nothing in it needs to start at zero): calls that overlap on one GPU (different
 * streams, or threads without ordering) race and must be ordered by the caller.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
MOE_API moe_status moe_layer_forward_noalloc(const moe_layer_weights* w, const void* x, float* logits,
                                             void* out, int out_dtype, const moe_shape* s,
                                             moe_layer_aux* aux, void** stage_events, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
