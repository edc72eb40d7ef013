/*
 * moe.h - C ABI of the MI355X (gfx950) MoE-layer forward, one GPU's share.
 *
 * The layer is the four-step expert-parallel pipeline: route, dispatch,
 * local expert compute, combine (Ultralytics glossary "Expert Parallelism",
 * section "How Tokens Move Between GPUs", numbered steps; ai360xpert "Expert
 * Parallelism", section "The All-to-All Bottleneck"; mbrenndoerfer "Expert
 * Parallelism > Summary", pipeline paragraph).  No inter-GPU traffic happens
 * here: dispatch produces the rank-major send layout an all-to-all would move.
 *
 * Conventions shared by every entry point
 *  - Every pointer argument is a DEVICE pointer owned by the caller, unless a
 *    comment says "host".  The library never allocates, frees or synchronises;
 *    all work is enqueued on the caller's hipStream_t (NULL = default stream)
 *    and is asynchronous.  Data-dependent sizes stay on the device: no call
 *    copies anything back to the host.
 *  - Layouts are dense row-major.  Weights use the [out, in] layout of a
 *    linear layer.  Token-major [T, k] arrays list the k choices of a token in
 *    order of decreasing selection key (ties: lower expert index first).
 *  - Dtype codes: MOE_F32 = float, MOE_BF16 = bfloat16 bit patterns (uint16),
 *    MOE_FP8_E4M3 = OCP e4m3fn bytes (expert weights only).
 *  - Device pointers must be 16-byte aligned.  Supported maxima: E <= 256,
 *    k <= 8.  d and h must be multiples of 128.
 *  - Argument errors return MOE_ERR_INVALID (unsupported combinations
 *    MOE_ERR_UNSUPPORTED, a too-small workspace MOE_ERR_WORKSPACE) before
 *    anything is launched; a failed launch returns MOE_ERR_HIP.  Faults inside
 *    kernels surface at the caller's next synchronisation.  moe_last_error()
 *    describes the most recent non-OK status of the calling thread.
 *  - Calls that share a workspace must be ordered on one stream.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID = -1,
  MOE_ERR_UNSUPPORTED = -2,
  MOE_ERR_WORKSPACE = -3,
  MOE_ERR_HIP = -4
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 } moe_dtype;
typedef enum { MOE_SOFTMAX = 0, MOE_SIGMOID = 1 } moe_score;
typedef enum { MOE_RELU = 0, MOE_GELU = 1, MOE_SWIGLU = 2 } moe_act;
/* Layout of expert weight matrices: the [out, in] row-major layout of a
 * linear layer, or the 16-row tiled layout moe_weight_tile produces. */
typedef enum { MOE_W_ROWMAJOR = 0, MOE_W_TILED16 = 1 } moe_w_layout;

#define MOE_MAX_EXPERTS 256
#define MOE_MAX_TOPK 8
/* Number of events moe_layer_forward records when moe_layer_args.events is
 * set: before route, after route, after dispatch, after the first expert
 * GEMM, after the expert FFN, after combine. */
#define MOE_LAYER_EVENTS 6

/* ------------------------------------------------------------------ route
 * Router scores and top-k (Ultralytics, "How Tokens Move Between GPUs",
 * step 1: a linear layer gives each token one score per expert, and each
 * token goes to its k highest-scoring experts).  logits = x W_r^T + b_router, in fp32.
 *   score = MOE_SOFTMAX: probabilities p = softmax(logits) over all E; the
 *           selection key is the logit itself (same order as p).
 *   score = MOE_SIGMOID: p = sigmoid(logits); the selection key is
 *           fp32(sigmoid(logit) evaluated in double) + b_select, in fp32.
 *           b_select only changes which experts are picked (Ultralytics,
 *           "Load Balancing and Capacity", bias-based balancing bullet).
 *   ids[t, :]     = the k best keys, ordered (key desc, expert asc).
 *   weights[t, j] = p[ids[t, j]] / sum_j' p[ids[t, j']]  (renorm = 1) or
 *                   p[ids[t, j]]                         (renorm = 0).
 * Identical-logits mode: x == NULL.  Then `logits` is an INPUT holding the
 * final fp32 logits (b_router must be NULL) and only scores and top-k run.
 * Group-limited selection (n_groups > 0, 0 < topk_groups < n_groups): the E
 * experts form n_groups contiguous equal groups (nodes); a token may only use
 * experts of its topk_groups best groups, a group's score being its largest
 * selection key (ties: lower group index); the other experts' keys count as
 * -infinity (DeepSeek-V3 limits each token to experts on 4 nodes: Ultralytics,
 * "Load Balancing and Capacity").  Requires n_groups <= 64, E % n_groups == 0,
 * E/n_groups a power of two or a multiple of 64, and k <= topk_groups*E/n_groups.
 */
typedef struct moe_route_args {
  int64_t T;              /* tokens */
  int32_t d, E, k;        /* model dim, experts, choices per token */
  int32_t act_dtype;      /* MOE_F32 or MOE_BF16: dtype of x and w_router */
  int32_t score;          /* moe_score */
  int32_t renorm;         /* 1: renormalise the weights over the k selected */
  int32_t n_groups;       /* expert groups for group-limited selection, 0 = off */
  int32_t topk_groups;    /* groups a token may use (0 or >= n_groups = no limit) */
  const void* x;          /* [T, d] hidden states, or NULL (see above) */
  const void* w_router;   /* [E, d] */
  const float* b_router;  /* [E] added to the logits, or NULL */
  const float* b_select;  /* [E] selection-only bias (MOE_SIGMOID), or NULL */
  float* logits;          /* [T, E]: optional output, or the input if x == NULL */
  int32_t* ids;           /* [T, k] out */
  float* weights;         /* [T, k] out */
} moe_route_args;

size_t moe_route_workspace_bytes(const moe_route_args* a);
moe_status moe_route(const moe_route_args* a, void* workspace, size_t ws_bytes,
                     hipStream_t stream);

/* --------------------------------------------------------------- dispatch
 * Histogram, capacity drop, offsets and the stable permutation into the
 * send buffer, plus the row pack.  Experts live on ranks in contiguous equal
 * blocks (rank = e / (E/R): Ultralytics listing; ai360xpert "Enter Expert
 * Parallelism"), so the expert-major layout is also rank-major.
 *   counts[e]      = number of (t, j) with ids[t, j] == e.
 *   kept[e]        = min(counts[e], capacity).  Assignments are visited in
 *                    token-major order; each expert keeps its first
 *                    `capacity`, the rest are dropped (Ultralytics, "Load
 *                    Balancing and Capacity", capacity bullet).
 *   expert_off     = exclusive prefix sum of kept, [E+1].
 *   rank_counts[r] = sum of kept over rank r's experts; rank_off[r] =
 *                    expert_off[r*E/R], rank_off[R] = expert_off[E].
 *   slot[t, j]     = expert_off[e] + position of (t, j) among e's
 *                    assignments, or -1 if dropped.
 *   src[s]         = token of send row s (token order within each expert:
 *                    mbrenndoerfer "Summary", buffer-management bullet).
 *   x_send[s, :]   = x[src[s], :].
 * Output sizes: src and x_send need moe_send_rows_max(T, k, E, capacity)
 * rows.  capacity = INT32_MAX means no limit.
 */
typedef struct moe_dispatch_args {
  int64_t T;
  int32_t d, E, k, R;
  int32_t capacity;       /* from moe_capacity() */
  int32_t act_dtype;      /* dtype of x / x_send */
  const int32_t* ids;     /* [T, k] */
  const void* x;          /* [T, d] */
  int32_t* counts;        /* [E] */
  int32_t* kept;          /* [E] */
  int32_t* expert_off;    /* [E + 1] */
  int32_t* rank_counts;   /* [R] */
  int32_t* rank_off;      /* [R + 1] */
  int32_t* slot;          /* [T, k] */
  int32_t* src;           /* [rows_max] */
  void* x_send;           /* [rows_max, d] */
} moe_dispatch_args;

/* ceil(cf * T * k / E), computed exactly from the binary value of cf (the
 * even share T*k/E scaled by the capacity factor: Ultralytics, "Load
 * Balancing and Capacity").  cf <= 0 means no limit and returns INT32_MAX.
 * Host function. */
int32_t moe_capacity(int64_t T, int32_t k, int32_t E, double cf);
/* min(T*k, E*capacity): the largest possible number of send rows.  Host. */
int64_t moe_send_rows_max(int64_t T, int32_t k, int32_t E, int32_t capacity);
size_t moe_dispatch_workspace_bytes(const moe_dispatch_args* a);
moe_status moe_dispatch(const moe_dispatch_args* a, void* workspace, size_t ws_bytes,
                        hipStream_t stream);

/* Bias-based balancing step (Ultralytics, "Load Balancing and Capacity",
 * bias bullet: after each step the selection bias of overloaded experts goes
 * down and of idle ones up).  With the raw per-expert counts of a dispatch
 * over T tokens and k choices:
 *   b_select[e] -= gamma * sign(counts[e] * E - T * k)
 * (the comparison with the mean load T*k/E made exactly in integers, the
 * update in fp32).  The pages give no step size; gamma is the caller's.
 * counts [E] and b_select [E] are device pointers; b_select is updated in
 * place.  E <= 256. */
moe_status moe_bias_update(const int32_t* counts, float* b_select, int32_t E, int64_t T,
                           int32_t k, float gamma, hipStream_t stream);

/* Auxiliary balancing loss value of one step, forward only (Ultralytics,
 * "Load Balancing and Capacity", auxiliary-loss bullet; ai360xpert, "Load
 * Balancing and Dropped Tokens": an extra loss term rewards the router for
 * spreading tokens evenly).  The pages give no formula; the
 * Switch-Transformer form is computed:
 *   P_e  = mean over the T tokens of the router probability of expert e
 *          (softmax of the logits, or for MOE_SIGMOID the sigmoids
 *          normalised per token),
 *   loss = alpha * E * sum_e counts[e] / (T * k) * P_e.
 * logits [T, E] fp32 are the router's final logits (moe_route's output),
 * counts [E] the raw per-expert assignment counts (moe_dispatch's output).
 * Writes prob_mean [E] and loss [1] (device).  Sums run in a fixed order
 * (deterministic).  T = 0 gives zeros.  Workspace: moe_aux_loss_workspace_bytes. */
size_t moe_aux_loss_workspace_bytes(int64_t T, int32_t E);
moe_status moe_aux_loss(const float* logits, const int32_t* counts, int64_t T, int32_t E,
                        int32_t k, int32_t score, float alpha, float* prob_mean, float* loss,
                        void* workspace, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------- expert FFN
 * Local expert compute (Ultralytics, "How Tokens Move Between GPUs", step 3;
 * experts are independent).  For each executed expert e in [e_begin, e_end)
 * and each send row s in [expert_off[e], expert_off[e+1]):
 *   y_send[s] = act(x_send[s] W1_e^T [, x_send[s] W3_e^T]) W2_e^T
 * with act = ReLU, GELU (erf form) or SwiGLU (silu(z1) * z3).  Rows of other
 * experts are not touched.  Optional dense (shared) expert over x_dense:
 *   y_dense = act(x_dense WS1^T [, x_dense WS3^T]) WS2^T.
 * Weights of local expert i = e - e_begin start at w1 + i*h*d etc.
 * fp8 weights carry one fp32 scale per 128x128 block: s1/s3 [E_x, h/128,
 * d/128], s2 [E_x, d/128, h/128]; the dequantised weight is q * scale.
 * Accumulation is fp32; the intermediate activation is stored in act_dtype.
 * max_rows bounds expert_off[e_end] - expert_off[e_begin] (host value; it
 * sizes the workspace and the grid; rows beyond it are a caller error).
 * w_layout applies to all six weight matrices (w1, w3, w2, ws1, ws3, ws2);
 * scales keep their layout.  MOE_W_TILED16 needs bf16 activations (bf16 or
 * fp8 weights).  Off the streaming path (more than 64 rows per executed
 * expert on average, or T_dense > 64) it also needs d and h multiples of 256
 * and, for fp8 weights, d and h at most 16384; otherwise
 * MOE_ERR_UNSUPPORTED.  Row-major weights have no such limits.
 */
typedef struct moe_ffn_args {
  int32_t d, h, E, e_begin, e_end;
  int32_t act;            /* moe_act */
  int32_t act_dtype;      /* MOE_F32 or MOE_BF16 */
  int32_t w_dtype;        /* MOE_F32 (with f32 acts), MOE_BF16 or MOE_FP8_E4M3 */
  int32_t w_layout;       /* moe_w_layout */
  int64_t max_rows;
  const void* x_send;     /* [*, d] */
  const int32_t* expert_off; /* [E + 1] */
  const void* w1;         /* [E_x, h, d] */
  const void* w3;         /* [E_x, h, d], SwiGLU only (else NULL) */
  const void* w2;         /* [E_x, d, h] */
  const float* s1;        /* fp8 scales, else NULL */
  const float* s3;
  const float* s2;
  void* y_send;           /* [*, d], same row numbering as x_send */
  int64_t T_dense;        /* rows of the shared expert (0 = none) */
  const void* x_dense;    /* [T_dense, d] */
  const void* ws1;        /* [h, d] */
  const void* ws3;        /* [h, d] (SwiGLU) */
  const void* ws2;        /* [d, h] */
  const float* ss1;
  const float* ss3;
  const float* ss2;
  void* y_dense;          /* [T_dense, d] */
} moe_ffn_args;

size_t moe_ffn_workspace_bytes(const moe_ffn_args* a);
moe_status moe_expert_ffn(const moe_ffn_args* a, void* workspace, size_t ws_bytes,
                          hipStream_t stream);

/* One-time re-layout of weights for streaming: n_mats row-major matrices of
 * `rows` rows of `row_bytes` bytes each (any dtype) are rewritten into the
 * 16-row tiled layout.  Within matrix i, tile t holds rows [16t, 16t + 16)
 * as row_bytes/64 consecutive 1 KB pieces; piece j holds bytes [64j, 64j + 64)
 * of the tile's rows, the 16 bytes at 64j + 16q of row 16t + r at offset
 * (16q + r) * 16.  This is the order in which a 64-lane wave feeding 16x16
 * matrix-core fragments reads a weight tile, so streaming the tiled matrix is
 * one contiguous read.  The matrices keep their sizes and their order;
 * w_tiled must not overlap w.  Requires rows % 16 == 0, row_bytes % 64 == 0,
 * 16-byte aligned pointers.  Computes nothing (a byte permutation). */
moe_status moe_weight_tile(const void* w, void* w_tiled, int64_t n_mats, int32_t rows,
                           int64_t row_bytes, hipStream_t stream);

/* ---------------------------------------------------------------- combine
 * Un-permute and weighted sum at the origin (Ultralytics, "How Tokens Move
 * Between GPUs", step 4), with the residual:
 *   y[t] = x[t] (+ shared_out[t]) + sum_j weights[t,j] * y_send[slot[t,j]]
 * over j with slot[t,j] >= 0 and e_begin <= ids[t,j] < e_end, accumulated in
 * fp32 and rounded once.  A token without contributions leaves as x[t]
 * bit for bit (Ultralytics, "Load Balancing and Capacity": a skipped token
 * passes through the residual unchanged).  Dropped assignments are not
 * renormalised away.
 */
typedef struct moe_combine_args {
  int64_t T;
  int32_t d, k, e_begin, e_end;
  int32_t act_dtype;
  const void* x;          /* [T, d] */
  const void* shared_out; /* [T, d] or NULL */
  const void* y_send;     /* [*, d] */
  const int32_t* ids;     /* [T, k] */
  const int32_t* slot;    /* [T, k] */
  const float* weights;   /* [T, k] */
  void* y;                /* [T, d] out (may not alias x) */
} moe_combine_args;

moe_status moe_combine(const moe_combine_args* a, hipStream_t stream);

/* ------------------------------------------------------------ whole layer
 * route -> dispatch -> expert FFN -> combine, enqueued on one stream with no
 * host synchronisation.  The four argument blocks must be consistent: the
 * same T, k, E, d and act_dtype, and the buffers one stage writes are the
 * ones the next reads (ids, weights, slot, x_send, expert_off, y_send; with a
 * shared expert, x_dense = dispatch.x, T_dense = T, shared_out = y_dense).
 * Every block and that wiring are checked before anything is launched, so an
 * error leaves the stream untouched.  If `events` is not
 * NULL it holds MOE_LAYER_EVENTS host-side hipEvent_t handles, recorded at
 * the stage boundaries listed at MOE_LAYER_EVENTS; a NULL entry is skipped.
 * Each recorded event delays the next kernel's start by a few microseconds,
 * so a caller timing one stage passes only the two events around it.
 */
typedef struct moe_layer_args {
  moe_route_args route;
  moe_dispatch_args dispatch;
  moe_ffn_args ffn;
  moe_combine_args combine;
  hipEvent_t* events;     /* host array of MOE_LAYER_EVENTS events (entries may
                             be NULL), or NULL */
} moe_layer_args;

size_t moe_workspace_bytes(const moe_layer_args* a);
moe_status moe_layer_forward(const moe_layer_args* a, void* workspace, size_t ws_bytes,
                             hipStream_t stream);

/* ------------------------------------------------- no-allocation variant
 * For callers that cannot allocate device memory or hand over a workspace
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  The same layer forward as moe_layer_forward, same arguments,
 * results and errors, with the workspace taken from a static device array
 * inside the library: MOE_STATIC_SCRATCH_BYTES on every GPU the library runs
 * on, held until the process ends.  The caller still owns and passes every
 * input and output.  A layer whose moe_workspace_bytes() exceeds the array
 * returns MOE_ERR_WORKSPACE before anything is launched.  The call allocates
 * and frees nothing.  All calls on one GPU share that GPU's array; nothing in
 * it has to start at zero, but calls that overlap on one GPU (on different
 * streams, or from threads without ordering between them) race on it. */
#define MOE_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status moe_layer_forward_noalloc(const moe_layer_args* a, hipStream_t stream);

/* Message for the calling thread's most recent non-OK status ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
