/*
 * moe.h -- C ABI of the MI355X (gfx950) top-k token-choice Mixture-of-Experts
 * layer forward, with expert-choice routing as a second routing mode.
 *
 * The layer (pages, cited by title and section or equation):
 *   aigrafen.se "Mixture of Experts": y = sum_{i in top-k} g_i E_i(x) with
 *     g = softmax(W_r x); L_aux = alpha N sum_i f_i P_i; capacity
 *     C = tokens / experts * capacity factor; the `MoE` module (softmax, top-k,
 *     renormalise, int(cf*T*k/N), per-expert `nonzero` order truncated to C).
 *   vanos001 "MoE Architecture": "Router Design" (top-k on logits, softmax over
 *     the k), "Expert Network Design" (SwiGLU and GELU experts), "Capacity and
 *     Token Dropping", "Shared vs Specialized Experts".
 *   learn.starphix.com "Mixture of Experts (MoE)": "Key Equations", "Top-k
 *     Gating", "Load Balancing (Critical)" (load_balancing_loss, z_loss),
 *     "Shared + Specialized", "Quantization".
 *   Expert choice: vanos001 "MoE Architecture" / "Router Design",
 *     Expert-Choice Router (softmax over the tokens, each expert takes its
 *     top-capacity tokens) and the router comparison table; chipfoundryservices
 *     glossary "Mixture of Experts (MoE)", Expert Choice Routing.
 *
 * Conventions for every entry point:
 *  - Memory: every pointer argument is DEVICE memory except the moe_shape /
 *    moe_weights / moe_stats structs themselves, which are read on the host
 *    during the call (the pointers inside them are device pointers, except
 *    moe_weights.w_bits / sw_bits, which are host arrays). The
 *    caller allocates and owns every buffer; the library never allocates,
 *    frees or keeps a pointer after returning. Buffers must stay valid until
 *    the work enqueued on `stream` has finished.
 *  - Asynchrony: work is enqueued on `stream` (0 = the null stream) and the
 *    call returns without synchronising. Results are valid after the caller
 *    synchronises with the stream.
 *  - Layout: row-major. Tokens are the flattened batch*sequence rows [T][d].
 *    Weights use the nn.Linear layout [out][in], stacked per expert:
 *    W_r [N][d], W1 and W3 [N][d_ff][d], W2 [N][d][d_ff].
 *  - Errors: arguments are validated on the host before anything is launched.
 *    A negative moe_status means nothing was enqueued, except MOE_ERR_HIP, which
 *    reports a failed launch (the HIP error code is kept per thread and read
 *    with moe_last_hip_error()). No C++ exception crosses this interface.
 *  - Workspace: `ws` is caller-provided device scratch of at least
 *    moe_workspace_size() bytes for that entry point, 256-byte aligned. Its
 *    contents on entry do not matter; they are clobbered.
 *  - Limits: 1 <= N <= 256, 1 <= k <= min(8, N), n_shared <= 4, d and d_ff
 *    multiples of 128 and at most 2^20, T <= 2^24, T*k*max(d, d_ff) < 2^31,
 *    weight row pitches (ld_up, ld_down) at most 2^21 elements. Expert choice:
 *    T <= 32768 and N*C*max(d, d_ff) < 2^31. Otherwise MOE_ERR_UNSUPPORTED.
 *  - Expert choice (gating MOE_GATE_EXPERT_CHOICE): top_k must be 1 and
 *    capacity is C, the tokens each expert takes, 0 <= C <= T (see
 *    moe_capacity); otherwise MOE_ERR_INVALID_ARG. The per-token arrays then
 *    change shape as each entry point states: topk_idx / topk_w become [N][C]
 *    (expert-major), inv_map [T][N], perm_token [N*C].
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null required pointer, bad shape, k > N, ... */
  MOE_ERR_UNSUPPORTED = -2, /* valid but outside the limits above */
  MOE_ERR_HIP = -3,         /* a launch failed; see moe_last_hip_error() */
  MOE_ERR_WORKSPACE = -4    /* ws is null, misaligned or smaller than required */
} moe_status;

/* MOE_INT_W: weight-only integers (starphix "Quantization": INT8 for
 * high-traffic experts, INT4 for the rest, the router kept in 16 bits). Each
 * expert has 8 or 4 bits (moe_weights.w_bits) and one fp32 scale per weight
 * row: W[r][c] = s_r * q[r][c], q symmetric two's complement. Expert matrices
 * keep byte rows (pitch ld_up / ld_down bytes, at least d / d_ff): an 8-bit
 * expert's row holds one int8 code per column; a 4-bit expert's row holds its
 * codes in its first d/2 (d_ff/2) bytes, each 8 consecutive columns 8m..8m+7
 * as one little-endian 32-bit word with column 8m + 2j in bits [4j, 4j + 4)
 * and column 8m + 2j + 1 in bits [16 + 4j, 20 + 4j), two's complement. (That
 * order lets the kernels turn two codes into a bf16 pair with one shift and
 * one and-or.) Activations stay bf16. */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2, MOE_INT_W = 3 } moe_dtype;

/* Expert FFN. GELU: y = W2 gelu(W1 x + b1) + b2 with the exact erf GELU
 * (aigrafen "Mixture of Experts", `MoE` module; vanos001 "Expert Network
 * Design", StandardExpert). SwiGLU: y = W2 (silu(W1 x) * W3 x), no biases
 * (vanos001 "Expert Network Design", SwiGLUExpert). */
typedef enum { MOE_ACT_GELU = 0, MOE_ACT_SWIGLU = 1 } moe_act;

/* Gates of the k selected experts S_t (selection is always the k largest fp32
 * logits, descending, exact ties to the lower expert index):
 *  SOFTMAX_TOPK:        g_j = softmax(l_t)[S_j]  (aigrafen, the y/g equation;
 *                       wiki.ai-engineering.at router/top-k figure)
 *  SOFTMAX_TOPK_RENORM: the same, divided by their sum (aigrafen `MoE` module)
 *  TOPK_SOFTMAX:        softmax over the k selected logits (vanos001
 *                       Token-Choice Router; starphix "Top-k Gating") --
 *                       equal to SOFTMAX_TOPK_RENORM in exact arithmetic.
 * EXPERT_CHOICE: no per-token selection. p[t][e] = softmax over the TOKENS t
 *                of column e of the logits; expert e takes the C tokens with
 *                the largest p[:, e] (exact ties to the lower token index),
 *                listed in ascending token order, with gates p[t][e] (vanos001
 *                Expert-Choice Router). A token may be taken by several
 *                experts or by none. */
typedef enum {
  MOE_GATE_SOFTMAX_TOPK = 0,
  MOE_GATE_SOFTMAX_TOPK_RENORM = 1,
  MOE_GATE_TOPK_SOFTMAX = 2,
  MOE_GATE_EXPERT_CHOICE = 3
} moe_gating;

typedef struct {
  int64_t T;          /* tokens in the call (batch * sequence) */
  int64_t d;          /* model width */
  int64_t d_ff;       /* expert hidden width */
  int32_t n_experts;  /* N routed experts */
  int32_t top_k;      /* k (1 under expert choice) */
  int32_t n_shared;   /* always-on shared experts, same shape and act (0..4) */
  int32_t act;        /* moe_act */
  int32_t gating;     /* moe_gating */
  int32_t act_dtype;  /* moe_dtype of x, W_r, the layer output: MOE_F32 or MOE_BF16 */
  int32_t w_dtype;    /* moe_dtype of expert weights: same as act_dtype, or
                         MOE_FP8_E4M3 or MOE_INT_W with act_dtype MOE_BF16 */
  int64_t capacity;   /* C pairs per expert; -1 = no limit (dropless).
                         Expert choice: C tokens per expert, 0 <= C <= T */
  float aux_alpha;    /* alpha of L_aux (the pages use about 0.01) */
} moe_shape;

typedef struct {
  const void* w_router;   /* [N][d], act_dtype (router stays 16/32-bit) */
  const float* b_router;  /* [N] fp32 logit bias or NULL */
  const void* w1;         /* [N][d_ff][d] w_dtype */
  const void* w3;         /* [N][d_ff][d] w_dtype (SwiGLU only, else NULL) */
  const void* w2;         /* [N][d][d_ff] w_dtype */
  const float* b1;        /* [N][d_ff] fp32 or NULL (GELU only) */
  const float* b2;        /* [N][d] fp32 or NULL (GELU only) */
  const float* w_scale;   /* [N][3] fp32 per-tensor scales of (W1, W3, W2) for
                             MOE_FP8_E4M3 (W = scale * code); for MOE_INT_W
                             [N][2 d_ff + d] row scales: W1's d_ff rows, W3's
                             d_ff rows (unused by GELU), W2's d rows; else NULL */
  const void* sw1;        /* shared experts: [n_shared][d_ff][d] */
  const void* sw3;        /* [n_shared][d_ff][d] (SwiGLU) */
  const void* sw2;        /* [n_shared][d][d_ff] */
  const float* sw_scale;  /* [n_shared][3] for MOE_FP8_E4M3, [n_shared][2 d_ff + d] for MOE_INT_W */
  /* Row pitches of the expert matrices, in elements (MOE_INT_W: bytes; 0 =
   * contiguous rows: d or d_ff elements, also for 4-bit experts).
   * ld_up applies to w1, w3, sw1, sw3: row j of expert e starts at element
   * (e * d_ff + j) * ld_up, ld_up >= d. ld_down applies to w2 and sw2:
   * (e * d + j) * ld_down, ld_down >= d_ff. Nonzero pitches must be multiples
   * of 16. A pitch of d + 64 (resp. d_ff + 64) keeps the rows of one k-column
   * from falling into the same few L2 channels when d or d_ff is a multiple
   * of 4096 and is the layout the prefill GEMM runs fastest on. */
  int64_t ld_up;
  int64_t ld_down;
  /* MOE_INT_W only: bits of each routed / shared expert, 8 or 4. These two are
   * HOST arrays (the one exception to the device-pointer rule): the width of
   * each expert decides the launches, and is read during the call. */
  const uint8_t* w_bits;  /* [N] */
  const uint8_t* sw_bits; /* [n_shared] */
} moe_weights;

/* Router statistics (aigrafen L_aux equation and `latest` dict; starphix
 * load_balancing_loss and z_loss). Every member is a device pointer; any
 * member may be NULL (not written). Written by moe_route (counts, f, P, l_aux,
 * z_loss, lse_mean, lse_sq_mean) and moe_permute (kept, n_dropped).
 * Expert choice balances by construction (vanos001 router comparison table):
 * counts and kept are C for every expert, n_dropped is the number of tokens
 * no expert took, z_loss / lse_mean / lse_sq_mean are as for token choice
 * (per-token logsumexp over the experts), and f, P and l_aux are not written. */
typedef struct {
  int32_t* counts;      /* [N] pairs that selected expert e, before capacity drops */
  int32_t* kept;        /* [N] pairs kept after the capacity cut */
  float* f;             /* [N] counts / (T k) */
  float* P;             /* [N] mean over tokens of the full softmax */
  float* l_aux;         /* [1] alpha * N * sum_e f_e P_e */
  float* z_loss;        /* [1] (mean_t logsumexp_t)^2 */
  float* lse_mean;      /* [1] mean_t logsumexp_t */
  float* lse_sq_mean;   /* [1] mean_t logsumexp_t^2 */
  int32_t* n_dropped;   /* [1] pairs dropped by the capacity cut */
} moe_stats;

/* Entry points whose workspace size can be queried. */
typedef enum {
  MOE_ENTRY_ROUTE = 0,
  MOE_ENTRY_PERMUTE = 1,
  MOE_ENTRY_GROUPED_FFN = 2,
  MOE_ENTRY_FORWARD = 3,
  MOE_ENTRY_BACKWARD = 4
} moe_entry;

/* Kernel family of the expert FFN (diagnostic; returned by moe_ffn_path). */
typedef enum {
  MOE_PATH_F32 = 0,     /* fp32 layers: FMA tiles */
  MOE_PATH_STREAM = 1,  /* few rows (decode): weights streamed once, GEMV for T <= 2 */
  MOE_PATH_REG128 = 2,  /* register-staged 128 x 128 MFMA tiles */
  MOE_PATH_DMA256 = 3,  /* LDS-DMA 256-row tiles, small groups and short group tails on 128-row tiles */
  MOE_PATH_DMA128 = 4,  /* LDS-DMA 128-row tiles */
  MOE_PATH_BGEMM = 5    /* moe_backward only: forward recompute on the backward GEMM */
} moe_path;

/* moe_route flag: take the fp32 logits from `logits` instead of computing the
 * router GEMM (x and w_router are then ignored and may be NULL). */
#define MOE_ROUTE_LOGITS_GIVEN 1u

/* MOE_ABI_VERSION of the loaded library. */
int moe_abi_version(void);

/* Static text for a moe_status (never NULL). */
const char* moe_status_string(int status);

/* hipError_t of the last MOE_ERR_HIP returned on this host thread (0 if none). */
int moe_last_hip_error(void);

/* Expert capacity C = floor(cf * T * k / N), evaluated in fp64 (aigrafen
 * capacity equation with the module's int(cf*T*k/N)). Returns -1 for cf < 0
 * (no limit) and for N < 1. With k = 1 it is the expert-choice capacity
 * int(T*cf/N) of the vanos001 Expert-Choice Router. Host function. */
int64_t moe_capacity(int64_t T, int32_t k, int32_t N, double cf);

/* Device workspace bytes that `entry` needs for `shape`. */
moe_status moe_workspace_size(const moe_shape* shape, int32_t entry, size_t* bytes);

/* Diagnostic, host only: the moe_path that the expert FFN of `entry`
 * (MOE_ENTRY_GROUPED_FFN or MOE_ENTRY_FORWARD) takes for `shape`, or, for
 * MOE_ENTRY_BACKWARD, the path of moe_backward's forward recompute (an FFN
 * path, or MOE_PATH_BGEMM). The choice depends on the shape only (dtypes,
 * widths and the capacity-bound row count), never on the routing. Returns a
 * negative moe_status for an invalid shape or entry. */
int32_t moe_ffn_path(const moe_shape* shape, int32_t entry);

/*
 * Router (aigrafen y/g equation; starphix "Key Equations" router_logits = x W_r^T;
 * vanos001 Token-Choice Router; starphix load_balancing_loss and z_loss).
 *   logits[t][e] = sum_i x[t][i] W_r[e][i] (+ b_router[e])   fp32 accumulation
 *   topk_idx[t][j], topk_w[t][j]: the k largest logits, descending (ties to the
 *   lower index), gates per shape->gating; statistics into `stats`.
 * x [T][d] act_dtype; logits [T][N] fp32 (written, or read with
 * MOE_ROUTE_LOGITS_GIVEN); topk_idx [T][k] int32; topk_w [T][k] fp32.
 * Expert choice: topk_idx [N][C] gets the tokens expert e takes (ascending)
 * and topk_w [N][C] their gates; the logits must not be NaN.
 * Deterministic: identical inputs give identical bits.
 */
moe_status moe_route(const moe_shape* shape, const void* x, const void* w_router,
                     const float* b_router, float* logits, uint32_t flags, int32_t* topk_idx,
                     float* topk_w, const moe_stats* stats, void* ws, size_t ws_bytes,
                     hipStream_t stream);

/*
 * Dispatch with expert capacity (aigrafen capacity equation and `MoE` module;
 * vanos001 "Capacity and Token Dropping"). For each expert e the pairs (t, j)
 * with topk_idx[t][j] == e, in ascending token order; the first
 * min(count, C) are kept, the rest dropped. Kept pairs are laid out expert by
 * expert, tokens ascending within an expert:
 *   expert_offsets [N+1]: offsets[e] = sum_{e'<e} kept[e'], offsets[N] = M
 *   perm_token [T*k]: token of permuted row r < M (rows >= M not written)
 *   inv_map [T][k]: permuted row of pair (t, j), or -1 when dropped
 *   x_perm [T*k][d] (act_dtype): x_perm[r] = x[perm_token[r]] for r < M
 * topk_idx [T][k] int32 with values in [0, N), distinct within a row.
 * Writes stats->kept and stats->n_dropped when given. Bit-deterministic.
 * Expert choice: topk_idx is moe_route's [N][C] (each row strictly ascending,
 * tokens in [0, T)); expert e's j-th token gets row e*C + j, so
 * offsets[e] = e*C, perm_token [N*C] is topk_idx itself, inv_map [T][N] holds
 * the row of (t, e) or -1, and x_perm has N*C rows.
 */
moe_status moe_permute(const moe_shape* shape, const int32_t* topk_idx, const void* x,
                       int32_t* expert_offsets, int32_t* perm_token, int32_t* inv_map,
                       void* x_perm, const moe_stats* stats, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/*
 * Grouped expert FFN (vanos001 "Expert Network Design" and "Efficient Batched
 * MoE"): for every expert e and every row r in [offsets[e], offsets[e+1]),
 *   y_perm[r] = E_e(x_perm[r]);
 * and, when shape->n_shared > 0 (starphix "Shared + Specialized"), for every
 * shared expert s and token t, y_shared[s][t] = E^sh_s(x[t]).
 * x_perm, y_perm [rows][d] act_dtype; expert_offsets [N+1] (device, as written
 * by moe_permute, nondecreasing, offsets[0] = 0, offsets[N] <= T*k);
 * x [T][d] and y_shared [n_shared][T][d] (required iff n_shared > 0).
 * The hidden activation is kept in act_dtype (bf16 for bf16 layers).
 */
moe_status moe_grouped_ffn(const moe_shape* shape, const void* x_perm,
                           const int32_t* expert_offsets, const void* x,
                           const moe_weights* weights, void* y_perm, void* y_shared, void* ws,
                           size_t ws_bytes, hipStream_t stream);

/*
 * Combine (aigrafen y = sum g_i E_i(x) and the module's out[index] += w * ...;
 * starphix "Shared + Specialized"):
 *   y[t] = sum_{j : inv_map[t][j] >= 0} topk_w[t][j] * y_perm[inv_map[t][j]]
 *          + sum_s y_shared[s][t]
 * A dropped pair adds 0 (the residual connection is outside this layer); the
 * gates are not renormalised after drops. y_shared may be NULL.
 * fp32 accumulation in a fixed order (slots ascending, then shared experts).
 * Expert choice: inv_map [T][N] and topk_w [N*C] indexed by row:
 *   y[t] = sum_{e : inv_map[t][e] >= 0} topk_w[inv_map[t][e]] * y_perm[inv_map[t][e]]
 *          + sum_s y_shared[s][t], experts ascending.
 */
moe_status moe_combine(const moe_shape* shape, const void* y_perm, const int32_t* inv_map,
                       const float* topk_w, const void* y_shared, void* y, hipStream_t stream);

/*
 * Whole layer: moe_route -> moe_permute -> moe_grouped_ffn (routed + shared)
 * -> moe_combine, enqueued on one stream with no host synchronisation.
 * x [T][d], y [T][d] act_dtype. logits [T][N], topk_idx/topk_w/inv_map [T][k],
 * expert_offsets [N+1], perm_token [T*k] are optional outputs (NULL: kept in
 * the workspace); under expert choice they have the shapes moe_route,
 * moe_permute and moe_combine give them. stats may be NULL.
 */
moe_status moe_forward(const moe_shape* shape, const void* x, const moe_weights* weights,
                       void* y, float* logits, int32_t* topk_idx, float* topk_w,
                       int32_t* expert_offsets, int32_t* perm_token, int32_t* inv_map,
                       const moe_stats* stats, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation, arguments and outputs as moe_forward, with the workspace
 * taken from a device array inside the library instead of `ws`. That array
 * holds MOE_NOALLOC_SCRATCH_BYTES on each GPU the call runs on; it is created
 * with the library's code on that GPU and kept until the process ends. The
 * call allocates nothing. Shapes whose MOE_ENTRY_FORWARD workspace
 * (moe_workspace_size) exceeds MOE_NOALLOC_SCRATCH_BYTES return
 * MOE_ERR_WORKSPACE and launch nothing: this covers decode-sized layers (the
 * Mixtral-shape layer up to 128 tokens) but not prefill. Every call on one GPU
 * uses that GPU's single array: calls that overlap on one GPU (concurrent
 * streams, or host threads) race and give undefined results; calls ordered on
 * one stream are safe. The array's contents between calls do not matter.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
moe_status moe_forward_noalloc(const moe_shape* shape, const void* x, const moe_weights* weights,
                               void* y, float* logits, int32_t* topk_idx, float* topk_w,
                               int32_t* expert_offsets, int32_t* perm_token, int32_t* inv_map,
                               const moe_stats* stats, hipStream_t stream);

/*
 * Gradients written by moe_backward. dx is required; every other member may be
 * NULL (that gradient is not computed). Weight gradients are fp32 in the
 * contiguous nn.Linear layout of the weights they belong to (no row pitch),
 * one matrix per expert, and are overwritten (not accumulated into).
 */
typedef struct {
  void* dx;          /* [T][d] act_dtype */
  float* dw_router;  /* [N][d] */
  float* db_router;  /* [N] */
  float* dw1;        /* [N][d_ff][d] */
  float* dw3;        /* [N][d_ff][d] (SwiGLU) */
  float* dw2;        /* [N][d][d_ff] */
  float* db1;        /* [N][d_ff] (GELU) */
  float* db2;        /* [N][d] (GELU) */
  float* dsw1;       /* [n_shared][d_ff][d] */
  float* dsw3;       /* [n_shared][d_ff][d] (SwiGLU) */
  float* dsw2;       /* [n_shared][d][d_ff] */
} moe_grads;

/*
 * Layer backward (the training step of the aigrafen `MoE` module, whose loss
 * adds alpha-weighted L_aux; starphix "Load Balancing (Critical)" adds the
 * z_loss): the gradients of
 *   L = sum_t <dy[t], y[t]> + c_aux * L_aux + c_z * z
 * with respect to x, W_r, b_r and every expert's (and shared expert's)
 * weights and GELU biases, where y is moe_forward's output for the same x and
 * weights. The routing decision (the selected experts, the capacity cut, the
 * counts behind f) is held fixed, as it is piecewise constant; the gates, P
 * and the logsumexp carry gradient. The fp32 rounding of the logits passes
 * the gradient unchanged. The forward is recomputed inside the call (nothing
 * is kept from an earlier moe_forward).
 * Token choice only (gating 0..2; expert choice gives MOE_ERR_UNSUPPORTED),
 * act_dtype = w_dtype = MOE_BF16 (else MOE_ERR_UNSUPPORTED). x, dy [T][d]
 * bf16. Intermediate products are rounded to bf16 where they feed a matrix
 * product (H, dY = g dy, dU, dV, the logit gradient as a bf16 pair);
 * accumulation is fp32. Deterministic: identical inputs give identical bits.
 */
moe_status moe_backward(const moe_shape* shape, const void* x, const moe_weights* weights, const void* dy,
                        float c_aux, float c_z, const moe_grads* grads, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/*
 * Stage timing, for profiling. Between moe_timing_start and moe_timing_stop
 * every entry point records a pair of hipEvents on its stream around each
 * stage below (ROUTE: router kernel + statistics finalize; PERMUTE: rank, scan
 * and scatter kernels; FFN_PLAN: the tile-plan kernel; FFN_UP / FFN_DOWN: the
 * up and down grouped GEMM kernels, one launch each; COMBINE: the combine
 * kernel). The events are host-side HIP objects created on the first start
 * (2 * max_launches of them) and kept until the process ends; no device memory
 * is allocated. moe_timing_stop waits for the recorded events and returns the
 * summed milliseconds and the number of recorded launches per stage; records
 * beyond max_launches are not taken. Process-wide state, serialised by a lock.
 */
typedef enum {
  MOE_STAGE_ROUTE = 0,
  MOE_STAGE_PERMUTE = 1,
  MOE_STAGE_FFN_PLAN = 2,
  MOE_STAGE_FFN_UP = 3,
  MOE_STAGE_FFN_DOWN = 4,
  MOE_STAGE_COMBINE = 5,
  MOE_N_STAGES = 6
} moe_stage;

moe_status moe_timing_start(int32_t max_launches);
moe_status moe_timing_stop(double* total_ms /* [MOE_N_STAGES] */, int32_t* launches /* [MOE_N_STAGES] */);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
