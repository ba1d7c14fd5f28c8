// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Stage timing hook (moe_timing_start / moe_timing_stop): records a hipEvent
// on `s` at the start (end = false) or end of a stage; no-op when disabled.
enum Stage { kStageRoute = 0, kStagePermute, kStageFfnPlan, kStageFfnUp, kStageFfnDown, kStageCombine, kNumStages };
void stage_mark(int stage, bool end, hipStream_t s);

// ---------------------------------------------------------------- router
struct RouteArgs {
  int64_t T, d;
  int32_t N, k, gating, act_dtype;
  bool logits_given;
  const void* x;
  const void* w_router;
  const float* b_router;
  float* logits;            // [T][N]
  int32_t* topk_idx;        // [T][k]
  float* topk_w;            // [T][k]
  // per-block partials (workspace), nb = ceil(T / kRouteTokens)
  float* part_P;            // [nb][N]
  int32_t* part_cnt;        // [nb][N]
  float* part_lse;          // [nb][2]
  float* part_logits;       // [splits][T][N] k-split partial logits (workspace)
  // expert choice (gating 3): topk_idx / topk_w are then [N][cap], the tokens
  // each expert takes (ascending) and their gates; logits_t [N][ld_lt] is the
  // column-major copy of the logits the per-expert selection reads (workspace)
  bool ec;
  int64_t cap;
  float* logits_t;
  int64_t ld_lt;
  // statistics outputs (any may be null)
  int32_t* counts;
  float *f, *P, *l_aux, *z_loss, *lse_mean, *lse_sq_mean;
  float aux_alpha;
};
constexpr int kRouteTokens = 64;  // tokens per route workgroup
constexpr int64_t kEcMaxTokens = 32768;  // expert choice: a column is held by one workgroup's registers
constexpr int kMaxRouteSplits = 16;  // k splits of the router GEMM (partial logit planes)
int route_splits(int64_t T, int64_t d, int32_t N);  // k splits of the router GEMM
int router_kstep(int64_t T, int64_t d, int32_t N);  // its k-step (64, 128 or 256)
// finalize = false: the statistics of more than one routing block are left
// to the permutation's scan pass (PermuteArgs::fin)
hipError_t launch_route(const RouteArgs& a, hipStream_t s, bool finalize = true);

// ---------------------------------------------------------------- FFN groups
// One group = one weight set applied to a contiguous block of rows.
struct GroupDesc {
  int32_t a_row0;   // first row in the A source (routed: x_perm / h, shared: x / h)
  int32_t c_row0;   // first row in the output
  int32_t rows;
  int32_t widx;     // expert index; shared experts are n_routed + s
};
constexpr int kMaxGroups = 260;  // routed experts (<= 256) plus shared experts (<= 4)
// Where and how the grouped FFN's group plan is written (row tiles of bm rows).
struct FfnPlan {
  GroupDesc* up;             // [G] up-GEMM groups
  GroupDesc* down;           // [G] down-GEMM groups
  int32_t* tile_start;       // [G + 1] row-tile prefix
  int32_t* active;           // [1 + G] count, then the groups with rows
  int32_t n_routed, n_shared, T, cap, bm;
  // tail tiles (bm_t > 0): a group whose last bm-row tile would hold at most
  // bm_t rows leaves those rows to a second launch of bm_t-row tiles
  GroupDesc* up_t;           // [G] the tails' up-GEMM groups
  GroupDesc* down_t;         // [G]
  int32_t* tile_start_t;     // [G + 1]
  int32_t bm_t;
  // integer layers with 8- and 4-bit experts (one launch per width): the
  // row-tile prefix of each width's groups alone, [width][plan][G + 1] (plan
  // 0: bm-row tiles, 1: bm_t-row tiles), so that each launch's tiles are dealt
  // over all XCDs; null for one width. Bit g of cls1: group g has the second
  // width (4 bits).
  int32_t* tile_start_c;
  uint32_t cls1[9];
};

// ---------------------------------------------------------------- permute
struct PermuteArgs {
  int64_t T, d;
  int32_t N, k, act_bytes;
  int64_t capacity;          // < 0: none
  const int32_t* topk_idx;
  const void* x;
  int32_t* offsets;          // [N+1]
  int32_t* perm_token;       // [T*k]
  int32_t* inv_map;          // [T*k]
  void* x_perm;              // [T*k] rows of pitch ld_out (may be null: no gather)
  int64_t ld_out;            // x_perm row pitch in elements (>= d)
  int32_t* kept;             // [N] (workspace if the caller gave none)
  int32_t* n_dropped;        // [1] (workspace if the caller gave none)
  // workspace
  int32_t* block_cnt;        // [nb][N]
  int32_t* block_base;       // [nb][N]
  int32_t* local_rank;       // [T*k]
  // with x_perm null and one workgroup (T <= kPermTokens): also write the FFN
  // group plan from the offsets (null plan.up: no plan)
  FfnPlan plan;
  // expert choice: topk_idx is [N][capacity], the tokens each expert takes in
  // ascending order; inv_map is [T][N]; n_dropped counts the tokens no expert
  // took (from per-block counts in ec_part, [ceil(T / 4)] ints of workspace)
  bool ec;
  int32_t* ec_part;
  // fin_nb > 0: the scan pass (more than one permutation block) also
  // finalizes the routing statistics of fin_nb routing blocks, with fin
  RouteArgs fin;
  int32_t fin_nb;
};
constexpr int kPermTokens = 256;  // tokens per permute workgroup
hipError_t launch_permute(const PermuteArgs& a, hipStream_t s);
// Decode front end: router GEMM, routing and the one-block permutation in one
// workgroup, for bf16 token-choice calls of at most 16 tokens and 64 experts
// whose FFN reads routed rows from x (front_fits).
bool front_fits(const RouteArgs& ra, const PermuteArgs& pa);
hipError_t launch_front(const RouteArgs& ra, const PermuteArgs& pa, hipStream_t s);

// ---------------------------------------------------------------- grouped FFN

struct FfnArgs {
  int64_t T, d, d_ff;
  int32_t n_routed, n_shared, act, act_dtype, w_dtype;
  int32_t routed_row_cap;     // rows reserved for routed experts in h (T*k or N*C)
  const int32_t* offsets;     // [n_routed+1] device
  const void* x_perm;         // routed A of the up GEMM, rows of pitch ld_xp
  int64_t ld_xp;              // x_perm row pitch (elements)
  const int32_t* gather;      // bf16 activations only: routed A row r is x row gather[r] (x_perm unused), or null
  int64_t ld_h;               // h row pitch (elements)
  int64_t ld_up, ld_down;     // weight row pitches (elements): W1/W3, W2
  const void* x;              // shared A of the up GEMM
  const void *w1, *w3, *w2;
  const float *b1, *b2, *w_scale;
  const void *sw1, *sw3, *sw2;
  const float* sw_scale;
  void* h;                    // [routed_row_cap + n_shared*T] rows of pitch ld_h, act dtype (workspace)
  void* y_perm;               // [*][d]
  void* y_shared;             // [n_shared][T][d]
  GroupDesc* groups;          // [2][n_routed + n_shared] (workspace)
  int32_t* tile_start;        // [n_routed + n_shared + 1] (workspace)
  GroupDesc* groups_t;        // [2][n_routed + n_shared]: tail tiles' groups (workspace)
  int32_t* tile_start_t;      // [n_routed + n_shared + 1] (workspace)
  int32_t* tile_start_c;      // [2][2][n_routed + n_shared + 1] per-width prefixes (workspace; integer weights)
  int32_t* active;            // [1 + n_routed + n_shared]: count, then the groups with rows (workspace)
  float* part;                // decode path: [splits][rows][d] fp32 partials (workspace)
  float* split_part;          // prefill path: k-split partial tiles, kSplitPartFloats (workspace) or null
  bool planned;               // groups, tile_start and active are already written (by the permutation)
  const uint8_t* w_bits;      // integer weights (w_dtype 3): HOST [n_routed], 8 or 4
  const uint8_t* sw_bits;     // HOST [n_shared]
  // the layer backward's forward recompute (DMA tiles only, else the launch
  // fails): fp32 W1 x (+ b1) and W3 x of every row (pitch ld_pre_up); null: none
  float *pre_up_u, *pre_up_v;
  int64_t ld_pre_up;
  bool up_only;  // the up GEMM alone (h and the copies above; no y)
  // one token, decode path: the combine folded into the down GEMM (see
  // ffn_fuses_combine), which then writes the layer output row fuse_y (bf16)
  // from the slots' rows (fuse_inv_map), experts and gates instead of y_perm
  const int32_t* fuse_inv_map;
  const int32_t* fuse_topk_idx;
  const float* fuse_topk_w;
  int32_t fuse_k;
  void* fuse_y;
};
// Whether the 256-column LDS-DMA tiles fit a layer: each GEMM's output width a
// multiple of the columns a tile yields (256; the SwiGLU up tile yields 128 of
// its 256 weight rows).
inline bool wide_tiles_fit(int32_t act, int64_t d, int64_t d_ff) {
  return d % 256 == 0 && (act == 1 ? d_ff % 128 == 0 : d_ff % 256 == 0);
}
// Whether the grouped FFN of these rows runs on the LDS-DMA tiles (bf16
// activations and weights, 2048 rows or more, widths that fit them).
inline bool ffn_uses_dma(int32_t act_dtype, int32_t w_dtype, int64_t rows, int32_t act, int64_t d, int64_t d_ff) {
  return act_dtype == 1 && w_dtype == 1 && rows >= 2048 && wide_tiles_fit(act, d, d_ff);
}
// Launch classes of a layer's weights: one for bf16 / e4m3 / uniform integer
// widths, two for mixed 8- and 4-bit experts (each launch skips, by group bit,
// the groups of the other width).
struct WeightClasses {
  int n;
  int wf[2];
  uint32_t skip[2][9];
};
WeightClasses weight_classes(const FfnArgs& a);
// The group plan the FFN launch would write for these arguments.
FfnPlan ffn_plan(const FfnArgs& a);
// fp32 floats of the prefill path's k-split partial tiles: 256 tiles of 256 x 256
constexpr int64_t kSplitPartFloats = 256LL * 256 * 256;

hipError_t launch_grouped_ffn(const FfnArgs& a, hipStream_t s);
// Groups of at most this many 128-row tiles run whole on the 128-row tiles
// next to the 256-row launch (see plan_groups).
constexpr int kSmallGroupTiles = 3;
// Kernel family launch_grouped_ffn takes for these arguments (the values of
// moe_ffn_path in moe.h).
enum FfnPath { kPathF32 = 0, kPathStream = 1, kPathReg128 = 2, kPathDma256 = 3, kPathDma128 = 4,
               kPathBgemm = 5 };
int ffn_path_of(const FfnArgs& a);

// Decode-sized layers (few rows per expert) stream expert weights instead of
// tiling rows: taken when all expert rows of the call fit in kSkinnyMaxRows.
constexpr int64_t kSkinnyMaxRows = 256;
// Elements added to the row pitch of the activation workspaces the library
// owns (x_perm inside moe_forward, h): with d or d_ff a multiple of 4096, rows
// a power of two apart put the lines of one k-column into few L2 channels.
constexpr int64_t kActPad = 64;
inline bool use_skinny(int32_t act_dtype, int64_t routed_row_cap, int32_t n_shared, int64_t T) {
  return act_dtype == 1 && routed_row_cap + n_shared * T <= kSkinnyMaxRows;
}
// whether a layer's FFN may take the prefill tiles (bf16 activations, any
// weight format), which use the k-split partial tiles
inline bool uses_prefill_gemm(int32_t act_dtype, int64_t routed_row_cap, int32_t n_shared, int64_t T) {
  return act_dtype == 1 && !use_skinny(act_dtype, routed_row_cap, n_shared, T);
}
// fp32 partial-sum floats the decode path needs (0 when no GEMM is split)
size_t skinny_part_floats(int64_t T, int64_t d, int64_t d_ff, int32_t n_routed, int32_t n_shared, int32_t act,
                          int64_t cap, int32_t w_dtype);
hipError_t launch_ffn_skinny(const FfnArgs& a, const GroupDesc* up, const GroupDesc* down, float* part,
                             hipStream_t s);
// Whether the decode down GEMM writes the layer output itself (fuse_y set,
// one token, bf16 or e4m3 weights on the GEMV path, k + n_shared <= 4): the
// caller then runs no combine.
bool ffn_fuses_combine(const FfnArgs& a);

// ---------------------------------------------------------------- backward GEMM
// C_g(m, n) (+)= sum_k A_g(m, k) B_g(k, n), bf16 operands, fp32 accumulation and output.
// Group g's rows are [off[g], off[g+1]) clamped to cap (off null: rows_all rows
// from 0 for every group). rows-M form: those rows are A's rows (A k-contiguous,
// lda) and C's rows, K fixed. rows-K form: they are the contraction, A m-
// contiguous (A(m, k) = A[(r0 + k) lda + m]), B(k, n) = B[(r0 + k) ldb + n], M
// fixed, one C matrix per group. B k-contiguous (b_kc): B(k, n) = B[n ldb + k],
// else n-contiguous. Per-group base offsets (elements): a_gs, b_gs, c_gs.
struct BGemm {
  const int32_t* off;
  int32_t n_groups, cap, rows_all;
  int32_t M, N, K;
  const uint16_t* A;
  int64_t lda, a_gs;
  const uint16_t* B;
  int64_t ldb, b_gs;
  void* C;
  int64_t ldc, c_gs;
  // bgemm_dma only: k >= k_split reads B2 (same layout, its row k - k_split)
  const uint16_t* B2;
  int32_t k_split;
};
// tile_start: [n_groups + 1] ints of workspace (rows-M form with offsets)
hipError_t launch_bgemm(const BGemm& p, bool rows_k, bool b_kc, bool acc, int32_t* tile_start, hipStream_t s);
// Rows-M products with B n-contiguous (dH = dY W2, dX = [dU dV] [W1; W3]) on
// LDS-DMA tiles: C = A B in fp32 (overwritten). Needs K a multiple of 128,
// k_split (if B2) a multiple of 32, lda and ldb multiples of 8, N a multiple
// of 8; otherwise hipErrorInvalidValue.
hipError_t launch_bgemm_dma(const BGemm& p, int32_t* tile_start, hipStream_t s);
// Rows-K products (dW = dY^T H, dU^T X, dV^T X) on the same tiles: C = A^T B
// in fp32 over each group's rows. Needs M, N, lda, ldb multiples of 8;
// otherwise hipErrorInvalidValue.
hipError_t launch_bgemm_dma_rk(const BGemm& p, hipStream_t s);

// ---------------------------------------------------------------- backward
// Token-choice layer backward, bf16 activations and weights. The caller has
// run the router (logits, topk_idx, topk_w, counts, lse_mean) and the
// permutation (offsets, inv_map, x_perm of pitch d). Routed rows are
// [0, cap), shared expert s owns rows [cap + s T, cap + (s+1) T) of every
// row-space buffer (U, V, H, dH, dU, dV, dX).
struct BwdArgs {
  int64_t T, d, d_ff, cap;
  int32_t N, k, S, act, gating, ldl;  // ldl: row pitch of dl_hi / dl_lo, N rounded up to 8
  int64_t ld_du;                      // row pitch of dU (2 d_ff for SwiGLU: dV = dU + d_ff, else d_ff)
  float aux_alpha, c_aux, c_z;
  const uint16_t *x, *dy, *w_router, *x_perm;
  const uint16_t *w1, *w3, *w2, *sw1, *sw3, *sw2;
  int64_t ld_up, ld_down;
  const float *b1, *b2;
  const float* logits;
  const int32_t *topk_idx, *inv_map, *offsets, *counts;
  const float *topk_w, *lse_mean;
  // workspace
  float *U, *V, *dH, *dX, *dl32, *dxr, *dg;
  uint16_t *H, *dY, *dU, *dV, *dl_hi, *dl_lo;
  // per routed row: dy of its token (unscaled), its (token, slot) pair index
  // and gate; dH holds dy W2 for those rows until the activation pass scales it
  uint16_t* dYu;
  int32_t* row_pair;
  float* row_gate;
  int32_t* tile_start;
  // dW_r = dl^T x over wr_splits token chunks (bounds wr_off [splits + 1]),
  // each into its own fp32 partial [N][d] of wr_part, summed in chunk order
  int32_t wr_splits;
  int32_t* wr_off;
  float* wr_part;
  // with use_ffn the forward recompute runs on the forward's grouped FFN
  // (ffn: its arguments; its up GEMM writes U, V and H)
  bool use_ffn;
  FfnArgs ffn;
  // outputs (weight gradients may be null: not computed)
  uint16_t* dx;
  float *dWr, *dbr, *dW1, *dW3, *dW2, *db1, *db2, *dsW1, *dsW3, *dsW2;
};
hipError_t launch_backward(const BwdArgs& a, hipStream_t s);
// Token chunks of dW_r: enough workgroups for a few experts' rows (about 512
// tiles), at least 64 tokens a chunk, at most 64 chunks and 2^25 partial floats.
inline int32_t bwd_router_splits(int64_t T, int32_t N, int64_t d) {
  const int64_t tiles = ((N + 127) / 128) * ((d + 255) / 256);
  int64_t sp = (512 + tiles - 1) / tiles;
  const int64_t by_tokens = (T + 63) / 64, by_mem = (int64_t{1} << 25) / (static_cast<int64_t>(N) * d);
  if (sp > by_tokens) sp = by_tokens;
  if (sp > 64) sp = 64;
  if (sp > by_mem) sp = by_mem;
  return static_cast<int32_t>(sp < 1 ? 1 : sp);
}

// ---------------------------------------------------------------- combine
struct CombineArgs {
  int64_t T, d;
  int32_t k, n_shared, act_dtype;
  bool ec;                    // expert choice: k = N slots per token, topk_w indexed by row
  const void* y_perm;
  const int32_t* inv_map;
  const float* topk_w;
  const void* y_shared;
  void* y;
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);

}  // namespace moe
