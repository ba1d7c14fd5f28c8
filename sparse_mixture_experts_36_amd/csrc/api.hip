// C ABI of the MoE layer forward: argument checks, workspace layout, and the
// launch sequence of every entry point. All validation happens on the host
// before anything is enqueued; nothing here allocates or synchronises.
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/moe.h"
#include "common.h"
#include "kernels.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int kMaxExperts = 256;
constexpr int kMaxTopK = 8;
constexpr int kMaxShared = 4;
constexpr int64_t kMaxWidth = int64_t{1} << 20;  // d, d_ff
constexpr int64_t kMaxPitch = int64_t{1} << 21;  // weight row pitches (elements)
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int act_bytes(int32_t dt) { return dt == MOE_F32 ? 4 : 2; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool is_ec(const moe_shape& s) { return s.gating == MOE_GATE_EXPERT_CHOICE; }

// Entries per token of inv_map (and of topk_idx / topk_w under token choice).
int64_t slots(const moe_shape& s) { return is_ec(s) ? s.n_experts : s.top_k; }

// Row pitch of the column-major logit copy of expert choice (16-byte rows).
int64_t ec_ld(const moe_shape& s) { return (s.T + 3) / 4 * 4; }

// Rows reserved for routed experts: every kept pair has one row (expert
// choice: exactly C per expert).
int64_t routed_row_cap(const moe_shape& s) {
  if (is_ec(s)) return static_cast<int64_t>(s.n_experts) * s.capacity;
  const int64_t tk = s.T * s.top_k;
  if (s.capacity < 0) return tk;
  const int64_t nc = static_cast<int64_t>(s.n_experts) * s.capacity;
  return nc < tk ? nc : tk;
}

moe_status check_shape(const moe_shape* s) {
  if (!s) return MOE_ERR_INVALID_ARG;
  if (s->T < 0 || s->d <= 0 || s->d_ff <= 0 || s->n_experts < 1 || s->top_k < 1 || s->top_k > s->n_experts ||
      s->n_shared < 0 || s->capacity < -1)
    return MOE_ERR_INVALID_ARG;
  if (s->act != MOE_ACT_GELU && s->act != MOE_ACT_SWIGLU) return MOE_ERR_INVALID_ARG;
  if (s->gating < MOE_GATE_SOFTMAX_TOPK || s->gating > MOE_GATE_EXPERT_CHOICE) return MOE_ERR_INVALID_ARG;
  if (s->gating == MOE_GATE_EXPERT_CHOICE && (s->top_k != 1 || s->capacity < 0 || s->capacity > s->T))
    return MOE_ERR_INVALID_ARG;
  if (s->act_dtype != MOE_F32 && s->act_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (s->w_dtype < MOE_F32 || s->w_dtype > MOE_INT_W) return MOE_ERR_INVALID_ARG;
  if (s->n_experts > kMaxExperts || s->top_k > kMaxTopK || s->n_shared > kMaxShared) return MOE_ERR_UNSUPPORTED;
  if (s->d % 128 != 0 || s->d_ff % 128 != 0) return MOE_ERR_UNSUPPORTED;
  // kernels form row offsets inside a tile or a pass in 32 bits
  if (s->d > kMaxWidth || s->d_ff > kMaxWidth) return MOE_ERR_UNSUPPORTED;
  if (s->w_dtype != s->act_dtype &&
      !((s->w_dtype == MOE_FP8_E4M3 || s->w_dtype == MOE_INT_W) && s->act_dtype == MOE_BF16))
    return MOE_ERR_UNSUPPORTED;
  if (s->T > (int64_t{1} << 24)) return MOE_ERR_UNSUPPORTED;
  if (s->gating == MOE_GATE_EXPERT_CHOICE && s->T > moe::kEcMaxTokens) return MOE_ERR_UNSUPPORTED;
  const int64_t rows = (s->gating == MOE_GATE_EXPERT_CHOICE ? s->n_experts * s->capacity : s->T * s->top_k) +
                       static_cast<int64_t>(s->n_shared) * s->T;
  const int64_t wmax = s->d > s->d_ff ? s->d : s->d_ff;
  if (rows * wmax >= (int64_t{1} << 31)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Workspace carving; the same walk serves the size query and the launch.
struct Carver {
  char* base;
  size_t off = 0;
  template <typename T>
  T* take(size_t count) {
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off = align_up(off + sizeof(T) * count);
    return p;
  }
};

struct RouteWs {
  float* part_P;
  int32_t* part_cnt;
  float* part_lse;
  float* part_logits;
  float* logits_t;  // expert choice: [N][ec_ld]
};
RouteWs carve_route(Carver& c, const moe_shape& s) {
  const size_t nb = static_cast<size_t>(moe::ceil_div(s.T, moe::kRouteTokens));
  RouteWs w;
  w.part_P = c.take<float>(nb * s.n_experts);
  w.part_cnt = c.take<int32_t>(nb * s.n_experts);
  w.part_lse = c.take<float>(2 * nb);
  w.part_logits = c.take<float>(static_cast<size_t>(moe::route_splits(s.T, s.d, s.n_experts)) * s.T * s.n_experts);
  w.logits_t = is_ec(s) ? c.take<float>(static_cast<size_t>(s.n_experts) * ec_ld(s)) : nullptr;
  return w;
}

struct PermWs {
  int32_t *block_cnt, *block_base, *local_rank, *kept, *n_dropped, *ec_part;
};
PermWs carve_perm(Carver& c, const moe_shape& s) {
  const size_t nb = static_cast<size_t>(moe::ceil_div(s.T, moe::kPermTokens));
  PermWs w;
  w.block_cnt = c.take<int32_t>(nb * s.n_experts);
  w.block_base = c.take<int32_t>(nb * s.n_experts);
  w.local_rank = c.take<int32_t>(static_cast<size_t>(s.T) * s.top_k);
  w.kept = c.take<int32_t>(s.n_experts);
  w.n_dropped = c.take<int32_t>(1);
  w.ec_part = is_ec(s) ? c.take<int32_t>(static_cast<size_t>(moe::ceil_div(s.T, 4))) : nullptr;
  return w;
}

struct FfnWs {
  void* h;
  moe::GroupDesc* groups;
  int32_t* tile_start;
  moe::GroupDesc* groups_t;
  int32_t* tile_start_t;
  int32_t* tile_start_c;
  int32_t* active;
  float* part;
  float* split_part;
};
// Workspace of one grouped-FFN launch set over n_routed routed experts (cap
// rows) and n_shared shared experts (T rows each).
FfnWs carve_ffn_for(Carver& c, const moe_shape& s, int32_t n_routed, int32_t n_shared, int64_t cap) {
  const size_t G = static_cast<size_t>(n_routed + n_shared);
  const size_t hrows = static_cast<size_t>(cap + static_cast<int64_t>(n_shared) * s.T);
  FfnWs w;
  w.h = c.take<char>(hrows * static_cast<size_t>(s.d_ff + moe::kActPad) * act_bytes(s.act_dtype));
  w.groups = c.take<moe::GroupDesc>(2 * G);
  w.tile_start = c.take<int32_t>(G + 1);
  w.groups_t = c.take<moe::GroupDesc>(2 * G);
  w.tile_start_t = c.take<int32_t>(G + 1);
  w.tile_start_c = s.w_dtype == MOE_INT_W ? c.take<int32_t>(4 * (G + 1)) : nullptr;
  w.active = c.take<int32_t>(G + 1);
  w.part = nullptr;
  if (moe::use_skinny(s.act_dtype, cap, n_shared, s.T))
    w.part = c.take<float>(moe::skinny_part_floats(s.T, s.d, s.d_ff, n_routed, n_shared, s.act, cap, s.w_dtype));
  w.split_part = nullptr;
  if (moe::uses_prefill_gemm(s.act_dtype, cap, n_shared, s.T))
    w.split_part = c.take<float>(static_cast<size_t>(moe::kSplitPartFloats));
  return w;
}

FfnWs carve_ffn(Carver& c, const moe_shape& s) {
  return carve_ffn_for(c, s, s.n_experts, s.n_shared, routed_row_cap(s));
}

struct FwdWs {
  float* logits;
  int32_t *topk_idx, *inv_map, *offsets, *perm_token;
  float* topk_w;
  void *x_perm, *y_perm, *y_shared;
};
// Whether moe_forward's expert kernels read routed rows from x through
// perm_token (no permuted copy): bf16 layers, except prefill-sized ones whose x
// rows are a multiple of 4 KB apart. Those rows, fetched at one k-column, fall
// into few L2 channels, so they are copied into x_perm with padded rows; the
// decode path reads its few rows either way.
bool fwd_gathers(const moe_shape& s) {
  if (s.act_dtype != MOE_BF16) return false;
  if (moe::use_skinny(s.act_dtype, routed_row_cap(s), s.n_shared, s.T)) return true;
  return (s.d * 2) % 4096 != 0;
}

FwdWs carve_fwd(Carver& c, const moe_shape& s) {
  const size_t T = static_cast<size_t>(s.T), k = static_cast<size_t>(slots(s));
  const size_t cap = static_cast<size_t>(routed_row_cap(s));
  const size_t rowb = static_cast<size_t>(s.d) * act_bytes(s.act_dtype);
  const size_t sel = is_ec(s) ? cap : T * k;  // topk_idx / topk_w entries
  FwdWs w;
  w.logits = c.take<float>(T * s.n_experts);
  w.topk_idx = c.take<int32_t>(sel);
  w.topk_w = c.take<float>(sel);
  w.inv_map = c.take<int32_t>(T * k);
  w.offsets = c.take<int32_t>(s.n_experts + 1);
  w.perm_token = c.take<int32_t>(is_ec(s) ? cap : T * k);
  w.x_perm = nullptr;
  if (!fwd_gathers(s)) w.x_perm = c.take<char>(cap * static_cast<size_t>(s.d + moe::kActPad) * act_bytes(s.act_dtype));
  w.y_perm = c.take<char>(cap * rowb);
  w.y_shared = c.take<char>(static_cast<size_t>(s.n_shared) * T * rowb);
  return w;
}

// Backward: the recomputed routing, then every row-space product of the
// routed rows [0, cap) and the shared experts' T rows each.
struct BwdWs {
  float* logits;
  int32_t *topk_idx, *inv_map, *offsets, *perm_token, *counts, *tile_start;
  float *topk_w, *lse_mean;
  uint16_t* x_perm;
  float *U, *V, *dH, *dX, *dl32, *dxr, *dg;
  uint16_t *H, *dY, *dU, *dV, *dl_hi, *dl_lo, *dYu;
  int32_t* row_pair;
  float* row_gate;
  int32_t* wr_off;
  float* wr_part;
  // the forward's grouped FFN for the recompute (bwd_uses_ffn)
  moe::GroupDesc *groups, *groups_t;
  int32_t *ffn_tiles, *ffn_tiles_t, *active;
  float* split_part;
};
int64_t bwd_rows(const moe_shape& s) { return routed_row_cap(s) + static_cast<int64_t>(s.n_shared) * s.T; }
bool bwd_uses_ffn(const moe_shape& s) {
  return moe::ffn_uses_dma(s.act_dtype, s.w_dtype, bwd_rows(s), s.act, s.d, s.d_ff);
}
int32_t bwd_ldl(const moe_shape& s) { return (s.n_experts + 7) / 8 * 8; }
BwdWs carve_bwd(Carver& c, const moe_shape& s) {
  const size_t T = static_cast<size_t>(s.T), k = static_cast<size_t>(s.top_k), N = s.n_experts;
  const size_t cap = static_cast<size_t>(routed_row_cap(s));
  const size_t rows = cap + static_cast<size_t>(s.n_shared) * T;
  const size_t d = static_cast<size_t>(s.d), f = static_cast<size_t>(s.d_ff);
  const bool swi = s.act == MOE_ACT_SWIGLU;
  BwdWs w;
  w.logits = c.take<float>(T * N);
  w.topk_idx = c.take<int32_t>(T * k);
  w.topk_w = c.take<float>(T * k);
  w.inv_map = c.take<int32_t>(T * k);
  w.offsets = c.take<int32_t>(N + 1);
  w.perm_token = c.take<int32_t>(T * k);
  w.counts = c.take<int32_t>(N);
  w.lse_mean = c.take<float>(1);
  w.tile_start = c.take<int32_t>(N + 1);
  w.x_perm = c.take<uint16_t>(cap * d);
  w.U = c.take<float>(rows * f);
  w.V = swi ? c.take<float>(rows * f) : nullptr;
  w.H = c.take<uint16_t>(rows * f);
  w.dY = c.take<uint16_t>(cap * d);
  w.dYu = c.take<uint16_t>(cap * d);
  w.row_pair = c.take<int32_t>(cap);
  w.row_gate = c.take<float>(cap);
  w.dH = c.take<float>(rows * f);
  w.dU = c.take<uint16_t>(rows * f * (swi ? 2 : 1));  // [dU | dV] rows for SwiGLU
  w.dV = (swi && w.dU) ? w.dU + f : nullptr;
  w.dX = c.take<float>(rows * d);
  w.dg = c.take<float>(T * k);
  w.dl32 = c.take<float>(T * N);
  w.dl_hi = c.take<uint16_t>(T * static_cast<size_t>(bwd_ldl(s)));
  w.dl_lo = c.take<uint16_t>(T * static_cast<size_t>(bwd_ldl(s)));
  w.dxr = c.take<float>(T * d);
  const int32_t sp = moe::bwd_router_splits(s.T, s.n_experts, s.d);
  w.wr_off = c.take<int32_t>(static_cast<size_t>(sp) + 1);
  w.wr_part = sp > 1 ? c.take<float>(static_cast<size_t>(sp) * N * d) : nullptr;
  w.groups = w.groups_t = nullptr;
  w.ffn_tiles = w.ffn_tiles_t = w.active = nullptr;
  w.split_part = nullptr;
  if (bwd_uses_ffn(s)) {
    const size_t G = static_cast<size_t>(s.n_experts + s.n_shared);
    w.groups = c.take<moe::GroupDesc>(2 * G);
    w.groups_t = c.take<moe::GroupDesc>(2 * G);
    w.ffn_tiles = c.take<int32_t>(G + 1);
    w.ffn_tiles_t = c.take<int32_t>(G + 1);
    w.active = c.take<int32_t>(G + 1);
    w.split_part = c.take<float>(static_cast<size_t>(moe::kSplitPartFloats));
  }
  return w;
}

size_t ws_bytes_for(const moe_shape& s, int32_t entry) {
  Carver c{nullptr};
  switch (entry) {
    case MOE_ENTRY_ROUTE: carve_route(c, s); break;
    case MOE_ENTRY_PERMUTE: carve_perm(c, s); break;
    case MOE_ENTRY_GROUPED_FFN: carve_ffn(c, s); break;
    case MOE_ENTRY_BACKWARD:
      carve_route(c, s);
      carve_perm(c, s);
      carve_bwd(c, s);
      break;
    default:
      carve_route(c, s);
      carve_perm(c, s);
      carve_ffn(c, s);
      carve_fwd(c, s);
      break;
  }
  return c.off + kAlign;
}

moe_status check_ws(const moe_shape& s, int32_t entry, void* ws, size_t ws_bytes) {
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0) return MOE_ERR_WORKSPACE;
  if (ws_bytes < ws_bytes_for(s, entry)) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

moe_status hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  g_last_hip_error = static_cast<int>(e);
  return MOE_ERR_HIP;
}

moe::RouteArgs route_args(const moe_shape& s, const void* x, const void* w_router, const float* b_router,
                          float* logits, bool given, int32_t* topk_idx, float* topk_w, const moe_stats* st,
                          const RouteWs& w) {
  moe::RouteArgs a{};
  a.T = s.T;
  a.d = s.d;
  a.N = s.n_experts;
  a.k = s.top_k;
  a.gating = s.gating;
  a.act_dtype = s.act_dtype;
  a.logits_given = given;
  a.x = x;
  a.w_router = w_router;
  a.b_router = b_router;
  a.logits = logits;
  a.topk_idx = topk_idx;
  a.topk_w = topk_w;
  a.part_P = w.part_P;
  a.part_cnt = w.part_cnt;
  a.part_lse = w.part_lse;
  a.part_logits = w.part_logits;
  a.ec = is_ec(s);
  a.cap = s.capacity;
  a.logits_t = w.logits_t;
  a.ld_lt = ec_ld(s);
  if (st) {
    a.counts = st->counts;
    a.f = st->f;
    a.P = st->P;
    a.l_aux = st->l_aux;
    a.z_loss = st->z_loss;
    a.lse_mean = st->lse_mean;
    a.lse_sq_mean = st->lse_sq_mean;
  }
  a.aux_alpha = s.aux_alpha;
  return a;
}

moe::PermuteArgs perm_args(const moe_shape& s, const int32_t* topk_idx, const void* x, int32_t* offsets,
                           int32_t* perm_token, int32_t* inv_map, void* x_perm, int64_t ld_x_perm,
                           const moe_stats* st, const PermWs& w) {
  moe::PermuteArgs a{};
  a.T = s.T;
  a.d = s.d;
  a.N = s.n_experts;
  a.k = s.top_k;
  a.act_bytes = act_bytes(s.act_dtype);
  a.capacity = s.capacity;
  a.topk_idx = topk_idx;
  a.x = x;
  a.offsets = offsets;
  a.perm_token = perm_token;
  a.inv_map = inv_map;
  a.x_perm = x_perm;
  a.ld_out = ld_x_perm;
  a.kept = (st && st->kept) ? st->kept : w.kept;
  a.n_dropped = (st && st->n_dropped) ? st->n_dropped : w.n_dropped;
  a.block_cnt = w.block_cnt;
  a.block_base = w.block_base;
  a.local_rank = w.local_rank;
  a.ec = is_ec(s);
  a.ec_part = w.ec_part;
  if (a.ec) a.n_dropped = (st && st->n_dropped) ? st->n_dropped : nullptr;
  return a;
}

moe_status check_weights(const moe_shape& s, const moe_weights* w, bool need_router) {
  if (!w) return MOE_ERR_INVALID_ARG;
  if (need_router && !w->w_router) return MOE_ERR_INVALID_ARG;
  if (!w->w1 || !w->w2) return MOE_ERR_INVALID_ARG;
  if (s.act == MOE_ACT_SWIGLU && !w->w3) return MOE_ERR_INVALID_ARG;
  if ((s.w_dtype == MOE_FP8_E4M3 || s.w_dtype == MOE_INT_W) && !w->w_scale) return MOE_ERR_INVALID_ARG;
  if (s.n_shared > 0) {
    if (!w->sw1 || !w->sw2 || (s.act == MOE_ACT_SWIGLU && !w->sw3)) return MOE_ERR_INVALID_ARG;
    if ((s.w_dtype == MOE_FP8_E4M3 || s.w_dtype == MOE_INT_W) && !w->sw_scale) return MOE_ERR_INVALID_ARG;
  }
  if (s.w_dtype == MOE_INT_W) {  // bit widths: host arrays, 8 or 4 per expert
    if (!w->w_bits || (s.n_shared > 0 && !w->sw_bits)) return MOE_ERR_INVALID_ARG;
    for (int e = 0; e < s.n_experts; ++e)
      if (w->w_bits[e] != 8 && w->w_bits[e] != 4) return MOE_ERR_INVALID_ARG;
    for (int e = 0; e < s.n_shared; ++e)
      if (w->sw_bits[e] != 8 && w->sw_bits[e] != 4) return MOE_ERR_INVALID_ARG;
  }
  const void* ptrs[] = {w->w_router, w->w1, w->w3, w->w2, w->sw1, w->sw3, w->sw2};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return MOE_ERR_INVALID_ARG;
  if (w->ld_up != 0 && (w->ld_up < s.d || w->ld_up % 16 != 0)) return MOE_ERR_INVALID_ARG;
  if (w->ld_down != 0 && (w->ld_down < s.d_ff || w->ld_down % 16 != 0)) return MOE_ERR_INVALID_ARG;
  if (w->ld_up > kMaxPitch || w->ld_down > kMaxPitch) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe::FfnArgs ffn_args(const moe_shape& s, const void* x_perm, int64_t ld_x_perm, const int32_t* offsets,
                      const void* x, const moe_weights* w, void* y_perm, void* y_shared, const FfnWs& fw) {
  moe::FfnArgs a{};
  a.T = s.T;
  a.d = s.d;
  a.d_ff = s.d_ff;
  a.n_routed = s.n_experts;
  a.n_shared = s.n_shared;
  a.act = s.act;
  a.act_dtype = s.act_dtype;
  a.w_dtype = s.w_dtype;
  a.routed_row_cap = static_cast<int32_t>(routed_row_cap(s));
  a.offsets = offsets;
  a.x_perm = x_perm;
  a.ld_xp = ld_x_perm;
  a.ld_h = s.d_ff + moe::kActPad;
  a.ld_up = w->ld_up ? w->ld_up : s.d;
  a.ld_down = w->ld_down ? w->ld_down : s.d_ff;
  a.x = x;
  a.w1 = w->w1;
  a.w3 = w->w3;
  a.w2 = w->w2;
  a.b1 = w->b1;
  a.b2 = w->b2;
  a.w_scale = w->w_scale;
  a.sw1 = w->sw1;
  a.sw3 = w->sw3;
  a.sw2 = w->sw2;
  a.sw_scale = w->sw_scale;
  a.h = fw.h;
  a.y_perm = y_perm;
  a.y_shared = y_shared;
  a.groups = fw.groups;
  a.tile_start = fw.tile_start;
  a.groups_t = fw.groups_t;
  a.tile_start_t = fw.tile_start_t;
  a.tile_start_c = fw.tile_start_c;
  a.active = fw.active;
  a.part = fw.part;
  a.split_part = fw.split_part;
  a.w_bits = w->w_bits;
  a.sw_bits = w->sw_bits;
  return a;
}

// ---------------------------------------------------------------- stage timing
struct Timing {
  std::mutex mu;
  std::atomic<bool> on{false};
  std::vector<hipEvent_t> ev;  // pairs: 2i start, 2i+1 end
  std::vector<int> stage_of;
  int cap = 0, used = 0;
  int open[moe::kNumStages];
};
Timing& timing() {
  static Timing t;
  return t;
}

}  // namespace

namespace moe {
void stage_mark(int stage, bool end, hipStream_t s) {
  Timing& t = timing();
  if (!t.on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> g(t.mu);
  if (!t.on) return;
  if (!end) {
    if (t.used >= t.cap) {
      t.open[stage] = -1;
      return;
    }
    const int i = t.used++;
    t.stage_of[i] = stage;
    t.open[stage] = i;
    (void)hipEventRecord(t.ev[2 * i], s);
  } else {
    const int i = t.open[stage];
    if (i < 0) return;
    t.open[stage] = -1;
    (void)hipEventRecord(t.ev[2 * i + 1], s);
  }
}
}  // namespace moe

// moe_forward_noalloc's workspace: a file-scope device array, one copy per GPU
// the library runs on, held until the process ends. Its name is a host-side
// stand-in in host code (never passed to a kernel); the device address comes
// from hipGetSymbolAddress, once per device with that device current.
static __device__ __align__(256) char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

moe_status scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (!p) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}
}  // namespace


extern "C" {

moe_status moe_timing_start(int32_t max_launches) {
  if (max_launches < 1 || max_launches > (1 << 20)) return MOE_ERR_INVALID_ARG;
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  while (static_cast<int>(t.ev.size()) < 2 * max_launches) {
    hipEvent_t e;
    const hipError_t err = hipEventCreate(&e);
    if (err != hipSuccess) return hip_status(err);
    t.ev.push_back(e);
  }
  t.stage_of.assign(max_launches, 0);
  t.cap = max_launches;
  t.used = 0;
  for (int& o : t.open) o = -1;
  t.on = true;
  return MOE_OK;
}

moe_status moe_timing_stop(double* total_ms, int32_t* launches) {
  if (!total_ms || !launches) return MOE_ERR_INVALID_ARG;
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  t.on = false;
  for (int s = 0; s < moe::kNumStages; ++s) {
    total_ms[s] = 0.0;
    launches[s] = 0;
  }
  for (int i = 0; i < t.used; ++i) {
    hipError_t err = hipEventSynchronize(t.ev[2 * i + 1]);
    float ms = 0.f;
    if (err == hipSuccess) err = hipEventElapsedTime(&ms, t.ev[2 * i], t.ev[2 * i + 1]);
    if (err != hipSuccess) return hip_status(err);
    total_ms[t.stage_of[i]] += ms;
    launches[t.stage_of[i]] += 1;
  }
  t.used = 0;
  return MOE_OK;
}


int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MOE_ERR_HIP: return "HIP launch failed";
    case MOE_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    default: return "unknown status";
  }
}

int moe_last_hip_error(void) { return g_last_hip_error; }

int64_t moe_capacity(int64_t T, int32_t k, int32_t N, double cf) {
  if (cf < 0.0 || N < 1) return -1;
  const double c = cf * static_cast<double>(T) * static_cast<double>(k) / static_cast<double>(N);
  return static_cast<int64_t>(c);  // truncation = floor for c >= 0
}

moe_status moe_workspace_size(const moe_shape* shape, int32_t entry, size_t* bytes) {
  const moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!bytes || entry < MOE_ENTRY_ROUTE || entry > MOE_ENTRY_BACKWARD) return MOE_ERR_INVALID_ARG;
  *bytes = ws_bytes_for(*shape, entry);
  return MOE_OK;
}

int32_t moe_ffn_path(const moe_shape* shape, int32_t entry) {
  const moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (entry != MOE_ENTRY_GROUPED_FFN && entry != MOE_ENTRY_FORWARD && entry != MOE_ENTRY_BACKWARD)
    return MOE_ERR_INVALID_ARG;
  const moe_shape& s = *shape;
  if (entry == MOE_ENTRY_BACKWARD && !bwd_uses_ffn(s)) return moe::kPathBgemm;
  moe::FfnArgs a{};
  a.T = s.T;
  a.d = s.d;
  a.d_ff = s.d_ff;
  a.n_routed = s.n_experts;
  a.n_shared = s.n_shared;
  a.act = s.act;
  a.act_dtype = s.act_dtype;
  a.w_dtype = s.w_dtype;
  a.routed_row_cap = routed_row_cap(s);
  return moe::ffn_path_of(a);
}

moe_status moe_route(const moe_shape* shape, const void* x, const void* w_router, const float* b_router,
                     float* logits, uint32_t flags, int32_t* topk_idx, float* topk_w, const moe_stats* stats,
                     void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  const bool given = (flags & MOE_ROUTE_LOGITS_GIVEN) != 0;
  if ((flags & ~MOE_ROUTE_LOGITS_GIVEN) != 0) return MOE_ERR_INVALID_ARG;
  const bool no_sel = is_ec(*shape) && shape->capacity == 0;  // expert choice with C = 0: empty lists
  if (!logits || (!no_sel && (!topk_idx || !topk_w))) return MOE_ERR_INVALID_ARG;
  if (!given && (!x || !w_router || !aligned16(x) || !aligned16(w_router))) return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(*shape, MOE_ENTRY_ROUTE, ws, ws_bytes)) != MOE_OK) return st;
  Carver c{static_cast<char*>(ws)};
  const RouteWs w = carve_route(c, *shape);
  return hip_status(moe::launch_route(
      route_args(*shape, x, w_router, b_router, logits, given, topk_idx, topk_w, stats, w), stream));
}

moe_status moe_permute(const moe_shape* shape, const int32_t* topk_idx, const void* x, int32_t* expert_offsets,
                       int32_t* perm_token, int32_t* inv_map, void* x_perm, const moe_stats* stats, void* ws,
                       size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  const bool no_sel = is_ec(*shape) && shape->capacity == 0;  // expert choice with C = 0: no rows
  if (!expert_offsets || !inv_map || (!no_sel && (!topk_idx || !perm_token))) return MOE_ERR_INVALID_ARG;
  if (x_perm && (!x || !aligned16(x) || !aligned16(x_perm))) return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(*shape, MOE_ENTRY_PERMUTE, ws, ws_bytes)) != MOE_OK) return st;
  Carver c{static_cast<char*>(ws)};
  const PermWs w = carve_perm(c, *shape);
  return hip_status(moe::launch_permute(
      perm_args(*shape, topk_idx, x, expert_offsets, perm_token, inv_map, x_perm, shape->d, stats, w), stream));
}

moe_status moe_grouped_ffn(const moe_shape* shape, const void* x_perm, const int32_t* expert_offsets,
                           const void* x, const moe_weights* weights, void* y_perm, void* y_shared, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!expert_offsets || !x_perm || !y_perm || !aligned16(x_perm) || !aligned16(y_perm))
    return MOE_ERR_INVALID_ARG;
  if (shape->n_shared > 0 && (!x || !y_shared || !aligned16(x) || !aligned16(y_shared))) return MOE_ERR_INVALID_ARG;
  if ((st = check_weights(*shape, weights, false)) != MOE_OK) return st;
  if ((st = check_ws(*shape, MOE_ENTRY_GROUPED_FFN, ws, ws_bytes)) != MOE_OK) return st;
  if (shape->T == 0) return MOE_OK;
  Carver c{static_cast<char*>(ws)};
  const FfnWs fw = carve_ffn(c, *shape);
  return hip_status(
      moe::launch_grouped_ffn(ffn_args(*shape, x_perm, shape->d, expert_offsets, x, weights, y_perm, y_shared, fw),
                              stream));
}

moe_status moe_combine(const moe_shape* shape, const void* y_perm, const int32_t* inv_map, const float* topk_w,
                       const void* y_shared, void* y, hipStream_t stream) {
  const moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  const bool no_rows = is_ec(*shape) && shape->capacity == 0;  // expert choice with C = 0
  if (!inv_map || !y || !aligned16(y)) return MOE_ERR_INVALID_ARG;
  if (!no_rows && (!y_perm || !topk_w || !aligned16(y_perm))) return MOE_ERR_INVALID_ARG;
  if (y_shared && !aligned16(y_shared)) return MOE_ERR_INVALID_ARG;
  moe::CombineArgs a{};
  a.T = shape->T;
  a.d = shape->d;
  a.k = static_cast<int32_t>(slots(*shape));
  a.ec = is_ec(*shape);
  a.n_shared = shape->n_shared;
  a.act_dtype = shape->act_dtype;
  a.y_perm = y_perm;
  a.inv_map = inv_map;
  a.topk_w = topk_w;
  a.y_shared = y_shared;
  a.y = y;
  return hip_status(moe::launch_combine(a, stream));
}

moe_status moe_forward(const moe_shape* shape, const void* x, const moe_weights* weights, void* y, float* logits,
                       int32_t* topk_idx, float* topk_w, int32_t* expert_offsets, int32_t* perm_token,
                       int32_t* inv_map, const moe_stats* stats, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!x || !y || !aligned16(x) || !aligned16(y)) return MOE_ERR_INVALID_ARG;
  if ((st = check_weights(*shape, weights, true)) != MOE_OK) return st;
  if ((st = check_ws(*shape, MOE_ENTRY_FORWARD, ws, ws_bytes)) != MOE_OK) return st;
  if (shape->T == 0) return MOE_OK;
  const moe_shape& s = *shape;
  Carver c{static_cast<char*>(ws)};
  const RouteWs rw = carve_route(c, s);
  const PermWs pw = carve_perm(c, s);
  const FfnWs fw = carve_ffn(c, s);
  const FwdWs w = carve_fwd(c, s);
  const int64_t ld_xp = s.d + moe::kActPad;  // the internal x_perm has a padded row pitch
  if (!logits) logits = w.logits;
  if (!topk_idx) topk_idx = w.topk_idx;
  if (!topk_w) topk_w = w.topk_w;
  if (!inv_map) inv_map = w.inv_map;
  if (!expert_offsets) expert_offsets = w.offsets;
  if (!perm_token) perm_token = w.perm_token;

  const bool gather = fwd_gathers(s);  // then the permutation copies no rows
  const moe::RouteArgs ra =
      route_args(s, x, weights->w_router, weights->b_router, logits, false, topk_idx, topk_w, stats, rw);
  moe::FfnArgs fa = ffn_args(s, w.x_perm, ld_xp, expert_offsets, x, weights, w.y_perm, w.y_shared, fw);
  moe::PermuteArgs pa = perm_args(s, topk_idx, x, expert_offsets, perm_token, inv_map, gather ? nullptr : w.x_perm,
                                  ld_xp, stats, pw);
  if (gather) fa.gather = perm_token;
  if (!is_ec(s)) {  // a one-token call may fold the combine into the down GEMM
    fa.fuse_inv_map = inv_map;
    fa.fuse_topk_idx = topk_idx;
    fa.fuse_topk_w = topk_w;
    fa.fuse_k = static_cast<int32_t>(s.top_k);
    fa.fuse_y = y;
  }
  // the permutation writes the FFN's group plan where it forms the offsets
  // (its scan pass, or its one block), and expert choice's where they are fixed:
  // no plan launch
  pa.plan = moe::ffn_plan(fa);
  fa.planned = true;
  hipError_t e = hipSuccess;
  if (moe::front_fits(ra, pa)) {  // decode sizes: router GEMM, routing and permutation in one launch
    e = moe::launch_front(ra, pa, stream);
  } else {
    // with a scan pass (more than one permutation block) the permutation also
    // finishes the routing statistics: one launch fewer
    const bool defer = !is_ec(s) && s.T > moe::kPermTokens;
    if (defer) {
      pa.fin = ra;
      pa.fin_nb = static_cast<int32_t>((s.T + moe::kRouteTokens - 1) / moe::kRouteTokens);
    }
    e = moe::launch_route(ra, stream, !defer);
    if (e == hipSuccess) e = moe::launch_permute(pa, stream);
  }
  if (e == hipSuccess) e = moe::launch_grouped_ffn(fa, stream);
  if (e == hipSuccess && !moe::ffn_fuses_combine(fa)) {
    moe::CombineArgs a{};
    a.T = s.T;
    a.d = s.d;
    a.k = static_cast<int32_t>(slots(s));
    a.ec = is_ec(s);
    a.n_shared = s.n_shared;
    a.act_dtype = s.act_dtype;
    a.y_perm = w.y_perm;
    a.inv_map = inv_map;
    a.topk_w = topk_w;
    a.y_shared = s.n_shared > 0 ? w.y_shared : nullptr;
    a.y = y;
    e = moe::launch_combine(a, stream);
  }
  return hip_status(e);
}

moe_status moe_forward_noalloc(const moe_shape* shape, const void* x, const moe_weights* weights, void* y,
                               float* logits, int32_t* topk_idx, float* topk_w, int32_t* expert_offsets,
                               int32_t* perm_token, int32_t* inv_map, const moe_stats* stats, hipStream_t stream) {
  const moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (ws_bytes_for(*shape, MOE_ENTRY_FORWARD) > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  const moe_status sp = scratch_ptr(&ws);
  if (sp != MOE_OK) return sp;
  return moe_forward(shape, x, weights, y, logits, topk_idx, topk_w, expert_offsets, perm_token, inv_map, stats, ws,
                     MOE_NOALLOC_SCRATCH_BYTES, stream);
}

moe_status moe_backward(const moe_shape* shape, const void* x, const moe_weights* weights, const void* dy,
                        float c_aux, float c_z, const moe_grads* g, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape& s = *shape;
  if (is_ec(s) || s.act_dtype != MOE_BF16 || s.w_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (!x || !dy || !g || !g->dx || !aligned16(x) || !aligned16(dy) || !aligned16(g->dx)) return MOE_ERR_INVALID_ARG;
  if ((st = check_weights(s, weights, true)) != MOE_OK) return st;
  if ((st = check_ws(s, MOE_ENTRY_BACKWARD, ws, ws_bytes)) != MOE_OK) return st;
  if (s.T == 0) return MOE_OK;
  Carver c{static_cast<char*>(ws)};
  const RouteWs rw = carve_route(c, s);
  const PermWs pw = carve_perm(c, s);
  const BwdWs w = carve_bwd(c, s);
  moe_stats rst{};
  rst.counts = w.counts;
  rst.lse_mean = w.lse_mean;
  hipError_t e = moe::launch_route(route_args(s, x, weights->w_router, weights->b_router, w.logits, false,
                                              w.topk_idx, w.topk_w, &rst, rw),
                                   stream);
  if (e == hipSuccess)
    e = moe::launch_permute(
        perm_args(s, w.topk_idx, x, w.offsets, w.perm_token, w.inv_map, w.x_perm, s.d, nullptr, pw), stream);
  if (e != hipSuccess) return hip_status(e);
  moe::BwdArgs a{};
  a.T = s.T;
  a.d = s.d;
  a.d_ff = s.d_ff;
  a.cap = routed_row_cap(s);
  a.N = s.n_experts;
  a.k = s.top_k;
  a.S = s.n_shared;
  a.act = s.act;
  a.gating = s.gating;
  a.ldl = bwd_ldl(s);
  a.ld_du = s.act == MOE_ACT_SWIGLU ? 2 * s.d_ff : s.d_ff;
  a.aux_alpha = s.aux_alpha;
  a.c_aux = c_aux;
  a.c_z = c_z;
  a.x = static_cast<const uint16_t*>(x);
  a.dy = static_cast<const uint16_t*>(dy);
  a.w_router = static_cast<const uint16_t*>(weights->w_router);
  a.x_perm = w.x_perm;
  a.w1 = static_cast<const uint16_t*>(weights->w1);
  a.w3 = static_cast<const uint16_t*>(weights->w3);
  a.w2 = static_cast<const uint16_t*>(weights->w2);
  a.sw1 = static_cast<const uint16_t*>(weights->sw1);
  a.sw3 = static_cast<const uint16_t*>(weights->sw3);
  a.sw2 = static_cast<const uint16_t*>(weights->sw2);
  a.ld_up = weights->ld_up ? weights->ld_up : s.d;
  a.ld_down = weights->ld_down ? weights->ld_down : s.d_ff;
  a.b1 = weights->b1;
  a.b2 = weights->b2;
  a.logits = w.logits;
  a.topk_idx = w.topk_idx;
  a.inv_map = w.inv_map;
  a.offsets = w.offsets;
  a.counts = w.counts;
  a.topk_w = w.topk_w;
  a.lse_mean = w.lse_mean;
  a.U = w.U;
  a.V = w.V;
  a.dYu = w.dYu;
  a.row_pair = w.row_pair;
  a.row_gate = w.row_gate;
  a.dH = w.dH;
  a.dX = w.dX;
  a.dl32 = w.dl32;
  a.dxr = w.dxr;
  a.dg = w.dg;
  a.H = w.H;
  a.dY = w.dY;
  a.dU = w.dU;
  a.dV = w.dV;
  a.dl_hi = w.dl_hi;
  a.dl_lo = w.dl_lo;
  a.tile_start = w.tile_start;
  a.wr_splits = moe::bwd_router_splits(s.T, s.n_experts, s.d);
  a.wr_off = w.wr_off;
  a.wr_part = w.wr_part;
  a.use_ffn = bwd_uses_ffn(s);
  if (a.use_ffn) {  // U, V, H and Y from the forward's grouped FFN
    FfnWs fw{};
    fw.h = w.H;
    fw.groups = w.groups;
    fw.tile_start = w.ffn_tiles;
    fw.groups_t = w.groups_t;
    fw.tile_start_t = w.ffn_tiles_t;
    fw.active = w.active;
    fw.split_part = w.split_part;
    // only its up GEMM runs (the down GEMM's outputs would land in dY and dX)
    a.ffn = ffn_args(s, w.x_perm, s.d, w.offsets, x, weights, w.dY, w.dX, fw);
    a.ffn.ld_h = s.d_ff;
    a.ffn.pre_up_u = w.U;
    a.ffn.pre_up_v = w.V;
    a.ffn.ld_pre_up = s.d_ff;
    a.ffn.up_only = true;
  }
  a.dx = static_cast<uint16_t*>(g->dx);
  a.dWr = g->dw_router;
  a.dbr = g->db_router;
  a.dW1 = g->dw1;
  a.dW3 = s.act == MOE_ACT_SWIGLU ? g->dw3 : nullptr;
  a.dW2 = g->dw2;
  a.db1 = s.act == MOE_ACT_GELU ? g->db1 : nullptr;
  a.db2 = s.act == MOE_ACT_GELU ? g->db2 : nullptr;
  a.dsW1 = s.n_shared > 0 ? g->dsw1 : nullptr;
  a.dsW3 = (s.n_shared > 0 && s.act == MOE_ACT_SWIGLU) ? g->dsw3 : nullptr;
  a.dsW2 = s.n_shared > 0 ? g->dsw2 : nullptr;
  return hip_status(moe::launch_backward(a, stream));
}

}  // extern "C"
