// MoE layer forward -- CPU ORACLE. TEST INFRASTRUCTURE ONLY.
//
// Plain, slow, fp64 reference of what the GPU library computes. Only the test
// suite, the smoke check and the benchmark's CPU-baseline leg may load it. It
// shares no code, header or table with the GPU library (it has its own copies
// of the argument structs below and decodes bf16 / e4m3 itself).
//
// Sources (the pages this follows, cited by title and section):
//  [AIG]  aigrafen.se, "Mixture of Experts": the y = sum g_i E_i(x) and
//         g = softmax(W_r x) equation, the L_aux = alpha*N*sum f_i P_i equation,
//         the capacity equation C = tokens/N * cf, and the `MoE` module (router
//         softmax -> top-k -> renormalise, capacity int(cf*T*k/N), the
//         per-expert loop with `nonzero` order and truncation to C, f and P).
//  [MOEA] vanos001 placement notes, "MoE Architecture": section "Expert Network
//         Design" (SwiGLUExpert w2(silu(w1 x) * w3 x); StandardExpert
//         Linear-GELU-Linear), "Router Design / Token-Choice Router" (top-k on
//         logits, then softmax over the k), "Router Design / Expert-Choice
//         Router" (softmax over tokens, each expert's top-capacity tokens) and
//         the router comparison table, "Capacity and Token Dropping".
//  [SPX]  learn.starphix.com, "Mixture of Experts (MoE)": sections "Key
//         Equations", "Top-k Gating", "Load Balancing (Critical)"
//         (load_balancing_loss, z_loss), "Shared + Specialized".
//  [CFS]  chipfoundryservices.com glossary, "Mixture of Experts (MoE)": the
//         "Expert Choice Routing" item (experts pick their tokens; balanced).
//  [WIKI] wiki.ai-engineering.at, "Mixture of Experts (MoE)": the router /
//         softmax / top-k / weighted-combination figure and the `MoELayer`
//         snippet (top-k of the gate scores, softmax over the k).
//
// Readings where the pages are silent or disagree (all listed in the design
// notes of the repository):
//  - Router output is an fp32 tensor (the pages' modules run in PyTorch's
//    default float32). Logits are accumulated in fp64 and rounded once to fp32;
//    selection and everything after it use those fp32 values widened exactly.
//  - Top-k order: descending logit, exact ties go to the lower expert index.
//    Selection on logits equals selection on softmax probabilities because
//    softmax is strictly increasing.
//  - f_e = counts_e / (T*k) counted before drops; P_e = mean over tokens of the
//    full softmax; alpha multiplies the loss; z = (mean_t logsumexp_t)^2.
//  - Capacity: pairs of expert e in ascending token order, the first C kept;
//    a dropped pair adds 0 to the layer output (the residual is outside).
//  - GELU is the exact erf form; SiLU(u) = u / (1 + e^-u).
//  - e4m3 weights: W = s * q, q an OCP e4m3fn code, one fp32 scale per
//    (expert, matrix).
//  - Integer weights [SPX "Quantization": INT8 for high-traffic experts, INT4
//    for the rest, the router kept in 16 bits]: W[r][c] = s_r * q[r][c] with
//    one fp32 scale per weight row and symmetric codes (|q| <= 127 or <= 7);
//    the oracle reads one code per byte whatever the expert's bit width.
//  - Expert choice [MOEA Expert-Choice Router]: the softmax runs over the
//    tokens of each expert's column; an expert takes the C = int(T*cf/N)
//    tokens of largest probability, exact ties to the lower token index, and
//    lists them in ascending token order (the order inside an expert never
//    reaches the output). The router there returns only the assignments; the
//    gate of a taken (token, expert) pair is that column probability, and a
//    token no expert took gets only the shared experts.
//
// Every function returns 0 on success and -1 when the arguments fall outside
// the contract (k > N, N < 1, ...). Parallelism (OpenMP) only splits
// independent rows; every sum is accumulated sequentially in fp64.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <vector>

#include <omp.h>

extern "C" {

struct OrcShape {
  int64_t T, d, d_ff;
  int32_t n_experts, top_k, n_shared;
  int32_t act;        // 0 GELU expert (Linear+bias, GELU, Linear+bias), 1 SwiGLU
  int32_t gating;     // 0 softmax->top-k, 1 softmax->top-k->renormalise, 2 top-k->softmax,
                      // 3 expert choice (softmax over tokens, each expert takes C tokens)
  int32_t act_dtype;  // 0 fp32, 1 bf16 (x, router weight, layer output)
  int32_t w_dtype;    // 0 fp32, 1 bf16, 2 e4m3fn + per-(expert, matrix) fp32 scale,
                      // 3 integer codes (int8 storage, |q| <= 127 or <= 7) + per-row fp32 scale
  int64_t capacity;   // < 0: no capacity limit
  double aux_alpha;
};

struct OrcWeights {
  const void* w_router;        // [N][d], act dtype
  const float* b_router;       // [N] or null
  const void* w1;              // [N][d_ff][d]
  const void* w3;              // [N][d_ff][d] (SwiGLU) or null
  const void* w2;              // [N][d][d_ff]
  const float* b1;             // [N][d_ff] or null (GELU only)
  const float* b2;             // [N][d] or null (GELU only)
  const float* w_scale;        // [N][3] scales of (W1, W3, W2) for e4m3; for integer
                               // codes [N][2 d_ff + d] row scales: W1 rows, W3 rows, W2 rows
  const void* sw1;             // shared experts [S][d_ff][d]
  const void* sw3;             // [S][d_ff][d]
  const void* sw2;             // [S][d][d_ff]
  const float* sw_scale;       // [S][3]
};

}  // extern "C"

namespace {

double bf16_value(uint16_t b) {
  uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return static_cast<double>(f);
}

// OCP e4m3fn: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0
// is subnormal (m * 2^-9); no infinities; S.1111.111 is NaN (never produced).
double e4m3_value(uint8_t q) {
  const int e = (q >> 3) & 15, m = q & 7;
  double v = (e == 0) ? std::ldexp(static_cast<double>(m), -9)
                      : std::ldexp(1.0 + m / 8.0, e - 7);
  return (q & 0x80) ? -v : v;
}

// Element i of a tensor stored in `dtype`, times `scale` (e4m3 and integer
// codes only).
double elem(const void* p, int dtype, int64_t i, double scale) {
  switch (dtype) {
    case 0: return static_cast<double>(static_cast<const float*>(p)[i]);
    case 1: return bf16_value(static_cast<const uint16_t*>(p)[i]);
    case 2: return scale * e4m3_value(static_cast<const uint8_t*>(p)[i]);
    default: return scale * static_cast<double>(static_cast<const int8_t*>(p)[i]);
  }
}

bool shape_ok(const OrcShape* s) {
  return s && s->T >= 0 && s->d > 0 && s->d_ff > 0 && s->n_experts >= 1 && s->top_k >= 1 &&
         s->top_k <= s->n_experts && s->n_shared >= 0 && (s->act == 0 || s->act == 1) &&
         s->gating >= 0 && s->gating <= 3 && (s->act_dtype == 0 || s->act_dtype == 1) &&
         s->w_dtype >= 0 && s->w_dtype <= 3;
}

// token choice: gating 0..2
bool shape_ok_tc(const OrcShape* s) { return shape_ok(s) && s->gating != 3; }

// expert choice: gating 3, top_k 1, 0 <= C <= T
bool shape_ok_ec(const OrcShape* s) {
  return s && s->T >= 0 && s->d > 0 && s->d_ff > 0 && s->n_experts >= 1 && s->top_k == 1 &&
         s->n_shared >= 0 && (s->act == 0 || s->act == 1) && s->gating == 3 &&
         (s->act_dtype == 0 || s->act_dtype == 1) && s->w_dtype >= 0 && s->w_dtype <= 3 &&
         s->capacity >= 0 && s->capacity <= s->T;
}

double gelu(double u) { return 0.5 * u * (1.0 + std::erf(u / std::sqrt(2.0))); }
double silu(double u) { return u / (1.0 + std::exp(-u)); }

// One expert applied to n rows X [n][d] -> Y [n][d] (fp64).
// GELU expert [AIG `MoE` module; MOEA "Expert Network Design", StandardExpert]:
//   y = W2 gelu(W1 x + b1) + b2.
// SwiGLU expert [MOEA "Expert Network Design", SwiGLUExpert]:
//   y = W2 (silu(W1 x) * (W3 x)).
void expert_rows(const OrcShape* s, const OrcWeights* w, bool shared, int e, const double* X,
                 int64_t n, double* Y) {
  const int64_t d = s->d, f = s->d_ff;
  const void* W1 = shared ? w->sw1 : w->w1;
  const void* W3 = shared ? w->sw3 : w->w3;
  const void* W2 = shared ? w->sw2 : w->w2;
  const float* sc = shared ? w->sw_scale : w->w_scale;
  const float* b1 = shared ? nullptr : w->b1;
  const float* b2 = shared ? nullptr : w->b2;
  // e4m3: one scale per matrix; integer codes: one per weight row
  const bool rowsc = (s->w_dtype == 3);
  const int64_t rs0 = static_cast<int64_t>(e) * (2 * f + d);  // the expert's row scales
  auto s1 = [&](int64_t i) { return rowsc ? sc[rs0 + i] : (s->w_dtype == 2) ? sc[3 * e + 0] : 1.0; };
  auto s3 = [&](int64_t i) { return rowsc ? sc[rs0 + f + i] : (s->w_dtype == 2) ? sc[3 * e + 1] : 1.0; };
  auto s2 = [&](int64_t o) { return rowsc ? sc[rs0 + 2 * f + o] : (s->w_dtype == 2) ? sc[3 * e + 2] : 1.0; };
  const int64_t base1 = static_cast<int64_t>(e) * f * d;  // expert e in [N][d_ff][d]
  const int64_t base2 = static_cast<int64_t>(e) * d * f;  // expert e in [N][d][d_ff]
  std::vector<double> H(static_cast<size_t>(n * f));

#pragma omp parallel
  {
    std::vector<double> a(d), g(d);
#pragma omp for schedule(static)
    for (int64_t i = 0; i < f; ++i) {
      for (int64_t j = 0; j < d; ++j) a[j] = elem(W1, s->w_dtype, base1 + i * d + j, s1(i));
      if (s->act == 1)
        for (int64_t j = 0; j < d; ++j) g[j] = elem(W3, s->w_dtype, base1 + i * d + j, s3(i));
      for (int64_t r = 0; r < n; ++r) {
        const double* x = X + r * d;
        double u = 0.0;
        for (int64_t j = 0; j < d; ++j) u += a[j] * x[j];
        if (s->act == 0) {
          if (b1) u += static_cast<double>(b1[static_cast<int64_t>(e) * f + i]);
          H[r * f + i] = gelu(u);
        } else {
          double v = 0.0;
          for (int64_t j = 0; j < d; ++j) v += g[j] * x[j];
          H[r * f + i] = silu(u) * v;
        }
      }
    }
  }

#pragma omp parallel
  {
    std::vector<double> a(f);
#pragma omp for schedule(static)
    for (int64_t o = 0; o < d; ++o) {
      for (int64_t i = 0; i < f; ++i) a[i] = elem(W2, s->w_dtype, base2 + o * f + i, s2(o));
      for (int64_t r = 0; r < n; ++r) {
        const double* h = H.data() + r * f;
        double u = 0.0;
        for (int64_t i = 0; i < f; ++i) u += a[i] * h[i];
        if (s->act == 0 && b2) u += static_cast<double>(b2[static_cast<int64_t>(e) * d + o]);
        Y[r * d + o] = u;
      }
    }
  }
}

}  // namespace

extern "C" {

int orc_abi_version(void) { return 1; }

// Threads the oracle's parallel loops use (OpenMP default team size).
int orc_threads(void) {
  int n = 1;
#pragma omp parallel
  {
#pragma omp single
    n = omp_get_num_threads();
  }
  return n;
}

// Router logits [AIG, g = softmax(W_r x); SPX "Key Equations", router_logits =
// x W_router^T; WIKI `MoELayer`/`CapacityMoE` use a biased gate]:
//   l[t][e] = sum_i x[t][i] * W_r[e][i] (+ b_r[e]), accumulated in fp64.
// Outputs the fp64 value and the fp32 router output (one rounding).
int orc_router_logits(const OrcShape* s, const void* x, const OrcWeights* w, double* logits64,
                      float* logits32) {
  if (!shape_ok(s) || !x || !w || !w->w_router) return -1;
  const int64_t T = s->T, d = s->d, N = s->n_experts;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t e = 0; e < N; ++e) {
      double acc = 0.0;
      for (int64_t i = 0; i < d; ++i)
        acc += elem(x, s->act_dtype, t * d + i, 1.0) * elem(w->w_router, s->act_dtype, e * d + i, 1.0);
      if (w->b_router) acc += static_cast<double>(w->b_router[e]);
      if (logits64) logits64[t * N + e] = acc;
      if (logits32) logits32[t * N + e] = static_cast<float>(acc);
    }
  }
  return 0;
}

// Routing and statistics from fp32 router outputs `logits` [T][N].
//  softmax  p[t][e] = exp(l - m) / sum exp(l - m), m = max_e l;  lse = m + ln sum exp(l - m)
//  select   S_t = the k largest logits, descending, ties -> lower expert index
//  gates    mode 0 [AIG equation; WIKI figure]: g_j = p[t][S_j]
//           mode 1 [AIG `MoE` module]:          g_j = p[t][S_j] / sum_j' p[t][S_j']
//           mode 2 [MOEA Token-Choice Router; SPX "Top-k Gating"; WIKI `MoELayer`]:
//                                               g = softmax over l[t][S_t]
//  stats    [AIG L_aux equation and `MoE` module; SPX "Load Balancing"]:
//           counts_e = #{t : e in S_t} (before any capacity drop)
//           f_e = counts_e / (T k),  P_e = (1/T) sum_t p[t][e]
//           L_aux = alpha * N * sum_e f_e P_e
//           z = ((1/T) sum_t lse_t)^2  [SPX z_loss];  lse_sq_mean = (1/T) sum_t lse_t^2
//  margins  margin_set[t]   = l_(k) - l_(k+1) of the sorted logits (+inf when k = N)
//           margin_order[t] = min_j l_(j) - l_(j+1), j < k (+inf when k = 1)
// Any output pointer except topk_idx may be null.
int orc_route(const OrcShape* s, const float* logits, int32_t* topk_idx, double* topk_w,
              double* probs, double* lse_out, double* margin_set, double* margin_order,
              int64_t* counts, double* f, double* P, double* l_aux, double* z,
              double* lse_sq_mean) {
  if (!shape_ok_tc(s) || !logits || !topk_idx) return -1;
  const int64_t T = s->T, N = s->n_experts, k = s->top_k;
  std::vector<double> p_all(static_cast<size_t>(T * N));
  std::vector<double> lse(static_cast<size_t>(T));

#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    const float* l = logits + t * N;
    double m = -std::numeric_limits<double>::infinity();
    for (int64_t e = 0; e < N; ++e) m = std::max(m, static_cast<double>(l[e]));
    double sum = 0.0;
    for (int64_t e = 0; e < N; ++e) sum += std::exp(static_cast<double>(l[e]) - m);
    for (int64_t e = 0; e < N; ++e) p_all[t * N + e] = std::exp(static_cast<double>(l[e]) - m) / sum;
    lse[t] = m + std::log(sum);

    // selection: k rounds, each taking the largest remaining logit; scanning e
    // upward with a strict '>' keeps the lower index on exact ties.
    std::vector<char> taken(static_cast<size_t>(N), 0);
    int32_t* S = topk_idx + t * k;
    for (int64_t j = 0; j < k; ++j) {
      int64_t best = -1;
      for (int64_t e = 0; e < N; ++e)
        if (!taken[e] && (best < 0 || l[e] > l[best])) best = e;
      taken[best] = 1;
      S[j] = static_cast<int32_t>(best);
    }
    if (margin_set) {
      double next = -std::numeric_limits<double>::infinity();
      for (int64_t e = 0; e < N; ++e)
        if (!taken[e]) next = std::max(next, static_cast<double>(l[e]));
      margin_set[t] = (k == N) ? std::numeric_limits<double>::infinity()
                               : static_cast<double>(l[S[k - 1]]) - next;
    }
    if (margin_order) {
      double mo = std::numeric_limits<double>::infinity();
      for (int64_t j = 0; j + 1 < k; ++j)
        mo = std::min(mo, static_cast<double>(l[S[j]]) - static_cast<double>(l[S[j + 1]]));
      margin_order[t] = mo;
    }
    if (topk_w) {
      double* g = topk_w + t * k;
      if (s->gating == 0) {
        for (int64_t j = 0; j < k; ++j) g[j] = p_all[t * N + S[j]];
      } else if (s->gating == 1) {
        double den = 0.0;
        for (int64_t j = 0; j < k; ++j) den += p_all[t * N + S[j]];
        for (int64_t j = 0; j < k; ++j) g[j] = p_all[t * N + S[j]] / den;
      } else {
        const double m0 = static_cast<double>(l[S[0]]);  // largest selected logit
        double den = 0.0;
        for (int64_t j = 0; j < k; ++j) den += std::exp(static_cast<double>(l[S[j]]) - m0);
        for (int64_t j = 0; j < k; ++j) g[j] = std::exp(static_cast<double>(l[S[j]]) - m0) / den;
      }
    }
  }

  if (probs) std::memcpy(probs, p_all.data(), sizeof(double) * static_cast<size_t>(T * N));
  if (lse_out) std::memcpy(lse_out, lse.data(), sizeof(double) * static_cast<size_t>(T));

  std::vector<int64_t> cnt(static_cast<size_t>(N), 0);
  for (int64_t t = 0; t < T; ++t)
    for (int64_t j = 0; j < k; ++j) cnt[topk_idx[t * k + j]] += 1;
  std::vector<double> Pv(static_cast<size_t>(N), 0.0), fv(static_cast<size_t>(N), 0.0);
  for (int64_t e = 0; e < N; ++e) {
    double acc = 0.0;
    for (int64_t t = 0; t < T; ++t) acc += p_all[t * N + e];
    Pv[e] = (T > 0) ? acc / static_cast<double>(T) : 0.0;
    fv[e] = (T > 0) ? static_cast<double>(cnt[e]) / static_cast<double>(T * k) : 0.0;
  }
  double dot = 0.0;
  for (int64_t e = 0; e < N; ++e) dot += fv[e] * Pv[e];
  double lse_sum = 0.0, lse_sq = 0.0;
  for (int64_t t = 0; t < T; ++t) { lse_sum += lse[t]; lse_sq += lse[t] * lse[t]; }
  const double lse_mean = (T > 0) ? lse_sum / static_cast<double>(T) : 0.0;

  if (counts) std::memcpy(counts, cnt.data(), sizeof(int64_t) * static_cast<size_t>(N));
  if (f) std::memcpy(f, fv.data(), sizeof(double) * static_cast<size_t>(N));
  if (P) std::memcpy(P, Pv.data(), sizeof(double) * static_cast<size_t>(N));
  if (l_aux) *l_aux = s->aux_alpha * static_cast<double>(N) * dot;
  if (z) *z = lse_mean * lse_mean;
  if (lse_sq_mean) *lse_sq_mean = (T > 0) ? lse_sq / static_cast<double>(T) : 0.0;
  return 0;
}

// Dispatch with capacity [AIG capacity equation and `MoE` module;
// MOEA "Capacity and Token Dropping"]. For every expert e (ascending), the
// tokens that selected e in ascending token order; the first min(count, C)
// are kept. The kept pairs, experts ascending and tokens ascending within an
// expert, define the permuted row order:
//   kept[e], offsets[e] = sum_{e' < e} kept[e'] (offsets[N] = M),
//   perm_token[row] = token of that row (rows >= M are -1),
//   inv_map[t*k + j] = row of pair (t, S_t[j]), or -1 if dropped.
int orc_dispatch(const OrcShape* s, const int32_t* topk_idx, int32_t* kept, int32_t* offsets,
                 int32_t* perm_token, int32_t* inv_map, int64_t* n_dropped) {
  if (!shape_ok_tc(s) || !topk_idx) return -1;
  const int64_t T = s->T, N = s->n_experts, k = s->top_k;
  const int64_t C = s->capacity;
  std::vector<std::vector<std::pair<int64_t, int64_t>>> lists(static_cast<size_t>(N));
  for (int64_t t = 0; t < T; ++t)
    for (int64_t j = 0; j < k; ++j) {
      const int64_t e = topk_idx[t * k + j];
      if (e < 0 || e >= N) return -1;
      lists[e].push_back({t, j});
    }
  int64_t row = 0, dropped = 0;
  for (int64_t i = 0; i < T * k; ++i) {
    if (inv_map) inv_map[i] = -1;
    if (perm_token) perm_token[i] = -1;
  }
  for (int64_t e = 0; e < N; ++e) {
    const int64_t cnt = static_cast<int64_t>(lists[e].size());
    const int64_t keep = (C < 0) ? cnt : std::min(cnt, C);
    if (offsets) offsets[e] = static_cast<int32_t>(row);
    if (kept) kept[e] = static_cast<int32_t>(keep);
    for (int64_t r = 0; r < keep; ++r) {
      const auto& pr = lists[e][r];
      if (perm_token) perm_token[row] = static_cast<int32_t>(pr.first);
      if (inv_map) inv_map[pr.first * k + pr.second] = static_cast<int32_t>(row);
      ++row;
    }
    dropped += cnt - keep;
  }
  if (offsets) offsets[N] = static_cast<int32_t>(row);
  if (n_dropped) *n_dropped = dropped;
  return 0;
}

// Expert e (or shared expert e when `shared` != 0) applied to n rows given in
// the activation dtype: Y[r] = E_e(X[r]), fp64 output.
int orc_expert_rows(const OrcShape* s, const OrcWeights* w, int shared, int e, const void* X,
                    int64_t n, double* Y) {
  if (!shape_ok(s) || !w || !X || !Y) return -1;
  if (shared ? (e < 0 || e >= s->n_shared) : (e < 0 || e >= s->n_experts)) return -1;
  std::vector<double> Xd(static_cast<size_t>(n * s->d));
  for (int64_t i = 0; i < n * s->d; ++i) Xd[i] = elem(X, s->act_dtype, i, 1.0);
  expert_rows(s, w, shared != 0, e, Xd.data(), n, Y);
  return 0;
}

// Layer output for the tokens listed in `tokens` (n_tok of them), following
// the per-expert masked loop of [AIG `MoE` module] and the weighted sum
// y = sum_{i in top-k} g_i E_i(x) [AIG equation; SPX "Key Equations"], plus
// the always-on shared experts [SPX "Shared + Specialized"; MOEA "Shared vs
// Specialized Experts"]:
//   y_t = sum_{j : inv_map[t][j] >= 0} g[t][j] * E_{S_t[j]}(x_t) + sum_s E^sh_s(x_t)
// Dropped pairs (inv_map < 0) add nothing; the gates are not renormalised
// after drops. topk_idx, topk_w and inv_map cover all T tokens.
int orc_moe_output(const OrcShape* s, const void* x, const OrcWeights* w, const int32_t* topk_idx,
                   const double* topk_w, const int32_t* inv_map, const int64_t* tokens,
                   int64_t n_tok, double* y) {
  if (!shape_ok_tc(s) || !x || !w || !topk_idx || !topk_w || !tokens || !y) return -1;
  const int64_t d = s->d, k = s->top_k, N = s->n_experts;
  for (int64_t i = 0; i < n_tok * d; ++i) y[i] = 0.0;
  for (int64_t e = 0; e < N; ++e) {
    // mask: the listed tokens whose kept selection includes e
    std::vector<int64_t> which;   // position in `tokens`
    std::vector<double> gate;
    for (int64_t i = 0; i < n_tok; ++i) {
      const int64_t t = tokens[i];
      for (int64_t j = 0; j < k; ++j)
        if (topk_idx[t * k + j] == e && (!inv_map || inv_map[t * k + j] >= 0)) {
          which.push_back(i);
          gate.push_back(topk_w[t * k + j]);
        }
    }
    if (which.empty()) continue;
    const int64_t n = static_cast<int64_t>(which.size());
    std::vector<double> X(static_cast<size_t>(n * d)), Y(static_cast<size_t>(n * d));
    for (int64_t r = 0; r < n; ++r)
      for (int64_t c = 0; c < d; ++c) X[r * d + c] = elem(x, s->act_dtype, tokens[which[r]] * d + c, 1.0);
    expert_rows(s, w, false, static_cast<int>(e), X.data(), n, Y.data());
    for (int64_t r = 0; r < n; ++r)
      for (int64_t c = 0; c < d; ++c) y[which[r] * d + c] += gate[r] * Y[r * d + c];
  }
  if (s->n_shared > 0) {
    std::vector<double> X(static_cast<size_t>(n_tok * d)), Y(static_cast<size_t>(n_tok * d));
    for (int64_t r = 0; r < n_tok; ++r)
      for (int64_t c = 0; c < d; ++c) X[r * d + c] = elem(x, s->act_dtype, tokens[r] * d + c, 1.0);
    for (int sh = 0; sh < s->n_shared; ++sh) {
      expert_rows(s, w, true, sh, X.data(), n_tok, Y.data());
      for (int64_t i = 0; i < n_tok * d; ++i) y[i] += Y[i];
    }
  }
  return 0;
}

// Combine alone [AIG `MoE` module, out[index] += w * expert(x[index])]: given
// permuted expert outputs y_perm [M][d] (activation dtype), the pair -> row map
// and the gates, y_t = sum_{j : inv_map >= 0} g[t][j] * y_perm[inv_map[t][j]]
// (+ sum_s y_shared[s][t] when y_shared is given, [S][T][d] activation dtype).
int orc_combine(const OrcShape* s, const void* y_perm, const int32_t* inv_map, const float* topk_w,
                const void* y_shared, double* y) {
  if (!shape_ok_tc(s) || !y_perm || !inv_map || !topk_w || !y) return -1;
  const int64_t T = s->T, d = s->d, k = s->top_k;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int64_t j = 0; j < k; ++j) {
        const int64_t row = inv_map[t * k + j];
        if (row >= 0) acc += static_cast<double>(topk_w[t * k + j]) * elem(y_perm, s->act_dtype, row * d + c, 1.0);
      }
      if (y_shared)
        for (int64_t sh = 0; sh < s->n_shared; ++sh)
          acc += elem(y_shared, s->act_dtype, (sh * T + t) * d + c, 1.0);
      y[t * d + c] = acc;
    }
  }
  return 0;
}

// ---------------------------------------------------------------- expert choice
// [MOEA "Router Design", Expert-Choice Router and the router comparison table;
// AIG, the variants paragraph; chipfoundryservices glossary, "Expert Choice
// Routing"; SPX routing-variants table]. Every expert picks its own tokens:
//   probs[t][e] = exp(l[t][e] - m_e) / sum_t' exp(l[t'][e] - m_e), m_e = max_t l[t][e]
//                 (softmax over the TOKENS of column e)
//   expert e takes the C tokens with the largest probs[:, e] (exact ties to the
//   lower token index), C = capacity (0 <= C <= T), and lists them in
//   ascending token order; the gate of (t, e) is probs[t][e].
// A token may be taken by any number of experts, none included.
// Shape contract: gating 3, top_k 1, 0 <= capacity <= T.

// Selection and gates from fp32 logits [T][N]:
//   ec_token [N][C] the tokens of expert e, ascending; ec_gate [N][C] their
//   probs[t][e]; probs [T][N] (optional) the whole column softmax; lse [T]
//   (optional) and z / lse_sq_mean: the router's per-token logsumexp over the
//   experts, the same z statistics as token choice [SPX z_loss].
int orc_route_ec(const OrcShape* s, const float* logits, int32_t* ec_token, double* ec_gate, double* probs,
                 double* lse_out, double* z, double* lse_sq_mean) {
  if (!shape_ok_ec(s) || !logits || (s->capacity > 0 && (!ec_token || !ec_gate))) return -1;
  const int64_t T = s->T, N = s->n_experts, C = s->capacity;
  std::vector<double> p(static_cast<size_t>(T * N));
  for (int64_t e = 0; e < N; ++e) {
    double m = -std::numeric_limits<double>::infinity();
    for (int64_t t = 0; t < T; ++t) m = std::max(m, static_cast<double>(logits[t * N + e]));
    double sum = 0.0;
    for (int64_t t = 0; t < T; ++t) sum += std::exp(static_cast<double>(logits[t * N + e]) - m);
    for (int64_t t = 0; t < T; ++t) p[t * N + e] = std::exp(static_cast<double>(logits[t * N + e]) - m) / sum;

    // top-C of the column: tokens ordered by probability, descending; the
    // stable sort keeps ascending token order among equal probabilities
    std::vector<int64_t> order(static_cast<size_t>(T));
    for (int64_t t = 0; t < T; ++t) order[t] = t;
    std::stable_sort(order.begin(), order.end(),
                     [&](int64_t a, int64_t b) { return p[a * N + e] > p[b * N + e]; });
    std::vector<int64_t> pick(order.begin(), order.begin() + C);
    std::sort(pick.begin(), pick.end());
    for (int64_t j = 0; j < C; ++j) {
      ec_token[e * C + j] = static_cast<int32_t>(pick[j]);
      ec_gate[e * C + j] = p[pick[j] * N + e];
    }
  }
  if (probs) std::memcpy(probs, p.data(), sizeof(double) * static_cast<size_t>(T * N));
  double lse_sum = 0.0, lse_sq = 0.0;
  for (int64_t t = 0; t < T; ++t) {
    double m = -std::numeric_limits<double>::infinity();
    for (int64_t e = 0; e < N; ++e) m = std::max(m, static_cast<double>(logits[t * N + e]));
    double sum = 0.0;
    for (int64_t e = 0; e < N; ++e) sum += std::exp(static_cast<double>(logits[t * N + e]) - m);
    const double l = m + std::log(sum);
    if (lse_out) lse_out[t] = l;
    lse_sum += l;
    lse_sq += l * l;
  }
  const double lm = (T > 0) ? lse_sum / static_cast<double>(T) : 0.0;
  if (z) *z = lm * lm;
  if (lse_sq_mean) *lse_sq_mean = (T > 0) ? lse_sq / static_cast<double>(T) : 0.0;
  return 0;
}

// Row layout of the expert-choice assignments: expert e's j-th token sits in
// row e*C + j, so offsets[e] = e*C, perm_token[e*C + j] = ec_token[e][j],
// inv_map[t][e] = the row of (t, e) or -1, and n_untouched = the number of
// tokens no expert took. ec_token rows must be ascending and within [0, T).
int orc_dispatch_ec(const OrcShape* s, const int32_t* ec_token, int32_t* offsets, int32_t* perm_token,
                    int32_t* inv_map, int64_t* n_untouched) {
  if (!shape_ok_ec(s) || (s->capacity > 0 && !ec_token)) return -1;
  const int64_t T = s->T, N = s->n_experts, C = s->capacity;
  if (inv_map)
    for (int64_t i = 0; i < T * N; ++i) inv_map[i] = -1;
  std::vector<int32_t> taken(static_cast<size_t>(T), 0);
  for (int64_t e = 0; e < N; ++e) {
    if (offsets) offsets[e] = static_cast<int32_t>(e * C);
    for (int64_t j = 0; j < C; ++j) {
      const int64_t t = ec_token[e * C + j];
      if (t < 0 || t >= T || (j > 0 && t <= ec_token[e * C + j - 1])) return -1;
      if (perm_token) perm_token[e * C + j] = static_cast<int32_t>(t);
      if (inv_map) inv_map[t * N + e] = static_cast<int32_t>(e * C + j);
      taken[t] = 1;
    }
  }
  if (offsets) offsets[N] = static_cast<int32_t>(N * C);
  if (n_untouched) {
    int64_t n = 0;
    for (int64_t t = 0; t < T; ++t) n += taken[t] ? 0 : 1;
    *n_untouched = n;
  }
  return 0;
}

// Layer output of the listed tokens under expert choice: each expert runs on
// the tokens it took and adds gate * output into them, then the shared experts
// [SPX "Shared + Specialized"]:
//   y_t = sum_{e : t in ec_token[e]} probs[t][e] E_e(x_t) + sum_s E^sh_s(x_t)
int orc_moe_output_ec(const OrcShape* s, const void* x, const OrcWeights* w, const int32_t* ec_token,
                      const double* ec_gate, const int64_t* tokens, int64_t n_tok, double* y) {
  if (!shape_ok_ec(s) || !x || !w || !tokens || !y || (s->capacity > 0 && (!ec_token || !ec_gate))) return -1;
  const int64_t d = s->d, N = s->n_experts, C = s->capacity;
  for (int64_t i = 0; i < n_tok * d; ++i) y[i] = 0.0;
  for (int64_t e = 0; e < N; ++e) {
    std::vector<int64_t> which;  // position in `tokens`
    std::vector<double> gate;
    for (int64_t i = 0; i < n_tok; ++i)
      for (int64_t j = 0; j < C; ++j)
        if (ec_token[e * C + j] == tokens[i]) {
          which.push_back(i);
          gate.push_back(ec_gate[e * C + j]);
        }
    if (which.empty()) continue;
    const int64_t n = static_cast<int64_t>(which.size());
    std::vector<double> X(static_cast<size_t>(n * d)), Y(static_cast<size_t>(n * d));
    for (int64_t r = 0; r < n; ++r)
      for (int64_t c = 0; c < d; ++c) X[r * d + c] = elem(x, s->act_dtype, tokens[which[r]] * d + c, 1.0);
    expert_rows(s, w, false, static_cast<int>(e), X.data(), n, Y.data());
    for (int64_t r = 0; r < n; ++r)
      for (int64_t c = 0; c < d; ++c) y[which[r] * d + c] += gate[r] * Y[r * d + c];
  }
  if (s->n_shared > 0) {
    std::vector<double> X(static_cast<size_t>(n_tok * d)), Y(static_cast<size_t>(n_tok * d));
    for (int64_t r = 0; r < n_tok; ++r)
      for (int64_t c = 0; c < d; ++c) X[r * d + c] = elem(x, s->act_dtype, tokens[r] * d + c, 1.0);
    for (int sh = 0; sh < s->n_shared; ++sh) {
      expert_rows(s, w, true, sh, X.data(), n_tok, Y.data());
      for (int64_t i = 0; i < n_tok * d; ++i) y[i] += Y[i];
    }
  }
  return 0;
}

// Combine alone under expert choice: y_t = sum over experts e ascending with
// inv_map[t][e] >= 0 of gate_row[r] * y_perm[r], r = inv_map[t][e] (gates
// indexed by row, [N*C] fp32), plus the shared outputs when given.
int orc_combine_ec(const OrcShape* s, const void* y_perm, const int32_t* inv_map, const float* gate_row,
                   const void* y_shared, double* y) {
  if (!shape_ok_ec(s) || !y_perm || !inv_map || !gate_row || !y) return -1;
  const int64_t T = s->T, d = s->d, N = s->n_experts;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int64_t e = 0; e < N; ++e) {
        const int64_t row = inv_map[t * N + e];
        if (row >= 0) acc += static_cast<double>(gate_row[row]) * elem(y_perm, s->act_dtype, row * d + c, 1.0);
      }
      if (y_shared)
        for (int64_t sh = 0; sh < s->n_shared; ++sh)
          acc += elem(y_shared, s->act_dtype, (sh * T + t) * d + c, 1.0);
      y[t * d + c] = acc;
    }
  }
  return 0;
}

// ---------------------------------------------------------------- backward
// Gradients of the token-choice layer [AIG y/g equation, `MoE` module and L_aux
// equation; SPX "Key Equations", "Load Balancing (Critical)" z_loss; MOEA
// "Expert Network Design"], for the scalar
//   loss = sum_t <dy_t, y_t> + c_aux * L_aux + c_z * z
// (dy is the gradient arriving at the layer output). The routing decision
// (which experts, which pairs the capacity keeps) is held fixed and the fp32
// rounding of the logits passes gradients through unchanged; everything else
// is differentiated exactly in fp64:
//  combine   dY_e[r] = g * dy_t for kept pair (t, j -> e, row r); dg_tj = <dy_t, E_e(x_t)>;
//            shared experts: dY = dy
//  expert    dH = dY W2;  dW2 += dY^T H;  db2 += sum dY
//            SwiGLU: dU = dH * V * silu'(U), dV = dH * silu(U); GELU: dU = dH * gelu'(U)
//            dW1 += dU^T X;  dW3 += dV^T X;  db1 += sum dU;  dx += dU W1 (+ dV W3)
//  gates     mode 0: dp_S += dg;  mode 1: g = p_S / s -> dp_S += (dg - <dg, g>) / s;
//            mode 2: dl_S += g * (dg - <dg, g>)
//  L_aux     f is a count (no gradient); P_e = mean_t p_te -> dp_te += c_aux alpha N f_e / T
//  z         z = (mean_t lse_t)^2 -> dl_te += c_z 2 mean(lse) / T * p_te
//  softmax   dl += p * (dp - <dp, p>)
//  router    dW_r += dl^T x;  db_r += sum_t dl;  dx += dl W_r
// Outputs (fp64, any may be null except dx): dx [T][d], dWr [N][d], dbr [N],
// dW1 / dW3 [N][d_ff][d], dW2 [N][d][d_ff], db1 [N][d_ff], db2 [N][d], and the
// shared experts' dsW1 / dsW3 [S][d_ff][d], dsW2 [S][d][d_ff].
int orc_backward(const OrcShape* s, const void* x, const OrcWeights* w, const void* dy, double c_aux, double c_z,
                 double* dx, double* dWr, double* dbr, double* dW1, double* dW3, double* dW2, double* db1,
                 double* db2, double* dsW1, double* dsW3, double* dsW2) {
  if (!shape_ok_tc(s) || !x || !w || !w->w_router || !dy || !dx) return -1;
  if (s->w_dtype >= 2) return -1;  // gradients of fp32 / bf16 weights only
  const int64_t T = s->T, d = s->d, f = s->d_ff, N = s->n_experts, k = s->top_k, S = s->n_shared;
  const bool swi = (s->act == 1);

  // forward decisions and values
  std::vector<double> l64(static_cast<size_t>(T * N));
  std::vector<float> l32(static_cast<size_t>(T * N));
  orc_router_logits(s, x, w, l64.data(), l32.data());
  std::vector<int32_t> idx(static_cast<size_t>(T * k));
  std::vector<double> gate(static_cast<size_t>(T * k)), p(static_cast<size_t>(T * N)), lse(static_cast<size_t>(T));
  std::vector<int64_t> counts(static_cast<size_t>(N));
  orc_route(s, l32.data(), idx.data(), gate.data(), p.data(), lse.data(), nullptr, nullptr, counts.data(), nullptr,
            nullptr, nullptr, nullptr, nullptr);
  std::vector<int32_t> inv(static_cast<size_t>(T * k));
  orc_dispatch(s, idx.data(), nullptr, nullptr, nullptr, inv.data(), nullptr);

  for (int64_t i = 0; i < T * d; ++i) dx[i] = 0.0;
  std::vector<double> dg(static_cast<size_t>(T * k), 0.0);
  auto zero = [](double* a, int64_t n) { if (a) for (int64_t i = 0; i < n; ++i) a[i] = 0.0; };
  zero(dWr, N * d); zero(dbr, N); zero(dW1, N * f * d); zero(dW3, N * f * d); zero(dW2, N * d * f);
  zero(db1, N * f); zero(db2, N * d); zero(dsW1, S * f * d); zero(dsW3, S * f * d); zero(dsW2, S * d * f);

  // one expert over rows X [n][d] with output gradients dY [n][d]: parameter
  // gradients into gW1/gW3/gW2/gb1/gb2 (may be null), input gradients into dX,
  // and the expert's outputs into Yout (may be null)
  auto expert_bwd = [&](bool shared, int e, const std::vector<double>& X, const std::vector<double>& dY, int64_t n,
                        double* gW1, double* gW3, double* gW2, double* gb1, double* gb2, std::vector<double>& dX) {
    const void* W1 = shared ? w->sw1 : w->w1;
    const void* W3 = shared ? w->sw3 : w->w3;
    const void* W2 = shared ? w->sw2 : w->w2;
    const float* b1 = shared ? nullptr : w->b1;
    const int64_t base1 = static_cast<int64_t>(e) * f * d, base2 = static_cast<int64_t>(e) * d * f;
    auto w1 = [&](int64_t i, int64_t j) { return elem(W1, s->w_dtype, base1 + i * d + j, 1.0); };
    auto w3 = [&](int64_t i, int64_t j) { return elem(W3, s->w_dtype, base1 + i * d + j, 1.0); };
    auto w2 = [&](int64_t o, int64_t i) { return elem(W2, s->w_dtype, base2 + o * f + i, 1.0); };
    std::vector<double> U(static_cast<size_t>(n * f)), V(static_cast<size_t>(n * f)), H(static_cast<size_t>(n * f));
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < f; ++i)
      for (int64_t r = 0; r < n; ++r) {
        double u = 0.0, v = 0.0;
        for (int64_t j = 0; j < d; ++j) {
          u += w1(i, j) * X[r * d + j];
          if (swi) v += w3(i, j) * X[r * d + j];
        }
        if (!swi && b1) u += static_cast<double>(b1[static_cast<int64_t>(e) * f + i]);
        U[r * f + i] = u;
        V[r * f + i] = v;
        H[r * f + i] = swi ? silu(u) * v : gelu(u);
      }
    // dH = dY W2, dW2 += dY^T H, db2 += sum dY
    std::vector<double> dH(static_cast<size_t>(n * f), 0.0);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < f; ++i)
      for (int64_t r = 0; r < n; ++r) {
        double a = 0.0;
        for (int64_t o = 0; o < d; ++o) a += dY[r * d + o] * w2(o, i);
        dH[r * f + i] = a;
      }
    if (gW2)
#pragma omp parallel for schedule(static)
      for (int64_t o = 0; o < d; ++o)
        for (int64_t i = 0; i < f; ++i) {
          double a = 0.0;
          for (int64_t r = 0; r < n; ++r) a += dY[r * d + o] * H[r * f + i];
          gW2[base2 + o * f + i] += a;
        }
    if (gb2)
      for (int64_t o = 0; o < d; ++o)
        for (int64_t r = 0; r < n; ++r) gb2[static_cast<int64_t>(e) * d + o] += dY[r * d + o];
    // activation backward
    std::vector<double> dU(static_cast<size_t>(n * f)), dV(static_cast<size_t>(n * f), 0.0);
    for (int64_t q = 0; q < n * f; ++q) {
      const double u = U[q];
      if (swi) {
        const double sg = 1.0 / (1.0 + std::exp(-u));
        dU[q] = dH[q] * V[q] * (sg + u * sg * (1.0 - sg));
        dV[q] = dH[q] * u * sg;
      } else {
        const double cdf = 0.5 * (1.0 + std::erf(u / std::sqrt(2.0)));
        const double pdf = std::exp(-0.5 * u * u) / std::sqrt(2.0 * 3.14159265358979323846);
        dU[q] = dH[q] * (cdf + u * pdf);
      }
    }
    // dW1 += dU^T X, dW3 += dV^T X, db1 += sum dU, dX = dU W1 (+ dV W3)
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < f; ++i)
      for (int64_t j = 0; j < d; ++j) {
        double a = 0.0, c = 0.0;
        for (int64_t r = 0; r < n; ++r) {
          a += dU[r * f + i] * X[r * d + j];
          if (swi) c += dV[r * f + i] * X[r * d + j];
        }
        if (gW1) gW1[base1 + i * d + j] += a;
        if (swi && gW3) gW3[base1 + i * d + j] += c;
      }
    if (gb1 && !swi)
      for (int64_t i = 0; i < f; ++i)
        for (int64_t r = 0; r < n; ++r) gb1[static_cast<int64_t>(e) * f + i] += dU[r * f + i];
    dX.assign(static_cast<size_t>(n * d), 0.0);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r)
      for (int64_t j = 0; j < d; ++j) {
        double a = 0.0;
        for (int64_t i = 0; i < f; ++i) {
          a += dU[r * f + i] * w1(i, j);
          if (swi) a += dV[r * f + i] * w3(i, j);
        }
        dX[r * d + j] = a;
      }
  };

  // routed experts: rows are the kept pairs of expert e in ascending token order
  for (int64_t e = 0; e < N; ++e) {
    std::vector<int64_t> tok, slot;
    for (int64_t t = 0; t < T; ++t)
      for (int64_t j = 0; j < k; ++j)
        if (idx[t * k + j] == e && inv[t * k + j] >= 0) {
          tok.push_back(t);
          slot.push_back(t * k + j);
        }
    const int64_t n = static_cast<int64_t>(tok.size());
    if (n == 0) continue;
    std::vector<double> X(static_cast<size_t>(n * d)), dY(static_cast<size_t>(n * d)), Y(static_cast<size_t>(n * d));
    for (int64_t r = 0; r < n; ++r)
      for (int64_t c = 0; c < d; ++c) {
        X[r * d + c] = elem(x, s->act_dtype, tok[r] * d + c, 1.0);
        dY[r * d + c] = gate[slot[r]] * elem(dy, s->act_dtype, tok[r] * d + c, 1.0);
      }
    expert_rows(s, w, false, static_cast<int>(e), X.data(), n, Y.data());
    for (int64_t r = 0; r < n; ++r) {
      double a = 0.0;
      for (int64_t c = 0; c < d; ++c) a += elem(dy, s->act_dtype, tok[r] * d + c, 1.0) * Y[r * d + c];
      dg[slot[r]] = a;
    }
    std::vector<double> dX;
    expert_bwd(false, static_cast<int>(e), X, dY, n, dW1, dW3, dW2, db1, db2, dX);
    for (int64_t r = 0; r < n; ++r)
      for (int64_t c = 0; c < d; ++c) dx[tok[r] * d + c] += dX[r * d + c];
  }
  // shared experts: every token, output gradient dy
  if (S > 0) {
    std::vector<double> X(static_cast<size_t>(T * d)), dY(static_cast<size_t>(T * d));
    for (int64_t i = 0; i < T * d; ++i) {
      X[i] = elem(x, s->act_dtype, i, 1.0);
      dY[i] = elem(dy, s->act_dtype, i, 1.0);
    }
    for (int sh = 0; sh < S; ++sh) {
      std::vector<double> dX;
      expert_bwd(true, sh, X, dY, T, dsW1, dsW3, dsW2, nullptr, nullptr, dX);
      for (int64_t i = 0; i < T * d; ++i) dx[i] += dX[i];
    }
  }

  // router: gates, L_aux and z to the logits, then to W_r, b_r and x
  std::vector<double> dl(static_cast<size_t>(T * N), 0.0);
  double lm = 0.0;
  for (int64_t t = 0; t < T; ++t) lm += lse[t];
  lm = (T > 0) ? lm / static_cast<double>(T) : 0.0;
  for (int64_t t = 0; t < T; ++t) {
    std::vector<double> dp(static_cast<size_t>(N), 0.0);
    const int32_t* St = idx.data() + t * k;
    const double* g = gate.data() + t * k;
    const double* dgt = dg.data() + t * k;
    double* dlt = dl.data() + t * N;
    const double* pt = p.data() + t * N;
    if (s->gating == 0) {
      for (int64_t j = 0; j < k; ++j) dp[St[j]] += dgt[j];
    } else if (s->gating == 1) {
      double ssum = 0.0, dot = 0.0;
      for (int64_t j = 0; j < k; ++j) { ssum += pt[St[j]]; dot += dgt[j] * g[j]; }
      for (int64_t j = 0; j < k; ++j) dp[St[j]] += (dgt[j] - dot) / ssum;
    } else {
      double dot = 0.0;
      for (int64_t j = 0; j < k; ++j) dot += dgt[j] * g[j];
      for (int64_t j = 0; j < k; ++j) dlt[St[j]] += g[j] * (dgt[j] - dot);
    }
    for (int64_t e = 0; e < N; ++e)
      dp[e] += c_aux * s->aux_alpha * static_cast<double>(N) * (static_cast<double>(counts[e]) /
                                                               static_cast<double>(T * k)) / static_cast<double>(T);
    double dpp = 0.0;
    for (int64_t e = 0; e < N; ++e) dpp += dp[e] * pt[e];
    for (int64_t e = 0; e < N; ++e) {
      dlt[e] += pt[e] * (dp[e] - dpp);
      dlt[e] += c_z * 2.0 * lm / static_cast<double>(T) * pt[e];
    }
  }
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t)
    for (int64_t c = 0; c < d; ++c) {
      double a = 0.0;
      for (int64_t e = 0; e < N; ++e) a += dl[t * N + e] * elem(w->w_router, s->act_dtype, e * d + c, 1.0);
      dx[t * d + c] += a;
    }
  if (dWr)
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < N; ++e)
      for (int64_t c = 0; c < d; ++c) {
        double a = 0.0;
        for (int64_t t = 0; t < T; ++t) a += dl[t * N + e] * elem(x, s->act_dtype, t * d + c, 1.0);
        dWr[e * d + c] = a;
      }
  if (dbr)
    for (int64_t e = 0; e < N; ++e) {
      double a = 0.0;
      for (int64_t t = 0; t < T; ++t) a += dl[t * N + e];
      dbr[e] = a;
    }
  return 0;
}

// Parts of the same gradients, for layers whose whole backward is too slow
// here: dx for the listed tokens, and for each listed (expert e, hidden unit i)
// pair, row i of dW1[e] and of dW3[e] (SwiGLU) and column i of dW2[e]. Each
// value follows orc_backward's definitions term by term; only the rows and
// units that these outputs need are formed. The router, the statistics and
// the capacity cut still run over all T tokens.
// tokens [n_tok] in [0, T); units [n_units][2] = (e, i), e in [0, N), i in
// [0, d_ff). Outputs: dx_rows [n_tok][d], dW1_rows / dW3_rows [n_units][d]
// (dW3_rows may be null), dW2_cols [n_units][d].
int orc_backward_sampled(const OrcShape* s, const void* x, const OrcWeights* w, const void* dy, double c_aux,
                         double c_z, const int32_t* tokens, int64_t n_tok, double* dx_rows, const int32_t* units,
                         int64_t n_units, double* dW1_rows, double* dW3_rows, double* dW2_cols) {
  if (!shape_ok_tc(s) || !x || !w || !w->w_router || !dy) return -1;
  if (s->w_dtype >= 2) return -1;
  const int64_t T = s->T, d = s->d, f = s->d_ff, N = s->n_experts, k = s->top_k, S = s->n_shared;
  const bool swi = (s->act == 1);
  if (n_tok > 0 && (!tokens || !dx_rows)) return -1;
  if (n_units > 0 && (!units || !dW1_rows || !dW2_cols)) return -1;
  for (int64_t a = 0; a < n_tok; ++a)
    if (tokens[a] < 0 || tokens[a] >= T) return -1;
  for (int64_t b = 0; b < n_units; ++b)
    if (units[2 * b] < 0 || units[2 * b] >= N || units[2 * b + 1] < 0 || units[2 * b + 1] >= f) return -1;

  std::vector<double> l64(static_cast<size_t>(T * N));
  std::vector<float> l32(static_cast<size_t>(T * N));
  orc_router_logits(s, x, w, l64.data(), l32.data());
  std::vector<int32_t> idx(static_cast<size_t>(T * k));
  std::vector<double> gate(static_cast<size_t>(T * k)), p(static_cast<size_t>(T * N)), lse(static_cast<size_t>(T));
  std::vector<int64_t> counts(static_cast<size_t>(N));
  orc_route(s, l32.data(), idx.data(), gate.data(), p.data(), lse.data(), nullptr, nullptr, counts.data(), nullptr,
            nullptr, nullptr, nullptr, nullptr);
  std::vector<int32_t> inv(static_cast<size_t>(T * k));
  orc_dispatch(s, idx.data(), nullptr, nullptr, nullptr, inv.data(), nullptr);
  double lm = 0.0;
  for (int64_t t = 0; t < T; ++t) lm += lse[t];
  lm = (T > 0) ? lm / static_cast<double>(T) : 0.0;

  auto xv = [&](int64_t t, int64_t c) { return elem(x, s->act_dtype, t * d + c, 1.0); };
  auto dyv = [&](int64_t t, int64_t c) { return elem(dy, s->act_dtype, t * d + c, 1.0); };
  auto W1 = [&](bool sh, int64_t e, int64_t i, int64_t j) {
    return elem(sh ? w->sw1 : w->w1, s->w_dtype, (e * f + i) * d + j, 1.0);
  };
  auto W3 = [&](bool sh, int64_t e, int64_t i, int64_t j) {
    return elem(sh ? w->sw3 : w->w3, s->w_dtype, (e * f + i) * d + j, 1.0);
  };
  auto W2 = [&](bool sh, int64_t e, int64_t o, int64_t i) {
    return elem(sh ? w->sw2 : w->w2, s->w_dtype, (e * d + o) * f + i, 1.0);
  };

  // dx of one token: its kept pairs, the shared experts, the router
  for (int64_t a = 0; a < n_tok; ++a) {
    const int64_t t = tokens[a];
    double* out = dx_rows + a * d;
    for (int64_t c = 0; c < d; ++c) out[c] = 0.0;
    std::vector<double> dg(static_cast<size_t>(k), 0.0);
    std::vector<double> U(f), V(f), H(f), Y(d), dY(d), dH(f), dU(f), dV(f), dX(d);
    auto expert = [&](bool sh, int64_t e, double g, double* dg_out) {
      const float* b1 = (!sh && !swi) ? w->b1 : nullptr;
      const float* b2 = (!sh && !swi) ? w->b2 : nullptr;
#pragma omp parallel for schedule(static)
      for (int64_t i = 0; i < f; ++i) {
        double u = 0.0, v = 0.0;
        for (int64_t j = 0; j < d; ++j) {
          u += W1(sh, e, i, j) * xv(t, j);
          if (swi) v += W3(sh, e, i, j) * xv(t, j);
        }
        if (b1) u += static_cast<double>(b1[e * f + i]);
        U[i] = u;
        V[i] = v;
        H[i] = swi ? silu(u) * v : gelu(u);
      }
      if (dg_out) {  // the expert's output, for the gate's gradient
#pragma omp parallel for schedule(static)
        for (int64_t o = 0; o < d; ++o) {
          double yo = 0.0;
          for (int64_t i = 0; i < f; ++i) yo += W2(sh, e, o, i) * H[i];
          if (b2) yo += static_cast<double>(b2[e * d + o]);
          Y[o] = yo;
        }
        double acc = 0.0;
        for (int64_t o = 0; o < d; ++o) acc += dyv(t, o) * Y[o];
        *dg_out = acc;
      }
      for (int64_t o = 0; o < d; ++o) dY[o] = g * dyv(t, o);
#pragma omp parallel for schedule(static)
      for (int64_t i = 0; i < f; ++i) {
        double h = 0.0;
        for (int64_t o = 0; o < d; ++o) h += dY[o] * W2(sh, e, o, i);
        const double u = U[i];
        if (swi) {
          const double sg = 1.0 / (1.0 + std::exp(-u));
          dU[i] = h * V[i] * (sg + u * sg * (1.0 - sg));
          dV[i] = h * u * sg;
        } else {
          const double cdf = 0.5 * (1.0 + std::erf(u / std::sqrt(2.0)));
          const double pdf = std::exp(-0.5 * u * u) / std::sqrt(2.0 * 3.14159265358979323846);
          dU[i] = h * (cdf + u * pdf);
          dV[i] = 0.0;
        }
      }
#pragma omp parallel for schedule(static)
      for (int64_t j = 0; j < d; ++j) {
        double acc = 0.0;
        for (int64_t i = 0; i < f; ++i) {
          acc += dU[i] * W1(sh, e, i, j);
          if (swi) acc += dV[i] * W3(sh, e, i, j);
        }
        dX[j] = acc;
      }
      for (int64_t j = 0; j < d; ++j) out[j] += dX[j];
    };
    for (int64_t j = 0; j < k; ++j)
      if (inv[t * k + j] >= 0) expert(false, idx[t * k + j], gate[t * k + j], &dg[j]);
    for (int64_t sh = 0; sh < S; ++sh) expert(true, sh, 1.0, nullptr);
    // router: the same chain as orc_backward for this token's row of dl
    std::vector<double> dp(static_cast<size_t>(N), 0.0), dl(static_cast<size_t>(N), 0.0);
    const int32_t* St = idx.data() + t * k;
    const double* g = gate.data() + t * k;
    const double* pt = p.data() + t * N;
    if (s->gating == 0) {
      for (int64_t j = 0; j < k; ++j) dp[St[j]] += dg[j];
    } else if (s->gating == 1) {
      double ssum = 0.0, dot = 0.0;
      for (int64_t j = 0; j < k; ++j) { ssum += pt[St[j]]; dot += dg[j] * g[j]; }
      for (int64_t j = 0; j < k; ++j) dp[St[j]] += (dg[j] - dot) / ssum;
    } else {
      double dot = 0.0;
      for (int64_t j = 0; j < k; ++j) dot += dg[j] * g[j];
      for (int64_t j = 0; j < k; ++j) dl[St[j]] += g[j] * (dg[j] - dot);
    }
    for (int64_t e = 0; e < N; ++e)
      dp[e] += c_aux * s->aux_alpha * static_cast<double>(N) * (static_cast<double>(counts[e]) /
                                                               static_cast<double>(T * k)) / static_cast<double>(T);
    double dpp = 0.0;
    for (int64_t e = 0; e < N; ++e) dpp += dp[e] * pt[e];
    for (int64_t e = 0; e < N; ++e) dl[e] += pt[e] * (dp[e] - dpp) + c_z * 2.0 * lm / static_cast<double>(T) * pt[e];
    for (int64_t c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int64_t e = 0; e < N; ++e) acc += dl[e] * elem(w->w_router, s->act_dtype, e * d + c, 1.0);
      out[c] += acc;
    }
  }

  // one hidden unit i of expert e over the expert's kept rows (ascending tokens)
  for (int64_t b = 0; b < n_units; ++b) {
    const int64_t e = units[2 * b], i = units[2 * b + 1];
    std::vector<int64_t> tok;
    std::vector<double> gr;
    for (int64_t t = 0; t < T; ++t)
      for (int64_t j = 0; j < k; ++j)
        if (idx[t * k + j] == e && inv[t * k + j] >= 0) {
          tok.push_back(t);
          gr.push_back(gate[t * k + j]);
        }
    const int64_t n = static_cast<int64_t>(tok.size());
    std::vector<double> H(n), dU(n), dV(n);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
      const int64_t t = tok[r];
      double u = 0.0, v = 0.0, h = 0.0;
      for (int64_t j = 0; j < d; ++j) {
        u += W1(false, e, i, j) * xv(t, j);
        if (swi) v += W3(false, e, i, j) * xv(t, j);
      }
      if (!swi && w->b1) u += static_cast<double>(w->b1[e * f + i]);
      for (int64_t o = 0; o < d; ++o) h += gr[r] * dyv(t, o) * W2(false, e, o, i);
      H[r] = swi ? silu(u) * v : gelu(u);
      if (swi) {
        const double sg = 1.0 / (1.0 + std::exp(-u));
        dU[r] = h * v * (sg + u * sg * (1.0 - sg));
        dV[r] = h * u * sg;
      } else {
        const double cdf = 0.5 * (1.0 + std::erf(u / std::sqrt(2.0)));
        const double pdf = std::exp(-0.5 * u * u) / std::sqrt(2.0 * 3.14159265358979323846);
        dU[r] = h * (cdf + u * pdf);
        dV[r] = 0.0;
      }
    }
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < d; ++c) {
      double a1 = 0.0, a3 = 0.0, a2 = 0.0;
      for (int64_t r = 0; r < n; ++r) {
        a1 += dU[r] * xv(tok[r], c);
        a3 += dV[r] * xv(tok[r], c);
        a2 += gr[r] * dyv(tok[r], c) * H[r];
      }
      dW1_rows[b * d + c] = a1;
      if (dW3_rows) dW3_rows[b * d + c] = swi ? a3 : 0.0;
      dW2_cols[b * d + c] = a2;
    }
  }
  return 0;
}

// Exact decoders, exported so that tests can pin them to library conversions.
double orc_bf16_value(uint16_t b) { return bf16_value(b); }
double orc_e4m3_value(uint8_t q) { return e4m3_value(q); }
double orc_gelu(double u) { return gelu(u); }
double orc_silu(double u) { return silu(u); }

}  // extern "C"
