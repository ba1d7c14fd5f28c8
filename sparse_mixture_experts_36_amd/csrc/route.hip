// Router: logits GEMM (k-split partial logits), then softmax / top-k / gates
// with per-block statistics, and a one-workgroup finalize of f, P, L_aux and z
// (done by the routing workgroup itself when one covers all tokens).
//
// Pages: aigrafen.se "Mixture of Experts" (g = softmax(W_r x); L_aux =
// alpha N sum f_i P_i; the `MoE` module's softmax -> top-k -> renormalise),
// vanos001 "MoE Architecture" / "Router Design" (top-k of the logits, softmax
// over the k), learn.starphix.com "Mixture of Experts (MoE)" / "Load Balancing
// (Critical)" (load_balancing_loss, z_loss).
//
// Layout on the GPU: a workgroup owns 64 consecutive tokens. In the router
// GEMM each of its four waves computes 16 tokens x N logits on MFMA; the
// routing workgroup has 16 waves, and quarter-wave q of wave w (lanes
// 16q..16q+15) owns token 4w + q, lane l%16 holding experts 16*nt + l%16. Every
// per-token step (max, sum, top-k) is then a 16-lane reduction inside one
// quarter. Reductions run in a fixed order, so the result is bit-for-bit
// reproducible.
#include <float.h>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kRK = 64;            // k-step of the router GEMM
constexpr int kWStride = kRK + 8;  // padded LDS row (bf16 elements): 144 B spreads the banks
constexpr int kMaxN = 256;

struct Sel {
  float v;
  int e;
};

// (v, e) total order: larger value first, lower expert index on exact ties.
__device__ __forceinline__ bool better(float v, int e, float v2, int e2) {
  return v > v2 || (v == v2 && e < e2);
}

// Router GEMM over one k range: partial logits of 64 tokens (4 waves x 16) for
// all experts. Grid (token blocks, k splits). bf16 runs on MFMA with the
// router-weight tile for all experts in LDS (double buffered); the next
// k-step's tile and token fragments are loaded while the current one computes.
template <int NT>
__global__ __launch_bounds__(kThreads) void router_gemm_kernel(RouteArgs a, float* part, int k_len) {
  __shared__ __attribute__((aligned(16))) uint16_t wtile[2][NT * 16 * kWStride];
  constexpr int WCH = (NT * 16 * (kRK / 8) + kThreads - 1) / kThreads;  // 16-byte weight chunks per thread
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, c16 = lane & 15;
  const int N = a.N;
  const int64_t T = a.T, d = a.d;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kRouteTokens + wave * 16;
  const int64_t k0 = static_cast<int64_t>(blockIdx.y) * k_len;
  float* out = part + static_cast<int64_t>(blockIdx.y) * T * N;

  floatx4_t acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  if (a.act_dtype == 1) {
    // Lane (row c16, k-group q) takes 16 consecutive k of its token row per step.
    const uint16_t* xr = static_cast<const uint16_t*>(a.x);
    const uint16_t* wr = static_cast<const uint16_t*>(a.w_router);
    int64_t trow = t0 + c16;
    if (trow > T - 1) trow = T - 1;  // rows past T compute garbage that is never stored
    const uint16_t* xrow = xr + trow * d + k0 + q * 16;
    const int nsteps = k_len / kRK;
    uint4 wv[WCH];
    auto wload = [&](int step) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < WCH; ++i) {
        const int c = tid + i * kThreads;
        const int e = c >> 3, kc = c & 7;
        wv[i] = make_uint4(0, 0, 0, 0);
        if (c < NT * 16 * 8 && e < N) wv[i] = *reinterpret_cast<const uint4*>(wr + e * d + k0 + step * kRK + kc * 8);
      }
    };
    auto wstore = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < WCH; ++i) {
        const int c = tid + i * kThreads;
        const int e = c >> 3, kc = c & 7;
        if (c < NT * 16 * 8) *reinterpret_cast<uint4*>(&wtile[buf][e * kWStride + kc * 8]) = wv[i];
      }
    };
    wload(0);
    uint4 x0 = *reinterpret_cast<const uint4*>(xrow);
    uint4 x1 = *reinterpret_cast<const uint4*>(xrow + 8);
    wstore(0);
    __syncthreads();
    for (int st = 0; st < nsteps; ++st) {
      const int nx = (st + 1 < nsteps) ? st + 1 : st;  // the last step re-reads itself into the idle buffer
      wload(nx);
      const uint4 y0 = *reinterpret_cast<const uint4*>(xrow + nx * kRK);
      const uint4 y1 = *reinterpret_cast<const uint4*>(xrow + nx * kRK + 8);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const uint16_t* wp = &wtile[st & 1][(16 * nt + c16) * kWStride + q * 16];
        const uint4 b0 = *reinterpret_cast<const uint4*>(wp);
        const uint4 b1 = *reinterpret_cast<const uint4*>(wp + 8);
        acc[nt] = mfma16x16x32(x0, b0, acc[nt]);
        acc[nt] = mfma16x16x32(x1, b1, acc[nt]);
      }
      wstore((st + 1) & 1);
      x0 = y0;
      x1 = y1;
      __syncthreads();
    }
  } else {
    // fp32: plain dot products straight into the same layout.
    const float* xr = static_cast<const float*>(a.x);
    const float* wr = static_cast<const float*>(a.w_router);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int e = 16 * nt + c16;
      if (e >= N) continue;
      const float4* w4 = reinterpret_cast<const float4*>(wr + e * d + k0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int64_t t = t0 + 4 * q + i;
        if (t > T - 1) t = T - 1;
        const float4* x4 = reinterpret_cast<const float4*>(xr + t * d + k0);
        float s = 0.f;
        for (int64_t j = 0; j < k_len / 4; ++j) {
          const float4 u = x4[j], w = w4[j];
          s = fmaf(u.x, w.x, s);
          s = fmaf(u.y, w.y, s);
          s = fmaf(u.z, w.z, s);
          s = fmaf(u.w, w.w, s);
        }
        acc[nt][i] = s;
      }
    }
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int e = 16 * nt + c16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t t = t0 + 4 * q + i;
      if (t < T && e < N) out[t * N + e] = acc[nt][i];
    }
  }
}

// Statistics from totals (fp64): counts, f = counts/(T k), P = sum/T, and
// the f P products for L_aux.
__device__ __forceinline__ void finalize_expert(const RouteArgs& a, int e, double p_sum, int64_t c, double* s_fp) {
  const double T = static_cast<double>(a.T);
  const double P = p_sum / T;
  const double f = static_cast<double>(c) / (T * a.k);
  if (a.counts) a.counts[e] = static_cast<int32_t>(c);
  if (a.f) a.f[e] = static_cast<float>(f);
  if (a.P) a.P[e] = static_cast<float>(P);
  s_fp[e] = f * P;
}

// L_aux = alpha N sum_e f P (summed in expert order), z = mean(lse)^2.
__device__ __forceinline__ void finalize_scalars(const RouteArgs& a, const double* s_fp, double lse_sum,
                                                 double lse_sq_sum) {
  const double T = static_cast<double>(a.T);
  double dot = 0.0;
  if (!a.ec)
    for (int e = 0; e < a.N; ++e) dot += s_fp[e];
  const double lm = lse_sum / T;
  if (a.l_aux && !a.ec) *a.l_aux = static_cast<float>(static_cast<double>(a.aux_alpha) * a.N * dot);
  if (a.z_loss) *a.z_loss = static_cast<float>(lm * lm);
  if (a.lse_mean) *a.lse_mean = static_cast<float>(lm);
  if (a.lse_sq_mean) *a.lse_sq_mean = static_cast<float>(lse_sq_sum / T);
}

// Logits of token t for experts 16 nt + c16: the given ones, or the sum of
// the k-split partial logits (in split order) plus the router bias, which is
// then also stored as the router output (and, for expert choice, into the
// column-major copy).
template <int NT>
__device__ __forceinline__ void token_logits(const RouteArgs& a, const float* part, int splits, int64_t t,
                                             bool live, int c16, float (&lg)[NT]) {
  const int N = a.N;
  const int64_t T = a.T;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int e = 16 * nt + c16;
    float v = 0.f;
    if (live && e < N) {
      if (a.logits_given) {
        v = a.logits[t * N + e];
      } else {
        // all split partials are loaded before the first add (one round
        // trip, not one per split), then summed in split order
        float pv[kMaxRouteSplits];
#pragma unroll
        for (int sp = 0; sp < kMaxRouteSplits; ++sp)
          if (sp < splits) pv[sp] = part[(static_cast<int64_t>(sp) * T + t) * N + e];
        v = pv[0];
#pragma unroll
        for (int sp = 1; sp < kMaxRouteSplits; ++sp)
          if (sp < splits) v += pv[sp];
        if (a.b_router) v += a.b_router[e];
        a.logits[t * N + e] = v;
      }
      if (a.ec) a.logits_t[e * a.ld_lt + t] = v;
    }
    lg[nt] = v;
  }
}

// Softmax / top-k / gates / block statistics over 64 tokens, one per
// quarter-wave (16 waves): lane (q, c16) of wave w holds the logits of token
// 4w + q for experts 16 nt + c16, so every per-token step is a 16-lane
// reduction and no wave walks tokens one after another. Logits are the given
// ones, or the sum of the k-split partial logits (in split order) plus the
// router bias, which is then also stored as the router output. A launch of one
// workgroup (T <= 64) also finishes the statistics itself.
constexpr int kRouteWaves = kRouteTokens / 4;
constexpr int kRouteThreads = 64 * kRouteWaves;

template <int NT>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(RouteArgs a, const float* part, int splits) {
  __shared__ int32_t s_cnt[kMaxN];
  __shared__ float s_P[kRouteWaves][kMaxN];
  __shared__ float s_lse[kRouteWaves][2];
  __shared__ double s_fp[kMaxN];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, c16 = lane & 15;
  const int N = a.N, k = a.k;
  const int64_t T = a.T;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kRouteTokens + wave * 4 + q;
  const bool live = t < T;  // uniform within the quarter

  for (int e = tid; e < kMaxN; e += kRouteThreads) s_cnt[e] = 0;

  float lg[NT];  // logit of expert 16 nt + c16
  token_logits<NT>(a, part, splits, t, live, c16, lg);
  __syncthreads();  // s_cnt cleared before any count below

  // selection: k rounds of a 16-lane arg-max under `better`
  uint32_t taken = 0;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
    if (16 * nt + c16 >= N) taken |= 1u << nt;
  float selv[8];
  int sele[8];
  for (int j = 0; j < k; ++j) {
    Sel b{-FLT_MAX, 0x7fffffff};
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int e = 16 * nt + c16;
      if (!(taken >> nt & 1u) && (b.e == 0x7fffffff || better(lg[nt], e, b.v, b.e))) {
        b.v = lg[nt];
        b.e = e;
      }
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) {
      const float v2 = __shfl_xor(b.v, o, 16);
      const int e2 = __shfl_xor(b.e, o, 16);
      if (e2 != 0x7fffffff && (b.e == 0x7fffffff || better(v2, e2, b.v, b.e))) {
        b.v = v2;
        b.e = e2;
      }
    }
    selv[j] = b.v;
    sele[j] = b.e;
    if ((b.e & 15) == c16) taken |= 1u << (b.e >> 4);
  }
  // softmax over all N: the largest logit is the first selected one
  const float m = selv[0];
  float s = 0.f;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
    if (16 * nt + c16 < N) s += expf(lg[nt] - m);
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) s += __shfl_xor(s, o, 16);
  const float inv_s = 1.0f / s;
  const float lse = m + logf(s);
  float pacc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) pacc[nt] = (live && 16 * nt + c16 < N) ? expf(lg[nt] - m) * inv_s : 0.f;
  const float lse_s = live ? lse : 0.f, lse_sq = live ? lse * lse : 0.f;
  if (live) {
    float g[8];
    if (a.gating == 0) {
      for (int j = 0; j < k; ++j) g[j] = expf(selv[j] - m) * inv_s;
    } else if (a.gating == 1) {
      float den = 0.f;
      for (int j = 0; j < k; ++j) {
        g[j] = expf(selv[j] - m) * inv_s;
        den += g[j];
      }
      for (int j = 0; j < k; ++j) g[j] = g[j] / den;
    } else {
      float den = 0.f;
      for (int j = 0; j < k; ++j) {
        g[j] = expf(selv[j] - m);
        den += g[j];
      }
      for (int j = 0; j < k; ++j) g[j] = g[j] / den;
    }
    for (int j = 0; j < k; ++j)
      if (c16 == j) {
        a.topk_idx[t * k + j] = sele[j];
        a.topk_w[t * k + j] = g[j];
        atomicAdd(&s_cnt[sele[j]], 1);
      }
  }

  // ---- block totals, fixed order: the wave's four tokens (xor 16, 32), then waves in order
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float v = pacc[nt];
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    if (q == 0) s_P[wave][16 * nt + c16] = v;
  }
  {
    const float a1 = __shfl(lse_s, 0) + __shfl(lse_s, 16) + __shfl(lse_s, 32) + __shfl(lse_s, 48);
    const float a2 = __shfl(lse_sq, 0) + __shfl(lse_sq, 16) + __shfl(lse_sq, 32) + __shfl(lse_sq, 48);
    if (lane == 0) {
      s_lse[wave][0] = a1;
      s_lse[wave][1] = a2;
    }
  }
  __syncthreads();
  const int b = blockIdx.x;
  const bool last = gridDim.x == 1;  // the only block: its totals are the layer's
  for (int e = tid; e < N; e += kRouteThreads) {
    float P = s_P[0][e];
#pragma unroll
    for (int w = 1; w < kRouteWaves; ++w) P += s_P[w][e];
    if (last) {
      finalize_expert(a, e, static_cast<double>(P), s_cnt[e], s_fp);
    } else {
      a.part_P[static_cast<int64_t>(b) * N + e] = P;
      a.part_cnt[static_cast<int64_t>(b) * N + e] = s_cnt[e];
    }
  }
  float l1 = s_lse[0][0], l2 = s_lse[0][1];
#pragma unroll
  for (int w = 1; w < kRouteWaves; ++w) {
    l1 += s_lse[w][0];
    l2 += s_lse[w][1];
  }
  if (last) {
    __syncthreads();  // every f P product is in s_fp
    if (tid == 0) finalize_scalars(a, s_fp, static_cast<double>(l1), static_cast<double>(l2));
  } else if (tid == 0) {
    a.part_lse[2 * b] = l1;
    a.part_lse[2 * b + 1] = l2;
  }
}

// One workgroup of 1024 threads: sums the block partials (fp64) and writes
// counts, f = counts/(T k), P = sum/T, L_aux = alpha N sum f P, z = mean(lse)^2.
// Expert e's nb partials are cut into S contiguous segments, one thread each
// (S <= 1024 / NP, NP the power of two >= N, and at least 16 blocks a segment);
// a segment is summed in block order with 16 loads in flight, then the
// segments in order. The lse sums run the same way over up to 64 lanes of
// wave 0. Every order is fixed.
constexpr int kFinThreads = 1024;
constexpr int kFinBatch = 16;

__global__ __launch_bounds__(kFinThreads) void route_finalize_kernel(RouteArgs a, int nb) {
  __shared__ double s_fp[kMaxN];
  __shared__ double s_segp[kFinThreads];
  __shared__ int64_t s_segc[kFinThreads];
  __shared__ double s_lse[2][64];
  const int tid = threadIdx.x;
  const int N = a.N;
  int NP = 1;
  while (NP < N) NP <<= 1;
  // at least one full batch of loads per segment
  const int S = min(kFinThreads / NP, max(1, (nb + kFinBatch - 1) / kFinBatch));
  const int e = tid % NP, seg = tid / NP;
  if (!a.ec && e < N && seg < S) {
    const int b0 = static_cast<int>((static_cast<int64_t>(seg) * nb) / S);
    const int b1 = static_cast<int>((static_cast<int64_t>(seg + 1) * nb) / S);
    double p = 0.0;
    int64_t c = 0;
    for (int b = b0; b < b1; b += kFinBatch) {
      float vp[kFinBatch];
      int32_t vc[kFinBatch];
#pragma unroll
      for (int i = 0; i < kFinBatch; ++i)
        if (b + i < b1) {
          vp[i] = a.part_P[static_cast<int64_t>(b + i) * N + e];
          vc[i] = a.part_cnt[static_cast<int64_t>(b + i) * N + e];
        }
#pragma unroll
      for (int i = 0; i < kFinBatch; ++i)
        if (b + i < b1) {
          p += static_cast<double>(vp[i]);
          c += vc[i];
        }
    }
    s_segp[tid] = p;
    s_segc[tid] = c;
  }
  const int SL = min(64, max(1, (nb + kFinBatch - 1) / kFinBatch));  // lse segments
  if (tid < SL) {  // lse: lane L takes blocks [L nb / SL, (L + 1) nb / SL)
    const int b0 = (tid * nb) / SL, b1 = ((tid + 1) * nb) / SL;
    double ls = 0.0, lq = 0.0;
    for (int b = b0; b < b1; b += kFinBatch) {
      float v1[kFinBatch], v2[kFinBatch];
#pragma unroll
      for (int i = 0; i < kFinBatch; ++i)
        if (b + i < b1) {
          v1[i] = a.part_lse[2 * (b + i)];
          v2[i] = a.part_lse[2 * (b + i) + 1];
        }
#pragma unroll
      for (int i = 0; i < kFinBatch; ++i)
        if (b + i < b1) {
          ls += static_cast<double>(v1[i]);
          lq += static_cast<double>(v2[i]);
        }
    }
    s_lse[0][tid] = ls;
    s_lse[1][tid] = lq;
  }
  __syncthreads();
  if (!a.ec && tid < N) {
    double p = 0.0;
    int64_t c = 0;
    for (int sg = 0; sg < S; ++sg) {
      p += s_segp[sg * NP + tid];
      c += s_segc[sg * NP + tid];
    }
    finalize_expert(a, tid, p, c, s_fp);
  }
  __syncthreads();
  if (tid == 0) {
    double ls = 0.0, lq = 0.0;
    for (int l = 0; l < SL; ++l) {
      ls += s_lse[0][l];
      lq += s_lse[1][l];
    }
    finalize_scalars(a, s_fp, ls, lq);
  }
}

// ---------------------------------------------------------------- expert choice
// vanos001 "MoE Architecture" / "Router Design", Expert-Choice Router: the
// softmax runs over the tokens of each expert's column and every expert takes
// the C tokens of largest probability. Ranking by that probability is ranking
// by the logit (the column softmax is strictly increasing), so the selection
// compares fp32 logits; exact ties go to the lower token index.

// Per-token pass: logits (and their column-major copy), the logsumexp over the
// experts for the z statistics; no per-token selection.
template <int NT>
__global__ __launch_bounds__(kRouteThreads) void route_ec_kernel(RouteArgs a, const float* part, int splits) {
  __shared__ float s_lse[kRouteWaves][2];
  __shared__ double s_fp[1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, c16 = lane & 15;
  const int N = a.N;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kRouteTokens + wave * 4 + q;
  const bool live = t < a.T;
  float lg[NT];
  token_logits<NT>(a, part, splits, t, live, c16, lg);
  float m = -FLT_MAX;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
    if (16 * nt + c16 < N) m = fmaxf(m, lg[nt]);
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 16));
  float s = 0.f;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
    if (16 * nt + c16 < N) s += expf(lg[nt] - m);
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) s += __shfl_xor(s, o, 16);
  const float lse = m + logf(s);
  const float lse_s = live ? lse : 0.f, lse_sq = live ? lse * lse : 0.f;
  {
    const float a1 = __shfl(lse_s, 0) + __shfl(lse_s, 16) + __shfl(lse_s, 32) + __shfl(lse_s, 48);
    const float a2 = __shfl(lse_sq, 0) + __shfl(lse_sq, 16) + __shfl(lse_sq, 32) + __shfl(lse_sq, 48);
    if (lane == 0) {
      s_lse[wave][0] = a1;
      s_lse[wave][1] = a2;
    }
  }
  __syncthreads();
  if (tid == 0) {
    float l1 = s_lse[0][0], l2 = s_lse[0][1];
    for (int w = 1; w < kRouteWaves; ++w) {
      l1 += s_lse[w][0];
      l2 += s_lse[w][1];
    }
    if (gridDim.x == 1) {
      finalize_scalars(a, s_fp, static_cast<double>(l1), static_cast<double>(l2));
    } else {
      a.part_lse[2 * blockIdx.x] = l1;
      a.part_lse[2 * blockIdx.x + 1] = l2;
    }
  }
}

constexpr int kEcThreads = 1024;
constexpr int kEcWaves = kEcThreads / 64;

// Order-preserving key of an fp32 value (larger value, larger key); -0 and +0
// share one key, as they compare equal.
__device__ __forceinline__ uint32_t ec_key(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The fp32 value of a key (-0 comes back as +0).
__device__ __forceinline__ float ec_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Exclusive prefix sum over the workgroup in thread order; `total` gets the
// sum of all. s_w holds one value per wave.
__device__ __forceinline__ uint32_t ec_scan(uint32_t v, uint32_t* s_w, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_w[wave] = x;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kEcWaves; ++w) {
    const uint32_t c = s_w[w];
    if (w < wave) base += c;
    tot += c;
  }
  __syncthreads();
  total = tot;
  return base + x - v;
}

// One workgroup per expert e; thread i holds tokens [CH i, CH i + CH) of the
// column (T <= 1024 CH). Column softmax: max, then the sum of exp (fp64,
// fixed order). Selection: a most-significant-digit radix select (4 passes of
// 8 bits over the order-preserving keys, per-wave histograms) finds the C-th
// largest key K and how many keys equal to K are taken; the tokens above K and
// the first of those equal to K in token order are kept. Two prefix sums in
// token order give each kept token its row e*C + j, so the list comes out in
// ascending token order. Every order is fixed: the output is reproducible.
template <int CH>
__global__ __launch_bounds__(kEcThreads) void ec_select_kernel(RouteArgs a) {
  __shared__ uint32_t s_hist[kEcWaves][256];
  __shared__ uint32_t s_w[kEcWaves];
  __shared__ float s_m[kEcWaves];
  __shared__ double s_s[kEcWaves];
  __shared__ uint32_t s_pick[2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int e = blockIdx.x;
  const int64_t T = a.T;
  const int C = static_cast<int>(a.cap);
  if (tid == 0 && a.counts) a.counts[e] = C;
  if (C == 0) return;
  const float* col = a.logits_t + static_cast<int64_t>(e) * a.ld_lt;
  const int t0 = tid * CH;
  uint32_t key[CH];  // the values are kept only as their keys (a bijection)
#pragma unroll
  for (int j = 0; j < CH; j += 4) {
    float4 q = make_float4(0.f, 0.f, 0.f, 0.f);
    if (t0 + j < T) q = *reinterpret_cast<const float4*>(col + t0 + j);  // ld_lt: a multiple of 4 >= T
    key[j] = ec_key(q.x);
    key[j + 1] = ec_key(q.y);
    key[j + 2] = ec_key(q.z);
    key[j + 3] = ec_key(q.w);
  }
  int nv = static_cast<int>(T) - t0;  // valid tokens of this thread
  nv = nv < 0 ? 0 : (nv > CH ? CH : nv);

  // column softmax denominators
  float m = -FLT_MAX;
#pragma unroll
  for (int i = 0; i < CH; ++i)
    if (i < nv) m = fmaxf(m, ec_value(key[i]));
  m = wave_max(m);
  if (lane == 0) s_m[wave] = m;
  __syncthreads();
  m = s_m[0];
#pragma unroll
  for (int w = 1; w < kEcWaves; ++w) m = fmaxf(m, s_m[w]);
  double S = 0.0;
#pragma unroll
  for (int i = 0; i < CH; ++i)
    if (i < nv) S += static_cast<double>(expf(ec_value(key[i]) - m));
  S = wave_sum(S);
  if (lane == 0) s_s[wave] = S;

  // radix select of the C-th largest key
  uint32_t prefix = 0, pmask = 0, rem = static_cast<uint32_t>(C);
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < kEcWaves * 256; i += kEcThreads) (&s_hist[0][0])[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < CH; ++i)
      if (i < nv && (key[i] & pmask) == prefix) atomicAdd(&s_hist[wave][(key[i] >> shift) & 255u], 1u);
    __syncthreads();
    if (wave == 0) {
      // lane l owns bins 255 - 4l - j, j < 4: lanes in ascending order walk the bins downward
      uint32_t c[4], loc = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int b = 255 - 4 * lane - j;
        uint32_t sum = 0;
#pragma unroll
        for (int w = 0; w < kEcWaves; ++w) sum += s_hist[w][b];
        c[j] = sum;
        loc += sum;
      }
      uint32_t inc = loc;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(inc, o);
        if (lane >= o) inc += y;
      }
      const uint32_t exc = inc - loc;
      if (exc < rem && rem <= inc) {
        uint32_t acc = exc;
        int pick = 0;
        uint32_t left = 0;
        bool found = false;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (!found && acc + c[j] >= rem) {
            pick = 255 - 4 * lane - j;
            left = rem - acc;
            found = true;
          }
          acc += c[j];
        }
        s_pick[0] = static_cast<uint32_t>(pick);
        s_pick[1] = left;
      }
    }
    __syncthreads();
    prefix |= s_pick[0] << shift;
    pmask |= 0xFFu << shift;
    rem = s_pick[1];
  }
  // prefix = K, rem = how many keys equal to K are taken (lowest tokens first)
  S = 0.0;
#pragma unroll
  for (int w = 0; w < kEcWaves; ++w) S += s_s[w];

  uint32_t neq = 0;
#pragma unroll
  for (int i = 0; i < CH; ++i)
    if (i < nv && key[i] == prefix) ++neq;
  uint32_t total;
  uint32_t eqr = ec_scan(neq, s_w, total);
  uint32_t sel = 0, nsel = 0;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    bool take = false;
    if (i < nv) {
      if (key[i] > prefix) {
        take = true;
      } else if (key[i] == prefix) {
        take = eqr < rem;
        ++eqr;
      }
    }
    if (take) {
      sel |= 1u << i;
      ++nsel;
    }
  }
  uint32_t pos = ec_scan(nsel, s_w, total);
  int32_t* tok = a.topk_idx + static_cast<int64_t>(e) * C;
  float* gate = a.topk_w + static_cast<int64_t>(e) * C;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    if ((sel >> i & 1u) && pos < static_cast<uint32_t>(C)) {
      tok[pos] = t0 + i;
      gate[pos] = static_cast<float>(static_cast<double>(expf(ec_value(key[i]) - m)) / S);
      ++pos;
    }
  }
}

template <int CH>
hipError_t launch_ec_select(const RouteArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(ec_select_kernel<CH>, dim3(a.N), dim3(kEcThreads), 0, s, a);
  return hipGetLastError();
}

template <int NT>
hipError_t launch_nt(const RouteArgs& a, int nb, int splits, hipStream_t s) {
  if (!a.logits_given) {
    hipLaunchKernelGGL(router_gemm_kernel<NT>, dim3(nb, splits), dim3(kThreads), 0, s, a, a.part_logits,
                       static_cast<int>(a.d / splits));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.ec)
    hipLaunchKernelGGL(route_ec_kernel<NT>, dim3(nb), dim3(kRouteThreads), 0, s, a, a.part_logits, splits);
  else
    hipLaunchKernelGGL(route_kernel<NT>, dim3(nb), dim3(kRouteThreads), 0, s, a, a.part_logits, splits);
  return hipGetLastError();
}

}  // namespace

int route_splits(int64_t T, int64_t d) {
  const int64_t nb = ceil_div(T, kRouteTokens), steps = d / kRK;
  int s = 1;
  while (nb * s < 256 && s < kMaxRouteSplits && steps % (2 * s) == 0 && steps / (2 * s) >= 4) s *= 2;
  return s;
}

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  const int nb = static_cast<int>(ceil_div(a.T, kRouteTokens));
  const int nt = static_cast<int>(ceil_div(a.N, 16));
  const int splits = a.logits_given ? 1 : route_splits(a.T, a.d);
  hipError_t err;
  stage_mark(kStageRoute, false, s);
  switch (nt) {
#define MOE_ROUTE_CASE(n) \
  case n: err = launch_nt<n>(a, nb, splits, s); break;
    MOE_ROUTE_CASE(1) MOE_ROUTE_CASE(2) MOE_ROUTE_CASE(3) MOE_ROUTE_CASE(4)
    MOE_ROUTE_CASE(5) MOE_ROUTE_CASE(6) MOE_ROUTE_CASE(7) MOE_ROUTE_CASE(8)
    MOE_ROUTE_CASE(9) MOE_ROUTE_CASE(10) MOE_ROUTE_CASE(11) MOE_ROUTE_CASE(12)
    MOE_ROUTE_CASE(13) MOE_ROUTE_CASE(14) MOE_ROUTE_CASE(15) MOE_ROUTE_CASE(16)
#undef MOE_ROUTE_CASE
    default: return hipErrorInvalidValue;
  }
  if (err != hipSuccess) return err;
  if (nb > 1) hipLaunchKernelGGL(route_finalize_kernel, dim3(1), dim3(kFinThreads), 0, s, a, nb);
  if (a.ec) {
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (a.T > kEcMaxTokens) return hipErrorInvalidValue;
    if (a.T <= 4 * kEcThreads) err = launch_ec_select<4>(a, s);
    else if (a.T <= 8 * kEcThreads) err = launch_ec_select<8>(a, s);
    else if (a.T <= 16 * kEcThreads) err = launch_ec_select<16>(a, s);
    else err = launch_ec_select<32>(a, s);
    if (err != hipSuccess) return err;
  }
  stage_mark(kStageRoute, true, s);
  return hipGetLastError();
}

}  // namespace moe
