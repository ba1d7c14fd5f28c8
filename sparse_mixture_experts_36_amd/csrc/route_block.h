// Routing of one token block (softmax, top-k, gates, statistics), shared by
// the routing kernel and the fused decode front end.
//
// Pages: aigrafen.se "Mixture of Experts" (g = softmax(W_r x); L_aux =
// alpha N sum f_i P_i; the `MoE` module's softmax -> top-k -> renormalise),
// vanos001 "MoE Architecture" / "Router Design" (top-k of the logits, softmax
// over the k), learn.starphix.com "Mixture of Experts (MoE)" / "Load Balancing
// (Critical)" (load_balancing_loss, z_loss).
#pragma once

#include <float.h>

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kRouteMaxN = 256;
constexpr int kRouteWaves = kRouteTokens / 4;
constexpr int kRouteThreads = 64 * kRouteWaves;

struct Sel {
  float v;
  int e;
};

// (v, e) total order: larger value first, lower expert index on exact ties.
__device__ __forceinline__ bool better(float v, int e, float v2, int e2) {
  return v > v2 || (v == v2 && e < e2);
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

// The routing of one token, held by the 16 lanes of a quarter-wave: lane
// c16 holds the logits lg[nt] of experts 16 nt + c16. Top-k selection (k
// rounds of a 16-lane arg-max under `better`), softmax over all N (the largest
// logit is the first selected one), gates in the call's gating mode. When
// live, the token's top-k list and gates are stored (topk_row: an LDS copy of
// the list, or null). Every lane of the quarter returns the selected experts;
// pacc[nt] is its experts' probability (0 when not live), lse the token's
// log-sum-exp (0 when not live).
template <int NT>
__device__ __forceinline__ void route_token(const RouteArgs& a, int64_t t, bool live, const float (&lg)[NT], int c16,
                                            int32_t* topk_row, int (&sele)[8], float (&pacc)[NT], float& lse_out) {
  const int N = a.N, k = a.k;
  uint32_t taken = 0;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
    if (16 * nt + c16 >= N) taken |= 1u << nt;
  float selv[8];
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
    // 16-lane arg-max by DPP exchanges (the order of the pairs does not
    // change the result: `better` is a total order)
    auto merge = [&](float v2, int e2) __attribute__((always_inline)) {
      if (e2 != 0x7fffffff && (b.e == 0x7fffffff || better(v2, e2, b.v, b.e))) {
        b.v = v2;
        b.e = e2;
      }
    };
    merge(dpp_row16<0>(b.v), dpp_row16<0>(b.e));
    merge(dpp_row16<1>(b.v), dpp_row16<1>(b.e));
    merge(dpp_row16<2>(b.v), dpp_row16<2>(b.e));
    merge(dpp_row16<3>(b.v), dpp_row16<3>(b.e));
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
  s = row16_sum(s);
  const float inv_s = 1.0f / s;
  const float lse = m + logf(s);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) pacc[nt] = (live && 16 * nt + c16 < N) ? expf(lg[nt] - m) * inv_s : 0.f;
  lse_out = live ? lse : 0.f;
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
        if (topk_row) topk_row[j] = sele[j];
        a.topk_w[t * k + j] = g[j];
      }
  }
}

// Softmax / top-k / gates / block statistics over 64 tokens, one per
// quarter-wave (16 waves): lane (q, c16) of wave w holds the logits of token
// 4w + q for experts 16 nt + c16, so every per-token step is a 16-lane
// reduction and no wave walks tokens one after another. Logits are the given
// ones, or the sum of the k-split partial logits (in split order) plus the
// router bias, which is then also stored as the router output. A launch of one
// workgroup (T <= 64) also finishes the statistics itself.

// The routing of one block of kRouteTokens tokens, run by all kRouteThreads
// threads: token t of lane (q, c16) of wave w (t = the block's first token +
// 4 w + q) arrives with its logits lg[nt] of experts 16 nt + c16. Block b
// writes its statistics partials, or, when it is the only block (last), the
// final statistics.
// With topk_lds, the token's top-k list is also kept there ([t - first][k]).
template <int NT>
__device__ __forceinline__ void route_block(const RouteArgs& a, int64_t t, bool live, const float (&lg)[NT], int b,
                                            bool last, int32_t* topk_lds = nullptr) {
  __shared__ int32_t s_cnt[kRouteMaxN];
  __shared__ float s_P[kRouteWaves][kRouteMaxN];
  __shared__ float s_lse[kRouteWaves][2];
  __shared__ double s_fp[kRouteMaxN];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, c16 = lane & 15;
  (void)q;
  const int N = a.N, k = a.k;

  for (int e = tid; e < kRouteMaxN; e += kRouteThreads) s_cnt[e] = 0;
  __syncthreads();  // s_cnt cleared before any count below

  int sele[8];
  float pacc[NT], lse;
  route_token<NT>(a, t, live, lg, c16, topk_lds ? topk_lds + (t - static_cast<int64_t>(b) * kRouteTokens) * k : nullptr,
                  sele, pacc, lse);
  if (live)
    for (int j = 0; j < k; ++j)
      if (c16 == j) atomicAdd(&s_cnt[sele[j]], 1);
  const float lse_s = lse, lse_sq = lse * lse;

  // ---- block totals, fixed order: the wave's four tokens (xor 16, 32), then waves in order
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float v = pacc[nt];
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    if (q == 0) s_P[wave][16 * nt + c16] = v;
  }
  {
    auto at = [](float v, int l) __attribute__((always_inline)) {
      return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
    };
    const float a1 = at(lse_s, 0) + at(lse_s, 16) + at(lse_s, 32) + at(lse_s, 48);
    const float a2 = at(lse_sq, 0) + at(lse_sq, 16) + at(lse_sq, 32) + at(lse_sq, 48);
    if (lane == 0) {
      s_lse[wave][0] = a1;
      s_lse[wave][1] = a2;
    }
  }
  __syncthreads();
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

constexpr int kFinThreads = 1024;
constexpr int kFinBatch = 16;

// Run by one workgroup of kFinThreads threads: sums the block partials (fp64)
// and writes counts, f = counts/(T k), P = sum/T, L_aux = alpha N sum f P, z = mean(lse)^2.
// Expert e's nb partials are cut into S contiguous segments, one thread each
// (S <= 1024 / NP, NP the power of two >= N, and at least 16 blocks a segment);
// a segment is summed in block order with 16 loads in flight, then the
// segments in order. The lse sums run the same way over up to 64 lanes of
// wave 0. Every order is fixed.
__device__ __forceinline__ void route_finalize_block(const RouteArgs& a, int nb) {
  __shared__ double s_fp[kRouteMaxN];
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

}  // namespace moe
