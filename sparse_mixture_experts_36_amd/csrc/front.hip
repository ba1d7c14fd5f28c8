// Decode front end in one workgroup: the router GEMM, the routing (softmax,
// top-k, gates, statistics) and the permutation (rank, scan, slots and the
// FFN group plan) of a call with at most 16 tokens and 64 experts, in one
// launch where the general path takes three (router GEMM, routing,
// permutation), each with its own launch latency and global round trip.
//
// Pages: aigrafen.se "Mixture of Experts" (g = softmax(W_r x), the capacity
// equation and the `MoE` module's `nonzero`-order dispatch); vanos001 "MoE
// Architecture" / "Router Design" and "Capacity and Token Dropping";
// learn.starphix.com "Mixture of Experts (MoE)" / "Load Balancing (Critical)".
#include "common.h"
#include "kernels.h"
#include "perm_block.h"
#include "route_block.h"

namespace moe {
namespace {

constexpr int kFrontTokens = 16;  // tokens the front end takes (one MFMA row block)
constexpr int kFrontMaxNT = 4;    // 16-expert column blocks (64 experts)
constexpr int kFrontWaves = kRouteThreads / 64;
static_assert(kFrontWaves == 16, "the k range is cut in 16 wave slices");

// One token: after the router GEMM, wave 0 alone routes it and builds the
// permutation (the general blocks' barriers and block reductions are not
// needed for one token), then the workgroup writes the FFN group plan. The
// outputs are those of route_block and perm_rank_block for a block holding
// only token 0, computed the same way: the token's routing by route_token
// (its quarters all hold the same logits, so every lane ends with the same
// selection), statistics from the one token's probabilities and log-sum-exp,
// the offsets as an exclusive scan of the kept counts over the expert lanes.
template <int NT>
__device__ __forceinline__ void front_one(const RouteArgs& ra, const PermuteArgs& pa, const float* logit) {
  __shared__ int32_t s_off[kPermMaxN + 1];
  __shared__ double s_fp[16 * kFrontMaxNT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = ra.N, k = ra.k;
  if (wave == 0) {
    const int c16 = lane & 15;
    float lg[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) lg[nt] = logit[16 * nt + c16];
    int sele[8];
    float pacc[NT], lse;
    route_token<NT>(ra, 0, lane < 16, lg, c16, nullptr, sele, pacc, lse);
    // statistics: count, f and P of each expert, then L_aux and z (T = 1)
    if (lane < 16) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int e = 16 * nt + c16;
        if (e >= N) continue;
        int c = 0;
        for (int j = 0; j < k; ++j) c += sele[j] == e;
        finalize_expert(ra, e, static_cast<double>(pacc[nt]), c, s_fp);
      }
    }
    if (lane == 0) finalize_scalars(ra, s_fp, static_cast<double>(lse), static_cast<double>(lse * lse));
    // permutation: expert e on lane e (N <= 64), kept counts, their
    // exclusive scan, the token's slots
    int cnt = 0;
    for (int j = 0; j < k; ++j) cnt += sele[j] == lane;
    const int kept = (pa.capacity >= 0 && cnt > pa.capacity) ? static_cast<int>(pa.capacity) : cnt;
    if (lane < N) {
      pa.block_base[lane] = 0;
      pa.kept[lane] = kept;
    }
    int incl = kept;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (lane >= o) incl += v;
    }
    const int off = incl - kept;
    if (lane < N) {
      s_off[lane] = off;
      pa.offsets[lane] = off;
    }
    const int total = __shfl(incl, 63);
    int drop = cnt - kept;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) drop += __shfl_xor(drop, o);
    if (lane == 0) {
      s_off[N] = total;
      pa.offsets[N] = total;
      *pa.n_dropped = drop;
    }
    for (int j = 0; j < k; ++j) {
      const int row = __shfl(off, sele[j]);  // the token is its expert's first row
      if (lane == 0) {
        pa.local_rank[j] = 0;
        const int32_t slot = (pa.capacity < 0 || pa.capacity > 0) ? row : -1;
        pa.inv_map[j] = slot;
        if (slot >= 0) pa.perm_token[slot] = 0;
      }
    }
  }
  __syncthreads();  // the offsets are in LDS
  if (pa.plan.up) {
    __shared__ int32_t s_mt[2 * kMaxGroups];
    plan_groups(s_off, pa.plan, s_mt, tid, kRouteThreads);
  }
}

// Router GEMM: wave w takes k [w d/16, (w + 1) d/16) of every token and
// expert as MFMA 16x16x32 products (tokens as rows, clamped to T - 1; experts
// 16 nt + c16 as columns), with SB k-steps of loads in flight; the 16 wave
// partials are then summed in wave order (fixed, so the logits are
// reproducible bit for bit). Then the routing of the 16-token block and the
// one-block permutation, as in the general kernels (one token: front_one).
template <int NT>
__global__ __launch_bounds__(kRouteThreads) void front_kernel(RouteArgs ra, PermuteArgs pa) {
  __shared__ floatx4_t s_part[kFrontWaves][NT][64];
  __shared__ float s_logit[kFrontTokens][NT * 16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, c16 = lane & 15;
  const int N = ra.N;
  const int64_t T = ra.T, d = ra.d;

  const int64_t kw = d / kFrontWaves;  // a multiple of 32
  const int64_t kb = wave * kw;
  const int64_t trow = c16 < T ? c16 : T - 1;
  const uint16_t* xr = static_cast<const uint16_t*>(ra.x) + trow * d + kb + q * 8;
  const uint16_t* wr = static_cast<const uint16_t*>(ra.w_router) + kb + q * 8;
  floatx4_t acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  const int steps = static_cast<int>(kw / 32);
  constexpr int SB = NT == 1 ? 8 : NT == 2 ? 6 : 4;  // (NT + 1) SB 16-byte loads a lane in flight
  for (int s0 = 0; s0 < steps; s0 += SB) {
    uint4 xa[SB], wb[SB][NT];
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      if (s0 + u >= steps) break;
      xa[u] = *reinterpret_cast<const uint4*>(xr + (s0 + u) * 32);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int e = 16 * nt + c16;
        wb[u][nt] = e < N ? *reinterpret_cast<const uint4*>(wr + static_cast<int64_t>(e) * d + (s0 + u) * 32)
                          : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      if (s0 + u >= steps) break;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nt] = mfma16x16x32(xa[u], wb[u][nt], acc[nt]);
    }
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) s_part[wave][nt][lane] = acc[nt];
  __syncthreads();
  // lane l of a fragment holds tokens 4 (l / 16) + i, i < 4, of expert column l % 16
  if (tid < kFrontTokens * NT * 16) {
    const int t = tid / (NT * 16), e = tid % (NT * 16);
    const int nt = e / 16, l = 16 * (t / 4) + (e % 16), i = t % 4;
    float v = s_part[0][nt][l][i];
#pragma unroll
    for (int w = 1; w < kFrontWaves; ++w) v += s_part[w][nt][l][i];
    if (e < N) {
      if (ra.b_router) v += ra.b_router[e];
      if (t < T) ra.logits[static_cast<int64_t>(t) * N + e] = v;
    }
    s_logit[t][e] = v;
  }
  __syncthreads();
  if (T == 1) {
    front_one<NT>(ra, pa, s_logit[0]);
    return;
  }

  // routing: token 4 w + q in the lanes of quarter q of wave w (waves 0..3)
  const int64_t t = wave * 4 + q;
  const bool live = t < T;
  float lg[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) lg[nt] = live ? s_logit[t][16 * nt + c16] : 0.f;
  __shared__ int32_t s_topk[kFrontTokens * kPermMaxK];
  route_block<NT>(ra, t, live, lg, 0, true, s_topk);
  __syncthreads();  // this block's top-k lists are in LDS

  perm_rank_block<kRouteThreads, true>(pa, 0, 1, s_topk);
}

// One token: the router logits by dot products instead of MFMA tiles (a
// 16-row tile would carry 15 copies of the token and load its row 16 times
// over; with one workgroup on one CU those redundant loads set the time).
// The token row goes to LDS once; thread (e, j) takes expert e's slice j of
// d (kRouteThreads / NP threads an expert, NP the power of two >= N, whole
// waves an expert), its weights straight from memory. Sums in fixed order:
// the slice in k order, the 64 lanes by a butterfly, the expert's waves in
// order. Then front_one.
constexpr int kOneMaxD = 16384;  // the token row in LDS (32 KB)
constexpr int kOneMaxSlice = 64;  // weights a thread (eight 16-byte loads)

template <int NT>
__global__ __launch_bounds__(kRouteThreads) void front1_kernel(RouteArgs ra, PermuteArgs pa) {
  __shared__ __attribute__((aligned(16))) uint16_t s_x[kOneMaxD];
  __shared__ float s_wsum[kFrontWaves];
  __shared__ float s_logit[NT * 16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = ra.N;
  const int d = static_cast<int>(ra.d);
  int np = 1;
  while (np < N) np <<= 1;
  const int tpe = kRouteThreads / np;  // a multiple of 64
  const int e = tid / tpe, j = tid % tpe;
  const int per = d / tpe;  // a multiple of 8, at most kOneMaxSlice
  uint4 w[kOneMaxSlice / 8];
  const uint4* wr = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(ra.w_router) +
                                                   static_cast<int64_t>(e) * d + j * per);
#pragma unroll
  for (int c = 0; c < kOneMaxSlice / 8; ++c)
    if (e < N && c < per / 8) w[c] = wr[c];
  const uint4* xg = reinterpret_cast<const uint4*>(ra.x);
  for (int c = tid; c < d / 8; c += kRouteThreads) reinterpret_cast<uint4*>(s_x)[c] = xg[c];
  __syncthreads();  // the token row is in LDS
  float v = 0.f;
  if (e < N) {
    const uint4* xs = reinterpret_cast<const uint4*>(s_x + j * per);
#pragma unroll
    for (int c = 0; c < kOneMaxSlice / 8; ++c) {
      if (c >= per / 8) break;
      const uint4 xv = xs[c];
      const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w}, ww[4] = {w[c].x, w[c].y, w[c].z, w[c].w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        v = fmaf(bf16_to_f32(static_cast<uint16_t>(xw[h] & 0xFFFFu)), bf16_to_f32(static_cast<uint16_t>(ww[h] & 0xFFFFu)), v);
        v = fmaf(bf16_to_f32(static_cast<uint16_t>(xw[h] >> 16)), bf16_to_f32(static_cast<uint16_t>(ww[h] >> 16)), v);
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if (lane == 0) s_wsum[wave] = v;
  __syncthreads();
  if (tid < NT * 16) {
    float l = 0.f;
    if (tid < N) {
      const int wpe = tpe / 64;
      l = s_wsum[tid * wpe];
      for (int i = 1; i < wpe; ++i) l += s_wsum[tid * wpe + i];
      if (ra.b_router) l += ra.b_router[tid];
      ra.logits[tid] = l;
    }
    s_logit[tid] = l;
  }
  __syncthreads();
  front_one<NT>(ra, pa, s_logit);
}

}  // namespace

bool front_fits(const RouteArgs& ra, const PermuteArgs& pa) {
  return ra.act_dtype == 1 && !ra.ec && !ra.logits_given && ra.T >= 1 && ra.T <= kFrontTokens && ra.N >= 1 &&
         ra.N <= 16 * kFrontMaxNT && ra.k >= 1 && ra.k <= kPermMaxK && ra.d % (32 * kFrontWaves) == 0 &&
         pa.x_perm == nullptr;
}

hipError_t launch_front(const RouteArgs& ra, const PermuteArgs& pa, hipStream_t s) {
  stage_mark(kStageRoute, false, s);
  int np = 1;
  while (np < ra.N) np <<= 1;
  const int64_t tpe = kRouteThreads / np;
  if (ra.T == 1 && ra.N <= 16 && ra.d <= kOneMaxD && ra.d % (tpe * 8) == 0 && ra.d / tpe <= kOneMaxSlice) {
    hipLaunchKernelGGL(front1_kernel<1>, dim3(1), dim3(kRouteThreads), 0, s, ra, pa);
    stage_mark(kStageRoute, true, s);
    return hipGetLastError();
  }
  switch ((ra.N + 15) / 16) {
    case 1: hipLaunchKernelGGL(front_kernel<1>, dim3(1), dim3(kRouteThreads), 0, s, ra, pa); break;
    case 2: hipLaunchKernelGGL(front_kernel<2>, dim3(1), dim3(kRouteThreads), 0, s, ra, pa); break;
    case 3: hipLaunchKernelGGL(front_kernel<3>, dim3(1), dim3(kRouteThreads), 0, s, ra, pa); break;
    case 4: hipLaunchKernelGGL(front_kernel<4>, dim3(1), dim3(kRouteThreads), 0, s, ra, pa); break;
    default: return hipErrorInvalidValue;
  }
  stage_mark(kStageRoute, true, s);
  return hipGetLastError();
}

}  // namespace moe
