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
#include "route_block.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxN = 256;
// s_waitcnt immediate: vmcnt(n), no wait on expcnt and lgkmcnt
constexpr int vmcnt_imm(int n) { return 0x0f70 | (n & 15) | (((n >> 4) & 3) << 14); }

// Router GEMM over one k range: partial logits of 64 tokens (4 waves x 16) for
// all experts. Grid (token blocks, k splits). bf16 runs on MFMA with the
// router-weight tile for all experts in LDS (double buffered); the next
// k-step's tile and token fragments are loaded while the current one computes.
// KR is the k-step: 64 for decode-sized calls (many k splits, little data a
// step), 128 or 256 for prefill, where each workgroup walks a long k range and
// wider steps keep more bytes in flight between its barriers.
template <int NT, int KR>
__global__ __launch_bounds__(kThreads) void router_gemm_kernel(RouteArgs a, float* part, int k_len) {
  constexpr int WS = KR + 8;                     // padded LDS row (bf16 elements)
  constexpr int KC = KR / 8;                     // 16-byte chunks of a weight row per step
  constexpr int XL = KR / 32;                    // 16-byte token chunks per lane and step
  __shared__ __attribute__((aligned(16))) uint16_t wtile[2][NT * 16 * WS];
  constexpr int WCH = (NT * 16 * KC + kThreads - 1) / kThreads;  // 16-byte weight chunks per thread
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
    // Lane (row c16, k-group q) takes KR/4 consecutive k of its token row per
    // step, as XL chunks of 8 (the same k order for the weight fragments).
    const uint16_t* xr = static_cast<const uint16_t*>(a.x);
    const uint16_t* wr = static_cast<const uint16_t*>(a.w_router);
    int64_t trow = t0 + c16;
    if (trow > T - 1) trow = T - 1;  // rows past T compute garbage that is never stored
    const uint16_t* xrow = xr + trow * d + k0 + q * (KR / 4);
    const int nsteps = k_len / KR;
    uint4 wv[WCH];
    auto wload = [&](int step) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < WCH; ++i) {
        const int c = tid + i * kThreads;
        const int e = c / KC, kc = c % KC;
        wv[i] = make_uint4(0, 0, 0, 0);
        if (c < NT * 16 * KC && e < N) wv[i] = *reinterpret_cast<const uint4*>(wr + e * d + k0 + step * KR + kc * 8);
      }
    };
    auto wstore = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < WCH; ++i) {
        const int c = tid + i * kThreads;
        const int e = c / KC, kc = c % KC;
        if (c < NT * 16 * KC) *reinterpret_cast<uint4*>(&wtile[buf][e * WS + kc * 8]) = wv[i];
      }
    };
    uint4 xc[XL], xn[XL];
    wload(0);
#pragma unroll
    for (int m = 0; m < XL; ++m) xc[m] = *reinterpret_cast<const uint4*>(xrow + m * 8);
    wstore(0);
    __syncthreads();
    for (int st = 0; st < nsteps; ++st) {
      const int nx = (st + 1 < nsteps) ? st + 1 : st;  // the last step re-reads itself into the idle buffer
      wload(nx);
#pragma unroll
      for (int m = 0; m < XL; ++m) xn[m] = *reinterpret_cast<const uint4*>(xrow + nx * KR + m * 8);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const uint16_t* wp = &wtile[st & 1][(16 * nt + c16) * WS + q * (KR / 4)];
#pragma unroll
        for (int m = 0; m < XL; ++m)
          acc[nt] = mfma16x16x32(xc[m], *reinterpret_cast<const uint4*>(wp + m * 8), acc[nt]);
      }
      wstore((st + 1) & 1);
#pragma unroll
      for (int m = 0; m < XL; ++m) xc[m] = xn[m];
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

// Router GEMM for prefill-sized calls (bf16): the same products and output
// layout as router_gemm_kernel, with more loads in flight. k-stages of 64:
// the router-weight rows of a stage (16 NT experts, padded to RP rows, 128
// bytes each, 16-byte chunk c of row r at c ^ (r & 7)) go to a ring of NS
// LDS buffers by global_load_lds, NS - 1 stages ahead; each wave loads its 16
// tokens' fragments of the same stages into registers, as far ahead. One
// barrier per stage. Expert rows past N load row N - 1 (computed, never
// stored). k_len is a multiple of 64 with at least NS - 1 stages.
template <int NT, int NS>
__global__ __launch_bounds__(kThreads) void router_gemm_dma_kernel(RouteArgs a, float* part, int k_len) {
  constexpr int RP = (NT + 1) / 2 * 32;  // weight rows of a stage: 8 per DMA instruction, the same count per wave
  constexpr int DI = RP / 32;            // DMA instructions per wave and stage
  constexpr int SB = RP * 128;           // stage bytes
  __shared__ __attribute__((aligned(16))) char wbuf[NS][SB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, c16 = lane & 15;
  const int N = a.N;
  const int64_t T = a.T, d = a.d;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kRouteTokens + wave * 16;
  const int64_t k0 = static_cast<int64_t>(blockIdx.y) * k_len;
  float* out = part + static_cast<int64_t>(blockIdx.y) * T * N;
  const int n_st = k_len / 64;

  // DMA sources: instruction i of this wave fills rows 32 i + 8 wave + lane / 8
  const char* wr = static_cast<const char*>(a.w_router) + k0 * 2;
  uint32_t woff[DI];
#pragma unroll
  for (int i = 0; i < DI; ++i) {
    const int r = 32 * i + 8 * wave + (lane >> 3);
    const int e = r < N ? r : N - 1;
    const int chunk = (lane & 7) ^ (r & 7);
    woff[i] = static_cast<uint32_t>(e * static_cast<int>(d) * 2 + chunk * 16);
  }
  // token fragments: lane (row c16, k-group q) takes k 8 q .. 8 q + 7 of each 32-wide half of a stage
  int64_t trow = t0 + c16;
  if (trow > T - 1) trow = T - 1;  // rows past T compute garbage that is never stored
  const char* xr = reinterpret_cast<const char*>(static_cast<const uint16_t*>(a.x) + trow * d + k0 + q * 8);
  // LDS read offsets of the two 32-wide halves: row 16 nt + c16, logical chunk 4 h + q
  int rd[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) rd[h] = c16 * 128 + (((4 * h + q) ^ (c16 & 7)) * 16);

  floatx4_t acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  uint4 xf[NS][2];
#define MOE_RDMA(S, ks)                                                                              \
  do {                                                                                               \
    const uint32_t ko_ = static_cast<uint32_t>(ks) * 128;                                            \
    _Pragma("unroll") for (int i_ = 0; i_ < DI; ++i_)                                                \
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(wr + (woff[i_] + ko_)),            \
                                         (__attribute__((address_space(3))) void*)(&wbuf[S][(32 * i_ + 8 * wave) * 128]), \
                                         16, 0, 0);                                                  \
    _Pragma("unroll") for (int h_ = 0; h_ < 2; ++h_)                                                 \
        xf[S][h_] = *reinterpret_cast<const uint4*>(xr + static_cast<int64_t>(ks) * 128 + h_ * 64); \
  } while (0)
  // stage ks in slot S: wait until only the newer NS - 2 stages' loads may
  // fly, barrier (every wave's DMA of stage ks has landed, and every wave is
  // done reading slot (ks - 1) mod NS), refill that slot with stage ks + NS - 1
  // (the last stage again past the end), then the products of stage ks
#define MOE_RSTAGE(S, ks)                                                                            \
  do {                                                                                               \
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * (DI + 2)));                                      \
    __builtin_amdgcn_s_waitcnt(0xc07f);                                                              \
    __builtin_amdgcn_s_barrier();                                                                    \
    asm volatile("" ::: "memory"); /* no LDS read moves above the barrier */                        \
    MOE_RDMA(((S) + NS - 1) % NS, min((ks) + NS - 1, n_st - 1));                                      \
    _Pragma("unroll") for (int h_ = 0; h_ < 2; ++h_)                                                 \
        _Pragma("unroll") for (int nt_ = 0; nt_ < NT; ++nt_) acc[nt_] =                              \
            mfma16x16x32(xf[S][h_], *reinterpret_cast<const uint4*>(&wbuf[S][nt_ * 2048 + rd[h_]]), acc[nt_]); \
  } while (0)
#pragma unroll
  for (int s0 = 0; s0 < NS - 1; ++s0) MOE_RDMA(s0, s0);
  const int n_round = n_st / NS * NS;
  for (int ks = 0; ks < n_round; ks += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) MOE_RSTAGE(u, ks + u);
  }
#pragma unroll
  for (int u = 0; u < NS - 1; ++u)
    if (n_round + u < n_st) MOE_RSTAGE(u, n_round + u);
#undef MOE_RSTAGE
#undef MOE_RDMA
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // the trailing refills have landed
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

// Softmax / top-k / gates / block statistics over 64 tokens, one per
// quarter-wave (16 waves): the logits are the given ones, or the sum of the
// k-split partial logits (in split order) plus the router bias, which is then
// also stored as the router output. A launch of one workgroup (T <= 64) also
// finishes the statistics itself.
template <int NT>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(RouteArgs a, const float* part, int splits) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, c16 = lane & 15;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kRouteTokens + wave * 4 + q;
  const bool live = t < a.T;  // uniform within the quarter
  float lg[NT];  // logit of expert 16 nt + c16
  token_logits<NT>(a, part, splits, t, live, c16, lg);
  route_block<NT>(a, t, live, lg, blockIdx.x, gridDim.x == 1);
}

// One workgroup of 1024 threads: the routing statistics from the block
// partials (route_finalize_block).
__global__ __launch_bounds__(kFinThreads) void route_finalize_kernel(RouteArgs a, int nb) { route_finalize_block(a, nb); }

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
    const int kr = router_kstep(a.T, a.d, a.N);
    const dim3 grid(nb, splits);
    const int k_len = static_cast<int>(a.d / splits);
    // prefill sizes, bf16: the LDS-DMA kernel, five stages ahead (three with
    // more than 160 experts, whose stages are larger)
    constexpr int NS = (NT + 1) / 2 * 32 <= 160 ? 6 : 4;
    if (a.T >= 1024 && a.act_dtype == 1 && k_len % 64 == 0 && k_len / 64 >= NS - 1) {
      hipLaunchKernelGGL((router_gemm_dma_kernel<NT, NS>), grid, dim3(kThreads), 0, s, a, a.part_logits, k_len);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    } else {
      if constexpr (NT <= 4) {  // the 256-wide weight tile fits LDS for at most 64 experts
        if (kr == 256)
          hipLaunchKernelGGL((router_gemm_kernel<NT, 256>), grid, dim3(kThreads), 0, s, a, a.part_logits, k_len);
      }
      if (kr == 256) {
        if constexpr (NT > 4) return hipErrorInvalidValue;
      } else if (kr == 128) {
        hipLaunchKernelGGL((router_gemm_kernel<NT, 128>), grid, dim3(kThreads), 0, s, a, a.part_logits, k_len);
      } else {
        hipLaunchKernelGGL((router_gemm_kernel<NT, 64>), grid, dim3(kThreads), 0, s, a, a.part_logits, k_len);
      }
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if (a.ec)
    hipLaunchKernelGGL(route_ec_kernel<NT>, dim3(nb), dim3(kRouteThreads), 0, s, a, a.part_logits, splits);
  else
    hipLaunchKernelGGL(route_kernel<NT>, dim3(nb), dim3(kRouteThreads), 0, s, a, a.part_logits, splits);
  return hipGetLastError();
}

}  // namespace

int router_kstep(int64_t T, int64_t d, int32_t N) {
  if (T < 1024) return 64;
  if (N <= 64 && d % 256 == 0) return 256;
  return 128;
}

int route_splits(int64_t T, int64_t d, int32_t N) {
  const int64_t nb = ceil_div(T, kRouteTokens), steps = d / router_kstep(T, d, N);
  int s = 1;
  while (nb * s < 256 && s < kMaxRouteSplits && steps % (2 * s) == 0 && steps / (2 * s) >= 4) s *= 2;
  return s;
}

hipError_t launch_route(const RouteArgs& a, hipStream_t s, bool finalize) {
  if (a.T <= 0) return hipSuccess;
  const int nb = static_cast<int>(ceil_div(a.T, kRouteTokens));
  const int nt = static_cast<int>(ceil_div(a.N, 16));
  const int splits = a.logits_given ? 1 : route_splits(a.T, a.d, a.N);
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
  if (nb > 1 && finalize) hipLaunchKernelGGL(route_finalize_kernel, dim3(1), dim3(kFinThreads), 0, s, a, nb);
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
