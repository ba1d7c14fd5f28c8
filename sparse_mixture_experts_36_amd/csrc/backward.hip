// Layer backward: gradients of sum_t <dy_t, y_t> + c_aux L_aux + c_z z with
// respect to x, the router weight and bias, and every expert's weights (and
// GELU biases), with the routing decision held fixed.
//
// Pages: aigrafen.se "Mixture of Experts" (y = sum g_i E_i(x); L_aux =
// alpha N sum f_i P_i; the `MoE` module), learn.starphix.com "Mixture of
// Experts (MoE)" / "Load Balancing (Critical)" (z_loss), vanos001 "MoE
// Architecture" / "Expert Network Design" (SwiGLU, GELU experts).
//
// Steps (all on the caller's stream):
//  1. forward again: router, permutation with the rows copied, U = X W1^T
//     (+ b1) and V = X W3^T in fp32, H = act(U, V) in bf16, shared experts on
//     all T rows (on the forward's grouped FFN, up GEMM only, when its DMA
//     tiles take the call). The layer output itself is not needed: the gate
//     gradient dg = <dy, E(x)> = <dy W2, H> (+ <dy, b2>) comes from dH;
//  2. combine backward: the kept rows' dy unscaled (dYu) and scaled by the
//     gate (dY = g dy, bf16);
//  3. dH = dYu W2 (fp32, LDS-DMA GEMM); per row dg, then dU, dV from g dH, U,
//     V (bf16, one [dU | dV] row each); dX = [dU dV] [W1; W3] (fp32, LDS-DMA);
//  4. dW2 = dY^T H, dW1 = dU^T X, dW3 = dV^T X (fp32, one matrix per expert,
//     LDS-DMA GEMM), b1 / b2 gradients as column sums;
//  5. router: dl from dg through the gates' mode, the L_aux and z terms and
//     the token softmax; dW_r = dl^T x and dx += dl W_r (dl split into two
//     bf16 halves whose sum is dl to about 2^-16), db_r = column sums of dl;
//  6. dx_t = sum of its kept rows of dX (slots ascending) + the shared rows +
//     the router term, bf16.
// Every sum runs in a fixed order: identical inputs give identical bits.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxSlots = 8;  // top-k limit

// H = act(U (+ b1), V) for every row; U takes the bias in place (GELU,
// routed rows: the row's expert from the offsets).
__global__ __launch_bounds__(kThreads) void act_fwd_kernel(BwdArgs a, float* U, const float* V, uint16_t* H,
                                                            int64_t rows) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= rows * a.d_ff) return;
  const int64_t r = i / a.d_ff, c = i % a.d_ff;
  float u = U[i];
  if (a.act == 0 && a.b1 && r < a.cap) {
    int lo = 0, hi = a.N - 1;  // expert of routed row r
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.offsets[mid] <= r) lo = mid; else hi = mid - 1;
    }
    u += a.b1[static_cast<int64_t>(lo) * a.d_ff + c];
    U[i] = u;
  }
  H[i] = f32_to_bf16(a.act == 1 ? silu(u) * V[i] : gelu_erf(u));
}

// Per token: for each kept slot j (routed row r), dy into row r as it is
// (dYu: the dH product's input) and scaled by the gate (dY = g dy, bf16: the
// dW2 product's input), the row's pair index and gate; dg = 0 for a dropped
// pair (kept pairs get theirs in act_bwd_kernel).
__global__ __launch_bounds__(kThreads) void combine_bwd_kernel(BwdArgs a) {
  const int64_t t = blockIdx.x;
  const uint4* dy = reinterpret_cast<const uint4*>(a.dy + t * a.d);
  const int64_t n8 = a.d / 8;
  for (int j = 0; j < a.k; ++j) {
    const int row = a.inv_map[t * a.k + j];  // uniform
    if (row < 0) {
      if (threadIdx.x == 0) a.dg[t * a.k + j] = 0.f;
      continue;
    }
    const float g = a.topk_w[t * a.k + j];
    uint4* du = reinterpret_cast<uint4*>(a.dYu + static_cast<int64_t>(row) * a.d);
    uint4* ds = reinterpret_cast<uint4*>(a.dY + static_cast<int64_t>(row) * a.d);
    for (int64_t c = threadIdx.x; c < n8; c += kThreads) {
      const uint4 v = dy[c];
      du[c] = v;
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[e] = static_cast<uint32_t>(f32_to_bf16(g * bf16_to_f32(static_cast<uint16_t>(w[e] & 0xFFFFu)))) |
               (static_cast<uint32_t>(f32_to_bf16(g * bf16_to_f32(static_cast<uint16_t>(w[e] >> 16)))) << 16);
      ds[c] = make_uint4(o[0], o[1], o[2], o[3]);
    }
    if (threadIdx.x == 0) {
      a.row_pair[row] = static_cast<int32_t>(t * a.k + j);
      a.row_gate[row] = g;
    }
  }
}

// One workgroup per row of the row space. dH holds dy W2 for the row (routed:
// its token's dy, unscaled; shared: dy); with the row's gate g (1 for shared
// rows) dH = g (dy W2), and dU, dV (bf16, row pitch ld_du) follow from dH, U, V:
// SwiGLU dU = dH V silu'(U), dV = dH silu(U); GELU dU = dH gelu'(U). A routed
// row also gives its pair's gate gradient dg = <dy, E(x)> = <dy W2, H> (+ <dy,
// b2> for GELU), summed in a fixed order.
__global__ __launch_bounds__(kThreads) void act_bwd_kernel(BwdArgs a) {
  __shared__ float s_red[kThreads / 64];
  const int64_t r = blockIdx.x;
  const bool routed = r < a.cap;
  if (routed && r >= a.offsets[a.N]) return;  // rows past the kept pairs (uniform)
  const int tid = threadIdx.x;
  const int64_t f = a.d_ff;
  const float g = routed ? a.row_gate[r] : 1.f;
  const float* dh = a.dH + r * f;
  const float* U = a.U + r * f;
  const float* V = a.act == 1 ? a.V + r * f : nullptr;
  const uint16_t* H = a.H + r * f;
  uint16_t* dU = a.dU + r * a.ld_du;
  uint16_t* dV = a.act == 1 ? a.dV + r * a.ld_du : nullptr;
  float dot = 0.f;
  // four elements a thread and step (d_ff is a multiple of 128: rows stay
  // 16-byte aligned). dH, U, V and H are read once, each wave load covering
  // whole lines: the loads carry the nontemporal hint (Mixtral shape 407 ->
  // 372 us a call).
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  for (int64_t i = 4 * tid; i < f; i += 4 * kThreads) {
    const f32x4 hq = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(dh + i));
    const f32x4 uq = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(U + i));
    const u32x2 hv = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(H + i));
    const float4 hp4 = make_float4(hq.x, hq.y, hq.z, hq.w), u4 = make_float4(uq.x, uq.y, uq.z, uq.w);
    const uint2 h2 = make_uint2(hv.x, hv.y);
    const float hp[4] = {hp4.x, hp4.y, hp4.z, hp4.w}, u[4] = {u4.x, u4.y, u4.z, u4.w};
    const uint16_t hb[4] = {static_cast<uint16_t>(h2.x & 0xFFFFu), static_cast<uint16_t>(h2.x >> 16),
                            static_cast<uint16_t>(h2.y & 0xFFFFu), static_cast<uint16_t>(h2.y >> 16)};
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (a.act == 1) {
      const f32x4 vq = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(V + i));
      const float4 v4 = make_float4(vq.x, vq.y, vq.z, vq.w);
      v[0] = v4.x; v[1] = v4.y; v[2] = v4.z; v[3] = v4.w;
    }
    uint16_t ou[4], ov[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float h = g * hp[e];
      dot = fmaf(hp[e], bf16_to_f32(hb[e]), dot);
      if (a.act == 1) {
        const float sg = 1.f / (1.f + expf(-u[e]));
        ou[e] = f32_to_bf16(h * v[e] * (sg + u[e] * sg * (1.f - sg)));
        ov[e] = f32_to_bf16(h * u[e] * sg);
      } else {
        const float cdf = 0.5f * (1.f + erff(u[e] * 0.70710678118654752f));
        const float pdf = expf(-0.5f * u[e] * u[e]) * 0.39894228040143268f;
        ou[e] = f32_to_bf16(h * (cdf + u[e] * pdf));
        ov[e] = 0;
      }
    }
    *reinterpret_cast<uint2*>(dU + i) = make_uint2(ou[0] | (static_cast<uint32_t>(ou[1]) << 16),
                                                   ou[2] | (static_cast<uint32_t>(ou[3]) << 16));
    if (a.act == 1)
      *reinterpret_cast<uint2*>(dV + i) = make_uint2(ov[0] | (static_cast<uint32_t>(ov[1]) << 16),
                                                     ov[2] | (static_cast<uint32_t>(ov[3]) << 16));
  }
  if (!routed) return;  // uniform
  const int32_t pair = a.row_pair[r];
  if (a.act == 0 && a.b2) {  // the output bias: <dy, b2_e>
    int lo = 0, hi = a.N - 1;  // expert of row r
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.offsets[mid] <= r) lo = mid; else hi = mid - 1;
    }
    const uint16_t* dy = a.dy + static_cast<int64_t>(pair / a.k) * a.d;
    const float* b2 = a.b2 + static_cast<int64_t>(lo) * a.d;
    for (int64_t o = tid; o < a.d; o += kThreads) dot = fmaf(bf16_to_f32(dy[o]), b2[o], dot);
  }
  dot = wave_sum(dot);
  if ((tid & 63) == 0) s_red[tid >> 6] = dot;
  __syncthreads();
  if (tid == 0) {
    float v = 0.f;
    for (int w = 0; w < kThreads / 64; ++w) v += s_red[w];
    a.dg[pair] = v;
  }
}

// Router backward, one token per quarter-wave (16 lanes): p from the logits,
// the gate gradient by mode, the L_aux and z terms, then through the softmax.
// dl is written in fp32 (for the bias gradient) and as two bf16 halves
// (hi = bf16(dl), lo = bf16(dl - hi)) of row pitch ldl, the pad columns zero.
__global__ __launch_bounds__(kThreads) void router_bwd_kernel(BwdArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 4, c16 = lane & 15;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 16 + wave * 4 + q;
  if (t >= a.T) return;  // uniform within the quarter
  const int N = a.N, k = a.k;
  const float* l = a.logits + t * N;
  float m = -3.0e38f;
  for (int e = c16; e < N; e += 16) m = fmaxf(m, l[e]);
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 16));
  float s = 0.f;
  for (int e = c16; e < N; e += 16) s += expf(l[e] - m);
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) s += __shfl_xor(s, o, 16);
  const float inv_s = 1.f / s;
  // <dg, g> and the sum of the selected p (renormalised gates)
  float dot = 0.f, psum = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxSlots; ++j) {
    if (j >= k) break;
    dot += a.dg[t * k + j] * a.topk_w[t * k + j];
    psum += expf(l[a.topk_idx[t * k + j]] - m) * inv_s;
  }
  const float zc = a.c_z * 2.f * (*a.lse_mean) / static_cast<float>(a.T);
  // d L_aux / d p_e = alpha N f_e / T with f_e = counts_e / (T k)
  const float ac = a.c_aux * a.aux_alpha * static_cast<float>(N) /
                   (static_cast<float>(a.T) * static_cast<float>(a.T) * static_cast<float>(k));
  // dp_e (gradient onto the full softmax) and dq_e (onto the logit directly:
  // the softmax over the k selected logits)
  auto grad_of = [&](int e, float& dq) {
    float dp = ac * static_cast<float>(a.counts[e]);
    dq = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxSlots; ++j) {
      if (j >= k) break;
      if (a.topk_idx[t * k + j] != e) continue;
      const float dgj = a.dg[t * k + j];
      if (a.gating == 0) dp += dgj;
      else if (a.gating == 1) dp += (dgj - dot) / psum;
      else dq += a.topk_w[t * k + j] * (dgj - dot);
    }
    return dp;
  };
  float dpp = 0.f;
  for (int e = c16; e < N; e += 16) {
    float dq;
    dpp += grad_of(e, dq) * expf(l[e] - m) * inv_s;
  }
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) dpp += __shfl_xor(dpp, o, 16);
  for (int e = c16; e < a.ldl; e += 16) {
    float dl = 0.f;
    if (e < N) {
      const float p = expf(l[e] - m) * inv_s;
      float dq;
      const float dp = grad_of(e, dq);
      dl = dq + p * (dp - dpp) + zc * p;
      a.dl32[t * N + e] = dl;
    }
    const uint16_t hi = f32_to_bf16(dl);
    a.dl_hi[t * a.ldl + e] = hi;
    a.dl_lo[t * a.ldl + e] = f32_to_bf16(dl - bf16_to_f32(hi));
  }
}

// Column sums over the rows of each group (fixed order): out[g][c] = sum_r
// in[r][c], rows [off[g], off[g+1]) (off null: rows [0, rows) as one group).
template <typename TI>
__global__ __launch_bounds__(kThreads) void colsum_kernel(const TI* in, int64_t ld, const int32_t* off, int32_t cap,
                                                          int64_t rows, int64_t cols, float* out) {
  const int g = blockIdx.y;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (c >= cols) return;
  int64_t r0 = 0, r1 = rows;
  if (off) {
    r0 = max(0, min(off[g], cap));
    r1 = max(static_cast<int>(r0), min(off[g + 1], cap));
  }
  float s = 0.f;
  for (int64_t r = r0; r < r1; ++r) {
    if constexpr (sizeof(TI) == 2) s += bf16_to_f32(in[r * ld + c]);
    else s += in[r * ld + c];
  }
  out[static_cast<int64_t>(g) * cols + c] = s;
}

// db_r[e] = sum_t dl[t][e]: one workgroup per expert, each thread a strided
// share of the tokens, then the waves in order.
__global__ __launch_bounds__(kThreads) void router_bias_grad_kernel(const float* dl, int64_t T, int32_t N,
                                                                    float* dbr) {
  __shared__ float s_w[kThreads / 64];
  const int e = blockIdx.x;
  float s = 0.f;
  for (int64_t t = threadIdx.x; t < T; t += kThreads) s += dl[t * N + e];
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) s_w[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    float v = 0.f;
    for (int w = 0; w < kThreads / 64; ++w) v += s_w[w];
    dbr[e] = v;
  }
}

// Bounds of `splits` equal token chunks: off[i] = i T / splits.
__global__ void split_bounds_kernel(int32_t* off, int32_t splits, int64_t T) {
  const int i = threadIdx.x;
  if (i <= splits) off[i] = static_cast<int32_t>(i * T / splits);
}

// out[i] = sum over chunks c (in order) of part[c][i].
__global__ __launch_bounds__(kThreads) void sum_parts_kernel(const float* part, int32_t splits, int64_t n,
                                                             float* out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= n) return;
  float v = 0.f;
  for (int c = 0; c < splits; ++c) v += part[c * n + i];
  out[i] = v;
}

// dx_t = sum over its kept slots of dX[row] (ascending) + the shared experts'
// rows + the router term, to bf16.
// dx of token t: its kept routed rows of dX in slot order, then its shared
// experts' rows, then the router's term, summed in that order in fp32. Four
// columns a thread (d is a multiple of 128), the loads of all terms of two
// column chunks issued before the sums; the rows are read once, in whole lines
// a wave, with the nontemporal hint (Mixtral shape: 85 -> 58 us a call against
// one column a thread and the terms loaded one after another). The sums are
// the same, in the same order.
constexpr int kDxTerms = 8 + 4 + 1;  // top-k, shared experts, router term
__global__ __launch_bounds__(kThreads) void dx_kernel(BwdArgs a, const float* dX, const float* dxr, uint16_t* dx) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const int64_t t = blockIdx.x;
  const int64_t d = a.d;
  // element offsets of the terms' rows, in summation order
  int64_t src[kDxTerms];
  const float* base[kDxTerms];
  int n = 0;
  for (int j = 0; j < a.k; ++j) {
    const int row = a.inv_map[t * a.k + j];
    if (row >= 0) {
      src[n] = static_cast<int64_t>(row) * d;
      base[n++] = dX;
    }
  }
  for (int sh = 0; sh < a.S; ++sh) {
    src[n] = (a.cap + static_cast<int64_t>(sh) * a.T + t) * d;
    base[n++] = dX;
  }
  src[n] = t * d;
  base[n++] = dxr;
  const int64_t nch = d / 4;
  for (int64_t c0 = threadIdx.x; c0 < nch; c0 += 2 * kThreads) {
    f32x4 v[2][kDxTerms];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t c = c0 + u * kThreads;
#pragma unroll
      for (int i = 0; i < kDxTerms; ++i)
        if (i < n && c < nch) v[u][i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(base[i] + src[i]) + c);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t c = c0 + u * kThreads;
      if (c >= nch) break;
      float sx = 0.f, sy = 0.f, sz = 0.f, sw = 0.f;
#pragma unroll
      for (int i = 0; i < kDxTerms; ++i)
        if (i < n) {
          sx += v[u][i].x;
          sy += v[u][i].y;
          sz += v[u][i].z;
          sw += v[u][i].w;
        }
      *reinterpret_cast<uint2*>(dx + t * d + 4 * c) =
          make_uint2(f32_to_bf16(sx) | (static_cast<uint32_t>(f32_to_bf16(sy)) << 16),
                     f32_to_bf16(sz) | (static_cast<uint32_t>(f32_to_bf16(sw)) << 16));
    }
  }
}

unsigned blocks_for(int64_t n) { return static_cast<unsigned>(ceil_div(n, kThreads)); }

}  // namespace

hipError_t launch_backward(const BwdArgs& a, hipStream_t s) {
  hipError_t e = hipSuccess;
  const int64_t T = a.T, d = a.d, f = a.d_ff, cap = a.cap, S = a.S;
  const int64_t rows = cap + S * T;  // routed rows, then T per shared expert
  const bool swi = (a.act == 1);
  auto ok = [&]() { return e == hipSuccess; };
  auto check = [&]() { if (e == hipSuccess) e = hipGetLastError(); };

  // ---- 1. forward again (router and permutation are done by the caller):
  // on the forward's grouped FFN when its DMA tiles take these rows (U, V,
  // H and Y in one up and one down launch), else on the backward GEMM
  if (a.use_ffn) {
    e = launch_grouped_ffn(a.ffn, s);
  } else {
    BGemm up{};  // U / V = X W^T: routed rows from x_perm, shared rows from x
    up.off = a.offsets; up.n_groups = a.N; up.cap = static_cast<int32_t>(cap); up.K = static_cast<int32_t>(d);
    up.N = static_cast<int32_t>(f); up.A = a.x_perm; up.lda = d; up.ldb = a.ld_up; up.b_gs = f * a.ld_up;
    up.ldc = f;
    for (int w = 0; w < (swi ? 2 : 1) && ok(); ++w) {
      up.B = w == 0 ? a.w1 : a.w3;
      up.C = w == 0 ? a.U : a.V;
      e = launch_bgemm(up, false, true, false, a.tile_start, s);
    }
    if (S > 0) {
      BGemm sh = up;
      sh.off = nullptr; sh.n_groups = static_cast<int32_t>(S); sh.rows_all = static_cast<int32_t>(T); sh.A = a.x;
      sh.c_gs = T * f;
      for (int w = 0; w < (swi ? 2 : 1) && ok(); ++w) {
        sh.B = w == 0 ? a.sw1 : a.sw3;
        sh.C = (w == 0 ? a.U : a.V) + cap * f;
        e = launch_bgemm(sh, false, true, false, a.tile_start, s);
      }
    }
    if (ok()) {
      hipLaunchKernelGGL(act_fwd_kernel, dim3(blocks_for(rows * f)), dim3(kThreads), 0, s, a, a.U, a.V, a.H, rows);
      check();
    }
  }
  // ---- 2. combine backward
  if (ok()) {
    hipLaunchKernelGGL(combine_bwd_kernel, dim3(static_cast<unsigned>(T)), dim3(kThreads), 0, s, a);
    check();
  }
  // ---- 3. dH, dU / dV, dX on the DMA tiles (B read along the weights' rows)
  const int64_t ldu = a.ld_du;  // dU and dV share rows: [dU | dV] (SwiGLU) or dU
  BGemm dh{};  // dH = dy W2 (routed rows: the token's dy, unscaled), dy W2s (shared)
  dh.off = a.offsets; dh.n_groups = a.N; dh.cap = static_cast<int32_t>(cap); dh.K = static_cast<int32_t>(d);
  dh.N = static_cast<int32_t>(f); dh.A = a.dYu; dh.lda = d; dh.B = a.w2; dh.ldb = a.ld_down; dh.b_gs = d * a.ld_down;
  dh.C = a.dH; dh.ldc = f;
  if (ok() && cap > 0) e = launch_bgemm_dma(dh, a.tile_start, s);
  if (ok() && S > 0) {
    BGemm sh = dh;
    sh.off = nullptr; sh.n_groups = static_cast<int32_t>(S); sh.rows_all = static_cast<int32_t>(T); sh.A = a.dy;
    sh.B = a.sw2; sh.C = a.dH + cap * f; sh.c_gs = T * f;
    e = launch_bgemm_dma(sh, a.tile_start, s);
  }
  if (ok()) {
    hipLaunchKernelGGL(act_bwd_kernel, dim3(static_cast<unsigned>(rows)), dim3(kThreads), 0, s, a);
    check();
  }
  // dX = [dU dV] [W1; W3]: one product over k = 2 d_ff, W3 past k = d_ff
  BGemm dxg{};
  dxg.off = a.offsets; dxg.n_groups = a.N; dxg.cap = static_cast<int32_t>(cap);
  dxg.K = static_cast<int32_t>(swi ? 2 * f : f); dxg.N = static_cast<int32_t>(d); dxg.A = a.dU; dxg.lda = ldu;
  dxg.B = a.w1; dxg.B2 = swi ? a.w3 : nullptr; dxg.k_split = static_cast<int32_t>(f); dxg.ldb = a.ld_up;
  dxg.b_gs = f * a.ld_up; dxg.C = a.dX; dxg.ldc = d;
  if (ok() && cap > 0) e = launch_bgemm_dma(dxg, a.tile_start, s);
  if (ok() && S > 0) {
    BGemm sh = dxg;
    sh.off = nullptr; sh.n_groups = static_cast<int32_t>(S); sh.rows_all = static_cast<int32_t>(T);
    sh.A = a.dU + cap * ldu; sh.a_gs = T * ldu; sh.B = a.sw1; sh.B2 = swi ? a.sw3 : nullptr;
    sh.C = a.dX + cap * d; sh.c_gs = T * d;
    e = launch_bgemm_dma(sh, a.tile_start, s);
  }
  // ---- 4. weight gradients: rows-K on the DMA tiles, one matrix per expert
  BGemm dw{};
  dw.off = a.offsets; dw.n_groups = a.N; dw.cap = static_cast<int32_t>(cap);
  if (ok() && a.dW2) {  // dW2 = dY^T H: [d][d_ff]
    dw.M = static_cast<int32_t>(d); dw.N = static_cast<int32_t>(f); dw.A = a.dY; dw.lda = d; dw.B = a.H; dw.ldb = f;
    dw.C = a.dW2; dw.ldc = f; dw.c_gs = d * f;
    e = launch_bgemm_dma_rk(dw, s);
  }
  for (int w = 0; w < (swi ? 2 : 1) && ok(); ++w) {  // dW1 = dU^T X, dW3 = dV^T X: [d_ff][d]
    float* out = w == 0 ? a.dW1 : a.dW3;
    if (!out) continue;
    dw.M = static_cast<int32_t>(f); dw.N = static_cast<int32_t>(d); dw.A = w == 0 ? a.dU : a.dV; dw.lda = ldu;
    dw.B = a.x_perm; dw.ldb = d; dw.C = out; dw.ldc = d; dw.c_gs = f * d;
    e = launch_bgemm_dma_rk(dw, s);
  }
  if (S > 0) {
    BGemm sw{};
    sw.n_groups = static_cast<int32_t>(S); sw.rows_all = static_cast<int32_t>(T);
    if (ok() && a.dsW2) {
      sw.M = static_cast<int32_t>(d); sw.N = static_cast<int32_t>(f); sw.A = a.dy; sw.lda = d;
      sw.B = a.H + cap * f; sw.ldb = f; sw.b_gs = T * f; sw.C = a.dsW2; sw.ldc = f; sw.c_gs = d * f;
      e = launch_bgemm_dma_rk(sw, s);
    }
    for (int w = 0; w < (swi ? 2 : 1) && ok(); ++w) {
      float* out = w == 0 ? a.dsW1 : a.dsW3;
      if (!out) continue;
      sw.M = static_cast<int32_t>(f); sw.N = static_cast<int32_t>(d); sw.A = (w == 0 ? a.dU : a.dV) + cap * ldu;
      sw.lda = ldu; sw.a_gs = T * ldu; sw.B = a.x; sw.ldb = d; sw.b_gs = 0; sw.C = out; sw.ldc = d; sw.c_gs = f * d;
      e = launch_bgemm_dma_rk(sw, s);
    }
  }
  if (ok() && !swi && a.db1) {
    hipLaunchKernelGGL(colsum_kernel<uint16_t>, dim3(blocks_for(f), a.N), dim3(kThreads), 0, s, a.dU, ldu, a.offsets,
                       static_cast<int32_t>(cap), cap, f, a.db1);
    check();
  }
  if (ok() && !swi && a.db2) {
    hipLaunchKernelGGL(colsum_kernel<uint16_t>, dim3(blocks_for(d), a.N), dim3(kThreads), 0, s, a.dY, d, a.offsets,
                       static_cast<int32_t>(cap), cap, d, a.db2);
    check();
  }
  // ---- 5. router
  if (ok()) {
    hipLaunchKernelGGL(router_bwd_kernel, dim3(static_cast<unsigned>(ceil_div(T, 16))), dim3(kThreads), 0, s, a);
    check();
  }
  const bool wr_split = a.dWr && a.wr_splits > 1;
  if (ok() && wr_split) {
    hipLaunchKernelGGL(split_bounds_kernel, dim3(1), dim3(128), 0, s, a.wr_off, a.wr_splits, T);
    check();
  }
  for (int h = 0; h < 2 && ok(); ++h) {  // dW_r = dl^T x and dx_r = dl W_r, each as hi + lo
    if (a.dWr) {  // token chunks as groups of a rows-K product, one partial matrix each
      BGemm r{};
      r.off = wr_split ? a.wr_off : nullptr; r.n_groups = wr_split ? a.wr_splits : 1;
      r.cap = static_cast<int32_t>(T); r.rows_all = static_cast<int32_t>(T);
      r.M = a.N; r.N = static_cast<int32_t>(d); r.A = h == 0 ? a.dl_hi : a.dl_lo; r.lda = a.ldl; r.B = a.x;
      r.ldb = d; r.C = wr_split ? a.wr_part : a.dWr; r.ldc = d; r.c_gs = wr_split ? a.N * d : 0;
      e = launch_bgemm(r, true, false, h == 1, a.tile_start, s);
      if (!ok()) break;
    }
    BGemm x{};
    x.n_groups = 1; x.rows_all = static_cast<int32_t>(T); x.K = a.N; x.N = static_cast<int32_t>(d);
    x.A = h == 0 ? a.dl_hi : a.dl_lo; x.lda = a.ldl; x.B = a.w_router; x.ldb = d; x.C = a.dxr; x.ldc = d;
    e = launch_bgemm(x, false, false, h == 1, a.tile_start, s);
  }
  if (ok() && wr_split) {
    hipLaunchKernelGGL(sum_parts_kernel, dim3(blocks_for(a.N * d)), dim3(kThreads), 0, s, a.wr_part, a.wr_splits,
                       a.N * d, a.dWr);
    check();
  }
  if (ok() && a.dbr) {
    hipLaunchKernelGGL(router_bias_grad_kernel, dim3(static_cast<unsigned>(a.N)), dim3(kThreads), 0, s, a.dl32, T,
                       a.N, a.dbr);
    check();
  }
  // ---- 6. dx
  if (ok()) {
    hipLaunchKernelGGL(dx_kernel, dim3(static_cast<unsigned>(T)), dim3(kThreads), 0, s, a, a.dX, a.dxr, a.dx);
    check();
  }
  return e;
}

}  // namespace moe
