// Combine: gate-weighted gather of the expert outputs back to token order.
//
// Pages: aigrafen.se "Mixture of Experts" (y = sum_{i in top-k} g_i E_i(x);
// the `MoE` module adds w * expert(x[index]) into out[index], so a token
// dropped by the capacity cut gets nothing from that expert),
// learn.starphix.com "Mixture of Experts (MoE)" / "Shared + Specialized"
// (shared outputs are added to the routed sum).
//
// Gather form instead of a scatter-add: each token reads its own k rows, so no
// atomics are needed and the sum order (slots ascending, then shared experts)
// is fixed -- the output is bit-for-bit reproducible.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxK = 8;

// TW tokens a workgroup (consecutive): every thread takes 16-byte chunks of
// all TW tokens' rows and issues the loads of U chunks x TW tokens x (k routed
// + shared) rows before the first sum, so the dependent chain (inv_map, row,
// store) of one token overlaps the others'. A token has KS = k + shared slots,
// at most 8 / TW (12 with TW = 1): the loads stay in registers.
// A 16-byte load with the nontemporal hint: the rows of y_perm and y_shared
// are read once, and a wave's loads of one row cover whole lines (fine-grained
// layer 4.03-4.04 -> 4.00-4.02 ms a call, the others unchanged).
__device__ __forceinline__ uint4 ld_nt16(const uint4* p) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <bool BF16, int TW>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineArgs a) {
  constexpr int KM = TW == 1 ? kMaxK + 4 : 8 / TW;  // slots a token may have
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * TW;
  const int k = a.k;
  const int nsh = a.y_shared ? a.n_shared : 0;
  // slot j < k: routed row (or -1, dropped) with its gate; j in [k, k + nsh): shared expert j - k
  int64_t row[TW][KM];
  float g[TW][KM];
#pragma unroll
  for (int w = 0; w < TW; ++w)
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      row[w][j] = -1;
      g[w][j] = 1.f;
      if (t0 + w < a.T) {
        if (j < k) {
          row[w][j] = a.inv_map[(t0 + w) * k + j];
          g[w][j] = a.topk_w[(t0 + w) * k + j];
        } else if (j < k + nsh) {
          row[w][j] = (j - k) * a.T + t0 + w;  // row of y_shared
        }
      }
    }
  constexpr int E = BF16 ? 8 : 4;     // elements per 16-byte chunk
  constexpr int U = TW == 1 ? 2 : 1;  // chunks per thread whose loads are in flight together
  const int64_t nch = a.d / E;
  for (int64_t c0 = threadIdx.x; c0 < nch; c0 += U * kThreads) {
    uint4 v[U][TW][KM];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + u * kThreads;
      if (c >= nch) break;
#pragma unroll
      for (int w = 0; w < TW; ++w)
#pragma unroll
        for (int j = 0; j < KM; ++j)
          if (row[w][j] >= 0)
            v[u][w][j] = ld_nt16(reinterpret_cast<const uint4*>(j < k ? a.y_perm : a.y_shared) + (row[w][j] * nch + c));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + u * kThreads;
      if (c >= nch) break;
#pragma unroll
      for (int w = 0; w < TW; ++w) {
        if (t0 + w >= a.T) break;
        float acc[E];
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = 0.f;
        // fixed order: routed slots ascending, then the shared experts
#pragma unroll
        for (int j = 0; j < KM; ++j) {
          if (row[w][j] < 0) continue;
          const uint4 x = v[u][w][j];
          const float wt = g[w][j];
          if constexpr (BF16) {
            const uint32_t w4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              acc[2 * e] = fmaf(wt, bf16_to_f32(static_cast<uint16_t>(w4[e] & 0xFFFFu)), acc[2 * e]);
              acc[2 * e + 1] = fmaf(wt, bf16_to_f32(static_cast<uint16_t>(w4[e] >> 16)), acc[2 * e + 1]);
            }
          } else {
            acc[0] = fmaf(wt, __uint_as_float(x.x), acc[0]);
            acc[1] = fmaf(wt, __uint_as_float(x.y), acc[1]);
            acc[2] = fmaf(wt, __uint_as_float(x.z), acc[2]);
            acc[3] = fmaf(wt, __uint_as_float(x.w), acc[3]);
          }
        }
        uint4 o;
        if constexpr (BF16) {
          o = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
                         pack_bf16x2(acc[6], acc[7]));
        } else {
          o = make_uint4(__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]),
                         __float_as_uint(acc[3]));
        }
        reinterpret_cast<uint4*>(a.y)[(t0 + w) * nch + c] = o;
      }
    }
  }
}

// Expert choice: a token has a row for every expert that took it (any number,
// none included). inv_map is [T][N]; the gates are indexed by row. The
// workgroup first lists the token's rows in expert order in LDS, then sums
// them eight at a time (loads of a group in flight together), then the shared
// experts: the same fixed order on every run.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void combine_ec_kernel(CombineArgs a) {
  __shared__ int32_t s_row[kThreads];
  __shared__ float s_g[kThreads];
  __shared__ int32_t s_wc[kThreads / 64];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = a.k;
  int32_t row = -1;
  if (tid < N) row = a.inv_map[t * N + tid];
  const uint64_t bal = __ballot(row >= 0);
  if (lane == 0) s_wc[wave] = __popcll(bal);
  __syncthreads();
  int base = 0, n = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    if (w < wave) base += s_wc[w];
    n += s_wc[w];
  }
  if (row >= 0) {
    const int i = base + __popcll(bal & ((uint64_t{1} << lane) - 1));
    s_row[i] = row;
    s_g[i] = a.topk_w[row];
  }
  __syncthreads();
  constexpr int E = BF16 ? 8 : 4;
  constexpr int U = 2;
  constexpr int G = 8;
  const int64_t nch = a.d / E;
  const int nsh = a.y_shared ? a.n_shared : 0;
  for (int64_t c0 = tid; c0 < nch; c0 += U * kThreads) {
    float acc[U][E];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < E; ++e) acc[u][e] = 0.f;
    auto add = [&](float (&ac)[E], const uint4& x, float w) {
      if constexpr (BF16) {
        const uint32_t w4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ac[2 * e] = fmaf(w, bf16_to_f32(static_cast<uint16_t>(w4[e] & 0xFFFFu)), ac[2 * e]);
          ac[2 * e + 1] = fmaf(w, bf16_to_f32(static_cast<uint16_t>(w4[e] >> 16)), ac[2 * e + 1]);
        }
      } else {
        ac[0] = fmaf(w, __uint_as_float(x.x), ac[0]);
        ac[1] = fmaf(w, __uint_as_float(x.y), ac[1]);
        ac[2] = fmaf(w, __uint_as_float(x.z), ac[2]);
        ac[3] = fmaf(w, __uint_as_float(x.w), ac[3]);
      }
    };
    for (int j0 = 0; j0 < n; j0 += G) {
      uint4 v[U][G];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t c = c0 + u * kThreads;
#pragma unroll
        for (int j = 0; j < G; ++j)
          if (c < nch && j0 + j < n) v[u][j] = reinterpret_cast<const uint4*>(a.y_perm)[s_row[j0 + j] * nch + c];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t c = c0 + u * kThreads;
#pragma unroll
        for (int j = 0; j < G; ++j)
          if (c < nch && j0 + j < n) add(acc[u], v[u][j], s_g[j0 + j]);
      }
    }
    uint4 vs[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + u * kThreads;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        if (c < nch && s < nsh) vs[u][s] = reinterpret_cast<const uint4*>(a.y_shared)[(s * a.T + t) * nch + c];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + u * kThreads;
      if (c >= nch) break;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        if (s < nsh) add(acc[u], vs[u][s], 1.0f);
      uint4 o;
      if constexpr (BF16) {
        o = make_uint4(pack_bf16x2(acc[u][0], acc[u][1]), pack_bf16x2(acc[u][2], acc[u][3]),
                       pack_bf16x2(acc[u][4], acc[u][5]), pack_bf16x2(acc[u][6], acc[u][7]));
      } else {
        o = make_uint4(__float_as_uint(acc[u][0]), __float_as_uint(acc[u][1]), __float_as_uint(acc[u][2]),
                       __float_as_uint(acc[u][3]));
      }
      reinterpret_cast<uint4*>(a.y)[t * nch + c] = o;
    }
  }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  stage_mark(kStageCombine, false, s);
  if (a.ec) {
    if (a.k > kThreads) return hipErrorInvalidValue;
    if (a.act_dtype == 1)
      hipLaunchKernelGGL(combine_ec_kernel<true>, dim3(static_cast<unsigned>(a.T)), dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL(combine_ec_kernel<false>, dim3(static_cast<unsigned>(a.T)), dim3(kThreads), 0, s, a);
  } else {
    // tokens a workgroup: as many as keep TW (k + shared) <= 8 loads in flight
    const int slots = a.k + (a.y_shared ? a.n_shared : 0);
    const int tw = slots <= 1 ? 8 : (slots <= 2 ? 4 : (slots <= 4 ? 2 : 1));
    const dim3 grid(static_cast<unsigned>(ceil_div(a.T, tw)));
    if (a.act_dtype == 1) {
      if (tw == 8) hipLaunchKernelGGL((combine_kernel<true, 8>), grid, dim3(kThreads), 0, s, a);
      else if (tw == 4) hipLaunchKernelGGL((combine_kernel<true, 4>), grid, dim3(kThreads), 0, s, a);
      else if (tw == 2) hipLaunchKernelGGL((combine_kernel<true, 2>), grid, dim3(kThreads), 0, s, a);
      else hipLaunchKernelGGL((combine_kernel<true, 1>), grid, dim3(kThreads), 0, s, a);
    } else {
      if (tw == 8) hipLaunchKernelGGL((combine_kernel<false, 8>), grid, dim3(kThreads), 0, s, a);
      else if (tw == 4) hipLaunchKernelGGL((combine_kernel<false, 4>), grid, dim3(kThreads), 0, s, a);
      else if (tw == 2) hipLaunchKernelGGL((combine_kernel<false, 2>), grid, dim3(kThreads), 0, s, a);
      else hipLaunchKernelGGL((combine_kernel<false, 1>), grid, dim3(kThreads), 0, s, a);
    }
  }
  stage_mark(kStageCombine, true, s);
  return hipGetLastError();
}

}  // namespace moe
