// Dispatch with expert capacity: histogram -> scan -> rank/drop -> gather.
//
// Pages: aigrafen.se "Mixture of Experts" (the capacity equation; the `MoE`
// module takes, per expert, the selecting tokens in `nonzero` (ascending
// token) order and truncates the list to the capacity), vanos001 "MoE
// Architecture" / "Capacity and Token Dropping".
//
// The rank of pair (t, j) with expert e is the number of tokens t' < t that
// also selected e. It is built without any order-dependent atomics:
//  1. rank kernel: per 256-token block, each wave ranks its 64 tokens with
//     ballots (one pass per distinct expert in the wave), waves are combined in
//     wave order, and the block's per-expert counts are written;
//  2. scan kernel (one workgroup): per expert, an exclusive scan of the block
//     counts in block order, the capacity cut, and the expert offsets;
//  3. scatter kernel: one wave per token writes inv_map / perm_token and copies
//     the token's row once into each of its kept slots (x read once).
// With at most 256 tokens the rank kernel's one block also does the scan, and
// when no rows are copied (the caller's FFN reads x through perm_token) it
// writes inv_map / perm_token itself: one launch instead of three.
#include "common.h"
#include "kernels.h"
#include "perm_block.h"
#include "route_block.h"
#include "plan.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxN = 256;
constexpr int kMaxK = 8;

__global__ __launch_bounds__(kThreads) void perm_rank_kernel(PermuteArgs a) {
  perm_rank_block<kThreads>(a, blockIdx.x, gridDim.x);
}

// One workgroup of 1024 threads: per expert, the exclusive scan of the block
// counts in block order (block_base), the capacity cut, and the expert
// offsets. Expert e's nb counts are cut into S contiguous segments, one
// thread each (S <= 1024 / NP, NP the power of two >= N, and at least 16
// blocks a segment): segment sums (16 loads in flight), an in-order scan of
// the segments, then each segment writes its blocks' bases. Integer
// arithmetic: the result is exact.
constexpr int kScanThreads = 1024;
constexpr int kScanBatch = 16;

__global__ __launch_bounds__(kScanThreads) void perm_scan_kernel(PermuteArgs a, int nb) {
  static_assert(kScanThreads == kFinThreads, "the routing finalize runs on the scan workgroup");
  if (a.fin_nb > 0) {  // the routing statistics first
    route_finalize_block(a.fin, a.fin_nb);
    __syncthreads();
  }
  __shared__ int32_t s_seg[kScanThreads];
  __shared__ int32_t s_kept[kMaxN];
  __shared__ int32_t s_drop[kMaxN];
  const int tid = threadIdx.x, N = a.N;
  int NP = 1;
  while (NP < N) NP <<= 1;
  // at least one full batch of loads per segment
  const int S = min(kScanThreads / NP, max(1, (nb + kScanBatch - 1) / kScanBatch));
  const int e = tid % NP, seg = tid / NP;
  const bool mine = e < N && seg < S;
  const int b0 = static_cast<int>((static_cast<int64_t>(seg) * nb) / S);
  const int b1 = static_cast<int>((static_cast<int64_t>(seg + 1) * nb) / S);
  if (mine) {
    int32_t sum = 0;
    for (int b = b0; b < b1; b += kScanBatch) {
      int32_t v[kScanBatch];
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i)
        if (b + i < b1) v[i] = a.block_cnt[static_cast<int64_t>(b + i) * N + e];
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i)
        if (b + i < b1) sum += v[i];
    }
    s_seg[tid] = sum;
  }
  __syncthreads();
  if (tid < N) {  // segments of expert tid in order: exclusive offsets, then the totals
    int32_t run = 0;
    for (int sg = 0; sg < S; ++sg) {
      const int32_t v = s_seg[sg * NP + tid];
      s_seg[sg * NP + tid] = run;
      run += v;
    }
    int32_t kept = run;
    if (a.capacity >= 0 && kept > a.capacity) kept = static_cast<int32_t>(a.capacity);
    s_kept[tid] = kept;
    s_drop[tid] = run - kept;
    a.kept[tid] = kept;
  }
  __syncthreads();
  if (mine) {
    int32_t run = s_seg[tid];
    for (int b = b0; b < b1; b += kScanBatch) {
      int32_t v[kScanBatch];
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i)
        if (b + i < b1) v[i] = a.block_cnt[static_cast<int64_t>(b + i) * N + e];
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i)
        if (b + i < b1) {
          a.block_base[static_cast<int64_t>(b + i) * N + e] = run;
          run += v[i];
        }
    }
  }
  // offsets: exclusive scan of the kept counts by wave 0, lane L owning
  // experts [4L, 4L + 4) (integer, exact)
  __shared__ int32_t s_off[kMaxN + 1];
  if (tid < 64) {
    const int lane = tid;
    int32_t kept4[4], sum = 0, drop = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int x = 4 * lane + i;
      kept4[i] = x < N ? s_kept[x] : 0;
      sum += kept4[i];
      drop += x < N ? s_drop[x] : 0;
    }
    int32_t incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t v = __shfl_up(incl, o);
      if (lane >= o) incl += v;
    }
    int32_t off = incl - sum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int x = 4 * lane + i;
      if (x < N) {
        a.offsets[x] = off;
        s_off[x] = off;
      }
      off += kept4[i];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) drop += __shfl_xor(drop, o);
    const int32_t total = __shfl(incl, 63);
    if (lane == 0) {
      a.offsets[N] = total;
      s_off[N] = total;
      *a.n_dropped = drop;
    }
  }
  if (a.plan.up) {  // the FFN's group plan from the offsets just formed
    __shared__ int32_t s_mt[2 * kMaxGroups];
    __syncthreads();
    plan_groups(s_off, a.plan, s_mt, tid, kScanThreads);
  }
}

// One wave per token. Copies move 16-byte chunks; x is read once per token.
__global__ __launch_bounds__(kThreads) void perm_scatter_kernel(PermuteArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  if (t >= a.T) return;
  const int N = a.N, k = a.k;
  const int64_t blk = t / kPermTokens;
  // the token's first 64*U chunks are loaded before the chain of index loads
  // below, so the two latencies overlap
  constexpr int U = 8;
  const int64_t nchunk = a.x_perm ? a.d * a.act_bytes / 16 : 0;
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(static_cast<const char*>(a.x) + t * a.d * a.act_bytes);
  u32x4_t v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t c = u * 64 + lane;
    if (c < nchunk) v[u] = src[c];
  }
  int64_t row[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    row[j] = -1;
    if (j < k) {
      const int e = a.topk_idx[t * k + j];
      const int r = a.local_rank[t * k + j];
      if (r >= 0 && e >= 0 && e < N) {
        const int64_t rank = static_cast<int64_t>(a.block_base[blk * N + e]) + r;
        if (a.capacity < 0 || rank < a.capacity) row[j] = a.offsets[e] + rank;
      }
      if (lane == 0) {
        a.inv_map[t * k + j] = static_cast<int32_t>(row[j]);
        if (row[j] >= 0) a.perm_token[row[j]] = static_cast<int32_t>(t);
      }
    }
  }
  if (!a.x_perm) return;
  // lane j keeps slot j's row, read back one slot at a time: a loop over the
  // slots then needs no per-slot registers for addresses
  int32_t rowv = -1;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    if (lane == j) rowv = static_cast<int32_t>(row[j]);
  const int64_t ochunk = a.ld_out * a.act_bytes / 16;  // 16-byte chunks per x_perm row
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(a.x_perm);
  for (int64_t c0 = 0; c0 < nchunk; c0 += 64 * U) {
    if (c0 > 0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t c = c0 + u * 64 + lane;
        if (c < nchunk) v[u] = src[c];
      }
    }
#pragma unroll 1
    for (int j = 0; j < k; ++j) {
      const int32_t r = __builtin_amdgcn_readlane(rowv, j);
      if (r < 0) continue;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t c = c0 + u * 64 + lane;
        if (c < nchunk) dst[static_cast<int64_t>(r) * ochunk + c] = v[u];
      }
    }
  }
}

// Expert choice: expert e's j-th token sits in row e*C + j, so the offsets are
// e*C. One wave per token finds, for every expert (a lane each), the token in
// that expert's ascending list by binary search; it writes inv_map[t][e] and
// perm_token, lists its rows in expert order, and copies the token's row (read
// once) into each of them. Block 0 writes the offsets (and the FFN group plan
// when asked). Tokens taken by no expert are counted per block.
__global__ __launch_bounds__(kThreads) void ec_permute_kernel(PermuteArgs a) {
  __shared__ int32_t s_off[kMaxN + 1];
  __shared__ int32_t s_mt[2 * kMaxGroups];
  __shared__ int32_t s_none[4];
  __shared__ int32_t s_rows[4][kMaxN];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = a.N;
  const int32_t C = static_cast<int32_t>(a.capacity);
  if (blockIdx.x == 0) {
    for (int e = tid; e <= N; e += kThreads) {
      a.offsets[e] = e * C;
      s_off[e] = e * C;
      if (e < N && a.kept) a.kept[e] = C;
    }
    if (a.plan.up) {
      __syncthreads();
      plan_groups(s_off, a.plan, s_mt, tid, kThreads);
    }
  }
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  const bool live = t < a.T;
  constexpr int U = 8;
  const int64_t nchunk = (a.x_perm && live) ? a.d * a.act_bytes / 16 : 0;
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(static_cast<const char*>(a.x) + (live ? t : 0) * a.d * a.act_bytes);
  // the token's first 64*U chunks are loaded before the searches, so the two
  // latencies overlap
  u32x4_t v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t c = u * 64 + lane;
    if (c < nchunk) v[u] = src[c];
  }
  int nrows = 0;  // rows of this token, listed in s_rows[wave] in expert order
  for (int e0 = 0; e0 < N; e0 += 64) {
    const int e = e0 + lane;
    int32_t row = -1;
    if (live && e < N) {
      if (C > 0) {
        const int32_t* list = a.topk_idx + static_cast<int64_t>(e) * C;
        int lo = 0, hi = C;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (list[mid] < t) lo = mid + 1;
          else hi = mid;
        }
        if (lo < C && list[lo] == t) row = e * C + lo;
      }
      a.inv_map[t * N + e] = row;
      if (row >= 0) a.perm_token[row] = static_cast<int32_t>(t);
    }
    const uint64_t found = __ballot(row >= 0);
    if (row >= 0) s_rows[wave][nrows + __popcll(found & ((uint64_t{1} << lane) - 1))] = row;
    nrows += __popcll(found);
  }
  __syncthreads();
  const int64_t ochunk = a.ld_out * a.act_bytes / 16;
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(a.x_perm);
  for (int64_t c0 = 0; c0 < nchunk; c0 += 64 * U) {
    if (c0 > 0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t c = c0 + u * 64 + lane;
        if (c < nchunk) v[u] = src[c];
      }
    }
    for (int j = 0; j < nrows; ++j) {
      const int64_t r = s_rows[wave][j];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t c = c0 + u * 64 + lane;
        if (c < nchunk) dst[r * ochunk + c] = v[u];
      }
    }
  }
  const bool taken = nrows > 0;
  if (a.n_dropped) {
    if (lane == 0) s_none[wave] = (live && !taken) ? 1 : 0;
    __syncthreads();
    if (tid == 0) a.ec_part[blockIdx.x] = s_none[0] + s_none[1] + s_none[2] + s_none[3];
  }
}

// Sum of the per-block counts of tokens no expert took.
__global__ __launch_bounds__(1024) void ec_untouched_kernel(PermuteArgs a, int nb) {
  __shared__ int32_t s_w[16];
  int32_t c = 0;
  for (int b = threadIdx.x; b < nb; b += 1024) c += a.ec_part[b];
  c = wave_sum(c);
  if ((threadIdx.x & 63) == 0) s_w[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t tot = 0;
    for (int w = 0; w < 16; ++w) tot += s_w[w];
    *a.n_dropped = tot;
  }
}

}  // namespace

hipError_t launch_permute(const PermuteArgs& a, hipStream_t s) {
  if (a.ec) {
    if (a.T <= 0) return hipSuccess;
    const int nb = static_cast<int>(ceil_div(a.T, 4));
    stage_mark(kStagePermute, false, s);
    hipLaunchKernelGGL(ec_permute_kernel, dim3(nb), dim3(kThreads), 0, s, a);
    if (a.n_dropped) hipLaunchKernelGGL(ec_untouched_kernel, dim3(1), dim3(1024), 0, s, a, nb);
    stage_mark(kStagePermute, true, s);
    return hipGetLastError();
  }
  if (a.T <= 0) {
    // no tokens: the scan over zero blocks writes the empty layout
    hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, a, 0);
    return hipGetLastError();
  }
  const int nb = static_cast<int>(ceil_div(a.T, kPermTokens));
  stage_mark(kStagePermute, false, s);
  hipLaunchKernelGGL(perm_rank_kernel, dim3(nb), dim3(kThreads), 0, s, a);
  // one rank block also scans, and without rows to copy also writes the slots
  if (nb > 1) hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, a, nb);
  if (nb > 1 || a.x_perm)
    hipLaunchKernelGGL(perm_scatter_kernel, dim3(static_cast<unsigned>(ceil_div(a.T, 4))), dim3(kThreads), 0, s,
                       a);
  stage_mark(kStagePermute, true, s);
  return hipGetLastError();
}

}  // namespace moe
