// Rank / scan / slot pass of the permutation for one block of tokens, shared
// by the permutation kernel and the fused decode front end.
//
// Pages: aigrafen.se "Mixture of Experts" (the capacity equation; the `MoE`
// module takes, per expert, the selecting tokens in `nonzero` (ascending
// token) order and truncates the list to the capacity), vanos001 "MoE
// Architecture" / "Capacity and Token Dropping".
#pragma once

#include "common.h"
#include "kernels.h"
#include "plan.h"

namespace moe {

constexpr int kPermMaxN = 256;
constexpr int kPermMaxK = 8;

// Rank of the pairs of permutation block `bid` (of nblocks) by NTH threads:
// the first four waves hold its 256 tokens (one a lane), further waves only
// join the barriers and the block-wide loops.
// TOPK_LDS: topk_lds holds the block's top-k lists in LDS ([token][k], as
// a.topk_idx, at most 16 tokens) and is read instead of a.topk_idx.
template <int NTH, bool TOPK_LDS = false>
__device__ __forceinline__ void perm_rank_block(const PermuteArgs& a, int bid, int nblocks,
                                                const int32_t* topk_lds = nullptr) {
  __shared__ int32_t s_wcnt[4][kPermMaxN];
  // per wave and expert: the lanes (tokens) that selected it
  __shared__ unsigned long long s_mask[4][kPermMaxN];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = a.N, k = a.k;
  const int64_t t = static_cast<int64_t>(bid) * kPermTokens + wave * 64 + lane;
  const bool live = wave < 4 && t < a.T;

  for (int i = tid; i < 4 * kPermMaxN; i += NTH) {
    (&s_wcnt[0][0])[i] = 0;
    (&s_mask[0][0])[i] = 0ull;
  }

  int ex[kPermMaxK], rank[kPermMaxK];
  int lk[kPermMaxK];  // the LDS lists, read before any use (the addresses are LDS, so no flat loads)
  if constexpr (TOPK_LDS) {
    const auto* tl = (const __attribute__((address_space(3))) int32_t*)(topk_lds);
    const int tt = live ? static_cast<int>(t - static_cast<int64_t>(bid) * kPermTokens) : 0;
#pragma unroll
    for (int j = 0; j < kPermMaxK; ++j) lk[j] = j < k ? tl[tt * k + j] : -1;
  }
#pragma unroll
  for (int j = 0; j < kPermMaxK; ++j) {
    ex[j] = -1;
    rank[j] = 0;
    if (j < k && live) {
      const int e = TOPK_LDS ? lk[j] : a.topk_idx[t * k + j];
      ex[j] = (e >= 0 && e < N) ? e : -1;  // out-of-range ids are treated as dropped
    }
  }
  __syncthreads();

  // Rank of pair (token, slot j) among the wave's pairs of its expert: the
  // lanes below it whose token selected the same expert. Each lane ORs its
  // bit into the masks of its experts (the OR does not depend on the order),
  // then counts the set bits below it. The wave's count of an expert is the
  // population of its mask.
  if (wave < 4) {
    const unsigned long long bit = 1ull << lane;
#pragma unroll
    for (int j = 0; j < kPermMaxK; ++j)
      if (ex[j] >= 0) atomicOr(&s_mask[wave][ex[j]], bit);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's ORs are done
    __builtin_amdgcn_wave_barrier();
    const unsigned long long below = bit - 1ull;
#pragma unroll
    for (int j = 0; j < kPermMaxK; ++j)
      if (ex[j] >= 0) rank[j] = __popcll(s_mask[wave][ex[j]] & below);
    for (int e = lane; e < N; e += 64) s_wcnt[wave][e] = __popcll(s_mask[wave][e]);
  }
  __syncthreads();

  if (live) {
#pragma unroll
    for (int j = 0; j < kPermMaxK; ++j) {
      if (j >= k) break;
      int r = -1;
      if (ex[j] >= 0) {
        r = rank[j];
        for (int w = 0; w < wave; ++w) r += s_wcnt[w][ex[j]];
      }
      a.local_rank[t * k + j] = r;  // -1: out-of-range expert id
    }
  }
  const int64_t b = bid;
  if (nblocks > 1) {
    for (int e = tid; e < N; e += NTH)
      a.block_cnt[b * N + e] = s_wcnt[0][e] + s_wcnt[1][e] + s_wcnt[2][e] + s_wcnt[3][e];
    return;
  }

  // One block holds every token (T <= kPermTokens): the scan is this block's
  // counts, block base 0. Wave 0 scans the kept counts: lane L owns experts
  // [4L, 4L + 4), then an inclusive wave scan over the lanes (integer, exact).
  __shared__ int32_t s_off[kPermMaxN + 1];
  if (wave == 0) {
    int32_t kept4[4], sum = 0, drop = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      int32_t cnt = 0, kept = 0;
      if (e < N) {
        cnt = s_wcnt[0][e] + s_wcnt[1][e] + s_wcnt[2][e] + s_wcnt[3][e];
        kept = (a.capacity >= 0 && cnt > a.capacity) ? static_cast<int32_t>(a.capacity) : cnt;
        a.block_base[e] = 0;
        a.kept[e] = kept;
      }
      kept4[i] = kept;
      sum += kept;
      drop += cnt - kept;
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
      const int e = 4 * lane + i;
      if (e < N) {
        s_off[e] = off;
        a.offsets[e] = off;
      }
      off += kept4[i];
    }
    const int32_t total = __shfl(incl, 63);
    if (lane == 0) {
      s_off[N] = total;
      a.offsets[N] = total;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) drop += __shfl_xor(drop, o);
    if (lane == 0) *a.n_dropped = drop;
  }
  // the FFN's group plan, when asked; with no rows to copy also the slots
  // (no scatter pass runs)
  __syncthreads();
  if (a.plan.up) {
    __shared__ int32_t s_mt[2 * kMaxGroups];
    plan_groups(s_off, a.plan, s_mt, tid, NTH);
  }
  if (a.x_perm || !live) return;
#pragma unroll
  for (int j = 0; j < kPermMaxK; ++j) {
    if (j >= k) break;
    int32_t row = -1;
    if (ex[j] >= 0) {
      int r = rank[j];
      for (int w = 0; w < wave; ++w) r += s_wcnt[w][ex[j]];
      if (a.capacity < 0 || r < a.capacity) row = s_off[ex[j]] + r;
    }
    a.inv_map[t * k + j] = row;
    if (row >= 0) a.perm_token[row] = static_cast<int32_t>(t);
  }
}

}  // namespace moe
