// Group plan of the grouped expert FFN, shared by the plan kernel and by the
// one-block permutation (which has the expert offsets at hand and so saves the
// plan's launch on decode-sized layers).
#pragma once

#include "kernels.h"

namespace moe {

// Group descriptors of both GEMMs and the row-tile prefix for tile height bm.
// Routed expert e: rows [offsets[e], offsets[e+1]) of x_perm / h / y_perm,
// clamped to the reserved routed rows. Shared expert s: the T token rows; its
// hidden rows sit after the routed ones in h, its outputs in y_shared[s].
// With bm_t > 0, a group of at most kSmallGroupTiles * bm_t rows goes to the
// second plan (bm_t-row tiles, a second launch) whole: its few row tiles then
// run side by side there and share each weight tile in L2, where a separate
// tail tile would stream the expert's weights from HBM a second time. A larger
// group whose last tile would hold r <= bm_t rows gives those r rows to the
// second plan (one tile) and keeps the rest: less padding in its last tile.
// active[0] = the number of groups with
// rows, active[1..] those groups in order. Run by all threads of one
// workgroup; s_mt holds 2 (n_routed + n_shared) ints of LDS. Ends with a
// workgroup barrier.
__device__ __forceinline__ void plan_groups(const int32_t* offsets, const FfnPlan& pl, int32_t* s_mt, int tid,
                                            int nthreads) {
  const int G = pl.n_routed + pl.n_shared;
  for (int g = tid; g < G; g += nthreads) {
    GroupDesc u, dn;
    if (g < pl.n_routed) {
      int r0 = offsets[g], r1 = offsets[g + 1];
      r0 = max(0, min(r0, pl.cap));
      r1 = max(r0, min(r1, pl.cap));
      u.a_row0 = u.c_row0 = dn.a_row0 = dn.c_row0 = r0;
      u.rows = dn.rows = r1 - r0;
    } else {
      const int s = g - pl.n_routed;
      u.a_row0 = 0;
      u.c_row0 = pl.cap + s * pl.T;
      dn.a_row0 = pl.cap + s * pl.T;
      dn.c_row0 = s * pl.T;
      u.rows = dn.rows = pl.T;
    }
    u.widx = dn.widx = g;
    int tail = 0;
    if (pl.bm_t > 0) {
      const int rem = u.rows % pl.bm;
      if (u.rows <= kSmallGroupTiles * pl.bm_t) tail = u.rows;
      else if (rem > 0 && rem <= pl.bm_t) tail = rem;
      const int keep = u.rows - tail;
      GroupDesc ut = u, dt = dn;
      ut.a_row0 += keep;
      ut.c_row0 += keep;
      dt.a_row0 += keep;
      dt.c_row0 += keep;
      ut.rows = dt.rows = tail;
      pl.up_t[g] = ut;
      pl.down_t[g] = dt;
      u.rows = dn.rows = keep;
      s_mt[G + g] = (tail + pl.bm_t - 1) / pl.bm_t;
    }
    pl.up[g] = u;
    pl.down[g] = dn;
    s_mt[g] = (u.rows + pl.bm - 1) / pl.bm;
  }
  __syncthreads();
  // The prefixes, one wave each, 64 groups at a time (a wave scan carried
  // across the chunks): job 0 the bm-row tile prefix and the active list
  // (compacted by ballot, in group order), job 1 the tail tiles' prefix,
  // jobs 2..5 the per-width prefixes (width c = (job - 2) / 2, plan t =
  // (job - 2) % 2). Integer sums: the same values as a serial loop.
  const int lane = tid & 63, wave = tid >> 6, nwaves = nthreads >> 6;
  for (int job = wave; job < 6; job += nwaves) {
    int32_t* ts = nullptr;
    int src = 0;            // s_mt offset of the counts summed
    uint32_t cls = 2u;      // per-width jobs: the width class summed (2: all groups)
    if (job == 0) {
      ts = pl.tile_start;
    } else if (job == 1) {
      if (pl.bm_t <= 0) continue;
      ts = pl.tile_start_t;
      src = G;
    } else {
      if (!pl.tile_start_c) continue;
      cls = static_cast<uint32_t>(job - 2) >> 1;
      const int t = (job - 2) & 1;
      if (t == 1 && pl.bm_t <= 0) continue;
      ts = pl.tile_start_c + (2 * cls + t) * (G + 1);
      src = t * G;
    }
    int32_t base = 0, n_active = 0;
    for (int g0 = 0; g0 < G; g0 += 64) {
      const int g = g0 + lane;
      int32_t v = 0;
      if (g < G && (cls == 2u || ((pl.cls1[g >> 5] >> (g & 31)) & 1u) == cls)) v = s_mt[src + g];
      int32_t incl = v;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int32_t u = __shfl_up(incl, o);
        if (lane >= o) incl += u;
      }
      if (g < G) ts[g] = base + incl - v;
      if (job == 0) {
        const bool act = g < G && s_mt[g] > 0;
        const uint64_t m = __ballot(act);
        if (act) pl.active[1 + n_active + __popcll(m & ((1ull << lane) - 1ull))] = g;
        n_active += __popcll(m);
      }
      base += __shfl(incl, 63);
    }
    if (lane == 0) {
      ts[G] = base;
      if (job == 0) pl.active[0] = n_active;
    }
  }
  __syncthreads();
}

}  // namespace moe
