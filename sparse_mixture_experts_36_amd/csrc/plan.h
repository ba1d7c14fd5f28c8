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
  if (tid == 0) {
    int32_t acc = 0, n_active = 0;
    for (int g = 0; g < G; ++g) {
      pl.tile_start[g] = acc;
      acc += s_mt[g];
      if (s_mt[g] > 0) pl.active[1 + n_active++] = g;
    }
    pl.tile_start[G] = acc;
    pl.active[0] = n_active;
  } else if (tid == 1 && pl.bm_t > 0) {
    int32_t acc = 0;
    for (int g = 0; g < G; ++g) {
      pl.tile_start_t[g] = acc;
      acc += s_mt[G + g];
    }
    pl.tile_start_t[G] = acc;
  } else if (pl.tile_start_c && tid >= 2 && tid < 6) {  // per-width prefixes: width c, plan t
    const uint32_t c = static_cast<uint32_t>(tid - 2) >> 1;
    const int t = (tid - 2) & 1;
    if (t == 0 || pl.bm_t > 0) {
      int32_t* ts = pl.tile_start_c + (2 * c + t) * (G + 1);
      int32_t acc = 0;
      for (int g = 0; g < G; ++g) {
        ts[g] = acc;
        if (((pl.cls1[g >> 5] >> (g & 31)) & 1u) == c) acc += s_mt[t * G + g];
      }
      ts[G] = acc;
    }
  }
  __syncthreads();
}

}  // namespace moe
