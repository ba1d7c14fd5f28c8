// Grouped GEMM with per-group row ranges taken from device offsets, in any of
// the operand layouts the layer's backward pass needs:
//   C_g(m, n) (+)= sum_k A_g(m, k) B_g(k, n),   bf16 operands, fp32 accumulation.
// Group g owns rows [r0, r1) of a row space (the permuted rows of expert g, or
// the T token rows of a shared expert). In rows-M form those rows are A's and
// C's rows; in rows-K form they are the contraction, so every group has its
// own k range and writes its own output matrix. The expert products of large
// layers run on the LDS-DMA kernels (the forward's grouped FFN for the
// recompute, bgemm_dma for the gradients); this register-staged kernel takes
// the router's products (dl^T x, dl W_r) and the recompute of layers below
// those kernels' row threshold (U = X W1^T, Y = H W2^T).
//
// Tiles of 128 x 256 outputs (m x n), 4 waves (2 x 2), each 64 x 128 as
// 4 x 8 MFMA 16x16x32 fragments; k-steps of 64 through LDS rows of 64 k (+8 pad), the
// next step's global loads in flight while the current one computes.
// An operand stored k-contiguous is copied in 16-byte chunks. One stored m-
// (or n-) contiguous is loaded as 4 k-rows x 8 columns per thread (four
// 16-byte loads), transposed in registers and written as eight 8-byte runs
// of 4 k. The 16-byte k-chunks of LDS row R sit at chunk ^ ((R / 8) % 8), so
// that those writes spread over the banks. Rows, columns and k past the ends
// load zeros; outputs past the ends are not written.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kT = 128;   // tile rows (m)
constexpr int kBN = 256;  // tile columns (n)
constexpr int kFN = kBN / 32;  // n fragments per wave
constexpr int kBK = 64;   // k per step
constexpr int kLS = kBK + 8;  // LDS row (bf16): 144 bytes

__device__ __forceinline__ int group_rows(const BGemm& p, int g, int& r0) {
  if (!p.off) {
    r0 = 0;
    return p.rows_all;
  }
  const int a = max(0, min(p.off[g], p.cap)), b = max(a, min(p.off[g + 1], p.cap));
  r0 = a;
  return b - a;
}

// Row-tile prefix of a rows-M GEMM from its offsets (one workgroup).
__global__ __launch_bounds__(kThreads) void bgemm_plan_kernel(BGemm p, int32_t* tile_start) {
  __shared__ int32_t s_mt[kMaxGroups];
  for (int g = threadIdx.x; g < p.n_groups; g += kThreads) {
    int r0;
    s_mt[g] = (group_rows(p, g, r0) + kT - 1) / kT;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t acc = 0;
    for (int g = 0; g < p.n_groups; ++g) {
      tile_start[g] = acc;
      acc += s_mt[g];
    }
    tile_start[p.n_groups] = acc;
  }
}

// LDS element offset of (row, 16-byte k-chunk c) with the chunk swizzle.
__device__ __forceinline__ int lds_at(int row, int c) { return row * kLS + ((c ^ ((row >> 3) & 7)) << 3); }

// One operand tile (ROWS rows x 64 k) per k-step. KC: element (row, k) at
// src[row * ld + k], ROWS / 32 16-byte chunks a thread; otherwise at
// src[k * ld + row], ROWS / 128 units of 4 k-rows x 8 rows a thread. Rows >=
// nrows and k >= nk read as zero.
template <bool KC, int ROWS>
struct Stage {
  static constexpr int NV = KC ? ROWS / 32 : 4 * (ROWS / 128);
  static constexpr int RC = ROWS / 8;  // 8-row chunks (transposed form)
  uint4 v[NV];
  __device__ __forceinline__ void load(const uint16_t* src, int64_t ld, int nrows, int nk, int k0, int tid) {
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = make_uint4(0, 0, 0, 0);
    if (KC) {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int c = tid + i * kThreads, row = c >> 3, k = k0 + (c & 7) * 8;
        if (row < nrows && k < nk) v[i] = *reinterpret_cast<const uint4*>(src + static_cast<int64_t>(row) * ld + k);
      }
    } else {
#pragma unroll
      for (int u = 0; u < NV / 4; ++u) {
        const int t = tid + u * kThreads, row = (t % RC) * 8, kq = t / RC;
        if (row < nrows) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int k = k0 + kq * 4 + i;
            if (k < nk) v[4 * u + i] = *reinterpret_cast<const uint4*>(src + static_cast<int64_t>(k) * ld + row);
          }
        }
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* S, int tid) const {
    if (KC) {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int c = tid + i * kThreads;
        *reinterpret_cast<uint4*>(S + lds_at(c >> 3, c & 7)) = v[i];
      }
    } else {
      // v[4u + i] holds rows 8mc..8mc+7 at k = 4kq + i; each row's four k go
      // to one 8-byte run
#pragma unroll
      for (int u = 0; u < NV / 4; ++u) {
        const int t = tid + u * kThreads, mc = t % RC, kq = t / RC;
        const uint4* x = v + 4 * u;
        const uint32_t w[4][4] = {{x[0].x, x[0].y, x[0].z, x[0].w}, {x[1].x, x[1].y, x[1].z, x[1].w},
                                  {x[2].x, x[2].y, x[2].z, x[2].w}, {x[3].x, x[3].y, x[3].z, x[3].w}};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint2 lo = make_uint2((w[0][j] & 0xFFFFu) | (w[1][j] << 16), (w[2][j] & 0xFFFFu) | (w[3][j] << 16));
          const uint2 hi = make_uint2((w[0][j] >> 16) | (w[1][j] & 0xFFFF0000u),
                                      (w[2][j] >> 16) | (w[3][j] & 0xFFFF0000u));
          const int r = mc * 8 + 2 * j;
          *reinterpret_cast<uint2*>(S + lds_at(r, kq >> 1) + (kq & 1) * 4) = lo;
          *reinterpret_cast<uint2*>(S + lds_at(r + 1, kq >> 1) + (kq & 1) * 4) = hi;
        }
      }
    }
  }
};

template <bool ROWS_K, bool B_KC, bool ACC>
__global__ __launch_bounds__(kThreads, 2) void bgemm_kernel(BGemm p, const int32_t* tile_start) {
  __shared__ __attribute__((aligned(16))) uint16_t As[kT * kLS];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kBN * kLS];
  const int ntn = (p.N + kBN - 1) / kBN;
  int g, mt, nt;
  if (ROWS_K || !p.off) {
    const int mtn = ((ROWS_K ? p.M : p.rows_all) + kT - 1) / kT;
    const int L = blockIdx.x;
    if (L >= p.n_groups * mtn * ntn) return;
    g = L / (mtn * ntn);
    nt = (L % (mtn * ntn)) / mtn;
    mt = L % mtn;
  } else {
    const int L = blockIdx.x;
    if (L >= tile_start[p.n_groups] * ntn) return;
    int lo = 0, hi = p.n_groups - 1;  // largest g with tile_start[g] * ntn <= L
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tile_start[mid] * ntn <= L) lo = mid; else hi = mid - 1;
    }
    g = lo;
    const int mtg = tile_start[g + 1] - tile_start[g];
    const int local = L - tile_start[g] * ntn;
    nt = local / mtg;  // the row tiles of one weight tile run next to each other
    mt = local % mtg;
  }
  int r0;
  const int rows = group_rows(p, g, r0);
  const int M = ROWS_K ? p.M : rows;
  const int K = ROWS_K ? rows : p.K;
  const int m0 = mt * kT, n0 = nt * kBN;
  if (!ROWS_K && m0 >= M) return;

  // A tile source: rows-M k-contiguous rows r0 + m0.., rows-K [k][m] from row r0
  const uint16_t* A = p.A + p.a_gs * g +
                      (ROWS_K ? static_cast<int64_t>(r0) * p.lda + m0 : static_cast<int64_t>(r0 + m0) * p.lda);
  const uint16_t* B = p.B + p.b_gs * g +
                      (B_KC ? static_cast<int64_t>(n0) * p.ldb
                            : static_cast<int64_t>(ROWS_K ? r0 : 0) * p.ldb + n0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int q = lane >> 4, c16 = lane & 15;

  floatx4_t acc[4][kFN];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < kFN; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  Stage<!ROWS_K, kT> sa;
  Stage<B_KC, kBN> sb;
  if (K > 0) {
    sa.load(A, p.lda, M - m0, K, 0, tid);
    sb.load(B, p.ldb, p.N - n0, K, 0, tid);
  }
  for (int k0 = 0; k0 < K; k0 += kBK) {
    sa.store(As, tid);
    sb.store(Bs, tid);
    __syncthreads();
    if (k0 + kBK < K) {  // in flight during this step's MFMAs
      sa.load(A, p.lda, M - m0, K, k0 + kBK, tid);
      sb.load(B, p.ldb, p.N - n0, K, k0 + kBK, tid);
    }
#pragma unroll
    for (int s2 = 0; s2 < kBK / 32; ++s2) {
      // the A fragments stay in registers; the B fragments are read one at a
      // time, so that the accumulators and both stages fit two waves a SIMD
      uint4 af[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = *reinterpret_cast<const uint4*>(As + lds_at(wm * 64 + i * 16 + c16, s2 * 4 + q));
#pragma unroll
      for (int j = 0; j < kFN; ++j) {
        const uint4 bf = *reinterpret_cast<const uint4*>(Bs + lds_at(wn * (kBN / 2) + j * 16 + c16, s2 * 4 + q));
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i][j] = mfma16x16x32(af[i], bf, acc[i][j]);
      }
    }
    __syncthreads();
  }

  // lane (q, c16) of fragment (i, j): rows 4q + r, column c16
  const int64_t crow0 = ROWS_K ? 0 : r0;
  float* Cg = static_cast<float*>(p.C) + p.c_gs * g;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + wm * 64 + i * 16 + q * 4 + r;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < kFN; ++j) {
        const int n = n0 + wn * (kBN / 2) + j * 16 + c16;
        if (n >= p.N) continue;
        float* C = Cg + (crow0 + m) * p.ldc + n;
        *C = ACC ? *C + acc[i][j][r] : acc[i][j][r];
      }
    }
}

}  // namespace

hipError_t launch_bgemm(const BGemm& p, bool rows_k, bool b_kc, bool acc, int32_t* tile_start, hipStream_t s) {
  if (p.n_groups <= 0 || p.N <= 0) return hipSuccess;
  const int ntn = (p.N + kBN - 1) / kBN;
  int64_t grid;
  if (rows_k || !p.off) {
    grid = static_cast<int64_t>(p.n_groups) * (((rows_k ? p.M : p.rows_all) + kT - 1) / kT) * ntn;
  } else {
    hipLaunchKernelGGL(bgemm_plan_kernel, dim3(1), dim3(kThreads), 0, s, p, tile_start);
    grid = (static_cast<int64_t>(p.cap) / kT + p.n_groups) * ntn;  // every group may end in a partial tile
  }
  if (grid <= 0) return hipSuccess;
  const dim3 gd(static_cast<unsigned>(grid));
#define MOE_BG(RK, BK, AC)                                                                          \
  if (rows_k == RK && b_kc == BK && acc == AC) {                                                    \
    hipLaunchKernelGGL((bgemm_kernel<RK, BK, AC>), gd, dim3(kThreads), 0, s, p, tile_start);        \
    return hipGetLastError();                                                                       \
  }
  MOE_BG(false, true, false)   // forward recompute: U = X W^T, Y = H W2^T
  MOE_BG(false, false, false)  // dH = dY W2, dX = dU W1, dl W_r
  MOE_BG(false, false, true)   // dX += dV W3, += dl_lo W_r
  MOE_BG(true, false, false)   // dW = dY^T H, dU^T X, dl^T x
  MOE_BG(true, false, true)    // dW_r += dl_lo^T x
#undef MOE_BG
  return hipErrorInvalidValue;
}

}  // namespace moe
