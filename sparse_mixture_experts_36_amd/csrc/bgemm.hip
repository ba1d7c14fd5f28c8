// Grouped GEMM with per-group row ranges taken from device offsets, in any of
// the operand layouts the layer's backward pass needs:
//   C_g(m, n) (+)= sum_k A_g(m, k) B_g(k, n),   bf16 operands, fp32 accumulation.
// Group g owns rows [r0, r1) of a row space (the permuted rows of expert g, or
// the T token rows of a shared expert). In rows-M form those rows are A's and
// C's rows (dH = dY W2, dX = dU W1, and the forward's U = X W1^T); in rows-K
// form they are the contraction (dW2 = dY^T H, dW1 = dU^T X), so every group
// has its own k range and writes its own output matrix.
//
// Tiles of 128 x 128 outputs, 4 waves (2 x 2), each 64 x 64 as 4 x 4 MFMA
// 16x16x32 fragments; k-steps of 32 through LDS rows of 32 k (+8 pad). An
// operand stored k-contiguous is copied to LDS in 16-byte chunks; one stored
// with m (or n) contiguous is loaded in 16-byte chunks along m and written to
// LDS transposed, one bf16 at a time. The next k-step's global loads are in
// flight while the current one computes. Rows, columns and k past the ends
// load zeros; outputs past the ends are not written.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kT = 128;   // tile edge
constexpr int kBK = 32;   // k per step
constexpr int kLS = kBK + 8;  // LDS row (bf16): 80 bytes

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

template <bool ROWS_K, bool B_KC, bool C_F32, bool ACC>
__global__ __launch_bounds__(kThreads) void bgemm_kernel(BGemm p, const int32_t* tile_start) {
  __shared__ __attribute__((aligned(16))) uint16_t As[kT * kLS];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kT * kLS];
  const int ntn = (p.N + kT - 1) / kT;
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
  const int m0 = mt * kT, n0 = nt * kT;
  if (!ROWS_K && m0 >= M) return;

  const uint16_t* A = p.A + p.a_gs * g + (ROWS_K ? 0 : static_cast<int64_t>(r0 + m0) * p.lda);
  const uint16_t* B = p.B + p.b_gs * g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int q = lane >> 4, c16 = lane & 15;

  // two 16-byte chunks per operand and thread and k-step
  auto load = [&](int k0, uint4 (&ra)[2], uint4 (&rb)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + i * kThreads;
      ra[i] = make_uint4(0, 0, 0, 0);
      rb[i] = make_uint4(0, 0, 0, 0);
      if (!ROWS_K) {  // A k-contiguous: row c / 4, k chunk c % 4
        const int r = c >> 2, k = k0 + (c & 3) * 8;
        if (m0 + r < M && k < K) ra[i] = *reinterpret_cast<const uint4*>(A + static_cast<int64_t>(r) * p.lda + k);
      } else {  // A m-contiguous: k row c / 16, m chunk c % 16
        const int kk = c >> 4, m = m0 + (c & 15) * 8;
        if (k0 + kk < K && m < M)
          ra[i] = *reinterpret_cast<const uint4*>(A + static_cast<int64_t>(r0 + k0 + kk) * p.lda + m);
      }
      if (B_KC) {  // B(k, n) at B[n ldb + k]: row n = c / 4, k chunk c % 4
        const int n = n0 + (c >> 2), k = k0 + (c & 3) * 8;
        if (n < p.N && k < K) rb[i] = *reinterpret_cast<const uint4*>(B + static_cast<int64_t>(n) * p.ldb + k);
      } else {  // B(k, n) at B[(k (+ r0)) ldb + n]: k row c / 16, n chunk c % 16
        const int kk = c >> 4, n = n0 + (c & 15) * 8;
        const int64_t brow = (ROWS_K ? r0 : 0) + k0 + kk;
        if (k0 + kk < K && n < p.N) rb[i] = *reinterpret_cast<const uint4*>(B + brow * p.ldb + n);
      }
    }
  };
  auto store = [&](const uint4 (&ra)[2], const uint4 (&rb)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + i * kThreads;
      if (!ROWS_K) {
        *reinterpret_cast<uint4*>(As + (c >> 2) * kLS + (c & 3) * 8) = ra[i];
      } else {
        const int kk = c >> 4, m = (c & 15) * 8;
        const uint32_t w[4] = {ra[i].x, ra[i].y, ra[i].z, ra[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          As[(m + 2 * e) * kLS + kk] = static_cast<uint16_t>(w[e] & 0xFFFFu);
          As[(m + 2 * e + 1) * kLS + kk] = static_cast<uint16_t>(w[e] >> 16);
        }
      }
      if (B_KC) {
        *reinterpret_cast<uint4*>(Bs + (c >> 2) * kLS + (c & 3) * 8) = rb[i];
      } else {
        const int kk = c >> 4, n = (c & 15) * 8;
        const uint32_t w[4] = {rb[i].x, rb[i].y, rb[i].z, rb[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          Bs[(n + 2 * e) * kLS + kk] = static_cast<uint16_t>(w[e] & 0xFFFFu);
          Bs[(n + 2 * e + 1) * kLS + kk] = static_cast<uint16_t>(w[e] >> 16);
        }
      }
    }
  };

  floatx4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  uint4 ra[2], rb[2];
  if (K > 0) load(0, ra, rb);
  for (int k0 = 0; k0 < K; k0 += kBK) {
    store(ra, rb);
    __syncthreads();
    if (k0 + kBK < K) load(k0 + kBK, ra, rb);  // in flight during this step's MFMAs
    uint4 af[4], bf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      af[i] = *reinterpret_cast<const uint4*>(As + (wm * 64 + i * 16 + c16) * kLS + q * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      bf[j] = *reinterpret_cast<const uint4*>(Bs + (wn * 64 + j * 16 + c16) * kLS + q * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(af[i], bf[j], acc[i][j]);
    __syncthreads();
  }

  // lane (q, c16) of fragment (i, j): rows 4q + r, column c16
  const int64_t crow0 = ROWS_K ? 0 : r0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + wm * 64 + i * 16 + q * 4 + r;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + wn * 64 + j * 16 + c16;
        if (n >= p.N) continue;
        const int64_t ci = p.c_gs * g + (crow0 + m) * p.ldc + n;
        if (C_F32) {
          float* C = static_cast<float*>(p.C) + ci;
          *C = ACC ? *C + acc[i][j][r] : acc[i][j][r];
        } else {
          uint16_t* C = static_cast<uint16_t*>(p.C) + ci;
          *C = f32_to_bf16(ACC ? bf16_to_f32(*C) + acc[i][j][r] : acc[i][j][r]);
        }
      }
    }
}

}  // namespace

hipError_t launch_bgemm(const BGemm& p, bool rows_k, bool b_kc, bool c_f32, bool acc, int32_t* tile_start,
                        hipStream_t s) {
  if (p.n_groups <= 0 || p.N <= 0) return hipSuccess;
  const int ntn = (p.N + kT - 1) / kT;
  int64_t grid;
  if (rows_k || !p.off) {
    grid = static_cast<int64_t>(p.n_groups) * (((rows_k ? p.M : p.rows_all) + kT - 1) / kT) * ntn;
  } else {
    hipLaunchKernelGGL(bgemm_plan_kernel, dim3(1), dim3(kThreads), 0, s, p, tile_start);
    grid = (static_cast<int64_t>(p.cap) / kT + p.n_groups) * ntn;  // every group may end in a partial tile
  }
  if (grid <= 0) return hipSuccess;
  const dim3 gd(static_cast<unsigned>(grid));
#define MOE_BG(RK, BK, CF, AC)                                                                      \
  if (rows_k == RK && b_kc == BK && c_f32 == CF && acc == AC) {                                     \
    hipLaunchKernelGGL((bgemm_kernel<RK, BK, CF, AC>), gd, dim3(kThreads), 0, s, p, tile_start);    \
    return hipGetLastError();                                                                       \
  }
  MOE_BG(false, true, true, false)   // forward recompute: U = X W^T, Y = H W2^T (fp32)
  MOE_BG(false, false, true, false)  // dH = dY W2, dX = dU W1 (fp32)
  MOE_BG(false, false, true, true)   // dX += dV W3
  MOE_BG(true, false, true, false)   // dW = dY^T H, dU^T X (fp32)
  MOE_BG(true, false, true, true)    // dW_r += dl_lo^T x
#undef MOE_BG
  return hipErrorInvalidValue;
}

}  // namespace moe
