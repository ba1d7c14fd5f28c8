// Grouped rows-M GEMM of the layer backward with B stored n-contiguous, on
// LDS DMA: C_g = A_g B_g in fp32, A_g the group's rows (k-contiguous), B_g
// element (k, n) at B[k ldb + n] (the weights in their [out][in] layout read
// along their rows: dH = dY W2; dX = [dU dV] [W1; W3] with B2 = W3 past
// k_split = d_ff).
//
// Tile 256 x 256, 8 waves (4 x 2), each 64 x 128 as 4 x 8 MFMA 16x16x32
// fragments. k-stages of 32 in a ring of four LDS buffers per operand (16 KB
// each), filled by global_load_lds three stages ahead: no VGPR staging, so
// the loads in flight are bounded by LDS, not by registers.
//  - A stage: 256 rows x 64 bytes; 16-byte chunk c of row r at c ^ ((r >> 1) & 3).
//  - B stage: 32 k-rows x 256 columns (512 bytes), as stored; chunk c of k-row
//    k at c ^ key(k). The MFMA operand (8 consecutive k of one column per lane)
//    comes from two ds_read_b64_tr_b16: in each 16-lane group, lane i receives
//    element i mod 4 of the 8-byte runs that lanes 4j + i/4 (j = 0..3) point
//    at, so lane s points at k-row k0 + s/4, columns n0 + 4 (s mod 4), and
//    lane i gets k0..k0+3 of column n0 + i. key(k) spreads the eight k-rows one
//    half-wave reads over all banks.
// Rows past a group's end and columns past N load clamped (valid) data that
// is computed and never stored.
//
// Rows-K form (RK): C_g = A_g^T B_g over the group's rows r (dW2 = dY^T H,
// dW1 = dU^T X, dW3 = dV^T X): both operands are stored [r][m] / [r][n], so
// both take the B path above (k-rows of 512 bytes, transpose reads). The k
// range is the group's row count; k-rows past it load the group's last row
// (the stage count is padded to a multiple of four), and on those stages the
// A fragment values of k past the range are set to zero before the MFMAs.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kNT = 512;          // 8 waves
constexpr int kTM = 256, kTN = 256, kTK = 32;
constexpr int kSA = kTM * kTK * 2;  // A stage bytes (16 KB)
constexpr int kSB = kTK * kTN * 2;  // B stage bytes (16 KB)
constexpr int kXcd = 8;

// s_waitcnt immediates: vmcnt(n) alone; lgkmcnt(0) alone
constexpr int vm_wait(int n) { return 0x0f70 | (n & 15) | (((n >> 4) & 3) << 14); }
constexpr int kLgkm0 = 0xc07f;

__device__ __forceinline__ int group_rows(const BGemm& p, int g, int& r0) {
  if (!p.off) {
    r0 = 0;
    return p.rows_all;
  }
  const int a = max(0, min(p.off[g], p.cap)), b = max(a, min(p.off[g + 1], p.cap));
  r0 = a;
  return b - a;
}

__device__ __forceinline__ int bkey(int k) { return ((k & 3) << 1) | (((k >> 3) & 1) << 3); }

__global__ __launch_bounds__(256) void dma_plan_kernel(BGemm p, int32_t* tile_start) {
  __shared__ int32_t s_mt[kMaxGroups];
  for (int g = threadIdx.x; g < p.n_groups; g += 256) {
    int r0;
    s_mt[g] = (group_rows(p, g, r0) + kTM - 1) / kTM;
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

typedef short v4s __attribute__((ext_vector_type(4)));
#define MOE_L(x) ((__attribute__((address_space(3))) void*)(x))

// The workgroup's tile (group g, row tile mt, column tile nt): consecutive
// tiles (the row tiles of one column tile) on one XCD. False past the last tile.
template <bool RK>
__device__ __forceinline__ bool tile_of_block(const BGemm& p, const int32_t* tile_start, int& g, int& mt, int& nt) {
  const int per_xcd = gridDim.x / kXcd;
  const int L = (blockIdx.x % kXcd) * per_xcd + blockIdx.x / kXcd;
  const int ntn = (p.N + kTN - 1) / kTN;
  if (RK || !p.off) {
    const int mtn = ((RK ? p.M : p.rows_all) + kTM - 1) / kTM;
    if (L >= p.n_groups * mtn * ntn) return false;
    g = L / (mtn * ntn);
    const int in = L % (mtn * ntn);
    if (RK && p.M > p.N) {
      // rows-K with the wider A (dW1, dW3: A = dU or dV, M = d_ff): the column
      // tiles of one row tile run together and share its A slab, the larger
      // operand (the B slabs, of X, are re-read from cache)
      mt = in / ntn;
      nt = in % ntn;
    } else {
      nt = in / mtn;
      mt = in % mtn;
    }
  } else {
    if (L >= tile_start[p.n_groups] * ntn) return false;
    int lo = 0, hi = p.n_groups - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tile_start[mid] * ntn <= L) lo = mid; else hi = mid - 1;
    }
    g = lo;
    const int mtg = tile_start[g + 1] - tile_start[g];
    const int local = L - tile_start[g] * ntn;
    nt = local / mtg;
    mt = local % mtg;
  }
  return true;
}

template <bool RK>
__global__ __launch_bounds__(kNT) void bgemm_dma_kernel(BGemm p, const int32_t* tile_start) {
  __shared__ __attribute__((aligned(16))) char A0[kSA];
  __shared__ __attribute__((aligned(16))) char A1[kSA];
  __shared__ __attribute__((aligned(16))) char A2[kSA];
  __shared__ __attribute__((aligned(16))) char A3[kSA];
  __shared__ __attribute__((aligned(16))) char B0[kSB];
  __shared__ __attribute__((aligned(16))) char B1[kSB];
  __shared__ __attribute__((aligned(16))) char B2s[kSB];
  __shared__ __attribute__((aligned(16))) char B3[kSB];

  int g, mt, nt;
  if (!tile_of_block<RK>(p, tile_start, g, mt, nt)) return;
  int r0;
  const int rows = group_rows(p, g, r0);
  const int M = RK ? p.M : rows;
  const int m0 = mt * kTM, n0 = nt * kTN;
  if (m0 >= M) return;
  const int K = RK ? rows : p.K;
  const int KS = ((K + kTK - 1) / kTK + 3) / 4 * 4;  // rows-M: K / 32, a multiple of 4

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int q = lane >> 4, c16 = lane & 15;

  // DMA sources: wave-uniform bases, 32-bit lane offsets (elements). Rows-M:
  // A rows r0 + m0.. (k-contiguous); rows-K: A k-rows r0.. of 256 columns m0..
  const uint16_t* Ab = p.A + p.a_gs * g +
                       (RK ? static_cast<int64_t>(r0) * p.lda + m0 : static_cast<int64_t>(r0 + m0) * p.lda);
  const uint16_t* Bb = p.B + p.b_gs * g + (RK ? static_cast<int64_t>(r0) * p.ldb : 0) + n0;
  const uint16_t* B2b = p.B2 ? p.B2 + p.b_gs * g + n0 : nullptr;
  uint32_t offa[2], offb[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int krow = wave * 4 + t * 2 + (lane >> 5);
    if (RK) {
      const int lastm = (min(kTM, M - m0) >> 3) - 1;                   // columns past M: clamped
      const int ac = min((lane & 31) ^ bkey(krow), lastm);
      offa[t] = static_cast<uint32_t>(ac * 8);  // + the k-row's offset, per stage
    } else {
      const int row = wave * 32 + t * 16 + (lane >> 2);               // tile row this lane fills
      const int chunk = (lane & 3) ^ ((row >> 1) & 3);                // its global k-chunk
      const int srow = min(row, M - m0 - 1);                         // rows past the group: clamped
      offa[t] = static_cast<uint32_t>(srow * static_cast<int>(p.lda) + chunk * 8);
    }
    const int lastc = (min(kTN, p.N - n0) >> 3) - 1;                   // columns past N: clamped
    const int bc = min((lane & 31) ^ bkey(krow), lastc);
    offb[t] = static_cast<uint32_t>((RK ? 0 : krow * static_cast<int>(p.ldb)) + bc * 8);
  }
  const int dsta = RK ? wave * 4 * 512 : wave * 32 * 64, dstb = wave * 4 * 512;  // byte offsets in a stage

  floatx4_t acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  // LDS read addresses (bytes) inside a stage
  int rda[4];  // rows-M: the swizzled 64-byte A rows
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = wm * 64 + i * 16 + c16;
    rda[i] = row * 64 + ((q ^ ((row >> 1) & 3)) << 4);
  }
  // rows-K: A fragment i, half h through the transpose read, chunk
  // ((8 wm + 2i) ^ key_h) + x of k-row kr_h (as for B, with m for n)
  int abase[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int krow = 8 * q + 4 * h + (c16 >> 2);
    abase[h] = krow * 512 + (((c16 & 3) >> 1) << 4) + (c16 & 1) * 8;
  }
  // B fragment j, half h: k-row kr_h = 8q + 4h + c16/4, column wn 128 + 16j +
  // 4 (c16 mod 4), i.e. chunk 16 wn + 2j + x (x = (c16 mod 4) / 2) at half
  // c16 mod 2; bkey is even, so the swizzled chunk is 16 wn + ((2j) ^ key_h) + x
  int rbase[2], rkey[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int krow = 8 * q + 4 * h + (c16 >> 2);
    rbase[h] = krow * 512 + ((wn * 16 + ((c16 & 3) >> 1)) << 4) + (c16 & 1) * 8;
    rkey[h] = bkey(krow);
  }

#define MOE_DMA(SA, SB, ks)                                                                          \
  do {                                                                                               \
    const int k0_ = (ks) * kTK;                                                                      \
    if (RK) {                                                                                        \
      _Pragma("unroll") for (int t_ = 0; t_ < 2; ++t_) {                                             \
        /* this lane's k-row k0 + 4 wave + 2 t + lane / 32, past the group: its last row */          \
        const int kr_ = min(k0_ + wave * 4 + 2 * t_ + (lane >> 5), K - 1);                           \
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(Ab + (static_cast<int64_t>(kr_) * p.lda + offa[t_])), \
                                         MOE_L((SA) + dsta + t_ * 1024), 16, 0, 0);                  \
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(Bb + (static_cast<int64_t>(kr_) * p.ldb + offb[t_])), \
                                         MOE_L((SB) + dstb + t_ * 1024), 16, 0, 0);                  \
      }                                                                                              \
    } else {                                                                                         \
      const uint16_t* ba_ = Ab + k0_;                                                                \
      const uint16_t* bb_ = (B2b && k0_ >= p.k_split) ? B2b + static_cast<int64_t>(k0_ - p.k_split) * p.ldb \
                                                      : Bb + static_cast<int64_t>(k0_) * p.ldb;      \
      _Pragma("unroll") for (int t_ = 0; t_ < 2; ++t_) {                                             \
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(ba_ + offa[t_]), MOE_L((SA) + dsta + t_ * 1024), 16, 0, 0); \
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(bb_ + offb[t_]), MOE_L((SB) + dstb + t_ * 1024), 16, 0, 0); \
      }                                                                                              \
    }                                                                                                \
  } while (0)
  // the B fragment of column block j + 1 is read while block j's MFMAs run
#define MOE_BFRAG(SB, j, OUT)                                                                        \
  do {                                                                                               \
    const v4s lo_ = __builtin_amdgcn_ds_read_tr16_b64_v4i16(                                         \
        (__attribute__((address_space(3))) v4s*)((SB) + rbase[0] + (((2 * (j)) ^ rkey[0]) << 4)));    \
    const v4s hi_ = __builtin_amdgcn_ds_read_tr16_b64_v4i16(                                         \
        (__attribute__((address_space(3))) v4s*)((SB) + rbase[1] + (((2 * (j)) ^ rkey[1]) << 4)));    \
    const uint2 l2_ = __builtin_bit_cast(uint2, lo_), h2_ = __builtin_bit_cast(uint2, hi_);          \
    OUT = make_uint4(l2_.x, l2_.y, h2_.x, h2_.y);                                                    \
  } while (0)
#define MOE_COMPUTE(SA, SB, ks)                                                                      \
  do {                                                                                               \
    uint4 af_[4], bc_, bn_;                                                                          \
    if (RK) {                                                                                        \
      _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_) {                                             \
        const v4s lo_ = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)( \
            (SA) + abase[0] + (((8 * wm + 2 * i_) ^ rkey[0]) << 4)));                                \
        const v4s hi_ = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)( \
            (SA) + abase[1] + (((8 * wm + 2 * i_) ^ rkey[1]) << 4)));                                \
        const uint2 l2_ = __builtin_bit_cast(uint2, lo_), h2_ = __builtin_bit_cast(uint2, hi_);      \
        af_[i_] = make_uint4(l2_.x, l2_.y, h2_.x, h2_.y);                                            \
      }                                                                                              \
      const int kv_ = K - (ks) * kTK;  /* valid k of this stage; lane holds k 8q .. 8q + 7 */        \
      if (kv_ < kTK) {                                                                               \
        _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_) {                                           \
          uint32_t w_[4] = {af_[i_].x, af_[i_].y, af_[i_].z, af_[i_].w};                             \
          _Pragma("unroll") for (int e_ = 0; e_ < 4; ++e_) {                                         \
            if (8 * q + 2 * e_ >= kv_) w_[e_] &= 0xFFFF0000u;                                        \
            if (8 * q + 2 * e_ + 1 >= kv_) w_[e_] &= 0x0000FFFFu;                                    \
          }                                                                                          \
          af_[i_] = make_uint4(w_[0], w_[1], w_[2], w_[3]);                                          \
        }                                                                                            \
      }                                                                                              \
    } else {                                                                                         \
      _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_) af_[i_] = *reinterpret_cast<const uint4*>((SA) + rda[i_]); \
    }                                                                                                \
    MOE_BFRAG(SB, 0, bc_);                                                                           \
    _Pragma("unroll") for (int j_ = 0; j_ < 8; ++j_) {                                               \
      if (j_ + 1 < 8) MOE_BFRAG(SB, j_ + 1, bn_);                                                    \
      _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_) acc[i_][j_] = mfma16x16x32(af_[i_], bc_, acc[i_][j_]); \
      bc_ = bn_;                                                                                     \
    }                                                                                                \
  } while (0)
  // stage ks from buffers (SA, SB): wait until at most VM DMA instructions
  // (the next stages') are in flight, barrier, refill (SAN, SBN) with stage
  // ks + 3 when DMA, then compute. The main loop runs unconditionally (every
  // stage refills; a conditional refill made the compiler drain all DMA at the
  // loop head); the last four stages are written out with their own waits.
#define MOE_STAGE(SA, SB, SAN, SBN, ks, VM, DMA)                                                     \
  do {                                                                                               \
    __builtin_amdgcn_s_waitcnt(vm_wait(VM));                                                         \
    __builtin_amdgcn_s_waitcnt(kLgkm0);                                                              \
    __builtin_amdgcn_s_barrier();                                                                    \
    if (DMA) MOE_DMA(SAN, SBN, (ks) + 3);                                                            \
    MOE_COMPUTE(SA, SB, ks);                                                                         \
  } while (0)

  if (KS > 0) {
  MOE_DMA(A0, B0, 0);
  MOE_DMA(A1, B1, 1);
  MOE_DMA(A2, B2s, 2);
  int ks = 0;
  for (; ks + 4 < KS; ks += 4) {  // every stage refills: ks + 6 < KS
    MOE_STAGE(A0, B0, A3, B3, ks, 8, true);
    MOE_STAGE(A1, B1, A0, B0, ks + 1, 8, true);
    MOE_STAGE(A2, B2s, A1, B1, ks + 2, 8, true);
    MOE_STAGE(A3, B3, A2, B2s, ks + 3, 8, true);
  }
  // the last four stages: ks = KS - 4
  MOE_STAGE(A0, B0, A3, B3, ks, 8, true);
  MOE_STAGE(A1, B1, A0, B0, ks + 1, 8, false);
  MOE_STAGE(A2, B2s, A1, B1, ks + 2, 4, false);
  MOE_STAGE(A3, B3, A2, B2s, ks + 3, 0, false);
  }
#undef MOE_STAGE
#undef MOE_COMPUTE
#undef MOE_BFRAG
#undef MOE_DMA

  // lane (q, c16) of fragment (i, j): rows 4q + r, column c16
  float* C = static_cast<float*>(p.C) + p.c_gs * g + static_cast<int64_t>((RK ? 0 : r0) + m0) * p.ldc + n0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = wm * 64 + i * 16 + q * 4 + r;
      if (m >= M - m0) continue;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int n = wn * 128 + j * 16 + c16;
        if (n0 + n < p.N) C[static_cast<int64_t>(m) * p.ldc + n] = acc[i][j][r];
      }
    }
}
// Rows-M products (dH, dX) with k-stages of 64 in five 32 KB LDS buffers
// (160 KB): A (routed rows) in a ring of two, filled one stage ahead, B (the
// weights) in a ring of three, filled two stages ahead. A stage is two 32-k
// MFMA steps behind one barrier, and each step's fragments are read from LDS
// while the previous step's MFMAs run.
//  - A stage: 256 rows x 128 bytes, chunk c of row r at c ^ (r mod 8).
//  - B stage: 64 k-rows x 256 columns; element (k, 16 jj + 8 x + e) at byte
//    256 (jj + 16 k2 + 32 (k >> 4)) + 32 rho(k) + 16 x + 2 e, with k2 = bit 2
//    of k and rho(k) = (k mod 4) + 4 (bit 3 of k). The eight k-rows a
//    half-wave's transpose read takes (k mod 4 and bit 3 vary, bit 2 and
//    k >> 4 do not) fill one 256-byte line, all banks once; and a fragment's
//    column block jj is a whole multiple of 256 bytes away from block 0, so
//    its reads differ only by immediate offsets (an XOR swizzle costs a
//    register per fragment and buffer, and those pushed the kernel into
//    spilling).
// The rows-K form (dW) stays on bgemm_dma_kernel: on this layout it ran
// faster for dW2 but slower for dW1 and dW3.
constexpr int kTK2 = 64;
constexpr int kS2 = 32768;  // one operand of one stage
constexpr int kDma2 = 4;    // DMA instructions per wave, operand and stage

__global__ __launch_bounds__(kNT, 1) void bgemm_dma64_kernel(BGemm p, const int32_t* tile_start) {
  __shared__ __attribute__((aligned(16))) char SA0[kS2];
  __shared__ __attribute__((aligned(16))) char SA1[kS2];
  __shared__ __attribute__((aligned(16))) char SB0[kS2];
  __shared__ __attribute__((aligned(16))) char SB1[kS2];
  __shared__ __attribute__((aligned(16))) char SB2[kS2];

  int g, mt, nt;
  if (!tile_of_block<false>(p, tile_start, g, mt, nt)) return;
  int r0;
  const int M = group_rows(p, g, r0);
  const int m0 = mt * kTM, n0 = nt * kTN;
  if (m0 >= M) return;
  const int n_st = p.K / kTK2;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int q = lane >> 4, c16 = lane & 15;

  const char* Ab = reinterpret_cast<const char*>(p.A + p.a_gs * g + static_cast<int64_t>(r0 + m0) * p.lda);
  const char* Bb = reinterpret_cast<const char*>(p.B + p.b_gs * g + n0);
  const char* B2b = p.B2 ? reinterpret_cast<const char*>(p.B2 + p.b_gs * g + n0) : nullptr;
  // DMA instruction t of this wave fills bytes [1024 (4 wave + t), + 1024) of
  // a stage. A: row 32 wave + 8t + l / 8, the global k-chunk that lands at
  // chunk l mod 8 of the LDS row. B: lane l takes k-row kl (the same for
  // every t) and 8-column chunk 8t + 2 (l >> 4) + (l mod 2).
  const int kl = ((lane >> 1) & 3) | ((wave & 1) << 2) | (((lane >> 3) & 1) << 3) | ((wave >> 1) << 4);
  const int cc0 = 2 * (lane >> 4) + (lane & 1);
  uint32_t offa[kDma2], offb[kDma2];  // bytes
#pragma unroll
  for (int t = 0; t < kDma2; ++t) {
    const int row = wave * 32 + t * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ (row & 7);
    const int srow = min(row, M - m0 - 1);  // rows past the group: clamped
    offa[t] = static_cast<uint32_t>(srow * static_cast<int>(p.lda) * 2 + chunk * 16);
    const int lastc = (min(kTN, p.N - n0) >> 3) - 1;  // columns past N: clamped
    offb[t] = static_cast<uint32_t>(kl * static_cast<int>(p.ldb) * 2 + min(8 * t + cc0, lastc) * 16);
  }
  const int dst = wave * 4096;

  floatx4_t acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  // LDS read offsets (bytes). A, step h: row wm 64 + 16 i + c16, chunk
  // 4h + q. B through transpose reads (see bgemm_dma_kernel): lane (q, c16)
  // points at k-row 8q + 4hh + c16 / 4 of the step, columns 4 (c16 mod 4) of
  // the fragment's block; hh = 1 is 4096 bytes on, step 1 16384 bytes on.
  int rda[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) rda[h] = (wm * 64 + c16) * 128 + (((4 * h + q) ^ (c16 & 7)) << 4);
  const int rb = 8192 * (q >> 1) + 32 * ((c16 >> 2) | ((q & 1) << 2)) + 16 * ((c16 & 3) >> 1) + 8 * (c16 & 1) +
                 256 * 8 * wn;  // B fragment j: + 256 j

#define MOE_TR(ADDR) __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(ADDR)))
#define MOE_DMA_A(S, ks)                                                                             \
  do {                                                                                               \
    const uint32_t k0b_ = static_cast<uint32_t>((ks) * kTK2 * 2);                                    \
    _Pragma("unroll") for (int t_ = 0; t_ < kDma2; ++t_)                                             \
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(Ab + (offa[t_] + k0b_)), MOE_L((S) + dst + t_ * 1024), 16, 0, 0); \
  } while (0)
  // piece t of stage ks's B (B2 past k_split)
#define MOE_DMA_B1(S, ks, t)                                                                         \
  do {                                                                                               \
    const int k0_ = (ks) * kTK2;                                                                     \
    const char* bb_ = (B2b && k0_ >= p.k_split) ? B2b + static_cast<int64_t>(k0_ - p.k_split) * p.ldb * 2 \
                                                : Bb + static_cast<int64_t>(k0_) * p.ldb * 2;        \
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(bb_ + offb[t]), MOE_L((S) + dst + (t) * 1024), 16, 0, 0); \
  } while (0)
#define MOE_READ_B(SB, H, j, OUT)                                                                    \
  do {                                                                                               \
    const uint2 l_ = MOE_TR((SB) + (H) * 16384 + rb + 256 * (j));                                   \
    const uint2 h_ = MOE_TR((SB) + (H) * 16384 + 4096 + rb + 256 * (j));                            \
    OUT = make_uint4(l_.x, l_.y, h_.x, h_.y);                                                        \
  } while (0)
  // One 32-k step: the MFMAs of A fragments AC with the B fragments in bf,
  // column block by column block. The slot of block j holds its four MFMAs,
  // the refill of bf[j] with block j of step H of the stage in (SA, SB), for
  // j < 4 A fragment j of that step (into AN), and with WITH_DMA, for
  // j < kDma2, piece j of stage DKS's B into DS: one LDS read after each of
  // the first MFMAs, the DMA after the last. Slots are fenced, so only one
  // set of B fragments is held.
#define MOE_PHASE(AC, AN, SA, SB, H, WITH_DMA, DS, DKS)                                              \
  do {                                                                                               \
    _Pragma("unroll") for (int j_ = 0; j_ < 8; ++j_) {                                               \
      _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_) acc[i_][j_] = mfma16x16x32(AC[i_], bf[j_], acc[i_][j_]); \
      MOE_READ_B(SB, H, j_, bf[j_]);                                                                 \
      if (j_ < 4) AN[j_] = *reinterpret_cast<const uint4*>((SA) + j_ * 16 * 128 + rda[H]);          \
      if (WITH_DMA && j_ < kDma2) MOE_DMA_B1(DS, DKS, j_);                                           \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                             \
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                             \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                             \
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                             \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                             \
      if (j_ < 4) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                 \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                             \
      if (WITH_DMA && j_ < kDma2) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                 \
      __builtin_amdgcn_sched_barrier(0);                                                             \
    }                                                                                                \
  } while (0)
  // Stage ks in (SAC, SBC), its first step's A fragments in af0 and B
  // fragments in bf: run the first step, reading the second's; wait until only
  // stage ks + 2's B DMA may fly (stage ks + 1 has landed), barrier (every
  // wave is done with SAC / SBC), refill SAC with stage ks + 2's A and SBC
  // with stage ks + 3's B (the A DMA first, so that it is older than the B DMA
  // the next wait leaves in flight), run the second step, reading stage
  // ks + 1's first.
#define MOE_STAGE(SAC, SBC, SAN, SBN, ks)                                                            \
  do {                                                                                               \
    MOE_PHASE(af0, af1, SAC, SBC, 1, false, SBC, 0);                                                 \
    __builtin_amdgcn_s_waitcnt(vm_wait(kDma2));                                                      \
    __builtin_amdgcn_s_waitcnt(kLgkm0);                                                              \
    __builtin_amdgcn_s_barrier();                                                                    \
    MOE_DMA_A(SAC, min((ks) + 2, n_st - 1));                                                         \
    __builtin_amdgcn_sched_barrier(0);                                                               \
    MOE_PHASE(af1, af0, SAN, SBN, 0, true, SBC, min((ks) + 3, n_st - 1));                            \
  } while (0)
  // a wave whose rows or columns all lie past the tile's: DMA and barriers only
#define MOE_STAGE_IDLE(SAC, SBC, SAN, SBN, ks)                                                       \
  do {                                                                                               \
    __builtin_amdgcn_s_waitcnt(vm_wait(kDma2));                                                      \
    __builtin_amdgcn_s_barrier();                                                                    \
    MOE_DMA_A(SAC, min((ks) + 2, n_st - 1));                                                         \
    __builtin_amdgcn_sched_barrier(0);                                                               \
    _Pragma("unroll") for (int t_ = 0; t_ < kDma2; ++t_) MOE_DMA_B1(SBC, min((ks) + 3, n_st - 1), t_); \
  } while (0)
  // whole rounds of six stages (A buffers cycle by 2, B buffers by 3), then
  // the 0..5 stages left
#define MOE_STAGES(STAGE)                                                                            \
  do {                                                                                               \
    const int n_round = n_st / 6 * 6;                                                                \
    for (int ks = 0; ks < n_round; ks += 6) {                                                        \
      STAGE(SA0, SB0, SA1, SB1, ks);                                                                 \
      STAGE(SA1, SB1, SA0, SB2, ks + 1);                                                             \
      STAGE(SA0, SB2, SA1, SB0, ks + 2);                                                             \
      STAGE(SA1, SB0, SA0, SB1, ks + 3);                                                             \
      STAGE(SA0, SB1, SA1, SB2, ks + 4);                                                             \
      STAGE(SA1, SB2, SA0, SB0, ks + 5);                                                             \
    }                                                                                                \
    const int left_ = n_st - n_round;                                                                \
    if (left_ > 0) STAGE(SA0, SB0, SA1, SB1, n_round);                                               \
    if (left_ > 1) STAGE(SA1, SB1, SA0, SB2, n_round + 1);                                           \
    if (left_ > 2) STAGE(SA0, SB2, SA1, SB0, n_round + 2);                                           \
    if (left_ > 3) STAGE(SA1, SB0, SA0, SB1, n_round + 3);                                           \
    if (left_ > 4) STAGE(SA0, SB1, SA1, SB2, n_round + 4);                                           \
  } while (0)

  if (n_st > 0) {
    uint4 af0[4], af1[4], bf[8];
    MOE_DMA_A(SA0, 0);
#pragma unroll
    for (int t = 0; t < kDma2; ++t) MOE_DMA_B1(SB0, 0, t);
    MOE_DMA_A(SA1, min(1, n_st - 1));
#pragma unroll
    for (int t = 0; t < kDma2; ++t) MOE_DMA_B1(SB1, min(1, n_st - 1), t);
#pragma unroll
    for (int t = 0; t < kDma2; ++t) MOE_DMA_B1(SB2, min(2, n_st - 1), t);
    __builtin_amdgcn_s_waitcnt(vm_wait(3 * kDma2));  // stage 0 landed
    __builtin_amdgcn_s_barrier();
    if (wm * 64 < M - m0 && wn * 128 < p.N - n0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) af0[i] = *reinterpret_cast<const uint4*>(SA0 + i * 16 * 128 + rda[0]);
#pragma unroll
      for (int j = 0; j < 8; ++j) MOE_READ_B(SB0, 0, j, bf[j]);
      MOE_STAGES(MOE_STAGE);
    } else {
      MOE_STAGES(MOE_STAGE_IDLE);
    }
    __builtin_amdgcn_s_waitcnt(vm_wait(0));  // the trailing DMAs have landed
    __builtin_amdgcn_s_waitcnt(kLgkm0);
    __builtin_amdgcn_s_barrier();
  }
#undef MOE_STAGES
#undef MOE_STAGE_IDLE
#undef MOE_STAGE
#undef MOE_PHASE
#undef MOE_READ_B
#undef MOE_DMA_B1
#undef MOE_DMA_A
#undef MOE_TR

  // lane (q, c16) of fragment (i, j): rows 4q + r, column c16
  float* C = static_cast<float*>(p.C) + p.c_gs * g + static_cast<int64_t>(r0 + m0) * p.ldc + n0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = wm * 64 + i * 16 + q * 4 + r;
      if (m >= M - m0) continue;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int n = wn * 128 + j * 16 + c16;
        if (n0 + n < p.N) C[static_cast<int64_t>(m) * p.ldc + n] = acc[i][j][r];
      }
    }
}
#undef MOE_L

}  // namespace

hipError_t launch_bgemm_dma(const BGemm& p, int32_t* tile_start, hipStream_t s) {
  if (p.n_groups <= 0 || p.N <= 0) return hipSuccess;
  if (p.K % 128 != 0 || p.lda % 8 != 0 || p.ldb % 8 != 0 || p.N % 8 != 0) return hipErrorInvalidValue;
  if (p.B2 && (p.k_split % kTK != 0 || p.k_split <= 0)) return hipErrorInvalidValue;
  const int ntn = (p.N + kTN - 1) / kTN;
  int64_t grid;
  if (!p.off) {
    grid = static_cast<int64_t>(p.n_groups) * ((p.rows_all + kTM - 1) / kTM) * ntn;
  } else {
    hipLaunchKernelGGL(dma_plan_kernel, dim3(1), dim3(256), 0, s, p, tile_start);
    grid = (static_cast<int64_t>(p.cap) / kTM + p.n_groups) * ntn;
  }
  if (grid <= 0) return hipSuccess;
  grid = (grid + kXcd - 1) / kXcd * kXcd;
  if (p.K % kTK2 == 0 && (!p.B2 || p.k_split % kTK2 == 0))
    hipLaunchKernelGGL(bgemm_dma64_kernel, dim3(static_cast<unsigned>(grid)), dim3(kNT), 0, s, p, tile_start);
  else
    hipLaunchKernelGGL(bgemm_dma_kernel<false>, dim3(static_cast<unsigned>(grid)), dim3(kNT), 0, s, p, tile_start);
  return hipGetLastError();
}

hipError_t launch_bgemm_dma_rk(const BGemm& p, hipStream_t s) {
  if (p.n_groups <= 0 || p.N <= 0 || p.M <= 0) return hipSuccess;
  if (p.M % 8 != 0 || p.N % 8 != 0 || p.lda % 8 != 0 || p.ldb % 8 != 0) return hipErrorInvalidValue;
  int64_t grid = static_cast<int64_t>(p.n_groups) * ((p.M + kTM - 1) / kTM) * ((p.N + kTN - 1) / kTN);
  grid = (grid + kXcd - 1) / kXcd * kXcd;
  hipLaunchKernelGGL(bgemm_dma_kernel<true>, dim3(static_cast<unsigned>(grid)), dim3(kNT), 0, s, p, nullptr);
  return hipGetLastError();
}

}  // namespace moe
