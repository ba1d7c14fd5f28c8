// Grouped GEMMs of the layer backward on LDS DMA, fp32 out.
//
// Rows-M form: C_g = A_g B_g, A_g the group's rows (k-contiguous), B_g
// element (k, n) at B[k ldb + n] (the weights in their [out][in] layout read
// along their rows: dH = dY W2; dX = [dU dV] [W1; W3] with B2 = W3 past
// k_split = d_ff).
// Rows-K form (RK): C_g = A_g^T B_g over the group's rows r (dW2 = dY^T H,
// dW1 = dU^T X, dW3 = dV^T X): both operands are stored [r][m] / [r][n].
//
// Tile 256 x 256, 8 waves (4 x 2), each 64 x 128 as 4 x 8 MFMA 16x16x32
// fragments. k-stages of 64 in five 32 KB LDS buffers (160 KB), filled by
// DMA (no VGPR staging): A in a ring of two, filled one stage ahead, B in a
// ring of three, filled two stages ahead (the weights, or the larger operand
// of dW, get the longer lead). A stage is two 32-k MFMA steps behind one
// barrier, and each step's fragments are read from LDS while the previous
// step's MFMAs run.
//  - Rows-M A stage: 256 rows x 128 bytes, 16-byte chunk c of row r at
//    c ^ (r mod 8).
//  - k-row stage (B, and A of rows-K): 64 k-rows x 256 columns as stored in
//    memory (n or m contiguous). The MFMA operand (8 consecutive k of one
//    column per lane) comes from two ds_read_b64_tr_b16: in each 16-lane
//    group, lane i receives element i mod 4 of the 8-byte runs that lanes
//    4j + i/4 (j = 0..3) point at, so lane s points at k-row k0 + s/4,
//    columns 4 (s mod 4) of the fragment's 16, and lane i gets k0..k0+3 of
//    column i. Element (k, 16 jj + 8 x + e) sits at byte 256 (jj + 16 k2 +
//    32 (k >> 4)) + 32 rho(k) + 16 x + 2 e, with k2 = bit 2 of k and
//    rho(k) = (k mod 4) + 4 (bit 3 of k). The eight k-rows a half-wave's
//    read takes (k mod 4 and bit 3 vary, bit 2 and k >> 4 do not) fill one
//    256-byte line, all banks once; and a fragment's column block jj is a
//    whole multiple of 256 bytes away from block 0, so its reads differ only
//    by immediate offsets (an XOR swizzle costs a register per fragment and
//    buffer).
// Rows past a group's end and columns past N load clamped (valid) data that
// is computed and never stored. Rows-K: a stage's k-rows come through a
// buffer resource that ends at the group's last row; a load past the end of a
// buffer resource returns zeros, so the k-rows past the group's rows add
// nothing to the sums.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kNT = 512;          // 8 waves
constexpr int kTM = 256, kTN = 256;
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
// tiles (the row tiles of one column tile, or for rows-K with M > N the
// column tiles of one row tile) on one XCD. False past the last tile.
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

constexpr int kTK = 64;
constexpr int kSt = 32768;  // one operand of one stage
constexpr int kDma = 4;     // DMA instructions per wave, operand and stage

// Buffer resource over whole k-rows [k0, min(k0 + 64, K)) of a rows-K operand
// (row stride ld elements, base at k-row 0, column 0), moved on by `skip`
// bytes (its end stays): loads past its end return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t kstage_rsrc(const char* base, int k0, int K, int64_t ld, int skip) {
  const int kv = min(K - k0, kTK);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base + static_cast<int64_t>(k0) * ld * 2 + skip), 0,
                                           max(kv * static_cast<int>(ld) * 2 - skip, 0), 0x00020000);
}

template <bool RK>
__global__ __launch_bounds__(kNT, 1) void bgemm_dma_kernel(BGemm p, const int32_t* tile_start) {
  __shared__ __attribute__((aligned(16))) char SA0[kSt];
  __shared__ __attribute__((aligned(16))) char SA1[kSt];
  __shared__ __attribute__((aligned(16))) char SB0[kSt];
  __shared__ __attribute__((aligned(16))) char SB1[kSt];
  __shared__ __attribute__((aligned(16))) char SB2[kSt];

  int g, mt, nt;
  if (!tile_of_block<RK>(p, tile_start, g, mt, nt)) return;
  int r0;
  const int rows = group_rows(p, g, r0);
  const int M = RK ? p.M : rows;
  const int m0 = mt * kTM, n0 = nt * kTN;
  if (m0 >= M) return;
  const int K = RK ? rows : p.K;
  const int n_st = (K + kTK - 1) / kTK;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int q = lane >> 4, c16 = lane & 15;

  // Rows-M: A at the tile's first row, B at column n0. Rows-K: both at the
  // group's first row, column 0 (the tile's columns are in the lane offsets).
  const char* Ab = reinterpret_cast<const char*>(
      p.A + p.a_gs * g + static_cast<int64_t>(RK ? r0 : r0 + m0) * p.lda);
  const char* Bb = reinterpret_cast<const char*>(p.B + p.b_gs * g + (RK ? static_cast<int64_t>(r0) * p.ldb : n0));
  const char* B2b = p.B2 ? reinterpret_cast<const char*>(p.B2 + p.b_gs * g + n0) : nullptr;
  // DMA instruction t of this wave fills bytes [1024 (4 wave + t), + 1024) of
  // a stage. k-row form: lane l takes k-row kl (the same for every t) and
  // 8-column chunk 8t + 2 (l >> 4) + (l mod 2); rows-M A: row 32 wave + 8t +
  // l / 8, the global k-chunk that lands at chunk l mod 8 of the LDS row.
  const int kl = ((lane >> 1) & 3) | ((wave & 1) << 2) | (((lane >> 3) & 1) << 3) | ((wave >> 1) << 4);
  const int cc0 = 2 * (lane >> 4) + (lane & 1);
  uint32_t offa[kDma], offb[kDma];  // bytes (rows-M)
#pragma unroll
  for (int t = 0; t < kDma; ++t) {
    const int row = wave * 32 + t * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ (row & 7);
    const int srow = min(row, M - m0 - 1);  // rows past the group: clamped
    offa[t] = static_cast<uint32_t>(srow * static_cast<int>(p.lda) * 2 + chunk * 16);
    const int lastc = (min(kTN, p.N - n0) >> 3) - 1;  // columns past N: clamped
    offb[t] = static_cast<uint32_t>(kl * static_cast<int>(p.ldb) * 2 + min(8 * t + cc0, lastc) * 16);
  }
  // rows-K: the lane's byte offset in a stage's buffer range (chunk t is 128
  // bytes on). k-rows past the group's rows lie past the range and load
  // zeros, which add nothing; columns past M or N run into the next k-row or
  // past the range: they feed only outputs that are never stored.
  const uint32_t oka = static_cast<uint32_t>(kl * static_cast<int>(p.lda) * 2 + (m0 + 8 * cc0) * 2);
  const uint32_t okb = static_cast<uint32_t>(kl * static_cast<int>(p.ldb) * 2 + (n0 + 8 * cc0) * 2);
  const int dst = wave * 4096;

  floatx4_t acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  // LDS read offsets (bytes). Rows-M A, step h: row wm 64 + 16 i + c16, chunk
  // 4h + q. Transpose reads (see the top of this file): lane (q, c16) points at
  // k-row 8q + 4hh + c16 / 4 of the step, columns 4 (c16 mod 4) of the
  // fragment's block; hh = 1 is 4096 bytes on, step 1 16384 bytes on.
  int rda[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) rda[h] = (wm * 64 + c16) * 128 + (((4 * h + q) ^ (c16 & 7)) << 4);
  const int lo = 8192 * (q >> 1) + 32 * ((c16 >> 2) | ((q & 1) << 2)) + 16 * ((c16 & 3) >> 1) + 8 * (c16 & 1);
  const int rb = lo + 256 * 8 * wn;  // B fragment j: + 256 j
  const int ra = lo + 256 * 4 * wm;  // rows-K A fragment i: + 256 i

#define MOE_TR(ADDR) __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(ADDR)))
  // the four 1 KB pieces of a rows-K operand's stage: chunk t is 128 bytes
  // on, by a resource moved on by 128t bytes (not by the instruction's offset
  // field, which a buffer load into LDS adds to the LDS address too, and not
  // by a lane offset per piece, four more registers)
#define MOE_BUF4(BASE, ks, LD, S, OFF)                                                               \
  do {                                                                                               \
    _Pragma("unroll") for (int t_ = 0; t_ < kDma; ++t_)                                             \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kstage_rsrc(BASE, (ks) * kTK, K, LD, 128 * t_),    \
                                                 MOE_L((S) + dst + t_ * 1024), 16, OFF, 0, 0, 0);    \
  } while (0)
#define MOE_DMA_A(S, ks)                                                                             \
  do {                                                                                               \
    const int k0_ = (ks) * kTK;                                                                     \
    if (RK) {                                                                                        \
      MOE_BUF4(Ab, ks, p.lda, S, oka);                                                               \
    } else {                                                                                         \
      _Pragma("unroll") for (int t_ = 0; t_ < kDma; ++t_)                                           \
          __builtin_amdgcn_global_load_lds(static_cast<const void*>(Ab + (offa[t_] + static_cast<uint32_t>(k0_ * 2))), \
                                           MOE_L((S) + dst + t_ * 1024), 16, 0, 0);                  \
    }                                                                                                \
  } while (0)
#define MOE_DMA_B(S, ks)                                                                             \
  do {                                                                                               \
    _Pragma("unroll") for (int t_ = 0; t_ < kDma; ++t_) MOE_DMA_B1(S, ks, t_);                      \
  } while (0)
  // piece t of a stage's B
#define MOE_DMA_B1(S, ks, t)                                                                         \
  do {                                                                                               \
    const int k0_ = (ks) * kTK;                                                                     \
    if (RK) {                                                                                        \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kstage_rsrc(Bb, k0_, K, p.ldb, 128 * (t)),             \
                                               MOE_L((S) + dst + (t) * 1024), 16, okb, 0, 0, 0);     \
    } else {                                                                                         \
      const char* bb_ = (B2b && k0_ >= p.k_split) ? B2b + static_cast<int64_t>(k0_ - p.k_split) * p.ldb * 2 \
                                                  : Bb + static_cast<int64_t>(k0_) * p.ldb * 2;      \
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(bb_ + offb[t]), MOE_L((S) + dst + (t) * 1024), 16, 0, 0); \
    }                                                                                                \
  } while (0)
  // the A fragments of 32-k step H of the stage in SA; B fragment j of the
  // stage in SB
#define MOE_READ_A(SA, H, AF)                                                                        \
  do {                                                                                               \
    _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_) {                                               \
      if (RK) {                                                                                      \
        const uint2 l_ = MOE_TR((SA) + (H) * 16384 + ra + 256 * i_);                                 \
        const uint2 h_ = MOE_TR((SA) + (H) * 16384 + 4096 + ra + 256 * i_);                          \
        AF[i_] = make_uint4(l_.x, l_.y, h_.x, h_.y);                                                 \
      } else {                                                                                       \
        AF[i_] = *reinterpret_cast<const uint4*>((SA) + i_ * 16 * 128 + rda[H]);                     \
      }                                                                                              \
    }                                                                                                \
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
  // j < kDma, piece j of stage DKS's B into DS. Slots are fenced, so the
  // reads and DMAs spread over the step and only one set of B fragments is
  // held. Rows-M pins the order inside a slot too (MFMA, read, MFMA, read,
  // ..., the DMA after the fourth MFMA; the compiler's own order clumped the
  // reads and ran slower); pinning it in the rows-K form pushed that form
  // into spilling, so there the compiler orders inside a slot.
#define MOE_PHASE(AC, AN, SA, SB, H, WITH_DMA, DS, DKS)                                              \
  do {                                                                                               \
    _Pragma("unroll") for (int j_ = 0; j_ < 8; ++j_) {                                               \
      _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_) acc[i_][j_] = mfma16x16x32(AC[i_], bf[j_], acc[i_][j_]); \
      MOE_READ_B(SB, H, j_, bf[j_]);                                                                 \
      if (RK && j_ < 4) {                                                                            \
        const uint2 l_ = MOE_TR((SA) + (H) * 16384 + ra + 256 * j_);                                 \
        const uint2 h_ = MOE_TR((SA) + (H) * 16384 + 4096 + ra + 256 * j_);                          \
        AN[j_] = make_uint4(l_.x, l_.y, h_.x, h_.y);                                                 \
      } else if (j_ < 4) {                                                                           \
        AN[j_] = *reinterpret_cast<const uint4*>((SA) + j_ * 16 * 128 + rda[H]);                     \
      }                                                                                              \
      if (WITH_DMA && j_ < kDma) MOE_DMA_B1(DS, DKS, j_);                                           \
      if (!RK) {                                                                                     \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                           \
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                           \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                           \
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                           \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                           \
        if (j_ < 4) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                               \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                           \
        if (WITH_DMA && j_ < kDma) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);               \
      }                                                                                              \
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
    MOE_PHASE(af0, af1, SAC, SBC, 1, false, SBC, 0);                                                \
    __builtin_amdgcn_s_waitcnt(vm_wait(kDma));                                                      \
    __builtin_amdgcn_s_waitcnt(kLgkm0);                                                              \
    __builtin_amdgcn_s_barrier();                                                                    \
    MOE_DMA_A(SAC, min((ks) + 2, n_st - 1));                                                         \
    __builtin_amdgcn_sched_barrier(0);                                                               \
    MOE_PHASE(af1, af0, SAN, SBN, 0, true, SBC, min((ks) + 3, n_st - 1));                            \
  } while (0)
  // a wave whose rows or columns all lie past the tile's: DMA and barriers only
#define MOE_STAGE_IDLE(SAC, SBC, SAN, SBN, ks)                                                       \
  do {                                                                                               \
    __builtin_amdgcn_s_waitcnt(vm_wait(kDma));                                                      \
    __builtin_amdgcn_s_barrier();                                                                    \
    MOE_DMA_A(SAC, min((ks) + 2, n_st - 1));                                                         \
    __builtin_amdgcn_sched_barrier(0);                                                               \
    MOE_DMA_B(SBC, min((ks) + 3, n_st - 1));                                                         \
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
    MOE_DMA_B(SB0, 0);
    MOE_DMA_A(SA1, min(1, n_st - 1));
    MOE_DMA_B(SB1, min(1, n_st - 1));
    MOE_DMA_B(SB2, min(2, n_st - 1));
    __builtin_amdgcn_s_waitcnt(vm_wait(3 * kDma));  // stage 0 landed
    __builtin_amdgcn_s_barrier();
    if (wm * 64 < M - m0 && wn * 128 < p.N - n0) {
      MOE_READ_A(SA0, 0, af0);
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
#undef MOE_READ_A
#undef MOE_DMA_B
#undef MOE_DMA_B1
#undef MOE_DMA_A
#undef MOE_BUF4
#undef MOE_TR

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
