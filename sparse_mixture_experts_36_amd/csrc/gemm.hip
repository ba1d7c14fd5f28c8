// Grouped expert FFN: up GEMM with fused activation, then down GEMM.
//
// Pages: vanos001 "MoE Architecture" / "Expert Network Design" (SwiGLUExpert:
// w2(silu(w1 x) * w3 x); StandardExpert: Linear -> GELU -> Linear) and
// "Efficient Batched MoE" (all experts' weights stacked and run as grouped
// operations instead of a per-expert loop); aigrafen.se "Mixture of Experts"
// (`MoE` module experts: Linear(d, hidden) -> GELU -> Linear(hidden, d));
// learn.starphix.com "Mixture of Experts (MoE)" / "Shared + Specialized"
// (always-on shared experts) and "Quantization" (low-precision expert
// weights; here OCP e4m3 with one fp32 scale per expert matrix).
//
// Both GEMMs are "NT": C[m][n] = sum_k A[m][k] * B[n][k], A rows and weight
// rows both contiguous in k (the nn.Linear layout). A group is one weight set
// over a contiguous block of rows: the routed experts over their slices of the
// permuted rows, then the shared experts over all T tokens, all in one launch.
//
// Tile schedule: the plan kernel turns the device-resident expert offsets into
// per-group row-tile counts and their prefix (no host round trip). Tile L runs
// group g's n-tile (L - base_g) / mt_g and m-tile (L - base_g) % mt_g, so the
// row tiles that share one weight tile are consecutive; consecutive L are
// mapped onto one XCD (workgroup ids reach the 8 XCDs round-robin), so they
// run together and share that weight tile in the XCD's L2.
#include "common.h"
#include "kernels.h"
#include "plan.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kXcds = 8;

// k-steps of global loads in flight in the bf16 GEMM (1 or 2)
#ifndef MOE_GEMM_PF
#define MOE_GEMM_PF 1
#endif

struct GemmParams {
  const void* A_r;        // routed A rows
  const int32_t* gather;  // routed A row r of a group is row gather[a_row0 + r] of A_r, or null (row a_row0 + r)
  const void* A_s;        // shared A rows
  int64_t lda_r, lda_s;   // A row pitches (elements, >= K)
  const void* B_r;        // routed weights [n_routed][Nout][K] (W1 or W2)
  const void* B3_r;       // routed W3 (SwiGLU up GEMM) or null
  const void* B_s;        // shared weights
  const void* B3_s;
  int64_t ldb;            // weight row pitch (elements, >= K)
  int64_t b_stride;       // elements per expert matrix = Nout * ldb
  const float* bias;      // [n_routed][Nout] or null (routed GELU experts only)
  const float* scale_r;   // [n_routed][3] (e4m3), [n_routed][scale_pitch] row scales (integer weights), or null
  const float* scale_s;   // [n_shared][3] or [n_shared][scale_pitch]
  int scale_col;          // 0 for the up GEMM (W1, W3 at +1), 2 for the down GEMM
  int32_t scale_pitch;    // integer weights: floats per expert in the row-scale arrays (2 d_ff + d)
  int32_t scale_row0;     // integer weights: offset of this GEMM's matrix rows (W1 0, W2 2 d_ff)
  int32_t scale_row3;     // integer weights: offset of W3's rows (d_ff)
  uint32_t skip[9];       // bit g set: group g is left to another launch (its experts' other bit width)
  uint32_t bits4[9];      // mixed-width launches (kWIntMix): bit g set: group g has 4-bit codes, else 8
  int32_t col_scaled;     // 1: the bf16 weights are integer codes; output column n takes row scale n
  int32_t mat_scaled;     // 1: e4m3 weights on the DMA tiles; the epilogue applies the per-matrix scales
  void* C_r;
  void* C_s;
  int64_t ldc;            // = Nout
  int32_t K, Nout;
  int32_t n_routed, n_groups;
  const GroupDesc* groups;
  const int32_t* tile_start;  // [n_groups+1] row-tile prefix
  float* split_part;          // fp32 partial tiles of the k-split tail, or null (no split)
  int32_t ncu;                // compute units of the device
  // fp32 copies of the up GEMM's values before the activation, for the layer
  // backward (DMA tiles only; null: not written): pre_u gets W1 x (+ b1),
  // pre_v gets W3 x; _r for routed groups, _s for shared ones; row c_row0 + r
  // of the group, pitch ld_pre
  float *pre_u_r, *pre_u_s, *pre_v_r, *pre_v_s;
  int64_t ld_pre;
};

enum Epi { EPI_GELU = 0, EPI_SWIGLU = 1, EPI_PLAIN = 2 };

// Largest g < n with ts[g] <= m (ts nondecreasing, ts[0] = 0 <= m).
__device__ __forceinline__ int find_group(const int32_t* ts, int n, int m) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (ts[mid] <= m) lo = mid; else hi = mid - 1;
  }
  return lo;
}

struct TileInfo {
  int g, m_tile, n_tile, rows;
  GroupDesc gd;
};

// Tile L of the launch: tiles run group by group, n-tile by n-tile, with the
// row tile fastest, so that consecutive tiles share a weight tile.
template <int BM, int BNO>
__device__ __forceinline__ void tile_from_linear(const GemmParams& p, int L, TileInfo& ti) {
  const int nt = p.Nout / BNO;
  const int g = find_group(p.tile_start, p.n_groups, L / nt);
  const int base = p.tile_start[g] * nt;
  const int mt = p.tile_start[g + 1] - p.tile_start[g];
  const int local = L - base;
  ti.g = g;
  ti.n_tile = local / mt;
  ti.m_tile = local % mt;
  ti.gd = p.groups[g];
  ti.rows = min(BM, ti.gd.rows - ti.m_tile * BM);
}

// Maps this workgroup to a tile; false when it has none. Consecutive tiles go
// to one XCD (workgroups are dealt to the 8 XCDs round-robin), so the tiles
// sharing a weight tile also share that XCD's L2.
template <int BM, int BNO>
__device__ __forceinline__ bool decode_tile(const GemmParams& p, TileInfo& ti) {
  const int total = p.tile_start[p.n_groups] * (p.Nout / BNO);
  const int per_xcd = (total + kXcds - 1) / kXcds;
  const int bid = blockIdx.x;
  const int slot = bid / kXcds;
  if (slot >= per_xcd) return false;
  const int L = (bid % kXcds) * per_xcd + slot;
  if (L >= total) return false;
  tile_from_linear<BM, BNO>(p, L, ti);
  return true;
}

// k-split of the last, partial round of tiles. With r = total mod ncu tiles
// left after the full rounds, and r <= ncu / 2, each of those r tiles is cut
// into s k-chunks (s * r <= ncu), run as s * r workgroups that write fp32
// partial tiles; a fix-up pass sums each tile's chunks in chunk order and
// applies the epilogue. The result then does not depend on timing.
constexpr int kSplitUnits = 256;  // partial tiles the workspace holds
// at most 4 chunks a tile: with 8, the Switch layer's up GEMM (K = 1024, its
// last round 32 tiles) ran chunks of two k-stages and a fix-up over 33 MB of
// partials; with 4 the layer took 0.279-0.281 ms against 0.289, the Mixtral
// and fine-grained layers unchanged
constexpr int kMaxSplit = 4;
struct SplitPlan {
  int total, full, r, s;
};
template <int BNO>
__device__ __forceinline__ SplitPlan split_plan(const GemmParams& p, int ks_pairs) {
  SplitPlan sp;
  sp.total = p.tile_start[p.n_groups] * (p.Nout / BNO);
  sp.r = sp.total % p.ncu;
  sp.s = 1;
  // the full rounds are then a multiple of the CU count; their XCD-ordered
  // mapping needs that to be a multiple of the XCD count as well
  if (p.split_part && sp.r > 0 && 2 * sp.r <= p.ncu && p.ncu % kXcds == 0)
    sp.s = min(min(p.ncu / sp.r, kMaxSplit), min(kSplitUnits / sp.r, ks_pairs));
  if (sp.s < 2) sp.s = 1;
  sp.full = sp.s > 1 ? sp.total - sp.r : sp.total;
  return sp;
}

// ------------------------------------------------------------------ bf16 MFMA
// WGM x WGN waves; a wave owns BM/WGM rows and BNB/WGN weight rows of the tile
// (for SwiGLU the matching halves of W1 and W3, so silu(a) * b is formed in
// registers). Weight tile rows: [0, BNO) from W1 (or W), [BNO, 2 BNO) from W3.
// Main loop: k-steps of 64 through two LDS buffers; the next step's global
// loads are in flight while the current one computes. LDS rows are 128 B (8
// chunks of 16 B) stored with chunk c of row r at position c ^ (r & 7): the 16
// rows of an MFMA operand read then hit distinct banks, so ds_read_b128 runs at
// the full 256 B/clk of a gfx950 CU (a 16-byte row pad only reaches half of
// it). The epilogue stages the bf16 output tile through LDS for 16-byte stores.
template <int BM, int BNB, int WGM, int WGN, int EPI, int WF, int PF>
__global__ __launch_bounds__(64 * WGM * WGN, 1) void gemm_bf16_kernel(GemmParams p) {
  constexpr int NTH = 64 * WGM * WGN;
  constexpr bool SWI = (EPI == EPI_SWIGLU);
  constexpr int BNO = SWI ? BNB / 2 : BNB;   // output columns per tile
  constexpr int BK = 64;
  constexpr int S = BK;                      // LDS row (bf16 elements), swizzled chunks
  constexpr int WTM = BM / WGM;              // rows per wave
  constexpr int WTB = BNB / WGN;             // weight rows per wave
  constexpr int WTO = SWI ? WTB / 2 : WTB;   // output columns per wave
  constexpr int FM = WTM / 16;
  constexpr int FN = WTB / 16;
  constexpr int FNO = WTO / 16;
  constexpr int A_CH = BM * (BK / 8) / NTH;  // 16-byte chunks per thread
  constexpr bool BYTE = WF != kWBf16;         // e4m3 / int8 / int4 codes, decoded in registers
  // 16-byte weight chunks per row and k-step: 8 bf16, 16 e4m3 or int8, 32 int4 weights each
  constexpr int CPR = WF == kWBf16 ? BK / 8 : (WF == kWInt4 ? BK / 32 : BK / 16);
  constexpr int DCH = (BK / 8) / CPR;          // bf16 chunks one weight chunk decodes to
  constexpr int B_CH = BNB * CPR / NTH;
  constexpr int STAGE = (BM + BNB) * S;      // elements per LDS buffer
  constexpr int SO = BNO + 8;                // output staging row (elements)
  static_assert(A_CH >= 1 && B_CH >= 1 && BM * (BK / 8) % NTH == 0 && BNB * CPR % NTH == 0, "tile/threads");
  constexpr int SMEM = (2 * STAGE > BM * SO) ? 2 * STAGE : BM * SO;  // operands, then the output tile

  __shared__ __attribute__((aligned(16))) uint16_t smem[SMEM];

  TileInfo ti;
  if (!decode_tile<BM, BNO>(p, ti)) return;
  if ((p.skip[ti.g >> 5] >> (ti.g & 31)) & 1u) return;  // the other bit width's launch takes this group

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int q = lane >> 4, c16 = lane & 15;
  const bool shared = ti.g >= p.n_routed;
  const int widx = ti.gd.widx;
  const int ew = shared ? widx - p.n_routed : widx;
  const int n0 = ti.n_tile * BNO;
  const int K = p.K;

  const int64_t lda = shared ? p.lda_s : p.lda_r;
  const int32_t* gth = shared ? nullptr : p.gather;
  const int arow0 = ti.gd.a_row0 + ti.m_tile * BM;  // the tile's first row in the group's A rows
  const uint16_t* A = static_cast<const uint16_t*>(shared ? p.A_s : p.A_r) + (gth ? 0 : static_cast<int64_t>(arow0) * lda);
  constexpr int EB = BYTE ? 1 : 2;  // bytes per row-pitch element
  const char* Bw = static_cast<const char*>(shared ? p.B_s : p.B_r) + static_cast<int64_t>(ew) * p.b_stride * EB;
  const char* B3w = SWI ? static_cast<const char*>(shared ? p.B3_s : p.B3_r) +
                              static_cast<int64_t>(ew) * p.b_stride * EB
                        : Bw;

  // per-thread chunk offsets (elements from A / bytes from the weight bases)
  uint32_t a_off[A_CH];
  int a_dst[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int c = tid + i * NTH;
    int r = c >> 3;
    const int kc = c & 7;
    a_dst[i] = r * S + ((kc ^ (r & 7)) * 8);
    if (r > ti.rows - 1) r = ti.rows - 1;  // rows past the group compute garbage, never stored
    const int src = gth ? gth[arow0 + r] : r;
    a_off[i] = static_cast<uint32_t>(src) * static_cast<uint32_t>(lda) + kc * 8;
  }
  // For SwiGLU the W3 rows are [BNO, 2 BNO). When that split falls on a chunk
  // boundary of every thread (chunks i >= B_CH / 2), the base choice is static.
  constexpr bool SPLIT = (B_CH % 2 == 0 && BNO * CPR == NTH * (B_CH / 2));
  uint32_t b_off[B_CH];
  int b_dst[B_CH];
  bool b_w3[B_CH];
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    const int c = tid + i * NTH;
    const int r = c / CPR, kc = c % CPR;
    // bf16: one chunk; codes: chunk kc decodes to the bf16 chunks DCH kc .. DCH kc + DCH - 1
    b_dst[i] = BM * S + r * S + (BYTE ? 0 : ((kc ^ (r & 7)) * 8));
    b_w3[i] = SWI && (SPLIT ? (i >= B_CH / 2) : (r >= BNO));
    const int wr = n0 + (b_w3[i] ? r - BNO : r);
    b_off[i] = static_cast<uint32_t>(wr) * static_cast<uint32_t>(p.ldb) * EB + kc * 16;
  }

  floatx4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

#define MOE_GLOAD(RA, RB, kb)                                                                       \
  do {                                                                                              \
    _Pragma("unroll") for (int i = 0; i < A_CH; ++i) RA[i] =                                        \
        *reinterpret_cast<const uint4*>(A + a_off[i] + (kb));                                       \
    _Pragma("unroll") for (int i = 0; i < B_CH; ++i) RB[i] = *reinterpret_cast<const uint4*>(       \
        ((SPLIT ? (SWI && i >= B_CH / 2) : b_w3[i]) ? B3w : Bw) + b_off[i] +                        \
        (WF == kWBf16 ? 2u : 1u) * static_cast<uint32_t>(kb) / (WF == kWInt4 ? 2u : 1u));          \
  } while (0)
#define MOE_LSTORE(RA, RB, buf)                                                                     \
  do {                                                                                              \
    uint16_t* st_ = smem + (buf) * STAGE;                                                           \
    _Pragma("unroll") for (int i = 0; i < A_CH; ++i)                                                \
        *reinterpret_cast<uint4*>(st_ + a_dst[i]) = RA[i];                                          \
    _Pragma("unroll") for (int i = 0; i < B_CH; ++i) {                                              \
      if constexpr (WF == kWE4m3 || WF == kWInt8) {                                                 \
        const int r_ = (tid + i * NTH) / CPR, k2_ = 2 * ((tid + i * NTH) % CPR);                    \
        const uint2 x0 = WF == kWE4m3 ? e4m3x4_to_bf16x4(RB[i].x) : int8x4_to_bf16x4(RB[i].x);      \
        const uint2 x1 = WF == kWE4m3 ? e4m3x4_to_bf16x4(RB[i].y) : int8x4_to_bf16x4(RB[i].y);      \
        const uint2 x2 = WF == kWE4m3 ? e4m3x4_to_bf16x4(RB[i].z) : int8x4_to_bf16x4(RB[i].z);      \
        const uint2 x3 = WF == kWE4m3 ? e4m3x4_to_bf16x4(RB[i].w) : int8x4_to_bf16x4(RB[i].w);      \
        *reinterpret_cast<uint4*>(st_ + b_dst[i] + ((k2_ ^ (r_ & 7)) * 8)) =                        \
            make_uint4(x0.x, x0.y, x1.x, x1.y);                                                     \
        *reinterpret_cast<uint4*>(st_ + b_dst[i] + (((k2_ + 1) ^ (r_ & 7)) * 8)) =                  \
            make_uint4(x2.x, x2.y, x3.x, x3.y);                                                     \
      } else if constexpr (WF == kWInt4) {                                                          \
        const int r_ = (tid + i * NTH) / CPR, k4_ = DCH * ((tid + i * NTH) % CPR);                  \
        const uint32_t q_[4] = {RB[i].x, RB[i].y, RB[i].z, RB[i].w};                                \
        _Pragma("unroll") for (int m_ = 0; m_ < 4; ++m_)                                            \
            *reinterpret_cast<uint4*>(st_ + b_dst[i] + (((k4_ + m_) ^ (r_ & 7)) * 8)) =             \
                int4x8_to_bf16x8(q_[m_]);                                                           \
      } else {                                                                                      \
        *reinterpret_cast<uint4*>(st_ + b_dst[i]) = RB[i];                                          \
      }                                                                                             \
    }                                                                                               \
  } while (0)

#define MOE_COMPUTE(SA)                                                                             \
  do {                                                                                              \
    const uint16_t* sA_ = (SA);                                                                     \
    const uint16_t* sB_ = sA_ + BM * S;                                                             \
    _Pragma("unroll") for (int kk = 0; kk < BK / 32; ++kk) {                                        \
      uint4 af[FM], bf[FN];                                                                         \
      /* operand rows start at multiples of 16, so row & 7 == c16 & 7 */                            \
      const int ch = ((kk * 4 + q) ^ (c16 & 7)) * 8;                                                \
      _Pragma("unroll") for (int i = 0; i < FM; ++i) af[i] =                                        \
          *reinterpret_cast<const uint4*>(sA_ + (wm * WTM + i * 16 + c16) * S + ch);                \
      _Pragma("unroll") for (int j = 0; j < FN; ++j) {                                              \
        const int brow = SWI ? ((j < FN / 2) ? wn * (WTB / 2) + j * 16                              \
                                             : BNO + wn * (WTB / 2) + (j - FN / 2) * 16)            \
                             : wn * WTB + j * 16;                                                   \
        bf[j] = *reinterpret_cast<const uint4*>(sB_ + (brow + c16) * S + ch);                       \
      }                                                                                             \
      _Pragma("unroll") for (int i = 0; i < FM; ++i)                                                \
          _Pragma("unroll") for (int j = 0; j < FN; ++j) acc[i][j] =                                \
              mfma16x16x32(af[i], bf[j], acc[i][j]);                                                \
    }                                                                                               \
  } while (0)

  const int KT = K / BK;
  if constexpr (PF == 1) {
    uint4 ra[A_CH], rb[B_CH];
    MOE_GLOAD(ra, rb, 0);
    MOE_LSTORE(ra, rb, 0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
      // prefetch the next k-step (the last iteration re-reads its own step;
      // the copy lands in the idle buffer and is never read)
      const int kn = (kt + 1 < KT) ? (kt + 1) * BK : kt * BK;
      MOE_GLOAD(ra, rb, kn);
      MOE_COMPUTE(smem + (kt & 1) * STAGE);
      MOE_LSTORE(ra, rb, (kt + 1) & 1);
      __syncthreads();
    }
  } else {
    // two k-steps in flight: registers hold step kt+1 while step kt+2 loads.
    // K is a multiple of 128, so the number of 64-wide k-steps is even; steps
    // past the end re-read the last one into buffers that are never read.
    uint4 ra0[A_CH], rb0[B_CH], ra1[A_CH], rb1[B_CH];
    MOE_GLOAD(ra0, rb0, 0);
    MOE_GLOAD(ra1, rb1, BK);
    MOE_LSTORE(ra0, rb0, 0);
    __syncthreads();
    for (int kt = 0; kt < KT; kt += 2) {
      MOE_GLOAD(ra0, rb0, min(kt + 2, KT - 1) * BK);
      MOE_COMPUTE(smem);
      MOE_LSTORE(ra1, rb1, 1);
      __syncthreads();
      MOE_GLOAD(ra1, rb1, min(kt + 3, KT - 1) * BK);
      MOE_COMPUTE(smem + STAGE);
      MOE_LSTORE(ra0, rb0, 0);
      __syncthreads();
    }
  }
#undef MOE_GLOAD
#undef MOE_LSTORE
#undef MOE_COMPUTE

  // ---- epilogue: activation in registers, bf16 tile staged in LDS, 16-byte stores
  const float* sc = shared ? p.scale_s : p.scale_r;
  float s_a = 1.f, s_b = 1.f;
  if (WF == kWE4m3 && sc) {
    s_a = sc[ew * 3 + p.scale_col];
    if (SWI) s_b = sc[ew * 3 + p.scale_col + 1];
  }
  // integer weights: one scale per weight row (output column)
  const float* rs = (WF == kWInt8 || WF == kWInt4) ? sc + static_cast<int64_t>(ew) * p.scale_pitch + n0 : nullptr;
  const float* bias = (!shared && p.bias) ? p.bias + static_cast<int64_t>(ew) * p.Nout + n0 : nullptr;
  uint16_t* so = smem;
#pragma unroll
  for (int j = 0; j < FNO; ++j) {
    const int col = wn * WTO + j * 16 + c16;
    const float bv = bias ? bias[col] : 0.f;
    if (rs) {
      s_a = rs[p.scale_row0 + col];
      if (SWI) s_b = rs[p.scale_row3 + col];
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wm * WTM + i * 16 + q * 4 + r;
        float v;
        if constexpr (EPI == EPI_SWIGLU) {
          v = silu(acc[i][j][r] * s_a) * (acc[i][j + FN / 2][r] * s_b);
        } else if constexpr (EPI == EPI_GELU) {
          v = gelu_erf(acc[i][j][r] * s_a + bv);
        } else {
          v = acc[i][j][r] * s_a + bv;
        }
        so[row * SO + col] = f32_to_bf16(v);
      }
    }
  }
  __syncthreads();
  uint16_t* C = static_cast<uint16_t*>(shared ? p.C_s : p.C_r) +
                (static_cast<int64_t>(ti.gd.c_row0) + static_cast<int64_t>(ti.m_tile) * BM) * p.ldc + n0;
  constexpr int OCH = BNO / 8;  // 16-byte chunks per output row
  for (int c = tid; c < BM * OCH; c += NTH) {
    const int row = c / OCH, cc = c % OCH;
    if (row < ti.rows)
      *reinterpret_cast<uint4*>(C + static_cast<int64_t>(row) * p.ldc + cc * 8) =
          *reinterpret_cast<const uint4*>(so + row * SO + cc * 8);
  }
}

// ------------------------------------------------------------------ bf16 MFMA, LDS DMA pipeline
// BM x 256 tile, 8 waves (2 x 4, each BM/2 rows x 64 weight rows), k-stages of
// 64 through LDS stage buffers. gemm_dma_kernel runs the 128-row tile with
// three shared 48 KB buffers (two stages in flight); gemm_dma5_kernel runs the
// 256-row tile with separate activation and weight buffers. Operands move from
// memory to LDS with global_load_lds (no VGPR staging, no ds_write): each wave
// instruction writes 1 KB = 8 rows x 128 B, so every fetched 128-byte line is
// used whole, and the source address each lane fetches puts 16-byte chunk c of
// row r at position c ^ (r & 7), at which the MFMA operand reads (16 rows, one
// chunk each) run conflict-free. A stage feeds two MFMA k-steps of 32; the
// fragments of the next k-step are read from LDS while the current one's
// MFMAs run. The stage buffers are separate LDS objects so that the
// compiler's wait for a DMA store only blocks reads of that buffer. Before
// every barrier a wave waits for its own LDS reads, so no DMA can overwrite
// data still being read.
namespace dma {
constexpr int BNB = 256, WGM = 2;
constexpr int BK = 64;      // k per stage
constexpr int RB = BK * 2;  // row bytes in a stage
// Cache policy of a weight-row DMA (global_load_lds's aux operand): bit 1 is
// the nontemporal hint. It is used where no other tile reads the weight
// tile: a group with one 128-row tile (bf16 rows, whole lines a stage; the
// Mixtral layer's short tails, most small groups of the Switch and
// fine-grained layers). Measured: Mixtral layer 2.597-2.613 -> 2.559-2.580
// ms, Switch 0.303-0.305 -> 0.290-0.291 ms, fine-grained unchanged. With the
// hint on every 128-row tile the fine-grained layer's down GEMM was slower
// (1.543 -> 1.573 ms): groups of two or three row tiles share each weight
// tile in L2, and the later tiles found fewer of its lines there.
constexpr int kAuxNT = 2;
constexpr int bno(int epi) { return epi == EPI_SWIGLU ? BNB / 2 : BNB; }
// BM x 256 tile on W waves (2 x W/2): a wave owns BM/2 rows and 512/W weight
// rows as FM x FN MFMA fragments, and moves BM/W A rows and 256/W weight rows
// of each stage from memory to LDS.
template <int BM, int W>
struct Cfg {
  static_assert((BM == 256 || BM == 128) && (W == 8 || W == 4), "DMA tile shape");
  static constexpr int NTH = 64 * W;
  static constexpr int WGN = W / WGM;
  static constexpr int WTM = BM / WGM;               // rows per wave
  static constexpr int WTB = BNB / WGN;              // weight rows per wave
  static constexpr int FM = WTM / 16, FN = WTB / 16;
  static constexpr int NSTAGE = BM == 256 ? 2 : 3;
  static constexpr int SBYTES = (BM + BNB) * RB;     // one stage buffer
  static constexpr int AROWS = BM / W, BROWS = BNB / W;
  static constexpr int ADMA = AROWS / 8, BDMA = BROWS / 8;  // DMA instructions per wave and stage
  static constexpr int NDMA = ADMA + BDMA;
};
// s_waitcnt immediate: vmcnt(n), no wait on expcnt and lgkmcnt
constexpr int vmcnt_imm(int n) { return 0x0f70 | (n & 15) | (((n >> 4) & 3) << 14); }
}  // namespace dma

// Epilogue of a DMA tile held as per-wave MFMA fragments: bias and activation
// (or the SwiGLU product of the W1 and W3 halves), bf16, straight from the
// registers to memory. Every wave converts its own fragments at once (no LDS,
// no barrier). A fragment gives lane l rows 4 (l / 16) + r, r < 4, of column
// l % 16; the quad transpose turns that into four consecutive columns of row
// 4 (l / 16) + l % 4, stored as 8 bytes.
template <int EPI, int BM, int W>
__device__ __forceinline__ void dma_store_tile(const GemmParams& p, const TileInfo& ti,
                                               floatx4_t (&acc)[dma::Cfg<BM, W>::FM][dma::Cfg<BM, W>::FN],
                                               int wave) {
  using namespace dma;
  using C_ = Cfg<BM, W>;
  constexpr int BNO = bno(EPI);
  constexpr int WTB = C_::WTB, FN = C_::FN, FM = C_::FM, WGN = C_::WGN, WTM = C_::WTM;
  constexpr int WTO = EPI == EPI_SWIGLU ? WTB / 2 : WTB;
  constexpr int FNO = WTO / 16;
  const int lane = threadIdx.x & 63;
  const int wm = wave / WGN, wn = wave % WGN;
  const int q = lane >> 4, c16 = lane & 15, t = lane & 3;
  const bool shared = ti.g >= p.n_routed;
  const int ew = shared ? ti.gd.widx - p.n_routed : ti.gd.widx;
  const int n0 = ti.n_tile * BNO;
  const float* bias = (!shared && p.bias) ? p.bias + static_cast<int64_t>(ew) * p.Nout + n0 : nullptr;
  // integer codes as bf16 weights: one scale per output column (weight row)
  const float* rs = p.col_scaled ? (shared ? p.scale_s : p.scale_r) + static_cast<int64_t>(ew) * p.scale_pitch + n0
                                 : nullptr;
  // e4m3 weights: one scale per expert matrix (W1 or W2, and W3)
  float ma = 1.f, mb = 1.f;
  if (p.mat_scaled) {
    const float* ms = (shared ? p.scale_s : p.scale_r) + ew * 3 + p.scale_col;
    ma = ms[0];
    if (EPI == EPI_SWIGLU) mb = ms[1];
  }
  uint16_t* C = static_cast<uint16_t*>(shared ? p.C_s : p.C_r) +
                (static_cast<int64_t>(ti.gd.c_row0) + static_cast<int64_t>(ti.m_tile) * BM) * p.ldc + n0;
#pragma unroll
  for (int j = 0; j < FNO; ++j) {
    const int col = wn * WTO + j * 16 + c16;         // this lane's column in the fragments
    const int ocol = wn * WTO + j * 16 + 4 * (c16 >> 2);  // the four columns it stores
    const float bv = bias ? bias[col] : 0.f;
    const float sa = rs ? rs[p.scale_row0 + col] : ma;
    const float sb = (rs && EPI == EPI_SWIGLU) ? rs[p.scale_row3 + col] : mb;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (EPI == EPI_SWIGLU) v[r] = silu(acc[i][j][r] * sa) * (acc[i][j + FN / 2][r] * sb);
        else if constexpr (EPI == EPI_GELU) v[r] = gelu_erf(acc[i][j][r] * sa + bv);
        else v[r] = acc[i][j][r] * sa + bv;
      }
      uint32_t r01, r23;
      quad_transpose_bf16(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), t, r01, r23);
      const int row = wm * WTM + i * 16 + q * 4 + t;
      if (row < ti.rows)
        *reinterpret_cast<uint2*>(C + static_cast<int64_t>(row) * p.ldc + ocol) = make_uint2(r01, r23);
    }
  }
}

// fp32 copies of an up-GEMM DMA tile's values before the activation, for the
// layer backward (bf16 weights): W1 x (+ b1) into pre_u and W3 x into pre_v,
// straight from the fragments (16 lanes write 64 contiguous bytes of a row).
template <int EPI, int BM, int W>
__device__ __forceinline__ void dma_store_pre(const GemmParams& p, const TileInfo& ti,
                                              floatx4_t (&acc)[dma::Cfg<BM, W>::FM][dma::Cfg<BM, W>::FN], int wave) {
  using namespace dma;
  using C_ = Cfg<BM, W>;
  constexpr int BNO = bno(EPI);
  constexpr int WTB = C_::WTB, FN = C_::FN, WGN = C_::WGN, WTM = C_::WTM;
  constexpr int WTO = EPI == EPI_SWIGLU ? WTB / 2 : WTB;
  constexpr int FNO = WTO / 16;
  const bool shared = ti.g >= p.n_routed;
  float* pu = shared ? p.pre_u_s : p.pre_u_r;
  if (!pu) return;
  float* pv = EPI == EPI_SWIGLU ? (shared ? p.pre_v_s : p.pre_v_r) : nullptr;
  const int lane = threadIdx.x & 63;
  const int wm = wave / WGN, wn = wave % WGN;
  const int q = lane >> 4, c16 = lane & 15;
  const int ew = shared ? ti.gd.widx - p.n_routed : ti.gd.widx;
  const int n0 = ti.n_tile * BNO;
  const float* bias = (!shared && p.bias) ? p.bias + static_cast<int64_t>(ew) * p.Nout + n0 : nullptr;
  const int64_t off = (static_cast<int64_t>(ti.gd.c_row0) + static_cast<int64_t>(ti.m_tile) * BM) * p.ld_pre + n0;
#pragma unroll
  for (int i = 0; i < C_::FM; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = wm * WTM + i * 16 + q * 4 + r;
      if (row >= ti.rows) continue;
#pragma unroll
      for (int j = 0; j < FNO; ++j) {
        const int col = wn * WTO + j * 16 + c16;
        const int64_t o = off + static_cast<int64_t>(row) * p.ld_pre + col;
        pu[o] = acc[i][j][r] + (bias ? bias[col] : 0.f);
        if (pv) pv[o] = acc[i][j + FN / 2][r];
      }
    }
}

// fp32 partial tile of a k-chunk, in fragment order: fragment (wave, i, j) is
// 64 lanes x 4 floats, 1 KB contiguous.
template <int BM, int W>
__device__ __forceinline__ float* dma_part_frag(float* part, int unit, int wave, int i, int j) {
  using namespace dma;
  using C_ = Cfg<BM, W>;
  return part + static_cast<int64_t>(unit) * (BM * BNB) + ((wave * C_::FM + i) * C_::FN + j) * 256;
}

// A weight fragment's 8 codes as read from LDS: 8 bytes (e4m3, int8) or one
// 32-bit word (int4), and their exact bf16 values.
template <int WF>
struct CodeFrag {
  typedef uint2 type;
};
template <>
struct CodeFrag<kWInt4> {
  typedef uint32_t type;
};
template <int WF>
__device__ __forceinline__ uint4 frag_to_bf16(uint2 c) {
  const uint2 lo = WF == kWE4m3 ? e4m3x4_to_bf16x4(c.x) : int8x4_to_bf16x4(c.x);
  const uint2 hi = WF == kWE4m3 ? e4m3x4_to_bf16x4(c.y) : int8x4_to_bf16x4(c.y);
  return make_uint4(lo.x, lo.y, hi.x, hi.y);
}
template <int WF>
__device__ __forceinline__ uint4 frag_to_bf16(uint32_t c) {
  return int4x8_to_bf16x8(c);
}

// Weight codes (WF other than kWBf16) arrive in LDS as stored and are turned
// into bf16 fragments exactly, after a wave's reads land and before its MFMAs:
// - kWE4m3 and kWInt8: one byte a weight, 64-byte stage rows. A fragment is 8
//   bytes; chunk c of row r sits at position c ^ ((r >> 2) & 3), where the
//   8-byte reads of 16 rows are conflict-free, and one DMA instruction fills
//   16 rows. e4m3 decodes in hardware; the epilogue applies the per-matrix
//   scales.
// - kWInt4: half a byte a weight, 32-byte stage rows. A fragment is one
//   32-bit word of 8 codes; chunk c of row r sits at c ^ ((r >> 3) & 1), and
//   one DMA instruction fills 32 rows.
// Integer codes take the row scales in the epilogue, one per output column.
// Bytes of one stage buffer (activation rows, then weight rows) and the
// number of stage buffers of the DMA tile for weight format WF.
template <int BM, int WF>
constexpr int dma_stage_bytes() {
  return BM * dma::RB + dma::BNB * ((WF == kWE4m3 || WF == kWInt8) ? dma::RB / 2 : (WF == kWInt4 ? dma::RB / 4 : dma::RB));
}
template <int BM, int W, int WF>
constexpr int dma_nstage() { return WF != kWBf16 ? 3 : dma::Cfg<BM, W>::NSTAGE; }

// One tile (or k-chunk ks_begin .. ks_end of a tile; unit >= 0: a k-split
// chunk whose raw partial sums go to the split workspace) with the stage
// buffers S0, S1, S2 in LDS.
template <int EPI, int BM, int W, int WF, int BAUX = 0>
__device__ __forceinline__ void dma_tile_body(const GemmParams& p, const TileInfo& ti, int ks_begin, int ks_end,
                                              int unit, char* S0, char* S1, char* S2) {
  using namespace dma;
  using C_ = Cfg<BM, W>;
  constexpr bool SWI = (EPI == EPI_SWIGLU);
  constexpr int BNO = bno(EPI);
  constexpr int FM = C_::FM, FN = C_::FN, WTM = C_::WTM, WTB = C_::WTB, WGN = C_::WGN;
  constexpr bool F8 = (WF == kWE4m3 || WF == kWInt8);  // byte codes
  constexpr bool I4 = (WF == kWInt4);
  constexpr bool CODES = F8 || I4;
  static_assert(!I4 || C_::BROWS % 32 == 0, "int4 rows go 32 to a DMA instruction");
  constexpr int RBB = F8 ? RB / 2 : (I4 ? RB / 4 : RB);  // weight row bytes in a stage
  constexpr int ADMA = C_::ADMA, BDMA = F8 ? C_::BROWS / 16 : (I4 ? C_::BROWS / 32 : C_::BDMA), NDMA = ADMA + BDMA;
  constexpr int NSTAGE = dma_nstage<BM, W, WF>();
  typedef typename CodeFrag<WF>::type BQT;
  // stage j of the loops below loads k-column ks_begin + j; all tiles walk k
  // in the same order, so tiles that share a weight tile or A rows read the
  // same lines at about the same time and L2 keeps them
  const int n_st = ks_end - ks_begin;
#define MOE_COL(j) (ks_begin + (j))
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: wave-level pointers stay in SGPRs
  const int wm = wave / WGN, wn = wave % WGN;
  const int q = lane >> 4, c16 = lane & 15;
  const bool shared = ti.g >= p.n_routed;
  const int ew = shared ? ti.gd.widx - p.n_routed : ti.gd.widx;
  const int n0 = ti.n_tile * BNO;
  const int64_t lda = shared ? p.lda_s : p.lda_r;
  const int32_t* gth = shared ? nullptr : p.gather;
  const int arow0 = ti.gd.a_row0 + ti.m_tile * BM;  // the tile's first row in the group's A rows
  const char* A = static_cast<const char*>(shared ? p.A_s : p.A_r) + (gth ? 0 : static_cast<int64_t>(arow0) * lda * 2);
  // This wave loads A rows [AROWS w, AROWS (w + 1)) and weight rows
  // [BROWS w, BROWS (w + 1)), in instructions of 8 rows each. For SwiGLU the
  // weight rows [0, 128) of the tile are W1 rows and [128, 256) the matching
  // W3 rows, so one wave's weight rows come from one matrix.
  const int ar0 = wave * C_::AROWS, wr0 = wave * C_::BROWS;
  const bool w3 = SWI && wr0 >= BNO;
  const char* Bw = static_cast<const char*>(w3 ? (shared ? p.B3_s : p.B3_r) : (shared ? p.B_s : p.B_r)) +
                   (static_cast<int64_t>(ew) * p.b_stride + static_cast<int64_t>(n0 + (w3 ? wr0 - BNO : wr0)) * p.ldb) *
                       (CODES ? 1 : 2);  // code pitches are in bytes
  // Lane L of an instruction over rows [r0, r0 + 8) fills row r0 + L/8,
  // position L%8 with logical chunk (L%8) ^ (row & 7); byte offsets are
  // relative to the tile's first A row and the wave's first weight row.
  uint32_t offa[ADMA], offb[BDMA];
#pragma unroll
  for (int i = 0; i < ADMA; ++i) {
    const int r = ar0 + i * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ (r & 7);
    const int rr = r > ti.rows - 1 ? ti.rows - 1 : r;  // rows past the group compute garbage, never stored
    const int src = gth ? gth[arow0 + rr] : rr;
    offa[i] = static_cast<uint32_t>(src * static_cast<int>(lda) * 2 + chunk * 16);
  }
#pragma unroll
  for (int i = 0; i < BDMA; ++i) {
    if constexpr (F8) {  // 16 rows of 64 bytes an instruction: lane L fills row r0 + L/4, position L%4
      const int r = wr0 + i * 16 + (lane >> 2);
      const int chunk = (lane & 3) ^ ((r >> 2) & 3);
      offb[i] = static_cast<uint32_t>((i * 16 + (lane >> 2)) * static_cast<int>(p.ldb) + chunk * 16);
    } else if constexpr (I4) {  // 32 rows of 32 bytes an instruction: lane L fills row r0 + L/2, position L%2
      const int r = wr0 + i * 32 + (lane >> 1);
      const int chunk = (lane & 1) ^ ((r >> 3) & 1);
      offb[i] = static_cast<uint32_t>((i * 32 + (lane >> 1)) * static_cast<int>(p.ldb) + chunk * 16);
    } else {
      const int r = wr0 + i * 8 + (lane >> 3);
      const int chunk = (lane & 7) ^ (r & 7);
      offb[i] = static_cast<uint32_t>((i * 8 + (lane >> 3)) * static_cast<int>(p.ldb) * 2 + chunk * 16);
    }
  }
  const int dst_a = ar0 * RB, dst_b = BM * RB + wr0 * RBB;  // byte offsets inside a stage
// (the source pointer is passed as const void*: with a char* argument the host
// compilation pass silently drops the kernel's launch stub)
#define MOE_LDS(x) ((__attribute__((address_space(3))) void*)(x))
#define MOE_DMA(S, ks)                                                                               \
  do {                                                                                               \
    const uint32_t ko_ = static_cast<uint32_t>(ks) * RB, kb_ = static_cast<uint32_t>(ks) * RBB;      \
    _Pragma("unroll") for (int i_ = 0; i_ < ADMA; ++i_)                                              \
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(A + (offa[i_] + ko_)), MOE_LDS((S) + dst_a + i_ * 1024), 16, 0, 0); \
    _Pragma("unroll") for (int i_ = 0; i_ < BDMA; ++i_)                                              \
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(Bw + (offb[i_] + kb_)), MOE_LDS((S) + dst_b + i_ * 1024), 16, 0, BAUX); \
  } while (0)

  floatx4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  // operand read offsets of the two k-steps of a stage: logical chunk
  // u * 4 + q of row c16 (mod 8) sits at position (u * 4 + q) ^ (c16 & 7)
  const int rd0 = c16 * RB + ((q ^ (c16 & 7)) * 16);
  const int rd1 = c16 * RB + (((4 + q) ^ (c16 & 7)) * 16);
  // byte-code weight fragments: k-step u, lane group q takes bytes
  // [32 u + 8 q, +8) of row c16: chunk 2 u + q / 2, half q % 2. int4: bytes
  // [16 u + 4 q, +4): chunk u, word q.
  const int rdb0 = I4 ? c16 * RBB + ((c16 >> 3) & 1) * 16 + q * 4
                      : c16 * RBB + (((q >> 1) ^ ((c16 >> 2) & 3)) * 16) + (q & 1) * 8;
  const int rdb1 = I4 ? c16 * RBB + ((1 ^ ((c16 >> 3) & 1)) * 16) + q * 4
                      : c16 * RBB + (((2 + (q >> 1)) ^ ((c16 >> 2) & 3)) * 16) + (q & 1) * 8;
  // reads a k-step's fragments: A into AF; weights into BF (bf16) or, raw, into BQ (codes)
#define MOE_READ(S, RD, RDB, AF, BF, BQ)                                                             \
  do {                                                                                               \
    _Pragma("unroll") for (int i = 0; i < FM; ++i) AF[i] =                                           \
        *reinterpret_cast<const uint4*>((S) + (wm * WTM + i * 16) * RB + RD);                        \
    _Pragma("unroll") for (int j = 0; j < FN; ++j) {                                                 \
      const int brow = SWI ? ((j < FN / 2) ? wn * (WTB / 2) + j * 16                                 \
                                           : BNO + wn * (WTB / 2) + (j - FN / 2) * 16)               \
                           : wn * WTB + j * 16;                                                      \
      if constexpr (CODES) BQ[j] = *reinterpret_cast<const BQT*>((S) + BM * RB + brow * RBB + RDB);  \
      else BF[j] = *reinterpret_cast<const uint4*>((S) + BM * RB + brow * RB + RD);                  \
    }                                                                                                \
  } while (0)
  // codes -> bf16, exact (after the reads have arrived)
#define MOE_CVT(BQ, BF)                                                                              \
  do {                                                                                               \
    if constexpr (CODES) {                                                                           \
      _Pragma("unroll") for (int j = 0; j < FN; ++j) {                                               \
        BF[j] = frag_to_bf16<WF>(BQ[j]);                                                             \
        if constexpr (I4) __builtin_amdgcn_sched_barrier(0); /* one fragment's temporaries at a time */ \
      }                                                                                              \
    }                                                                                                \
  } while (0)
#define MOE_MFMA(AC, BC)                                                                             \
  _Pragma("unroll") for (int i = 0; i < FM; ++i)                                                     \
      _Pragma("unroll") for (int j = 0; j < FN; ++j) acc[i][j] = mfma16x16x32(AC[i], BC[j], acc[i][j])
  // Issue order inside a k-step: one fragment read per two MFMAs, then the
  // remaining MFMAs; in the k-step after the barrier the MFMAs come first (the
  // MFMA unit restarts at once) and the DMA instructions are spread among
  // them. Left alone, the scheduler sinks each read down to its first use in
  // the next k-step and waits there.
  constexpr int REST = FM * FN - 2 * (FM + FN);
  static_assert(REST >= 0 && NDMA <= FM + FN, "schedule shape");
#define MOE_SCHEDULE(WITH_DMA)                                                                       \
  do {                                                                                               \
    _Pragma("unroll") for (int g_ = 0; g_ < FM + FN; ++g_) {                                         \
      if constexpr (WITH_DMA) {                                                                      \
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                                           \
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                           \
        if (g_ < NDMA) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                            \
      } else {                                                                                       \
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                           \
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                                           \
      }                                                                                              \
    }                                                                                                \
    if constexpr (REST > 0) __builtin_amdgcn_sched_group_barrier(0x008, REST, 0);                    \
    __builtin_amdgcn_sched_barrier(0);                                                               \
  } while (0)
  // Stage ks lives in buffer SC; its first k-step's fragments are in af0/bf0.
  // First half: read the second k-step's fragments, run the first's MFMAs.
  // Second half: wait for stage ks+1 (this wave's DMA, then the barrier for
  // everyone's, which also tells that all reads of SC are done), refill SC
  // with stage ks+NSTAGE, read stage ks+1's first fragments from SN, run the
  // second k-step's MFMAs.
#define MOE_STAGE(SC, SN, ks)                                                                        \
  do {                                                                                               \
    __builtin_amdgcn_s_waitcnt(0xc07f); /* lgkmcnt(0): af0/bf0 have arrived */                       \
    MOE_CVT(bq0, bf0);                                                                               \
    MOE_READ(SC, rd1, rdb1, af1, bf1, bq1);                                                          \
    MOE_MFMA(af0, bf0);                                                                              \
    MOE_SCHEDULE(false);                                                                             \
    /* stage ks+1 landed; the DMA of the NSTAGE-2 later stages may still fly */                      \
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((NSTAGE - 2) * NDMA));                                     \
    __builtin_amdgcn_s_waitcnt(0xc07f); /* lgkmcnt(0): my reads of SC are done */                    \
    __builtin_amdgcn_s_barrier();                                                                    \
    MOE_DMA(SC, MOE_COL(min((ks) + NSTAGE, n_st - 1)));                                              \
    MOE_CVT(bq1, bf1);                                                                               \
    MOE_READ(SN, rd0, rdb0, af0, bf0, bq0);                                                          \
    MOE_MFMA(af1, bf1);                                                                              \
    MOE_SCHEDULE(true);                                                                              \
  } while (0)

  // A stage of a wave whose rows all lie past the group's end (a tile's
  // second half when the tile holds at most BM/2 rows): no reads and no MFMAs,
  // but the same DMA and barriers as the other waves.
#define MOE_STAGE_IDLE(SC, ks)                                                                       \
  do {                                                                                               \
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((NSTAGE - 2) * NDMA));                                     \
    __builtin_amdgcn_s_barrier();                                                                    \
    MOE_DMA(SC, MOE_COL(min((ks) + NSTAGE, n_st - 1)));                                              \
  } while (0)
  // Loops over the stages: whole rounds of the stage buffers in the loop (a
  // conditional exit inside it makes the compiler drain every DMA at the loop
  // head), then the one or two stages left when NSTAGE is 3 (chunks hold whole
  // stage pairs).
#define MOE_STAGES(STAGE0, STAGE1, STAGE2)                                                           \
  do {                                                                                               \
    if constexpr (NSTAGE == 2) {                                                                     \
      for (int ks = 0; ks < n_st; ks += 2) {                                                         \
        STAGE0(ks);                                                                                  \
        STAGE1(ks + 1);                                                                              \
      }                                                                                              \
    } else {                                                                                         \
      const int ks_round = n_st / 3 * 3;                                                             \
      for (int ks = 0; ks < ks_round; ks += 3) {                                                     \
        STAGE0(ks);                                                                                  \
        STAGE1(ks + 1);                                                                              \
        STAGE2(ks + 2);                                                                              \
      }                                                                                              \
      if (ks_round < n_st) {                                                                         \
        STAGE0(ks_round);                                                                            \
        if (ks_round + 1 < n_st) STAGE1(ks_round + 1);                                               \
      }                                                                                              \
    }                                                                                                \
  } while (0)
#define MOE_LIVE0(ks) MOE_STAGE(S0, S1, ks)
#define MOE_LIVE1(ks) MOE_STAGE(S1, (NSTAGE == 2 ? S0 : S2), ks)
#define MOE_LIVE2(ks) MOE_STAGE(S2, S0, ks)
#define MOE_IDLE0(ks) MOE_STAGE_IDLE(S0, ks)
#define MOE_IDLE1(ks) MOE_STAGE_IDLE(S1, ks)
#define MOE_IDLE2(ks) MOE_STAGE_IDLE(S2, ks)

  uint4 af0[FM], bf0[FN], af1[FM], bf1[FN];
  BQT bq0[FN], bq1[FN];  // raw code fragments (unused for bf16 weights)
  MOE_DMA(S0, MOE_COL(0));
  MOE_DMA(S1, MOE_COL(1));
  if constexpr (NSTAGE == 3) MOE_DMA(S2, MOE_COL(min(2, n_st - 1)));
  __builtin_amdgcn_s_waitcnt(vmcnt_imm((NSTAGE - 1) * NDMA));  // the first stage landed
  __builtin_amdgcn_s_barrier();
  if (wm * WTM < ti.rows) {
    MOE_READ(S0, rd0, rdb0, af0, bf0, bq0);
    MOE_STAGES(MOE_LIVE0, MOE_LIVE1, MOE_LIVE2);
  } else {
    MOE_STAGES(MOE_IDLE0, MOE_IDLE1, MOE_IDLE2);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // the trailing DMAs have landed
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_s_barrier();
#undef MOE_LIVE0
#undef MOE_LIVE1
#undef MOE_LIVE2
#undef MOE_IDLE0
#undef MOE_IDLE1
#undef MOE_IDLE2
#undef MOE_STAGES
#undef MOE_STAGE_IDLE
#undef MOE_STAGE
#undef MOE_SCHEDULE
#undef MOE_MFMA
#undef MOE_READ
#undef MOE_CVT
#undef MOE_DMA
#undef MOE_COL
#undef MOE_LDS

  if (unit >= 0) {  // a k-chunk: raw fp32 partial sums, summed by the fix-up pass
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        *reinterpret_cast<floatx4_t*>(dma_part_frag<BM, W>(p.split_part, unit, wave, i, j) + lane * 4) = acc[i][j];
    return;
  }
  dma_store_pre<EPI, BM, W>(p, ti, acc, wave);
  dma_store_tile<EPI, BM, W>(p, ti, acc, wave);
}

template <int EPI, int BM, int W, int WF>
__global__ __launch_bounds__(64 * W, 1) void gemm_dma_kernel(GemmParams p) {
  using namespace dma;
  constexpr int BNO = bno(EPI);
  // a mixed-width launch holds the larger of the two formats' buffers
  constexpr int SBY = WF == kWIntMix ? dma_stage_bytes<BM, kWInt8>() : dma_stage_bytes<BM, WF>();
  constexpr int NSTAGE = dma_nstage<BM, W, WF>();
  __shared__ __attribute__((aligned(16))) char S0[SBY];
  __shared__ __attribute__((aligned(16))) char S1[SBY];
  __shared__ __attribute__((aligned(16))) char S2[NSTAGE == 3 ? SBY : 16];

  const int K = p.K;
  const int KS = K / BK;  // even: K is a multiple of 128
  TileInfo ti;
  int ks_begin = 0, ks_end = KS, unit = -1;
  {
    const SplitPlan sp = split_plan<BNO>(p, KS / 2);
    const int bid = blockIdx.x;
    if (sp.s == 1) {
      if (!decode_tile<BM, BNO>(p, ti)) return;
    } else if (bid < sp.full) {  // full rounds; sp.full is a multiple of the XCD count
      const int per_xcd = sp.full / kXcds;
      tile_from_linear<BM, BNO>(p, (bid % kXcds) * per_xcd + bid / kXcds, ti);
    } else {
      unit = bid - sp.full;
      if (unit >= sp.r * sp.s) return;
      const int c = unit % sp.s;
      tile_from_linear<BM, BNO>(p, sp.full + unit / sp.s, ti);
      ks_begin = 2 * ((c * (KS / 2)) / sp.s);  // chunks of whole stage pairs
      ks_end = 2 * (((c + 1) * (KS / 2)) / sp.s);
    }
  }
  if ((p.skip[ti.g >> 5] >> (ti.g & 31)) & 1u) return;  // the other bit width's launch takes this group
  if constexpr (WF == kWIntMix) {  // each tile takes its group's width
    if ((p.bits4[ti.g >> 5] >> (ti.g & 31)) & 1u)
      dma_tile_body<EPI, BM, W, kWInt4>(p, ti, ks_begin, ks_end, unit, S0, S1, S2);
    else
      dma_tile_body<EPI, BM, W, kWInt8>(p, ti, ks_begin, ks_end, unit, S0, S1, S2);
  } else if constexpr (WF == kWBf16 && BM == 128) {
    if (ti.gd.rows <= BM)  // the group's only row tile: nobody else reads its weight tiles
      dma_tile_body<EPI, BM, W, WF, kAuxNT>(p, ti, ks_begin, ks_end, unit, S0, S1, S2);
    else
      dma_tile_body<EPI, BM, W, WF>(p, ti, ks_begin, ks_end, unit, S0, S1, S2);
  } else {
    dma_tile_body<EPI, BM, W, WF>(p, ti, ks_begin, ks_end, unit, S0, S1, S2);
  }
}

// The 256 x 256 DMA tile with operands in separate buffers: two 32 KB buffers
// of activation rows, filled one stage ahead, and a ring of three 32 KB
// buffers of weight rows, filled two stages ahead (all 160 KB of LDS). The
// weight rows come from HBM, so they get the longer lead; the activation rows
// of a tile's group are mostly L2 hits. Waves, fragments, reads and the
// epilogue follow dma::Cfg<256, 8>, as gemm_dma_kernel's do for its tile.
template <int EPI>
__global__ __launch_bounds__(512, 1) void gemm_dma5_kernel(GemmParams p) {
  using namespace dma;
  using C_ = Cfg<256, 8>;
  constexpr int BM = 256, W = 8;
  constexpr bool SWI = (EPI == EPI_SWIGLU);
  constexpr int BNO = bno(EPI);
  constexpr int FM = C_::FM, FN = C_::FN, WTM = C_::WTM, WTB = C_::WTB, WGN = C_::WGN;
  constexpr int ADMA = C_::ADMA, BDMA = C_::BDMA, NDMA = C_::NDMA;
  constexpr int HB = BM * RB;  // one operand of one stage (32 KB)
  __shared__ __attribute__((aligned(16))) char SA0[HB];
  __shared__ __attribute__((aligned(16))) char SA1[HB];
  __shared__ __attribute__((aligned(16))) char SB0[HB];
  __shared__ __attribute__((aligned(16))) char SB1[HB];
  __shared__ __attribute__((aligned(16))) char SB2[HB];

  const int K = p.K;
  const int KS = K / BK;  // even: K is a multiple of 128
  TileInfo ti;
  int ks_begin = 0, ks_end = KS, unit = -1;
  {
    const SplitPlan sp = split_plan<BNO>(p, KS / 2);
    const int bid = blockIdx.x;
    if (sp.s == 1) {
      if (!decode_tile<BM, BNO>(p, ti)) return;
    } else if (bid < sp.full) {  // full rounds; sp.full is a multiple of the XCD count
      const int per_xcd = sp.full / kXcds;
      tile_from_linear<BM, BNO>(p, (bid % kXcds) * per_xcd + bid / kXcds, ti);
    } else {
      unit = bid - sp.full;
      if (unit >= sp.r * sp.s) return;
      const int c = unit % sp.s;
      tile_from_linear<BM, BNO>(p, sp.full + unit / sp.s, ti);
      ks_begin = 2 * ((c * (KS / 2)) / sp.s);  // chunks of whole stage pairs
      ks_end = 2 * (((c + 1) * (KS / 2)) / sp.s);
    }
  }
  const int n_st = ks_end - ks_begin;  // even
#define MOE_COL(j) (ks_begin + (j))
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: wave-level pointers stay in SGPRs
  const int wm = wave / WGN, wn = wave % WGN;
  const int q = lane >> 4, c16 = lane & 15;
  const bool shared = ti.g >= p.n_routed;
  const int ew = shared ? ti.gd.widx - p.n_routed : ti.gd.widx;
  const int n0 = ti.n_tile * BNO;
  const int64_t lda = shared ? p.lda_s : p.lda_r;
  const int32_t* gth = shared ? nullptr : p.gather;
  const int arow0 = ti.gd.a_row0 + ti.m_tile * BM;  // the tile's first row in the group's A rows
  const char* A = static_cast<const char*>(shared ? p.A_s : p.A_r) + (gth ? 0 : static_cast<int64_t>(arow0) * lda * 2);
  const int ar0 = wave * C_::AROWS, wr0 = wave * C_::BROWS;
  const bool w3 = SWI && wr0 >= BNO;
  const char* Bw = static_cast<const char*>(w3 ? (shared ? p.B3_s : p.B3_r) : (shared ? p.B_s : p.B_r)) +
                   (static_cast<int64_t>(ew) * p.b_stride + static_cast<int64_t>(n0 + (w3 ? wr0 - BNO : wr0)) * p.ldb) * 2;
  uint32_t offa[ADMA], offb[BDMA];
#pragma unroll
  for (int i = 0; i < ADMA; ++i) {
    const int r = ar0 + i * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ (r & 7);
    const int rr = r > ti.rows - 1 ? ti.rows - 1 : r;  // rows past the group compute garbage, never stored
    const int src = gth ? gth[arow0 + rr] : rr;
    offa[i] = static_cast<uint32_t>(src * static_cast<int>(lda) * 2 + chunk * 16);
  }
#pragma unroll
  for (int i = 0; i < BDMA; ++i) {
    const int r = wr0 + i * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ (r & 7);
    offb[i] = static_cast<uint32_t>((i * 8 + (lane >> 3)) * static_cast<int>(p.ldb) * 2 + chunk * 16);
  }
  const int dst_a = ar0 * RB, dst_b = wr0 * RB;  // byte offsets inside a buffer
#define MOE_LDS(x) ((__attribute__((address_space(3))) void*)(x))
#define MOE_DMA_A(S, ks)                                                                             \
  do {                                                                                               \
    const uint32_t ko_ = static_cast<uint32_t>(ks) * RB;                                             \
    _Pragma("unroll") for (int i_ = 0; i_ < ADMA; ++i_)                                              \
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(A + (offa[i_] + ko_)), MOE_LDS((S) + dst_a + i_ * 1024), 16, 0, 0); \
  } while (0)
#define MOE_DMA_B(S, ks)                                                                             \
  do {                                                                                               \
    const uint32_t ko_ = static_cast<uint32_t>(ks) * RB;                                             \
    _Pragma("unroll") for (int i_ = 0; i_ < BDMA; ++i_)                                              \
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(Bw + (offb[i_] + ko_)), MOE_LDS((S) + dst_b + i_ * 1024), 16, 0, 0); \
  } while (0)

  floatx4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  const int rd0 = c16 * RB + ((q ^ (c16 & 7)) * 16);
  const int rd1 = c16 * RB + (((4 + q) ^ (c16 & 7)) * 16);
#define MOE_READ(SA, SB, RD, AF, BF)                                                                 \
  do {                                                                                               \
    _Pragma("unroll") for (int i = 0; i < FM; ++i) AF[i] =                                           \
        *reinterpret_cast<const uint4*>((SA) + (wm * WTM + i * 16) * RB + RD);                       \
    _Pragma("unroll") for (int j = 0; j < FN; ++j) {                                                 \
      const int brow = SWI ? ((j < FN / 2) ? wn * (WTB / 2) + j * 16                                 \
                                           : BNO + wn * (WTB / 2) + (j - FN / 2) * 16)               \
                           : wn * WTB + j * 16;                                                      \
      BF[j] = *reinterpret_cast<const uint4*>((SB) + brow * RB + RD);                                \
    }                                                                                                \
  } while (0)
#define MOE_MFMA(AC, BC)                                                                             \
  _Pragma("unroll") for (int i = 0; i < FM; ++i)                                                     \
      _Pragma("unroll") for (int j = 0; j < FN; ++j) acc[i][j] = mfma16x16x32(AC[i], BC[j], acc[i][j])
  constexpr int REST = FM * FN - 2 * (FM + FN);
  static_assert(REST >= 0 && BDMA <= FM + FN, "schedule shape");
  // as in gemm_dma_kernel; after the barrier the B DMA instructions are spread
  // among the MFMAs (the A ones go first, see MOE_STAGE5)
#define MOE_SCHEDULE(WITH_DMA)                                                                       \
  do {                                                                                               \
    _Pragma("unroll") for (int g_ = 0; g_ < FM + FN; ++g_) {                                         \
      if constexpr (WITH_DMA) {                                                                      \
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                                           \
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                           \
        if (g_ < BDMA) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                            \
      } else {                                                                                       \
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                           \
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                                           \
      }                                                                                              \
    }                                                                                                \
    if constexpr (REST > 0) __builtin_amdgcn_sched_group_barrier(0x008, REST, 0);                    \
    __builtin_amdgcn_sched_barrier(0);                                                               \
  } while (0)
  // Stage ks: activation rows in SAC, weight rows in SBC, first k-step's
  // fragments in af0/bf0. First half: read the second k-step's fragments, run
  // the first's MFMAs. Then wait until only the newest weight DMA (stage
  // ks + 2) may still fly, so stage ks + 1 has landed; barrier (everyone's
  // stage ks + 1 is in, and all reads of SAC / SBC are done); refill SAC with
  // stage ks + 2's activation rows and SBC with stage ks + 3's weight rows
  // (the activation DMA first, so that it is older than the weight DMA that
  // the next wait leaves in flight); read stage ks + 1's first fragments, run
  // the second k-step's MFMAs.
#define MOE_STAGE5(SAC, SBC, SAN, SBN, ks)                                                           \
  do {                                                                                               \
    __builtin_amdgcn_s_waitcnt(0xc07f); /* lgkmcnt(0): af0/bf0 have arrived */                       \
    MOE_READ(SAC, SBC, rd1, af1, bf1);                                                               \
    MOE_MFMA(af0, bf0);                                                                              \
    MOE_SCHEDULE(false);                                                                             \
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(BDMA));                                                     \
    __builtin_amdgcn_s_waitcnt(0xc07f); /* lgkmcnt(0): my reads of SAC / SBC are done */             \
    __builtin_amdgcn_s_barrier();                                                                    \
    MOE_DMA_A(SAC, MOE_COL(min((ks) + 2, n_st - 1)));                                                \
    __builtin_amdgcn_sched_barrier(0);                                                               \
    MOE_DMA_B(SBC, MOE_COL(min((ks) + 3, n_st - 1)));                                                \
    MOE_READ(SAN, SBN, rd0, af0, bf0);                                                               \
    MOE_MFMA(af1, bf1);                                                                              \
    MOE_SCHEDULE(true);                                                                              \
  } while (0)
  // a stage of a wave whose rows all lie past the group's end: the same DMA
  // and barriers, no reads or MFMAs
#define MOE_STAGE5_IDLE(SAC, SBC, SAN, SBN, ks)                                                      \
  do {                                                                                               \
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(BDMA));                                                     \
    __builtin_amdgcn_s_barrier();                                                                    \
    MOE_DMA_A(SAC, MOE_COL(min((ks) + 2, n_st - 1)));                                                \
    __builtin_amdgcn_sched_barrier(0);                                                               \
    MOE_DMA_B(SBC, MOE_COL(min((ks) + 3, n_st - 1)));                                                \
  } while (0)
  // whole rounds of six stages (activation buffers cycle by 2, weight buffers
  // by 3) with no exit inside the loop, then the 0, 2 or 4 stages left
#define MOE_STAGES5(STAGE)                                                                           \
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
    if (n_round < n_st) {                                                                            \
      STAGE(SA0, SB0, SA1, SB1, n_round);                                                            \
      STAGE(SA1, SB1, SA0, SB2, n_round + 1);                                                        \
      if (n_round + 2 < n_st) {                                                                      \
        STAGE(SA0, SB2, SA1, SB0, n_round + 2);                                                      \
        STAGE(SA1, SB0, SA0, SB1, n_round + 3);                                                      \
      }                                                                                              \
    }                                                                                                \
  } while (0)

  uint4 af0[FM], bf0[FN], af1[FM], bf1[FN];
  MOE_DMA_A(SA0, MOE_COL(0));
  MOE_DMA_B(SB0, MOE_COL(0));
  MOE_DMA_A(SA1, MOE_COL(1));
  MOE_DMA_B(SB1, MOE_COL(1));
  MOE_DMA_B(SB2, MOE_COL(min(2, n_st - 1)));
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(ADMA + 2 * BDMA));  // stage 0 landed
  __builtin_amdgcn_s_barrier();
  if (wm * WTM < ti.rows) {
    MOE_READ(SA0, SB0, rd0, af0, bf0);
    MOE_STAGES5(MOE_STAGE5);
  } else {
    MOE_STAGES5(MOE_STAGE5_IDLE);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // the trailing DMAs have landed
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_s_barrier();
#undef MOE_STAGES5
#undef MOE_STAGE5_IDLE
#undef MOE_STAGE5
#undef MOE_SCHEDULE
#undef MOE_MFMA
#undef MOE_READ
#undef MOE_DMA_B
#undef MOE_DMA_A
#undef MOE_LDS
#undef MOE_COL

  if (unit >= 0) {  // a k-chunk: raw fp32 partial sums, summed by the fix-up pass
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        *reinterpret_cast<floatx4_t*>(dma_part_frag<BM, W>(p.split_part, unit, wave, i, j) + lane * 4) = acc[i][j];
    return;
  }
  dma_store_pre<EPI, BM, W>(p, ti, acc, wave);
  dma_store_tile<EPI, BM, W>(p, ti, acc, wave);
}

// Fix-up of the k-split tiles: one wave per (split tile, wave of the tile's
// layout), kFixWaves waves a workgroup, so the r split tiles spread over W r
// waves on as many CUs instead of one workgroup each. A wave sums its
// fragments' s partial tiles in chunk order and runs that wave's part of the
// tile epilogue.
constexpr int kFixWaves = 4;
template <int EPI, int BM, int W>
__global__ __launch_bounds__(64 * kFixWaves) void gemm_split_fixup_kernel(GemmParams p) {
  using namespace dma;
  using C_ = Cfg<BM, W>;
  constexpr int BNO = bno(EPI);
  constexpr int FM = C_::FM, FN = C_::FN;
  const SplitPlan sp = split_plan<BNO>(p, p.K / BK / 2);
  const int gw = blockIdx.x * kFixWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = gw / W, wave = gw % W;
  if (sp.s == 1 || b >= sp.r) return;
  TileInfo ti;
  tile_from_linear<BM, BNO>(p, sp.full + b, ti);
  if ((p.skip[ti.g >> 5] >> (ti.g & 31)) & 1u) return;  // the other bit width's launch takes this group
  const int lane = threadIdx.x & 63;
  // two chunks in flight: the loads of chunk c + 1 are issued before chunk c
  // is added (the adds stay in chunk order); the 256-row tile's fragments go
  // in two halves, so that two chunks of them fit the registers
  constexpr int FG = FM * FN > 16 ? FM / 2 : FM;  // fragment rows a pass
  floatx4_t acc[FM][FN];
#pragma unroll
  for (int i0 = 0; i0 < FM; i0 += FG) {
    floatx4_t b0[FG][FN], b1[FG][FN];
    auto load = [&](floatx4_t (&dst)[FG][FN], int c) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < FG; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          dst[i][j] = *reinterpret_cast<const floatx4_t*>(
              dma_part_frag<BM, W>(p.split_part, b * sp.s + c, wave, i0 + i, j) + lane * 4);
    };
    auto add = [&](const floatx4_t (&src)[FG][FN], bool first) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < FG; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i0 + i][j] = first ? src[i][j] : acc[i0 + i][j] + src[i][j];
    };
    load(b0, 0);
    for (int c = 0; c < sp.s; c += 2) {  // s >= 2
      if (c + 1 < sp.s) load(b1, c + 1);
      add(b0, c == 0);
      if (c + 2 < sp.s) load(b0, c + 2);
      if (c + 1 < sp.s) add(b1, false);
    }
  }
  dma_store_pre<EPI, BM, W>(p, ti, acc, wave);
  dma_store_tile<EPI, BM, W>(p, ti, acc, wave);
}

// ------------------------------------------------------------------ fp32
// Plain FMA tiles (64 x 64 outputs, 4 x 4 per thread) for fp32 layers.
template <int EPI>
__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(GemmParams p) {
  constexpr bool SWI = (EPI == EPI_SWIGLU);
  constexpr int BM = 64, BNO = 64, BK = 16;
  constexpr int BNB = SWI ? 2 * BNO : BNO;
  __shared__ float sA[BK][BM + 4];
  __shared__ float sB[BK][BNB + 4];

  TileInfo ti;
  if (!decode_tile<BM, BNO>(p, ti)) return;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const bool shared = ti.g >= p.n_routed;
  const int widx = ti.gd.widx;
  const int ew = shared ? widx - p.n_routed : widx;
  const int n0 = ti.n_tile * BNO;
  const int K = p.K;
  const int64_t lda = shared ? p.lda_s : p.lda_r;
  const float* A = static_cast<const float*>(shared ? p.A_s : p.A_r) +
                   (static_cast<int64_t>(ti.gd.a_row0) + static_cast<int64_t>(ti.m_tile) * BM) * lda;
  const float* Bw = static_cast<const float*>(shared ? p.B_s : p.B_r) + static_cast<int64_t>(ew) * p.b_stride;
  const float* B3w = SWI ? static_cast<const float*>(shared ? p.B3_s : p.B3_r) + static_cast<int64_t>(ew) * p.b_stride
                         : nullptr;

  float acc[4][4] = {}, acc3[4][4] = {};
  for (int kb = 0; kb < K; kb += BK) {
    {
      int r = tid >> 2;
      const int k4 = (tid & 3) * 4;
      const int rr = r > ti.rows - 1 ? ti.rows - 1 : r;
      const float4 v = *reinterpret_cast<const float4*>(A + static_cast<int64_t>(rr) * lda + kb + k4);
      sA[k4 + 0][r] = v.x;
      sA[k4 + 1][r] = v.y;
      sA[k4 + 2][r] = v.z;
      sA[k4 + 3][r] = v.w;
    }
    for (int c = tid; c < BNB * 4; c += kThreads) {
      const int r = c >> 2, k4 = (c & 3) * 4;
      const float* src = (SWI && r >= BNO) ? B3w + static_cast<int64_t>(n0 + r - BNO) * p.ldb
                                           : Bw + static_cast<int64_t>(n0 + r) * p.ldb;
      const float4 v = *reinterpret_cast<const float4*>(src + kb + k4);
      sB[k4 + 0][r] = v.x;
      sB[k4 + 1][r] = v.y;
      sB[k4 + 2][r] = v.z;
      sB[k4 + 3][r] = v.w;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float av[4], bv[4], b3[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        av[i] = sA[kk][ty * 4 + i];
        bv[i] = sB[kk][tx * 4 + i];
        if (SWI) b3[i] = sB[kk][BNO + tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
          if (SWI) acc3[i][j] = fmaf(av[i], b3[j], acc3[i][j]);
        }
    }
    __syncthreads();
  }
  const float* bias = (!shared && p.bias) ? p.bias + static_cast<int64_t>(ew) * p.Nout : nullptr;
  float* C = static_cast<float*>(shared ? p.C_s : p.C_r) +
             (static_cast<int64_t>(ti.gd.c_row0) + static_cast<int64_t>(ti.m_tile) * BM) * p.ldc + n0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = ty * 4 + i;
    if (row >= ti.rows) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = tx * 4 + j;
      float v;
      if constexpr (EPI == EPI_SWIGLU) v = silu(acc[i][j]) * acc3[i][j];
      else if constexpr (EPI == EPI_GELU) v = gelu_erf(acc[i][j] + (bias ? bias[n0 + col] : 0.f));
      else v = acc[i][j] + (bias ? bias[n0 + col] : 0.f);
      C[static_cast<int64_t>(row) * p.ldc + col] = v;
    }
  }
}

// ------------------------------------------------------------------ plan
__global__ __launch_bounds__(kThreads) void plan_kernel(const int32_t* offsets, FfnPlan pl) {
  __shared__ int32_t s_mt[2 * kMaxGroups];
  plan_groups(offsets, pl, s_mt, threadIdx.x, kThreads);
}

template <int BM, int BNB, int WGM, int WGN, int EPI, int WF, int PF = MOE_GEMM_PF>
hipError_t run_bf16(const GemmParams& p, int64_t max_mtiles, hipStream_t s) {
  constexpr int BNO = (EPI == EPI_SWIGLU) ? BNB / 2 : BNB;
  if (p.Nout % BNO != 0) return hipErrorInvalidValue;
  int64_t grid = max_mtiles * (p.Nout / BNO);
  grid = ceil_div(grid, kXcds) * kXcds;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BNB, WGM, WGN, EPI, WF, PF>), dim3(static_cast<unsigned>(grid)),
                     dim3(64 * WGM * WGN), 0, s, p);
  return hipGetLastError();
}

// Tile configurations of the bf16-activation path (any weight format).
enum TileCfg {
  kReg128 = 0,  // register-staged 128 x 128, 4 waves: fewer than 2048 rows
  kDma256 = 1,  // LDS-DMA 256 x 256: many rows per group
  kDma128 = 2,  // LDS-DMA 128 x 256: few rows per group
};
constexpr int tile_rows(int cfg) { return cfg == kDma256 ? 256 : 128; }

template <int EPI, int BM, int W, int WF = kWBf16>
hipError_t run_dma(const GemmParams& p_in, int64_t max_mtiles, hipStream_t s) {
  GemmParams p = p_in;
  p.mat_scaled = WF == kWE4m3 ? 1 : 0;
  p.col_scaled = (WF == kWInt8 || WF == kWInt4 || WF == kWIntMix) ? 1 : 0;
  constexpr int BNO = dma::bno(EPI);
  if (p.Nout % BNO != 0 || p.K % 128 != 0) return hipErrorInvalidValue;
  int64_t grid = max_mtiles * (p.Nout / BNO);
  grid = ceil_div(grid, kXcds) * kXcds;
  if (grid <= 0) return hipSuccess;
  // a k-split tail runs at most total - r + kSplitUnits workgroups
  if (p.split_part) grid += kSplitUnits;
  constexpr int NTH = dma::Cfg<BM, W>::NTH;
  hipLaunchKernelGGL((gemm_dma_kernel<EPI, BM, W, WF>), dim3(static_cast<unsigned>(grid)), dim3(NTH), 0, s, p);
  if (p.split_part) {
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    // split tiles: r <= kSplitUnits / 2 (each is cut at least in two)
    hipLaunchKernelGGL((gemm_split_fixup_kernel<EPI, BM, W>), dim3(kSplitUnits / 2 * W / kFixWaves),
                       dim3(64 * kFixWaves), 0, s, p);
  }
  return hipGetLastError();
}

template <int EPI>
hipError_t run_dma5(const GemmParams& p, int64_t max_mtiles, hipStream_t s) {
  constexpr int BNO = dma::bno(EPI);
  if (p.Nout % BNO != 0 || p.K % 128 != 0) return hipErrorInvalidValue;
  int64_t grid = max_mtiles * (p.Nout / BNO);
  grid = ceil_div(grid, kXcds) * kXcds;
  if (grid <= 0) return hipSuccess;
  // a k-split tail runs at most total - r + kSplitUnits workgroups
  if (p.split_part) grid += kSplitUnits;
  hipLaunchKernelGGL((gemm_dma5_kernel<EPI>), dim3(static_cast<unsigned>(grid)), dim3(512), 0, s, p);
  if (p.split_part) {
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    // split tiles: r <= kSplitUnits / 2 (each is cut at least in two); the
    // partial tiles have the fragment layout of dma::Cfg<256, 8>
    hipLaunchKernelGGL((gemm_split_fixup_kernel<EPI, 256, 8>), dim3(kSplitUnits / 2 * 8 / kFixWaves),
                       dim3(64 * kFixWaves), 0, s, p);
  }
  return hipGetLastError();
}

template <int EPI>
hipError_t run_f32(const GemmParams& p, int64_t max_mtiles, hipStream_t s) {
  int64_t grid = max_mtiles * (p.Nout / 64);
  grid = ceil_div(grid, kXcds) * kXcds;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_f32_kernel<EPI>), dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <int EPI, int WF>
hipError_t run_cfg(int cfg, const GemmParams& p, int64_t max_mtiles, hipStream_t s) {
  if constexpr (WF == kWIntMix) {  // the DMA tiles only
    switch (cfg) {
      case kDma256: return run_dma<EPI, 256, 8, WF>(p, max_mtiles, s);
      case kDma128: return run_dma<EPI, 128, 8, WF>(p, max_mtiles, s);
      default: return hipErrorInvalidValue;
    }
  } else if constexpr (WF != kWBf16) {
    switch (cfg) {
      case kDma256: return run_dma<EPI, 256, 8, WF>(p, max_mtiles, s);
      case kDma128: return run_dma<EPI, 128, 8, WF>(p, max_mtiles, s);
      default: return run_bf16<128, 128, 2, 2, EPI, WF>(p, max_mtiles, s);
    }
  } else {
    switch (cfg) {
      case kDma256: return run_dma5<EPI>(p, max_mtiles, s);
      case kDma128: return run_dma<EPI, 128, 8>(p, max_mtiles, s);
      default: return run_bf16<128, 128, 2, 2, EPI, kWBf16>(p, max_mtiles, s);
    }
  }
}

template <int EPI>
hipError_t run_wf(int wf, int cfg, const GemmParams& p, int64_t max_mtiles, hipStream_t s) {
  switch (wf) {
    case kWE4m3: return run_cfg<EPI, kWE4m3>(cfg, p, max_mtiles, s);
    case kWInt8: return run_cfg<EPI, kWInt8>(cfg, p, max_mtiles, s);
    case kWInt4: return run_cfg<EPI, kWInt4>(cfg, p, max_mtiles, s);
    case kWIntMix: return run_cfg<EPI, kWIntMix>(cfg, p, max_mtiles, s);
    default: return run_cfg<EPI, kWBf16>(cfg, p, max_mtiles, s);
  }
}

// Tile configuration of a call (any weight format): register-staged tiles for
// few rows; for many rows the LDS-DMA tiles, 256 rows when the groups average
// at least 384 rows, else 128 (less padding in each group's last tile).
// Measured: the fine-grained layer (about 400 rows a group, two shared
// experts of 8192) runs 4 % faster on 256-row tiles, the Switch layer (at most
// 320) 11 % slower. Widths that the 256-column tiles do not fit take the
// 128 x 128 tiles.
int pick_cfg(const FfnArgs& a) {
  const int64_t rows = a.routed_row_cap + static_cast<int64_t>(a.n_shared) * a.T;
  if (rows < 2048 || !wide_tiles_fit(a.act, a.d, a.d_ff)) return kReg128;
  return rows >= 384LL * (a.n_routed + a.n_shared) ? kDma256 : kDma128;
}

// Compute units of the current device, cached per device.
int device_cus() {
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

}  // namespace

bool swi_layer(const FfnArgs& a) { return a.act == 1; }

int ffn_path_of(const FfnArgs& a) {
  if (use_skinny(a.act_dtype, a.routed_row_cap, a.n_shared, a.T)) return kPathStream;
  if (a.act_dtype == 0) return kPathF32;
  switch (pick_cfg(a)) {
    case kDma256: return kPathDma256;
    case kDma128: return kPathDma128;
    default: return kPathReg128;
  }
}

WeightClasses weight_classes(const FfnArgs& a) {
  WeightClasses wc{};
  if (a.w_dtype != 3) {
    wc.n = 1;
    wc.wf[0] = a.w_dtype == 2 ? kWE4m3 : kWBf16;
    return wc;
  }
  const int G = a.n_routed + a.n_shared;
  uint32_t m4[9] = {};
  bool any8 = false, any4 = false;
  for (int g = 0; g < G; ++g) {
    const int b = g < a.n_routed ? a.w_bits[g] : a.sw_bits[g - a.n_routed];
    if (b == 4) {
      m4[g >> 5] |= 1u << (g & 31);
      any4 = true;
    } else {
      any8 = true;
    }
  }
  if (any8) {
    wc.wf[wc.n] = kWInt8;
    for (int i = 0; i < 9; ++i) wc.skip[wc.n][i] = m4[i];
    ++wc.n;
  }
  if (any4) {
    wc.wf[wc.n] = kWInt4;
    for (int i = 0; i < 9; ++i) wc.skip[wc.n][i] = ~m4[i];
    ++wc.n;
  }
  return wc;
}

FfnPlan ffn_plan(const FfnArgs& a) {
  const int G = a.n_routed + a.n_shared;
  FfnPlan pl;
  pl.up = a.groups;
  pl.down = a.groups + G;
  pl.tile_start = a.tile_start;
  pl.active = a.active;
  pl.n_routed = a.n_routed;
  pl.n_shared = a.n_shared;
  pl.T = static_cast<int32_t>(a.T);
  pl.cap = a.routed_row_cap;
  const int cfg = a.act_dtype == 0 ? -1 : pick_cfg(a);
  pl.bm = a.act_dtype == 0 ? 64 : tile_rows(cfg);
  // 256-row tiles leave tails of at most 128 rows to 128-row tiles
  pl.bm_t = (cfg == kDma256 && a.groups_t && a.tile_start_t) ? 128 : 0;
  pl.up_t = a.groups_t;
  pl.down_t = a.groups_t ? a.groups_t + G : nullptr;
  pl.tile_start_t = a.tile_start_t;
  // per-width prefixes: mixed widths on the register-staged tiles (one launch
  // per width); the DMA tiles take both widths in one launch
  const WeightClasses wc = weight_classes(a);
  const bool per_width = wc.n == 2 && cfg != kDma256 && cfg != kDma128;
  pl.tile_start_c = per_width ? a.tile_start_c : nullptr;
  for (int i = 0; i < 9; ++i) pl.cls1[i] = per_width ? wc.skip[0][i] : 0u;  // width 0 skips the 4-bit groups
  return pl;
}

hipError_t launch_grouped_ffn(const FfnArgs& a_in, hipStream_t s) {
  FfnArgs a = a_in;
  const int G = a.n_routed + a.n_shared;
  if (G > kMaxGroups) return hipErrorInvalidValue;
  if (a.routed_row_cap + static_cast<int64_t>(a.n_shared) * a.T == 0) return hipSuccess;  // no rows at all
  const bool f32 = (a.act_dtype == 0);
  const int cfg = pick_cfg(a);
  if (a.pre_up_u && ((cfg != kDma256 && cfg != kDma128) || a.w_dtype != 1))
    return hipErrorInvalidValue;  // DMA tiles on bf16 weights only
  const FfnPlan pl = ffn_plan(a);
  const int bm = pl.bm;
  GroupDesc* up = pl.up;
  GroupDesc* down = pl.down;
  hipError_t err = hipSuccess;
  if (!a.planned) {
    stage_mark(kStageFfnPlan, false, s);
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kThreads), 0, s, a.offsets, pl);
    stage_mark(kStageFfnPlan, true, s);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (use_skinny(a.act_dtype, a.routed_row_cap, a.n_shared, a.T)) return launch_ffn_skinny(a, up, down, a.part, s);
  if (a.gather && f32) return hipErrorInvalidValue;  // the fp32 tiles read routed rows from x_perm only
  // upper bound on row tiles: every group may end in a partial tile
  const int64_t max_mtiles = ceil_div(a.routed_row_cap, bm) + a.n_routed + a.n_shared * ceil_div(a.T, bm);
  const bool swi = (a.act == 1);
  // integer weights with 8- and 4-bit experts: on the DMA tiles one launch
  // (kWIntMix, each tile taking its group's width); on the register-staged
  // tiles one launch per width, each skipping the other width's groups and
  // walking its own row-tile prefix
  WeightClasses wc = weight_classes(a);
  GemmParams p{};
  if (wc.n == 2 && !pl.tile_start_c) {
    for (int i = 0; i < 9; ++i) {
      p.bits4[i] = wc.skip[0][i];  // the 8-bit class skips the 4-bit groups
      wc.skip[0][i] = 0;
    }
    wc.n = 1;
    wc.wf[0] = kWIntMix;
  }

  p.pre_u_r = p.pre_u_s = a.pre_up_u;
  p.pre_v_r = p.pre_v_s = a.pre_up_v;
  p.ld_pre = a.ld_pre_up;
  p.split_part = a.split_part;
  p.ncu = device_cus();
  p.n_routed = a.n_routed;
  p.n_groups = G;
  p.tile_start = a.tile_start;
  // up GEMM: [rows][d] x [d_ff][d]^T -> h [rows][d_ff]; routed rows from
  // x_perm, or from x through the permutation's token list
  p.A_r = a.gather ? a.x : a.x_perm;
  p.gather = a.gather;
  p.A_s = a.x;
  p.lda_r = a.gather ? a.d : a.ld_xp;
  p.lda_s = a.d;
  p.B_r = a.w1;
  p.B3_r = a.w3;
  p.B_s = a.sw1;
  p.B3_s = a.sw3;
  p.ldb = a.ld_up;
  p.b_stride = a.d_ff * a.ld_up;
  p.bias = swi ? nullptr : a.b1;
  p.scale_r = a.w_scale;
  p.scale_s = a.sw_scale;
  p.scale_col = 0;
  p.scale_pitch = static_cast<int32_t>(2 * a.d_ff + a.d);
  p.scale_row0 = 0;
  p.scale_row3 = static_cast<int32_t>(a.d_ff);
  p.C_r = a.h;
  p.C_s = a.h;
  p.ldc = a.ld_h;
  p.K = static_cast<int32_t>(a.d);
  p.Nout = static_cast<int32_t>(a.d_ff);
  p.groups = up;
  stage_mark(kStageFfnUp, false, s);
  if (f32) {
    err = swi ? run_f32<EPI_SWIGLU>(p, max_mtiles, s) : run_f32<EPI_GELU>(p, max_mtiles, s);
  } else {
    for (int c = 0; c < wc.n && err == hipSuccess; ++c) {
      for (int i = 0; i < 9; ++i) p.skip[i] = wc.skip[c][i];
      if (pl.tile_start_c) p.tile_start = pl.tile_start_c + 2 * c * (G + 1);
      err = swi ? run_wf<EPI_SWIGLU>(wc.wf[c], cfg, p, max_mtiles, s) : run_wf<EPI_GELU>(wc.wf[c], cfg, p, max_mtiles, s);
    }
    if (pl.bm_t > 0) {  // small groups and the groups' short tails on 128-row tiles
      GemmParams pt = p;
      pt.groups = pl.up_t;
      pt.tile_start = pl.tile_start_t;
      const int64_t mt = static_cast<int64_t>(kSmallGroupTiles) * G;  // row tiles of the second plan, at most
      for (int c = 0; c < wc.n && err == hipSuccess; ++c) {
        for (int i = 0; i < 9; ++i) pt.skip[i] = wc.skip[c][i];
        if (pl.tile_start_c) pt.tile_start = pl.tile_start_c + (2 * c + 1) * (G + 1);
        err = swi ? run_wf<EPI_SWIGLU>(wc.wf[c], kDma128, pt, mt, s) : run_wf<EPI_GELU>(wc.wf[c], kDma128, pt, mt, s);
      }
    }
  }
  stage_mark(kStageFfnUp, true, s);
  if (err != hipSuccess || a.up_only) return err;

  // down GEMM: h [rows][d_ff] x [d][d_ff]^T -> y [rows][d]
  p.A_r = a.h;
  p.gather = nullptr;
  p.A_s = a.h;
  p.lda_r = a.ld_h;
  p.lda_s = a.ld_h;
  p.B_r = a.w2;
  p.B3_r = nullptr;
  p.B_s = a.sw2;
  p.B3_s = nullptr;
  p.ldb = a.ld_down;
  p.b_stride = a.d * a.ld_down;
  p.bias = swi ? nullptr : a.b2;
  p.scale_col = 2;
  p.scale_row0 = static_cast<int32_t>(2 * a.d_ff);
  p.scale_row3 = 0;
  p.C_r = a.y_perm;
  p.C_s = a.y_shared;
  p.ldc = a.d;
  p.pre_u_r = p.pre_u_s = p.pre_v_r = p.pre_v_s = nullptr;
  p.K = static_cast<int32_t>(a.d_ff);
  p.Nout = static_cast<int32_t>(a.d);
  p.groups = down;
  stage_mark(kStageFfnDown, false, s);
  if (f32) {
    err = run_f32<EPI_PLAIN>(p, max_mtiles, s);
  } else {
    for (int c = 0; c < wc.n && err == hipSuccess; ++c) {
      for (int i = 0; i < 9; ++i) p.skip[i] = wc.skip[c][i];
      if (pl.tile_start_c) p.tile_start = pl.tile_start_c + 2 * c * (G + 1);
      err = run_wf<EPI_PLAIN>(wc.wf[c], cfg, p, max_mtiles, s);
    }
    if (pl.bm_t > 0) {
      GemmParams pt = p;
      pt.groups = pl.down_t;
      pt.tile_start = pl.tile_start_t;
      const int64_t mt = static_cast<int64_t>(kSmallGroupTiles) * G;
      for (int c = 0; c < wc.n && err == hipSuccess; ++c) {
        for (int i = 0; i < 9; ++i) pt.skip[i] = wc.skip[c][i];
        if (pl.tile_start_c) pt.tile_start = pl.tile_start_c + (2 * c + 1) * (G + 1);
        err = run_wf<EPI_PLAIN>(wc.wf[c], kDma128, pt, mt, s);
      }
    }
  }
  stage_mark(kStageFfnDown, true, s);
  return err;
}

}  // namespace moe
