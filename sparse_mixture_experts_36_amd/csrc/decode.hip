// Grouped expert FFN for decode-sized row counts: expert-weight streaming.
//
// Pages: vanos001 "MoE Architecture" / "Expert Network Design" (SwiGLU and
// GELU experts), aigrafen.se "Mixture of Experts" (every expert must sit in
// memory while only the selected ones are used per token), learn.starphix.com
// "Mixture of Experts (MoE)" / "Shared + Specialized" and "Quantization".
//
// With a few rows per expert the layer is bound by reading each touched
// expert's weights once from HBM, so the design maximises bytes in flight:
//  - a wave owns 32 weight rows of one expert (SwiGLU up: the same 16 rows of
//    W1 and W3; otherwise 32 rows of W1 or W2) and a k range, and streams them
//    from memory straight into MFMA operand registers (no LDS): per 128-wide
//    k-step, each bf16 load instruction reads 64 contiguous bytes of each of
//    16 rows;
//  - every load of two (or four) k-steps is issued before the first MFMA that
//    needs them (a scheduling barrier keeps the compiler from interleaving and
//    draining): each row is then read in runs of 512 bytes or more, which HBM
//    serves better than the same bytes requested one step at a time;
//  - the token rows (16, 32 or 64 per pass, the MFMA's M) come from L2;
//  - waves run over the groups that have rows only (the plan kernel lists
//    them), so a token's two experts do not dispatch work for all eight;
//  - when few experts are touched, k is split across waves; fp32 partials are
//    then summed in split order by a second kernel that also applies the
//    activation or the bias (bit-for-bit reproducible).
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;  // 4 independent waves per workgroup
constexpr int KC = 128;        // k per step
// s_waitcnt immediate for vmcnt(n), the other counters left at their maximum
constexpr int vmcnt_imm(int n) { return 0x0f70 | (n & 15) | (((n >> 4) & 3) << 14); }
// KU: k-steps in flight per wave (a template argument: 1, 2 or 4; 4 when few
// waves run and each must keep more bytes in flight)

struct StreamParams {
  const uint16_t* A_r;       // routed A rows (x_perm or h; x when gathered)
  const int32_t* gather;     // routed A row r of a group is row gather[a_row0 + r] of A_r, or null
  const uint16_t* A_s;       // shared A rows (x or h)
  int64_t lda_r, lda_s;      // A row pitches (elements)
  int64_t ldb;               // weight row pitch (elements)
  const char* B_r;           // weights of routed experts (bytes)
  const char* B3_r;          // W3 (SwiGLU up) or null
  const char* B_s;
  const char* B3_s;
  int64_t b_stride;          // elements per expert matrix
  const float* bias;         // [n_routed][Nout] (routed GELU experts) or null
  const float* scale_r;      // e4m3 scales [n_routed][3]; integer weights: row scales [n_routed][scale_pitch]
  const float* scale_s;
  int scale_col;
  int32_t scale_pitch;       // integer weights: floats per expert in the row-scale arrays (2 d_ff + d)
  int32_t scale_row0;        // integer weights: offset of this GEMM's matrix rows (W1 0, W2 2 d_ff)
  int32_t scale_row3;        // integer weights: offset of W3's rows (d_ff)
  uint32_t skip[9];          // bit g set: group g is left to another launch (its experts' other bit width)
  uint32_t bits4[9];         // mixed-width launches (kWIntMix): bit g set: group g has 4-bit codes, else 8
  uint16_t* C_r;             // outputs (h / y_perm) for routed groups
  uint16_t* C_s;             //              (h / y_shared) for shared groups
  int64_t ldc;
  int32_t c_shared_base;     // partial-row base of shared groups (down: cap, up: 0)
  float* part;               // [splits][rows_total][width] or null (direct epilogue)
  int32_t rows_total, width; // partial buffer shape
  int32_t K, Nout, splits;
  int32_t n_routed, n_groups;
  int32_t epi;               // 0 GELU (+b1), 1 SwiGLU, 2 plain (+b2)
  const GroupDesc* groups;
  const int32_t* active;     // [0]: groups with rows, [1..]: those groups
};

// The combine folded into the decode down GEMM (one token): its slots' rows,
// gates and expert ids, and the layer output row.
struct FusedCombine {
  const int32_t* inv_map;   // [k] row of each routed slot, -1 dropped
  const int32_t* topk_idx;  // [k]
  const float* topk_w;      // [k]
  int32_t k, n_shared;
  void* y;                  // [d] bf16
};

// Bytes of k consecutive weights of a row: bf16 2k, e4m3 and int8 k, int4 k/2
// (integer rows live at a pitch of ldb bytes whatever the expert's bit width).
template <int WF>
__device__ __forceinline__ constexpr uint32_t kbytes(uint32_t k) {
  return WF == kWBf16 ? 2 * k : (WF == kWInt4 ? k / 2 : k);
}
// Bytes of one row-pitch element.
template <int WF>
constexpr int pitch_bytes() { return WF == kWBf16 ? 2 : 1; }
// Weight load instructions per k-step of one row (16 bytes each).
template <int WF>
constexpr int loads_per_step() { return WF == kWBf16 ? 4 : (WF == kWInt4 ? 1 : 2); }

// One 16-byte weight load with the nontemporal hint, where every load
// instruction covers whole 128-byte lines: the GEMVs (a wave reads 1 KB of one
// row) and the streaming kernel's bf16 line loads (load_w). A plain
// grid-stride read of 2 GiB measured 5.3-5.6 TB/s with ordinary 16-byte loads
// and 5.6-6.1 TB/s with the hint, at every unroll and grid tried; the Mixtral
// one-token step went from 134 to 125.6 us. Where an instruction reads only
// half of each line (the streaming kernel's former loads: 64 bytes of each of
// 16 rows, the next instruction the other half) the hint made the second
// request come from memory again (16-token step 512 -> 594 us); the integer
// codes keep ordinary loads for that reason.
__device__ __forceinline__ uint4 ld_weight16(const char* p) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// One k-step of a weight row for lane (row, q): 32 weights from byte offset
// `off` of a wave-uniform base, w[t] holding MFMA t's eight (e4m3 and int8
// codes in .x/.y, int4 codes in .x, decoded to bf16 in registers).
//
// bf16 rows (256 bytes a step) are read in whole 128-byte lines, so that the
// loads can carry the nontemporal hint: w[2p] covers line p of rows 0-7 of
// the 16-row tile and w[2p + 1] line p of rows 8-15 (offsets `off` and
// `off2`, see line_offsets); wfrag forms MFMA t's operand from them.
template <int WF>
__device__ __forceinline__ void load_w(const char* base, uint32_t off, uint32_t off2, uint4 (&w)[4]) {
  if constexpr (WF == kWE4m3 || WF == kWInt8) {
    const uint4 q0 = *reinterpret_cast<const uint4*>(base + off);
    const uint4 q1 = *reinterpret_cast<const uint4*>(base + (off + 16));
    w[0] = make_uint4(q0.x, q0.y, 0, 0);
    w[1] = make_uint4(q0.z, q0.w, 0, 0);
    w[2] = make_uint4(q1.x, q1.y, 0, 0);
    w[3] = make_uint4(q1.z, q1.w, 0, 0);
  } else if constexpr (WF == kWInt4) {
    const uint4 q0 = *reinterpret_cast<const uint4*>(base + off);
    w[0] = make_uint4(q0.x, 0, 0, 0);
    w[1] = make_uint4(q0.y, 0, 0, 0);
    w[2] = make_uint4(q0.z, 0, 0, 0);
    w[3] = make_uint4(q0.w, 0, 0, 0);
  } else {
#pragma unroll
    for (int l = 0; l < 2; ++l) {
      w[2 * l] = ld_weight16(base + (off + 128 * l));
      w[2 * l + 1] = ld_weight16(base + (off2 + 128 * l));
    }
  }
}

// Lane offsets of the whole-line bf16 loads of a 16-row tile (rows row0 ..
// row0 + 15, row pitch ldb_bytes), lane (c16, q): the first load of a line
// takes row row0 + (c16 & 7), the second row row0 + 8 + (c16 & 7), each at
// 16-byte chunk q of the line's first half for one half of the lanes and of
// its second half for the other, so that each load reads 8 whole lines.
__device__ __forceinline__ void line_offsets(int row0, int ldb_bytes, int c16, int q, uint32_t& off,
                                             uint32_t& off2) {
  const int r = row0 + (c16 & 7);
  off = static_cast<uint32_t>(r * ldb_bytes + 16 * q + (c16 >= 8 ? 64 : 0));
  off2 = static_cast<uint32_t>((r + 8) * ldb_bytes + 16 * q + (c16 < 8 ? 64 : 0));
}

// One dword of MFMA operand 2p + hi from the two loads a, b of line p: lane
// (c16, q) needs row c16, chunk 4 hi + q. For hi = 0 lanes 0-7 of each 16-lane
// row hold it in a and lanes 8-15 in b; for hi = 1 it sits 8 lanes over, in a
// for lanes 0-7 and in b for lanes 8-15 (DPP row rotation by 8, the second
// move writing banks 2-3 only).
__device__ __forceinline__ uint32_t line_pick(uint32_t a, uint32_t b, bool hi) {
  if (!hi) return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(a), static_cast<int>(b), 0xE4, 0xF, 0xC, false));
  const int r = __builtin_amdgcn_mov_dpp(static_cast<int>(a), 0x128, 0xF, 0xF, false);  // row_ror:8
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(r, static_cast<int>(b), 0x128, 0xF, 0xC, false));
}

template <int WF>
__device__ __forceinline__ uint4 as_bf16(const uint4& w) {
  if constexpr (WF == kWE4m3) {
    const uint2 a = e4m3x4_to_bf16x4(w.x), b = e4m3x4_to_bf16x4(w.y);
    return make_uint4(a.x, a.y, b.x, b.y);
  } else if constexpr (WF == kWInt8) {
    const uint2 a = int8x4_to_bf16x4(w.x), b = int8x4_to_bf16x4(w.y);
    return make_uint4(a.x, a.y, b.x, b.y);
  } else if constexpr (WF == kWInt4) {
    return int4x8_to_bf16x8_biased(w.x);  // q + 136: the kernels subtract 136 * sum(x)
  } else {
    return w;
  }
}

// MFMA t's B operand (bf16) from the loads of load_w.
template <int WF>
__device__ __forceinline__ uint4 wfrag(const uint4 (&w)[4], int t) {
  if constexpr (WF == kWBf16) {
    const uint4 a = w[2 * (t >> 1)], b = w[2 * (t >> 1) + 1];
    const bool hi = t & 1;
    return make_uint4(line_pick(a.x, b.x, hi), line_pick(a.y, b.y, hi), line_pick(a.z, b.z, hi),
                      line_pick(a.w, b.w, hi));
  } else {
    return as_bf16<WF>(w[t]);
  }
}

// MFMA B operand of bf16 136 in every element: A times it is 136 * sum(x) per
// token row, the correction of the biased int4 products.
__device__ __forceinline__ uint4 int4_bias_b() {
  return make_uint4(kInt4BiasPair, kInt4BiasPair, kInt4BiasPair, kInt4BiasPair);
}

// Whether group g is left to another launch (integer weights of the other bit width).
__device__ __forceinline__ bool skipped(const StreamParams& p, int g) { return (p.skip[g >> 5] >> (g & 31)) & 1u; }

// The scale of weight row `row` of matrix offset `moff` (integer weights: one
// per row), or the e4m3 scale of the matrix, or 1.
template <int WF>
__device__ __forceinline__ float wscale(const StreamParams& p, bool shared, int ew, int moff, int row, int col) {
  const float* sc = shared ? p.scale_s : p.scale_r;
  if constexpr (WF == kWE4m3) return sc[ew * 3 + col];
  if constexpr (WF == kWInt8 || WF == kWInt4) return sc[static_cast<int64_t>(ew) * p.scale_pitch + moff + row];
  return 1.f;
}

__device__ __forceinline__ float epilogue(int epi, float a, float b, float bias) {
  if (epi == 1) return silu(a) * b;
  if (epi == 0) return gelu_erf(a + bias);
  return a + bias;
}

// Wave -> (group g, block nb of 32 weight rows, k split sp).
//
// SHARED_A (RB >= 2, KU = 2): the four waves of a workgroup take four
// consecutive blocks of one expert at one k range, and the token rows of each
// burst (16 RB rows x 256 k) are brought into LDS once per workgroup by LDS DMA
// (the weight loads fly at the same time) instead of once per wave into
// registers. Row R's 16-byte chunk c sits at position c ^ (R & 15), so the 16
// lanes that read one chunk of 16 rows hit 16 different bank groups. The two
// LDS buffers alternate by burst, one barrier per burst; the host guarantees
// an even number of bursts per pass.
template <int RB, int KU, bool SHARED_A>
constexpr int stream_atile() { return SHARED_A ? 16 * RB * KU * KC * 2 : 16; }  // bytes of a burst's token rows

// Wave w's share of the streaming GEMM: group g (which has rows), block and k
// split from w; abuf0 / abuf1 hold the token rows of alternate bursts
// (SHARED_A).
template <int RB, int WF, int KU, bool SHARED_A>
__device__ __forceinline__ void stream_body(const StreamParams& p, char* abuf0, char* abuf1, int w, int g) {
  static_assert(!SHARED_A || KU == 2 || KU == 4, "shared token rows: two or four k-steps a burst");
  constexpr int AROWB = KU * KC * 2;                         // bytes of one token row per burst
  constexpr int ATILE = stream_atile<RB, KU, SHARED_A>();
  constexpr int ADMA = ATILE / (kThreads * 16);              // DMA instructions per lane and burst
  constexpr int FN = 2;  // 16-row weight tiles per wave
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4, c16 = lane & 15;
  const bool swi = (p.epi == 1);
  const int nblk = swi ? p.Nout / 16 : p.Nout / 32;  // blocks per expert
  const int per_g = nblk * p.splits;
  const GroupDesc gd = p.groups[g];
  if (gd.rows <= 0) return;
  const int nb = SHARED_A ? (w % per_g) % nblk : (w % per_g) / p.splits;
  const int sp = SHARED_A ? (w % per_g) / nblk : w % p.splits;
  const bool shared = g >= p.n_routed;
  const int ew = shared ? g - p.n_routed : g;
  constexpr int EB = pitch_bytes<WF>();
  constexpr bool BYTE = WF != kWBf16;  // a byte or half a byte per weight
  // k order inside a 128-wide step (the same for both operands, so any order
  // gives the same sums): bf16 MFMA t takes k [32t, 32t + 32), lane group q
  // its 8 k at 8q (the weight loads read whole lines and DPP moves form the
  // operands, see load_w); with e4m3 / int8 codes lane group q takes k
  // [32q, 32q + 32) in two 16-byte loads (int4: one), MFMA t its 8 k at 8t
  constexpr int QK = BYTE ? 32 : 8;        // k offset of lane group q
  constexpr int AT = BYTE ? 16 : 64;       // A bytes between MFMA t and t + 1
  const int K = p.K, ks = K / p.splits;
  const int kbeg = sp * ks, nsteps = ks / KC;
  // weight rows: SwiGLU up takes rows [n0, n0 + 16) of W1 (tile 0) and of W3
  // (tile 1), otherwise rows [n0, n0 + 32) of one matrix; the bases point at
  // (row n0, column kbeg), the lane offsets add row and k-group
  const int n0 = swi ? nb * 16 : nb * 32;
  const int64_t eoff = (static_cast<int64_t>(ew) * p.b_stride + static_cast<int64_t>(n0) * p.ldb) * EB +
                       kbytes<WF>(static_cast<uint32_t>(kbeg));
  const char* Bw = (shared ? p.B_s : p.B_r) + eoff;
  const char* B3w = swi ? (shared ? p.B3_s : p.B3_r) + eoff : Bw;
  const char* wbase[FN] = {Bw, swi ? B3w : Bw};
  uint32_t woff[FN], woff2[FN];
  float sw[FN];  // the scale of the lane's weight row in tile j
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int r = swi ? c16 : j * 16 + c16;
    if constexpr (BYTE) {
      woff[j] = static_cast<uint32_t>(r * static_cast<int>(p.ldb) * EB) + kbytes<WF>(static_cast<uint32_t>(q * QK));
      woff2[j] = woff[j];
    } else {
      line_offsets(r - c16, static_cast<int>(p.ldb) * EB, c16, q, woff[j], woff2[j]);
    }
    const bool third = swi && j == 1;
    sw[j] = wscale<WF>(p, shared, ew, third ? p.scale_row3 : p.scale_row0, n0 + r, p.scale_col + (third ? 1 : 0));
  }
  const int64_t lda = shared ? p.lda_s : p.lda_r;
  // A rows are addressed from the buffer's start (column kbeg): row r of the
  // group is buffer row a_row0 + r, or gather[a_row0 + r]
  const char* A = reinterpret_cast<const char*>((shared ? p.A_s : p.A_r) + kbeg);
  const int32_t* gth = shared ? nullptr : p.gather;

  for (int r0 = 0; r0 < gd.rows; r0 += 16 * RB) {
    // opaque to the optimiser, so that the first loads' addresses are formed
    // here from base + offset, not hoisted out of the pass loop as 64-bit pointers
#pragma unroll
    for (int j = 0; j < FN; ++j) asm volatile("" : "+v"(woff[j]), "+v"(woff2[j]));
    const char* Ap = A;
    uint32_t aoff[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int arow = gd.a_row0 + min(r0 + rb * 16 + c16, gd.rows - 1);  // rows past the group compute garbage
      const int src = gth ? gth[arow] : arow;
      aoff[rb] = static_cast<uint32_t>((src * static_cast<int>(lda) + q * QK) * 2);
    }
    floatx4_t acc[RB][FN];
    floatx4_t accc[RB];  // int4: 136 * sum(x) of each token row (the bias of the decoded codes)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      accc[rb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[rb][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    }

    if constexpr (SHARED_A) {
      // DMA instruction i of wave v fills bytes [1024 (v ADMA + i), +1024) of
      // the tile: lane L writes row R = (1024 (v ADMA + i) + 16 L) / AROWB at
      // position L' = L % (AROWB / 16), which holds logical chunk L' ^ (R & 15)
      // (k-step L' / 16 of the burst, k 8 (L' % 16) of that step)
      const int wv = (threadIdx.x >> 6);
      uint32_t doff[ADMA];
#pragma unroll
      for (int i = 0; i < ADMA; ++i) {
        const int byte = (wv * ADMA + i) * 1024 + lane * 16;
        const int R = byte / AROWB, pos = (byte % AROWB) / 16;
        const int c = pos ^ (R & 15);
        const int arow = gd.a_row0 + min(r0 + R, gd.rows - 1);
        const int src = gth ? gth[arow] : arow;
        doff[i] = static_cast<uint32_t>(src * static_cast<int>(lda) * 2 + (c >> 4) * (KC * 2) + (c & 15) * 16);
      }
      // lane (c16, q) of MFMA t, k-step u, row block rb: logical chunk u*16 + ch(t, q)
      auto burst = [&](char* abuf, int st) __attribute__((always_inline)) {
        const uint32_t kb = static_cast<uint32_t>(st * KC * 2);
#pragma unroll
        for (int i = 0; i < ADMA; ++i)
          __builtin_amdgcn_global_load_lds(static_cast<const void*>(Ap + (doff[i] + kb)),
                                           (__attribute__((address_space(3))) void*)(abuf + (wv * ADMA + i) * 1024),
                                           16, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        uint4 bw[KU][FN][4];
#pragma unroll
        for (int u = 0; u < KU; ++u) {
          const uint32_t kk = static_cast<uint32_t>((st + u) * KC);
#pragma unroll
          for (int j = 0; j < FN; ++j) load_w<WF>(wbase[j], woff[j] + kbytes<WF>(kk), woff2[j] + kbytes<WF>(kk), bw[u][j]);
        }
        __builtin_amdgcn_sched_barrier(0);
        // this wave's token-row DMA has landed (loads complete in issue order)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(KU * FN * loads_per_step<WF>()));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < KU; ++u)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int ch = u * 16 + (BYTE ? q * 4 + t : t * 4 + q);
            uint4 av[RB];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
              const int R = rb * 16 + c16;
              av[rb] = *reinterpret_cast<const uint4*>(abuf + R * AROWB + ((ch ^ (R & 15)) * 16));
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
              const uint4 b = wfrag<WF>(bw[u][j], t);
#pragma unroll
              for (int rb = 0; rb < RB; ++rb) acc[rb][j] = mfma16x16x32(av[rb], b, acc[rb][j]);
            }
            if constexpr (WF == kWInt4) {
#pragma unroll
              for (int rb = 0; rb < RB; ++rb) accc[rb] = mfma16x16x32(av[rb], int4_bias_b(), accc[rb]);
            }
          }
      };
      // the buffers alternate by burst; the barrier inside each burst also
      // tells that every wave is done with the buffer the next burst refills.
      // nsteps is a multiple of KU (the host checks), not always of 2 KU.
      for (int st = 0; st < nsteps; st += 2 * KU) {
        burst(abuf0, st);
        if (st + KU < nsteps) burst(abuf1, st + KU);
      }
    } else {
    for (int st = 0; st < nsteps; st += KU) {
      uint4 bw[KU][FN][4], a[KU][RB][4];
#pragma unroll
      for (int u = 0; u < KU; ++u) {
        const uint32_t kk = static_cast<uint32_t>(min(st + u, nsteps - 1) * KC);  // a step past the end re-reads the last one
#pragma unroll
        for (int j = 0; j < FN; ++j) load_w<WF>(wbase[j], woff[j] + kbytes<WF>(kk), woff2[j] + kbytes<WF>(kk), bw[u][j]);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int t = 0; t < 4; ++t)
            a[u][rb][t] = *reinterpret_cast<const uint4*>(Ap + (aoff[rb] + kk * 2 + t * AT));
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < KU; ++u) {
        if (st + u >= nsteps) break;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const uint4 b = wfrag<WF>(bw[u][j], t);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) acc[rb][j] = mfma16x16x32(a[u][rb][t], b, acc[rb][j]);
          }
          if constexpr (WF == kWInt4) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) accc[rb] = mfma16x16x32(a[u][rb][t], int4_bias_b(), accc[rb]);
          }
        }
      }
    }
    }
    if constexpr (WF == kWInt4) {  // remove the bias: sum((q + 136) x) - 136 sum(x)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[rb][j] -= accc[rb];
    }

    // tile j, lane (q, c16): rows r0 + rb*16 + 4q + i, weight row n of tile j
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = r0 + rb * 16 + q * 4 + i;
        if (row >= gd.rows) continue;
        if (p.part) {
          const int prow = (shared ? p.c_shared_base : 0) + gd.c_row0 + row;
          float* dst = p.part + (static_cast<int64_t>(sp) * p.rows_total + prow) * p.width;
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            // partial columns: SwiGLU [W1 results | W3 results], otherwise the output columns
            const int col = swi ? (j == 0 ? n0 + c16 : p.Nout + n0 + c16) : n0 + j * 16 + c16;
            dst[col] = acc[rb][j][i] * sw[j];
          }
        } else {
          uint16_t* C = (shared ? p.C_s : p.C_r) + (static_cast<int64_t>(gd.c_row0) + row) * p.ldc;
          const float* bias = (!shared && p.bias) ? p.bias + static_cast<int64_t>(ew) * p.Nout : nullptr;
          if (swi) {
            C[n0 + c16] = f32_to_bf16(epilogue(1, acc[rb][0][i] * sw[0], acc[rb][1][i] * sw[1], 0.f));
          } else {
#pragma unroll
            for (int j = 0; j < FN; ++j) {
              const int col = n0 + j * 16 + c16;
              C[col] = f32_to_bf16(epilogue(p.epi, acc[rb][j][i] * sw[j], 0.f, bias ? bias[col] : 0.f));
            }
          }
        }
      }
    }
  }
}

// Whether group g of a mixed-width launch has 4-bit codes.
__device__ __forceinline__ bool group_int4(const StreamParams& p, int g) { return (p.bits4[g >> 5] >> (g & 31)) & 1u; }

// The streaming GEMM: wave w -> group, block and k split. WF = kWIntMix runs
// the 8- and 4-bit experts of an integer layer in one launch, each wave taking
// its group's width.
template <int RB, int WF, int KU, bool SHARED_A>
__global__ __launch_bounds__(kThreads) void stream_kernel(StreamParams p) {
  constexpr int ATILE = stream_atile<RB, KU, SHARED_A>();
  __shared__ __attribute__((aligned(16))) char abuf0[ATILE];
  __shared__ __attribute__((aligned(16))) char abuf1[ATILE];
  const int nblk = p.epi == 1 ? p.Nout / 16 : p.Nout / 32;  // blocks per expert
  // the wave index is made wave-uniform, so that group, expert and base
  // pointers live in scalar registers and loads take a 32-bit lane offset
  const int w = blockIdx.x * (kThreads / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slot = w / (nblk * p.splits);  // waves run over the groups that have rows only
  if (slot >= p.active[0]) return;
  const int g = p.active[1 + slot];
  if (g >= p.n_groups || skipped(p, g)) return;
  if constexpr (WF == kWIntMix) {
    if (group_int4(p, g)) stream_body<RB, kWInt4, KU, SHARED_A>(p, abuf0, abuf1, w, g);
    else stream_body<RB, kWInt8, KU, SHARED_A>(p, abuf0, abuf1, w, g);
  } else {
    stream_body<RB, WF, KU, SHARED_A>(p, abuf0, abuf1, w, g);
  }
}

// Sums the split partials in split order, applies the activation / bias and
// writes bf16. Block (x, R): partial row R, columns [x*1024, x*1024 + 1024), four
// per thread; all split loads are issued before the fixed-order sum. Rows never
// written (past the routed rows) are skipped.
constexpr int kRedCols = 4 * kThreads;

__global__ __launch_bounds__(kThreads) void stream_reduce_kernel(StreamParams p, const int32_t* offsets,
                                                                  int32_t cap) {
  const int R = blockIdx.y;
  const int c = blockIdx.x * kRedCols + threadIdx.x * 4;
  if (c >= p.Nout) return;
  // the group that owns partial row R: routed rows first, then T rows per shared expert
  int g = -1, row = 0;
  if (R < cap) {
    const int routed_rows = min(offsets[p.n_routed], cap);
    if (R >= routed_rows) return;
    int lo = 0, hi = p.n_routed - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (offsets[mid] <= R) lo = mid; else hi = mid - 1;
    }
    g = lo;
    row = R - offsets[g];
  } else {
    const int T = (p.rows_total - cap) / (p.n_groups - p.n_routed);
    g = p.n_routed + (R - cap) / T;
    row = (R - cap) % T;
  }
  const GroupDesc gd = p.groups[g];
  const bool shared = g >= p.n_routed;
  uint16_t* C = (shared ? p.C_s : p.C_r) + (static_cast<int64_t>(gd.c_row0) + row) * p.ldc + c;
  const float* bias = (!shared && p.bias) ? p.bias + static_cast<int64_t>(g) * p.Nout + c : nullptr;
  const int64_t plane = static_cast<int64_t>(p.rows_total) * p.width;
  const float* src = p.part + static_cast<int64_t>(R) * p.width + c;
  constexpr int kMaxSplits = 16;
  float4 va[kMaxSplits], vb[kMaxSplits];
#pragma unroll
  for (int sp = 0; sp < kMaxSplits; ++sp)
    if (sp < p.splits) {
      va[sp] = *reinterpret_cast<const float4*>(src + sp * plane);
      if (p.epi == 1) vb[sp] = *reinterpret_cast<const float4*>(src + sp * plane + p.Nout);
    }
  float4 a = va[0], b = make_float4(0.f, 0.f, 0.f, 0.f);
  if (p.epi == 1) b = vb[0];
#pragma unroll
  for (int sp = 1; sp < kMaxSplits; ++sp)
    if (sp < p.splits) {
      a.x += va[sp].x; a.y += va[sp].y; a.z += va[sp].z; a.w += va[sp].w;
      if (p.epi == 1) { b.x += vb[sp].x; b.y += vb[sp].y; b.z += vb[sp].z; b.w += vb[sp].w; }
    }
  const float4 bv = bias ? *reinterpret_cast<const float4*>(bias) : make_float4(0.f, 0.f, 0.f, 0.f);
  const float o0 = epilogue(p.epi, a.x, b.x, bv.x), o1 = epilogue(p.epi, a.y, b.y, bv.y);
  const float o2 = epilogue(p.epi, a.z, b.z, bv.z), o3 = epilogue(p.epi, a.w, b.w, bv.w);
  *reinterpret_cast<uint2*>(C) = make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
}

// ---- at most two token rows per expert: a weight-row GEMV on the vector ALUs
//
// With one or two rows an MFMA tile would be 15/16 padding, and the k split it
// needs for enough waves costs a partials pass. Here a wave owns NR weight rows
// of one expert (SwiGLU up: NR/2 rows of W1 and the same NR/2 rows of W3) and
// reads each over the whole k range in 1 KB segments, lane l taking 16 bytes
// at 16 l. A burst loads U segments of all NR rows, so each row is read in runs
// of U KB. Products are bf16 pair dots accumulated in fp32; each lane's sums
// are reduced across the wave once, at the end (a fixed butterfly order).
constexpr int kSeg = 1024;  // bytes of one weight row per segment

// Wave w's NR weight rows of group g (which has rows).
template <int R, int WF, int NR, int U>
__device__ __forceinline__ void gemv_body(const StreamParams& p, int w, int g) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  const int lane = threadIdx.x & 63;
  const bool swi = (p.epi == 1);
  const int cols = swi ? NR / 2 : NR;  // output columns per wave
  const int nblk = p.Nout / cols;
  const GroupDesc gd = p.groups[g];
  if (gd.rows <= 0) return;
  const int n0 = (w % nblk) * cols;
  const bool shared = g >= p.n_routed;
  const int ew = shared ? g - p.n_routed : g;
  constexpr int EB = pitch_bytes<WF>();
  constexpr int KSEG = WF == kWBf16 ? kSeg / 2 : (WF == kWInt4 ? 2 * kSeg : kSeg);  // k per segment
  constexpr int XW = KSEG / 512;    // activation uint4 per lane and segment
  const int nseg = p.K / KSEG;
  const int64_t eoff = (static_cast<int64_t>(ew) * p.b_stride + static_cast<int64_t>(n0) * p.ldb) * EB;
  const char* Bw = (shared ? p.B_s : p.B_r) + eoff;
  const char* B3w = swi ? (shared ? p.B3_s : p.B3_r) + eoff : Bw;
  const char* wrow[NR];
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    const bool third = swi && j >= NR / 2;
    wrow[j] = (third ? B3w : Bw) + static_cast<int64_t>(third ? j - NR / 2 : j) * p.ldb * EB;
  }
  const int64_t lda = shared ? p.lda_s : p.lda_r;
  const char* A = reinterpret_cast<const char*>(shared ? p.A_s : p.A_r);
  const int32_t* gth = shared ? nullptr : p.gather;
  const char* arow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int ar = gd.a_row0 + min(r, gd.rows - 1);
    arow[r] = A + static_cast<int64_t>(gth ? gth[ar] : ar) * lda * 2;
  }
  // lane l: weight bytes [16 l, 16 l + 16) of a segment, i.e. k from
  // seg * KSEG + l * KSEG / 64, and the bf16 activations of those k
  const uint32_t wl = static_cast<uint32_t>(lane) * 16;
  const uint32_t al = static_cast<uint32_t>(lane) * 16 * XW;

  float acc[NR][R];
  float accc[R];  // int4: 136 * sum(x) over the lane's k (the bias of the decoded codes)
#pragma unroll
  for (int r = 0; r < R; ++r) {
    accc[r] = 0.f;
#pragma unroll
    for (int j = 0; j < NR; ++j) acc[j][r] = 0.f;
  }

  for (int s0 = 0; s0 < nseg; s0 += U) {
    uint4 wv[U][NR], xv[U][R][XW];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t sg = static_cast<uint32_t>(min(s0 + u, nseg - 1));  // a segment past the end re-reads the last one
#pragma unroll
      for (int j = 0; j < NR; ++j) wv[u][j] = ld_weight16(wrow[j] + (wl + sg * kSeg));
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int x = 0; x < XW; ++x)
          xv[u][r][x] = *reinterpret_cast<const uint4*>(arow[r] + (al + sg * (KSEG * 2) + 16 * x));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s0 + u >= nseg) break;
      if constexpr (WF == kWInt4) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float c = accc[r];
#pragma unroll
          for (int x = 0; x < XW; ++x) {
            const uint32_t xd[4] = {xv[u][r][x].x, xv[u][r][x].y, xv[u][r][x].z, xv[u][r][x].w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
              c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kInt4BiasPair),
                                                  __builtin_bit_cast(bf16x2, xd[i]), c, false);
          }
          accc[r] = c;
        }
      }
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        uint32_t wd[4 * XW];
        if constexpr (WF == kWE4m3 || WF == kWInt8) {
          const uint32_t q4[4] = {wv[u][j].x, wv[u][j].y, wv[u][j].z, wv[u][j].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint2 b = WF == kWE4m3 ? e4m3x4_to_bf16x4(q4[i]) : int8x4_to_bf16x4(q4[i]);
            wd[2 * i] = b.x;
            wd[2 * i + 1] = b.y;
          }
        } else if constexpr (WF == kWInt4) {
          const uint32_t q4[4] = {wv[u][j].x, wv[u][j].y, wv[u][j].z, wv[u][j].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint4 b = int4x8_to_bf16x8_biased(q4[i]);  // q + 136
            wd[4 * i] = b.x;
            wd[4 * i + 1] = b.y;
            wd[4 * i + 2] = b.z;
            wd[4 * i + 3] = b.w;
          }
        } else {
          wd[0] = wv[u][j].x; wd[1] = wv[u][j].y; wd[2] = wv[u][j].z; wd[3] = wv[u][j].w;
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float c = acc[j][r];
#pragma unroll
          for (int x = 0; x < XW; ++x) {
            const uint32_t xd[4] = {xv[u][r][x].x, xv[u][r][x].y, xv[u][r][x].z, xv[u][r][x].w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
              c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wd[4 * x + i]),
                                                  __builtin_bit_cast(bf16x2, xd[i]), c, false);
          }
          acc[j][r] = c;
        }
      }
    }
  }

#pragma unroll
  for (int j = 0; j < NR; ++j)
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) acc[j][r] += __shfl_xor(acc[j][r], o);
  if constexpr (WF == kWInt4) {  // remove the bias: sum((q + 136) x) - 136 sum(x)
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) accc[r] += __shfl_xor(accc[r], o);
#pragma unroll
      for (int j = 0; j < NR; ++j) acc[j][r] -= accc[r];
    }
  }

  // lane c < cols writes output column n0 + c of each row
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r >= gd.rows) break;
    uint16_t* C = (shared ? p.C_s : p.C_r) + (static_cast<int64_t>(gd.c_row0) + r) * p.ldc + n0;
    const float* bias = (!shared && p.bias) ? p.bias + static_cast<int64_t>(ew) * p.Nout + n0 : nullptr;
#pragma unroll
    for (int c = 0; c < NR; ++c) {
      if (c >= cols || lane != c) continue;
      const float s_a = wscale<WF>(p, shared, ew, p.scale_row0, n0 + c, p.scale_col);
      const float s_b = swi ? wscale<WF>(p, shared, ew, p.scale_row3, n0 + c, p.scale_col + 1) : s_a;
      const float v = swi ? epilogue(1, acc[c][r] * s_a, acc[(c + NR / 2) % NR][r] * s_b, 0.f)
                          : epilogue(p.epi, acc[c][r] * s_a, 0.f, bias ? bias[c] : 0.f);
      C[c] = f32_to_bf16(v);
    }
  }
}

// The GEMV: wave w -> group and row block. WF = kWIntMix runs the 8- and
// 4-bit experts in one launch (4-bit rows with half the segments a burst, as
// in their own launches).
template <int R, int WF, int NR, int U>
__global__ __launch_bounds__(kThreads) void gemv_kernel(StreamParams p) {
  const int nblk = p.Nout / (p.epi == 1 ? NR / 2 : NR);
  const int w = blockIdx.x * (kThreads / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slot = w / nblk;  // waves run over the groups that have rows only
  if (slot >= p.active[0]) return;
  const int g = p.active[1 + slot];
  if (g >= p.n_groups || skipped(p, g)) return;
  if constexpr (WF == kWIntMix) {
    if (group_int4(p, g)) gemv_body<R, kWInt4, NR, U / 2>(p, w, g);
    else gemv_body<R, kWInt8, NR, U>(p, w, g);
  } else {
    gemv_body<R, WF, NR, U>(p, w, g);
  }
}

// One token (T = 1): the down GEMM with the combine folded in. Wave w owns
// output columns [NC w, NC w + NC) and streams those W2 rows of every slot of
// the token -- its routed slots in order (a dropped one is skipped), then the
// shared experts -- against the slot's row of h, in 1 KB segments of each row
// as the GEMV does. Each lane's sums are reduced across the wave in a fixed
// order, then the slots are added with their gates in slot order (the
// combine's order) and the layer output is written in bf16. The expert
// outputs are not rounded to bf16 before that sum, as y_perm rows are.
template <int WF, int S, int NC, int U>
__global__ __launch_bounds__(kThreads) void gemv_combine_kernel(StreamParams p, FusedCombine f) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  static_assert(WF == kWBf16 || WF == kWE4m3, "bf16 or e4m3 weights");
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * (kThreads / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = w * NC;
  if (n0 >= p.Nout) return;
  constexpr int EB = pitch_bytes<WF>();
  constexpr int KSEG = WF == kWBf16 ? kSeg / 2 : kSeg;  // k per segment
  constexpr int XW = KSEG / 512;                        // activation uint4 per lane and segment
  const int nseg = p.K / KSEG;
  // slot s: group (-1: none), row of h, gate; all wave-uniform
  int grp[S], hrow[S];
  float gate[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    grp[s] = -1;
    hrow[s] = 0;
    gate[s] = 1.f;
    if (s < f.k) {
      const int r = f.inv_map[s];
      if (r >= 0) {
        grp[s] = f.topk_idx[s];
        hrow[s] = r;
        gate[s] = f.topk_w[s];
      }
    } else if (s < f.k + f.n_shared) {
      grp[s] = p.n_routed + (s - f.k);
      hrow[s] = p.groups[grp[s]].a_row0;
    }
    grp[s] = __builtin_amdgcn_readfirstlane(grp[s]);
    hrow[s] = __builtin_amdgcn_readfirstlane(hrow[s]);
  }
  const char* wrow[S][NC];
  const char* arow[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const bool shared = grp[s] >= p.n_routed;
    const int ew = grp[s] < 0 ? 0 : (shared ? grp[s] - p.n_routed : grp[s]);
    const char* base = (shared ? p.B_s : p.B_r) + (static_cast<int64_t>(ew) * p.b_stride + static_cast<int64_t>(n0) * p.ldb) * EB;
#pragma unroll
    for (int c = 0; c < NC; ++c) wrow[s][c] = base + static_cast<int64_t>(c) * p.ldb * EB;
    arow[s] = reinterpret_cast<const char*>(shared ? p.A_s : p.A_r) +
              static_cast<int64_t>(hrow[s]) * (shared ? p.lda_s : p.lda_r) * 2;
  }
  const uint32_t wl = static_cast<uint32_t>(lane) * 16;
  const uint32_t al = static_cast<uint32_t>(lane) * 16 * XW;
  float acc[S][NC];
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[s][c] = 0.f;

  for (int s0 = 0; s0 < nseg; s0 += U) {
    uint4 wv[U][S][NC], xv[U][S][XW];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t sg = static_cast<uint32_t>(min(s0 + u, nseg - 1));  // a segment past the end re-reads the last one
#pragma unroll
      for (int s = 0; s < S; ++s) {
        if (grp[s] < 0) continue;
#pragma unroll
        for (int c = 0; c < NC; ++c) wv[u][s][c] = ld_weight16(wrow[s][c] + (wl + sg * kSeg));
#pragma unroll
        for (int x = 0; x < XW; ++x)
          xv[u][s][x] = *reinterpret_cast<const uint4*>(arow[s] + (al + sg * (KSEG * 2) + 16 * x));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s0 + u >= nseg) break;
#pragma unroll
      for (int s = 0; s < S; ++s) {
        if (grp[s] < 0) continue;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          uint32_t wd[4 * XW];
          if constexpr (WF == kWE4m3) {
            const uint32_t q4[4] = {wv[u][s][c].x, wv[u][s][c].y, wv[u][s][c].z, wv[u][s][c].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint2 b = e4m3x4_to_bf16x4(q4[i]);
              wd[2 * i] = b.x;
              wd[2 * i + 1] = b.y;
            }
          } else {
            wd[0] = wv[u][s][c].x; wd[1] = wv[u][s][c].y; wd[2] = wv[u][s][c].z; wd[3] = wv[u][s][c].w;
          }
          float a = acc[s][c];
#pragma unroll
          for (int x = 0; x < XW; ++x) {
            const uint32_t xd[4] = {xv[u][s][x].x, xv[u][s][x].y, xv[u][s][x].z, xv[u][s][x].w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
              a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wd[4 * x + i]),
                                                  __builtin_bit_cast(bf16x2, xd[i]), a, false);
          }
          acc[s][c] = a;
        }
      }
    }
  }
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) acc[s][c] += __shfl_xor(acc[s][c], o);
  // lane c < NC writes output column n0 + c: slots in order, each scaled (and
  // biased, routed GELU experts) as its own output row would be
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (lane != c) continue;
    float y = 0.f;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      if (grp[s] < 0) continue;
      const bool shared = grp[s] >= p.n_routed;
      const int ew = shared ? grp[s] - p.n_routed : grp[s];
      const float sc = wscale<WF>(p, shared, ew, p.scale_row0, n0 + c, p.scale_col);
      const float b = (!shared && p.bias) ? p.bias[static_cast<int64_t>(ew) * p.Nout + n0 + c] : 0.f;
      y += gate[s] * (acc[s][c] * sc + b);
    }
    static_cast<uint16_t*>(f.y)[n0 + c] = f32_to_bf16(y);
  }
}

// k splits for one GEMM: double while the touched experts' blocks give fewer
// than 2048 waves (eight per CU) and every split keeps at least two 128-wide
// k-steps. Fewer splits means less partial traffic and, at one split, no
// reduction pass. With ordinary loads 1024 waves had been as fast; with the
// whole-line nontemporal loads the Mixtral down GEMM (1024 blocks of 32 rows)
// runs faster split in two (T = 16 step 471 -> 461 us, T = 64 462 -> 454 us),
// and a target of 4096 waves gained nothing more. Integer weights aim at 4096
// waves: a wave then has fewer bytes in flight per k-step and decodes the
// codes on the vector ALUs, which other waves on the SIMD must cover.
int pick_splits(int64_t K, int64_t blocks_touched, bool intw) {
  const int64_t steps = K / KC;
  const int64_t target = intw ? 4096 : 2048;
  int s = 1;
  while (blocks_touched * s < target && s < 16 && steps % (2 * s) == 0 && steps / (2 * s) >= 2) s *= 2;
  return s;
}

hipError_t run_stream(const StreamParams& p, int rb, int wf, int64_t blocks, hipStream_t s) {
  const int64_t waves = blocks * p.splits;
  if (waves <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(ceil_div(waves, kThreads / 64)));
  // 32 or 64 token rows: shared through LDS when the passes hold whole burst pairs
  const bool pairs = (p.K / p.splits / KC) % 4 == 0;
  const bool shared_a = rb >= 2 && pairs;
  // 16-row passes of integer codes: four k-steps a burst (runs of 256 or 512
  // bytes per weight row) with the token rows in LDS, which frees the
  // registers a wave would hold them in. Measured at 16 tokens (Mixtral
  // shape, INT8 x 2 + INT4 x 6): FFN 228 -> 213 us.
  const bool intw = wf == kWInt8 || wf == kWInt4 || wf == kWIntMix;
  if (intw && rb == 1 && (p.K / p.splits / KC) % 4 == 0) {
    if (wf == kWInt8) hipLaunchKernelGGL((stream_kernel<1, kWInt8, 4, true>), grid, dim3(kThreads), 0, s, p);
    else if (wf == kWInt4) hipLaunchKernelGGL((stream_kernel<1, kWInt4, 4, true>), grid, dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL((stream_kernel<1, kWIntMix, 4, true>), grid, dim3(kThreads), 0, s, p);
    return hipGetLastError();
  }
  // at most 8 waves per CU: 16-row passes take the 32-row shared kernel when
  // they can (measured faster there), else four k-steps per burst (whose
  // registers still fit 2 waves per SIMD)
  const bool deep = rb == 1 && waves <= 2048;
#define MOE_STREAM_LAUNCH(R, U, SA)                                                                        \
  switch (wf) {                                                                                            \
    case kWE4m3: hipLaunchKernelGGL((stream_kernel<R, kWE4m3, U, SA>), grid, dim3(kThreads), 0, s, p); break; \
    case kWInt8: hipLaunchKernelGGL((stream_kernel<R, kWInt8, U, SA>), grid, dim3(kThreads), 0, s, p); break; \
    case kWInt4: hipLaunchKernelGGL((stream_kernel<R, kWInt4, U, SA>), grid, dim3(kThreads), 0, s, p); break; \
    case kWIntMix: hipLaunchKernelGGL((stream_kernel<R, kWIntMix, U, SA>), grid, dim3(kThreads), 0, s, p); break; \
    default: hipLaunchKernelGGL((stream_kernel<R, kWBf16, U, SA>), grid, dim3(kThreads), 0, s, p); break;     \
  }
  if (deep && pairs) {
    MOE_STREAM_LAUNCH(2, 2, true)
  } else if (deep) {
    MOE_STREAM_LAUNCH(1, 4, false)
  } else if (rb == 1) {
    // integer codes: four k-steps a burst, so a wave keeps as many bytes in flight
    if (intw) { MOE_STREAM_LAUNCH(1, 4, false) } else { MOE_STREAM_LAUNCH(1, 2, false) }
  } else if (rb == 2) {
    if (shared_a) { MOE_STREAM_LAUNCH(2, 2, true) } else { MOE_STREAM_LAUNCH(2, 2, false) }
  } else {
    if (shared_a) { MOE_STREAM_LAUNCH(4, 2, true) } else { MOE_STREAM_LAUNCH(4, 2, false) }
  }
#undef MOE_STREAM_LAUNCH
  return hipGetLastError();
}

// The GEMV path: at most two rows per group and whole 1 KB segments per row
// (k per segment: bf16 512, e4m3 1024, integer weights 2048, which also
// covers the int8 experts' 1024).
bool use_gemv(const FfnArgs& a) {
  const int64_t kseg = a.w_dtype == 2 ? kSeg : (a.w_dtype == 3 ? 2 * kSeg : kSeg / 2);
  return a.T <= 2 && a.d % kseg == 0 && a.d_ff % kseg == 0;
}

// NR = 8 weight rows per wave while that still gives 2048 waves, else 4;
// each burst is 32 KB of one wave's rows (int4: 16 KB, as a segment's
// activations are four times those of bf16 and would not fit the registers).
// One token row with bf16 weights always takes NR = 4 with eight 1 KB
// segments of each row a burst: with the nontemporal loads the Mixtral T = 1
// FFN (up and down launches by their events) took 125.6-126.1 us with 8 rows x
// 4 segments, 123.0-123.6 with 4 x 8 (4 x 4 124.1-125.2, 8 x 2 126.3), the
// whole step within 0.5 us either way; the integer layer's T = 1 step went
// from 68 to 79 us with it.
hipError_t run_gemv(const StreamParams& p, int rows, int wf, int64_t slots, hipStream_t s) {
  const bool swi = (p.epi == 1);
  const bool long_rows = rows == 1 && wf == kWBf16;
  const int nr = long_rows ? 4 : (slots * p.Nout / (swi ? 4 : 8) >= 2048 ? 8 : 4);
  const int64_t waves = slots * p.Nout / (swi ? nr / 2 : nr);
  if (waves <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(ceil_div(waves, kThreads / 64)));
#define MOE_GEMV_LAUNCH(R, NR, U)                                                                          \
  switch (wf) {                                                                                            \
    case kWE4m3: hipLaunchKernelGGL((gemv_kernel<R, kWE4m3, NR, U>), grid, dim3(kThreads), 0, s, p); break;   \
    case kWInt8: hipLaunchKernelGGL((gemv_kernel<R, kWInt8, NR, U>), grid, dim3(kThreads), 0, s, p); break;   \
    case kWInt4: hipLaunchKernelGGL((gemv_kernel<R, kWInt4, NR, U / 2>), grid, dim3(kThreads), 0, s, p); break; \
    case kWIntMix: hipLaunchKernelGGL((gemv_kernel<R, kWIntMix, NR, U>), grid, dim3(kThreads), 0, s, p); break; \
    default: hipLaunchKernelGGL((gemv_kernel<R, kWBf16, NR, U>), grid, dim3(kThreads), 0, s, p); break;       \
  }
  if (rows == 1) {
    if (nr == 8) { MOE_GEMV_LAUNCH(1, 8, 4) } else { MOE_GEMV_LAUNCH(1, 4, 8) }
  } else {
    if (nr == 8) { MOE_GEMV_LAUNCH(2, 8, 4) } else { MOE_GEMV_LAUNCH(2, 4, 8) }
  }
#undef MOE_GEMV_LAUNCH
  return hipGetLastError();
}

struct SplitPlan {
  int rb, up_splits, down_splits;
};

SplitPlan plan_splits(int64_t T, int64_t d, int64_t d_ff, int32_t n_routed, int32_t n_shared, int32_t act,
                      int64_t cap, int32_t w_dtype) {
  const bool intw = (w_dtype == 3);
  SplitPlan sp;
  const int64_t rows = cap + n_shared * T;
  sp.rb = rows <= 32 ? 1 : (rows <= 128 ? 2 : 4);
  // experts that can have rows: at most one per routed row, plus the shared ones
  const int64_t touched = (cap < n_routed ? cap : n_routed) + n_shared;
  const int64_t up_blocks = (act == 1 ? d_ff / 16 : d_ff / 32);
  sp.up_splits = pick_splits(d, touched * up_blocks, intw);
  sp.down_splits = pick_splits(d_ff, touched * (d / 32), intw);
  return sp;
}

}  // namespace

bool ffn_fuses_combine(const FfnArgs& a) {
  return a.fuse_y && a.T == 1 && a.act_dtype == 1 && (a.w_dtype == 1 || a.w_dtype == 2) && a.fuse_k >= 1 &&
         a.fuse_k + a.n_shared <= 4 && use_skinny(a.act_dtype, a.routed_row_cap, a.n_shared, a.T) && use_gemv(a);
}

size_t skinny_part_floats(int64_t T, int64_t d, int64_t d_ff, int32_t n_routed, int32_t n_shared, int32_t act,
                          int64_t cap, int32_t w_dtype) {
  const SplitPlan sp = plan_splits(T, d, d_ff, n_routed, n_shared, act, cap, w_dtype);
  const int64_t rows = cap + n_shared * T;
  const int64_t up = sp.up_splits > 1 ? sp.up_splits * rows * (act == 1 ? 2 * d_ff : d_ff) : 0;
  const int64_t down = sp.down_splits > 1 ? sp.down_splits * rows * d : 0;
  return static_cast<size_t>(up > down ? up : down);
}

hipError_t launch_ffn_skinny(const FfnArgs& a, const GroupDesc* up, const GroupDesc* down, float* part,
                             hipStream_t s) {
  const int G = a.n_routed + a.n_shared;
  const bool swi = (a.act == 1);
  const SplitPlan sp = plan_splits(a.T, a.d, a.d_ff, a.n_routed, a.n_shared, a.act, a.routed_row_cap, a.w_dtype);
  StreamParams p{};
  p.n_routed = a.n_routed;
  p.n_groups = G;
  // integer weights: one launch per bit width present, each skipping the
  // groups of the other width
  const WeightClasses wc = weight_classes(a);
  p.scale_pitch = static_cast<int32_t>(2 * a.d_ff + a.d);
  // mixed 8- and 4-bit experts run in one launch per GEMM, each wave taking
  // its group's width: two launches would each leave the GPU part idle and
  // pay their own ramp and drain
  auto run_classes = [&](auto&& run) -> hipError_t {
    if (wc.n == 2) {
      for (int i = 0; i < 9; ++i) {
        p.skip[i] = 0;
        p.bits4[i] = wc.skip[0][i];  // the 8-bit class skips the 4-bit groups
      }
      return run(static_cast<int>(kWIntMix));
    }
    hipError_t e = hipSuccess;
    for (int c = 0; c < wc.n && e == hipSuccess; ++c) {
      for (int i = 0; i < 9; ++i) p.skip[i] = wc.skip[c][i];
      e = run(wc.wf[c]);
    }
    return e;
  };
  p.rows_total = a.routed_row_cap + a.n_shared * static_cast<int32_t>(a.T);

  // ---- up: [rows][d] x W1 (W3)^T -> h [rows][d_ff]
  // routed rows: x_perm, or x through the permutation's token list
  p.A_r = static_cast<const uint16_t*>(a.gather ? a.x : a.x_perm);
  p.gather = a.gather;
  p.A_s = static_cast<const uint16_t*>(a.x);
  p.lda_r = a.gather ? a.d : a.ld_xp;
  p.lda_s = a.d;
  p.B_r = static_cast<const char*>(a.w1);
  p.B3_r = static_cast<const char*>(a.w3);
  p.B_s = static_cast<const char*>(a.sw1);
  p.B3_s = static_cast<const char*>(a.sw3);
  p.ldb = a.ld_up;
  p.b_stride = a.d_ff * a.ld_up;
  p.bias = swi ? nullptr : a.b1;
  p.scale_r = a.w_scale;
  p.scale_s = a.sw_scale;
  p.scale_col = 0;
  p.scale_row0 = 0;
  p.scale_row3 = static_cast<int32_t>(a.d_ff);
  p.C_r = static_cast<uint16_t*>(a.h);
  p.C_s = static_cast<uint16_t*>(a.h);
  p.ldc = a.ld_h;
  p.c_shared_base = 0;  // up group descriptors already place shared rows after cap
  p.K = static_cast<int32_t>(a.d);
  p.Nout = static_cast<int32_t>(a.d_ff);
  p.epi = swi ? 1 : 0;
  p.splits = sp.up_splits;
  p.width = swi ? 2 * p.Nout : p.Nout;
  p.part = sp.up_splits > 1 ? part : nullptr;
  p.groups = up;
  p.active = a.active;
  // groups that can have rows: at most one routed expert per routed row, plus the shared ones
  const int64_t slots = std::min<int64_t>(a.routed_row_cap, a.n_routed) + a.n_shared;
  const int64_t up_blocks = slots * (swi ? a.d_ff / 16 : a.d_ff / 32);
  const bool gemv = use_gemv(a);
  if (gemv) {
    p.splits = 1;
    p.part = nullptr;
  }
  stage_mark(kStageFfnUp, false, s);
  hipError_t e = run_classes([&](int wf) {
    return gemv ? run_gemv(p, static_cast<int>(a.T), wf, slots, s) : run_stream(p, sp.rb, wf, up_blocks, s);
  });
  if (e == hipSuccess && p.part) {
    const dim3 rgrid(static_cast<unsigned>(ceil_div(p.Nout, kRedCols)), static_cast<unsigned>(p.rows_total));
    hipLaunchKernelGGL(stream_reduce_kernel, rgrid, dim3(kThreads), 0, s, p, a.offsets, a.routed_row_cap);
    e = hipGetLastError();
  }
  stage_mark(kStageFfnUp, true, s);
  if (e != hipSuccess) return e;

  // ---- down: h [rows][d_ff] x W2^T -> y [rows][d]
  p.A_r = static_cast<const uint16_t*>(a.h);
  p.gather = nullptr;
  p.A_s = static_cast<const uint16_t*>(a.h);
  p.lda_r = a.ld_h;
  p.lda_s = a.ld_h;
  p.B_r = static_cast<const char*>(a.w2);
  p.B3_r = nullptr;
  p.B_s = static_cast<const char*>(a.sw2);
  p.B3_s = nullptr;
  p.ldb = a.ld_down;
  p.b_stride = a.d * a.ld_down;
  p.bias = swi ? nullptr : a.b2;
  p.scale_col = 2;
  p.scale_row0 = static_cast<int32_t>(2 * a.d_ff);
  p.scale_row3 = 0;
  p.C_r = static_cast<uint16_t*>(a.y_perm);
  p.C_s = static_cast<uint16_t*>(a.y_shared);
  p.ldc = a.d;
  p.c_shared_base = a.routed_row_cap;  // down descriptors index y_shared; partial rows follow the routed ones
  p.K = static_cast<int32_t>(a.d_ff);
  p.Nout = static_cast<int32_t>(a.d);
  p.epi = 2;
  p.splits = sp.down_splits;
  p.width = p.Nout;
  p.part = sp.down_splits > 1 ? part : nullptr;
  p.groups = down;
  const int64_t down_blocks = slots * (a.d / 32);
  if (gemv) {
    p.splits = 1;
    p.part = nullptr;
  }
  stage_mark(kStageFfnDown, false, s);
  if (ffn_fuses_combine(a)) {  // one token: the combine runs in this launch
    FusedCombine f{a.fuse_inv_map, a.fuse_topk_idx, a.fuse_topk_w, a.fuse_k, a.n_shared, a.fuse_y};
    // one output column a wave, four segments of each slot's row a burst.
    // Measured at the Mixtral shape (T = 1 step): 2 columns a wave with 8 or 4
    // segments 143.6 us, 1 column with 8 segments 140.4, with 4 140.3; the
    // separate combine 142.3-143.1.
    constexpr int NC = 1;
    const dim3 grid(static_cast<unsigned>(ceil_div(ceil_div(a.d, NC), kThreads / 64)));
    const bool e4 = a.w_dtype == 2;
    if (a.fuse_k + a.n_shared <= 2) {
      if (e4) hipLaunchKernelGGL((gemv_combine_kernel<kWE4m3, 2, NC, 4>), grid, dim3(kThreads), 0, s, p, f);
      else hipLaunchKernelGGL((gemv_combine_kernel<kWBf16, 2, NC, 4>), grid, dim3(kThreads), 0, s, p, f);
    } else {
      if (e4) hipLaunchKernelGGL((gemv_combine_kernel<kWE4m3, 4, NC, 2>), grid, dim3(kThreads), 0, s, p, f);
      else hipLaunchKernelGGL((gemv_combine_kernel<kWBf16, 4, NC, 4>), grid, dim3(kThreads), 0, s, p, f);
    }
    e = hipGetLastError();
  } else {
    e = run_classes([&](int wf) {
      return gemv ? run_gemv(p, static_cast<int>(a.T), wf, slots, s) : run_stream(p, sp.rb, wf, down_blocks, s);
    });
  }
  if (e == hipSuccess && p.part) {
    const dim3 rgrid(static_cast<unsigned>(ceil_div(p.Nout, kRedCols)), static_cast<unsigned>(p.rows_total));
    hipLaunchKernelGGL(stream_reduce_kernel, rgrid, dim3(kThreads), 0, s, p, a.offsets, a.routed_row_cap);
    e = hipGetLastError();
  }
  stage_mark(kStageFfnDown, true, s);
  return e;
}

}  // namespace moe
