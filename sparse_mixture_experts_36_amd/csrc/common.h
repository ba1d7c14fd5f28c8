// Internal helpers shared by the gfx950 kernels of the MoE layer library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4_t;
// 16-byte chunk as a vector type: arrays of it stay in registers where arrays
// of the uint4 struct can be left in scratch memory.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even (hardware v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two values, round-to-nearest-even, lo in the low half (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// Four OCP e4m3fn codes (one per byte of `w`) -> four bf16 values, exactly:
// every e4m3fn value is representable in bf16. gfx950 decodes the OCP format
// in hardware (v_cvt_pk_f32_fp8); fp32 -> bf16 is then exact.
__device__ __forceinline__ uint2 e4m3x4_to_bf16x4(uint32_t w) {
  typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f2;
  f2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  f2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  uint2 r;
  r.x = (__float_as_uint(lo[0]) >> 16) | (__float_as_uint(lo[1]) & 0xFFFF0000u);
  r.y = (__float_as_uint(hi[0]) >> 16) | (__float_as_uint(hi[1]) & 0xFFFF0000u);
  return r;
}

// Weight storage formats of the expert kernels (template argument WF);
// kWIntMix: 8- and 4-bit integer experts in one launch, each group taking its
// own width.
enum WeightFormat { kWBf16 = 0, kWE4m3 = 1, kWInt8 = 2, kWInt4 = 3, kWIntMix = 4 };

// The bf16 pair (lo, hi) from the upper halves of two fp32 values: exact when
// both are small integers, as decoded integer codes are.
__device__ __forceinline__ uint32_t pack_hi16(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// Four int8 codes (byte i of w is code i) -> four bf16 values, exactly
// (|q| <= 128 fits bf16's 8-bit significand).
__device__ __forceinline__ uint2 int8x4_to_bf16x4(uint32_t w) {
  const float f0 = static_cast<float>(static_cast<int32_t>(w << 24) >> 24);
  const float f1 = static_cast<float>(static_cast<int32_t>(w << 16) >> 24);
  const float f2 = static_cast<float>(static_cast<int32_t>(w << 8) >> 24);
  const float f3 = static_cast<float>(static_cast<int32_t>(w) >> 24);
  return make_uint2(pack_hi16(f0, f1), pack_hi16(f2, f3));
}

// Eight int4 codes in one 32-bit word, two's complement: code 2j in bits
// [4j, 4j + 4), code 2j + 1 in bits [16 + 4j, 16 + 4j + 4), j < 4. This order
// puts codes 2j and 2j + 1 sixteen bits apart, where one shift and one
// and-or turn them into a bf16 pair (int4x8_to_bf16x8_biased).

// -> eight bf16 values, exactly, in code order.
__device__ __forceinline__ uint4 int4x8_to_bf16x8(uint32_t w) {
  float f[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[2 * j] = static_cast<float>(static_cast<int32_t>(w << (28 - 4 * j)) >> 28);
    f[2 * j + 1] = static_cast<float>(static_cast<int32_t>(w << (12 - 4 * j)) >> 28);
  }
  return make_uint4(pack_hi16(f[0], f[1]), pack_hi16(f[2], f[3]), pack_hi16(f[4], f[5]), pack_hi16(f[6], f[7]));
}

// -> the eight bf16 values q + 136, in code order: flipping each nibble's sign
// bit gives u = q + 8 in [0, 15], and 0x4300 | u is the bf16 of 128 + u
// (exact: bf16 steps by 1 between 128 and 256). About one instruction per
// weight; the caller subtracts 136 times the sum of the activations.
constexpr float kInt4Bias = 136.f;
constexpr uint32_t kInt4BiasPair = 0x43084308u;  // two bf16 136
__device__ __forceinline__ uint4 int4x8_to_bf16x8_biased(uint32_t w) {
  const uint32_t v = w ^ 0x88888888u;
  return make_uint4((v & 0x000F000Fu) | 0x43004300u, ((v >> 4) & 0x000F000Fu) | 0x43004300u,
                    ((v >> 8) & 0x000F000Fu) | 0x43004300u, ((v >> 12) & 0x000F000Fu) | 0x43004300u);
}

// D += A(16x32) * B(32x16), bf16 inputs, fp32 accumulation. Lane l supplies
// row (l % 16) of A and column (l % 16) of B, each as 8 consecutive k values of
// the k-group (l / 16); it receives D rows 4*(l/16) + i, i < 4, column l % 16.
__device__ __forceinline__ floatx4_t mfma16x16x32(const uint4& a, const uint4& b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// erf by Abramowitz and Stegun's formula 7.1.26 (absolute error at most
// 1.5e-7; here with the hardware exponential and reciprocal, about 3e-7): a
// fifth-degree polynomial in t = 1 / (1 + p |x|) times exp(-x^2), odd in x. A
// few instructions, no branches, where the library erff takes about thirty
// with divergent branches; the results feed bf16 values.
__device__ __forceinline__ float erf_as(float x) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * ax);
  const float poly =
      t * (0.254829592f + t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
  const float r = 1.0f - poly * __expf(-ax * ax);
  return copysignf(r, x);
}

__device__ __forceinline__ float gelu_erf(float u) {
  return 0.5f * u * (1.0f + erf_as(u * 0.70710678118654752f));
}

// silu(u) = u sigmoid(u) with the hardware exponential and reciprocal (about
// 1 ulp each in fp32; the results feed bf16 values).
__device__ __forceinline__ float silu(float u) { return u * __builtin_amdgcn_rcpf(1.0f + __expf(-u)); }

// 4 x 4 transpose of bf16 values across the four lanes of a quad (DPP moves,
// no LDS). On entry lane t (t = lane % 4) holds column t of the block as
// c01 = (M[0][t], M[1][t]) and c23 = (M[2][t], M[3][t]), low half first; on
// exit it holds row t as r01 = (M[t][0], M[t][1]) and r23 = (M[t][2], M[t][3]).
// The off-diagonal 2 x 2 blocks move between lanes t and t ^ 2, then each
// 2 x 2 block is transposed between lanes t and t ^ 1.
__device__ __forceinline__ void quad_transpose_bf16(uint32_t c01, uint32_t c23, int t, uint32_t& r01,
                                                    uint32_t& r23) {
  const bool hi2 = (t & 2) != 0, odd = (t & 1) != 0;
  const uint32_t send = hi2 ? c01 : c23;
  const uint32_t recv = static_cast<uint32_t>(
      __builtin_amdgcn_mov_dpp(static_cast<int>(send), 0x4E, 0xF, 0xF, false));  // quad_perm [2,3,0,1]
  const uint32_t q0 = hi2 ? recv : c01;
  const uint32_t q1 = hi2 ? c23 : recv;
  // even lanes pass on the high halves of q0, q1; odd lanes the low halves
  const uint32_t s = __builtin_amdgcn_perm(q1, q0, odd ? 0x05040100u : 0x07060302u);
  const uint32_t x = static_cast<uint32_t>(
      __builtin_amdgcn_mov_dpp(static_cast<int>(s), 0xB1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
  r01 = __builtin_amdgcn_perm(x, q0, odd ? 0x03020504u : 0x05040100u);
  r23 = __builtin_amdgcn_perm(x, q1, odd ? 0x03020706u : 0x07060100u);
}

// Lane exchanges inside each row of 16 lanes by DPP (no LDS round trip, as
// a __shfl through ds_bpermute takes): step 0 rotates the row by 8, step 1 by
// 4, step 2 swaps lanes at distance 2, step 3 neighbours. After the four
// steps of an all-reduce with a commutative, associative merge every lane of
// the row holds the result of all 16, and the lanes of a row combine their
// operands in the same pairs, so they agree bit for bit.
template <int STEP>
__device__ __forceinline__ int dpp_row16(int v) {
  static_assert(STEP >= 0 && STEP < 4, "four steps");
  constexpr int kCtrl = STEP == 0 ? 0x128 : STEP == 1 ? 0x124 : STEP == 2 ? 0x4E : 0xB1;  // row_ror:8, row_ror:4, quad [2,3,0,1], quad [1,0,3,2]
  return __builtin_amdgcn_mov_dpp(v, kCtrl, 0xF, 0xF, false);
}
template <int STEP>
__device__ __forceinline__ float dpp_row16(float v) {
  return __int_as_float(dpp_row16<STEP>(__float_as_int(v)));
}
// Sum over each row of 16 lanes (every lane gets the row's sum).
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_row16<0>(v);
  v += dpp_row16<1>(v);
  v += dpp_row16<2>(v);
  v += dpp_row16<3>(v);
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__host__ __device__ constexpr int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace moe
