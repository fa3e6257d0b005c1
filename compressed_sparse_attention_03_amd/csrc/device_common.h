// device_common.h -- types, constants and element conversions shared by the
// gfx950 kernels of the CSA2 library.
//
// Element formats (NVFP4 article, sections 3.1-3.2, lpnh.cn/news/2752702):
//   bf16   : upper half of an IEEE binary32 word.
//   E4M3FN : 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent 0 is
//            subnormal; S.1111.111 is NaN; no infinities (max 448).
//   E2M1   : 1 sign, 2 exponent (bias 1), 1 mantissa bit (0 .. 6).
//   NVFP4  : E2M1 codes, element 2i in the low nibble of byte i, times one
//            E4M3 scale per group of 16 elements.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

constexpr int D = 512;   // latent width (one shared KV head)
constexpr int HQ = 64;   // attention query heads
constexpr int HI = 32;   // index heads
constexpr int DI = 128;  // index head width
constexpr int BLK = 8;   // latents per candidate block

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16, round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two fp32 -> packed bf16 pair (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// E4M3FN code -> fp32, from the bit fields.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  const uint32_t s = (b & 0x80u) << 24;
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  if (e == 15u && m == 7u) return __uint_as_float(0x7fc00000u);
  if (e == 0u) return __uint_as_float(s | __float_as_uint((float)m * 0.001953125f));
  return __uint_as_float(s | ((e + 120u) << 23) | (m << 20));
}

// E4M3FN code -> bf16 bits (every finite E4M3 value is a bf16 value).
__device__ __forceinline__ uint32_t e4m3_to_bf16(uint32_t b) {
  return __float_as_uint(e4m3_to_f32(b)) >> 16;
}

// E2M1 code (low 4 bits) -> fp32.
__device__ __forceinline__ float e2m1_to_f32(uint32_t n) {
  const uint32_t s = (n & 8u) << 28;
  const uint32_t e = (n >> 1) & 3u, m = n & 1u;
  if (e == 0u) return __uint_as_float(s | (m ? 0x3f000000u : 0u));
  return __uint_as_float(s | ((e + 126u) << 23) | (m << 22));
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) short s16x2;

// The two bf16 values of w (low half first) -> two E4M3FN codes (bits 0-7
// and 8-15): nearest, ties to even, saturating to +-448 (infinities
// included).  The conversion instruction rounds exactly so for every
// magnitude up to 464 and makes larger ones NaN, so magnitudes above 448 are
// clamped to 448 first; NaN stays NaN.  (Checked against the format's
// definition over all 65,536 bf16 values.)
__device__ __forceinline__ uint32_t bf16x2_to_e4m3x2(uint32_t w) {
  float lo = __uint_as_float(w << 16), hi = __uint_as_float(w & 0xffff0000u);
  lo = fabsf(lo) > 448.0f ? copysignf(448.0f, lo) : lo;
  hi = fabsf(hi) > 448.0f ? copysignf(448.0f, hi) : hi;
  const s16x2 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32((s16x2){0, 0}, lo, hi, 1.0f, false);
  return (uint32_t)(uint16_t)r[0];
}

// Eight bf16 values (the four words of x, low half first) -> eight E2M1
// codes, value 2i in the low nibble of byte i: nearest, ties to even,
// saturating to +-6, by the conversion instruction, which gives the format's
// definition for every finite bf16 value (checked over all of them) but
// keeps the sign of -0 (code 8; its products are zeros either way).
// (Each word is copied to a scalar before the bit cast: a bit cast of a
// vector element reads the vector's first element.)
__device__ __forceinline__ uint32_t bf16x8_to_e2m1x8(const u32x4& x) {
  const uint32_t x0 = x[0], x1 = x[1], x2 = x[2], x3 = x[3];
  uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(0u, __builtin_bit_cast(bf16x2, x0), 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(bf16x2, x1), 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(bf16x2, x2), 1.0f, 2);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(bf16x2, x3), 1.0f, 3);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace csa2

namespace csa2 {

// ---- wave-level reductions and scans over 64 lanes ------------------------
// Within a row of 16 lanes the data moves by DPP (register-to-register):
// quad permutes, half-row and row mirrors; across rows by ds_bpermute (two
// steps) or, for the scan, by the row broadcasts of the GFX9 DPP set.  Every
// lane gets the result (reductions) or its inclusive prefix (scan).
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
}

template <typename F>
__device__ __forceinline__ uint32_t wave_allreduce(uint32_t v, F op) {
  v = op(v, dpp_mov<0xB1>(v));   // quad_perm [1,0,3,2]
  v = op(v, dpp_mov<0x4E>(v));   // quad_perm [2,3,0,1]
  v = op(v, dpp_mov<0x141>(v));  // row_half_mirror: lane i <- 7-i of its 8
  v = op(v, dpp_mov<0x140>(v));  // row_mirror: lane i <- 15-i of its 16
  v = op(v, (uint32_t)__shfl_xor((int)v, 16, 64));
  v = op(v, (uint32_t)__shfl_xor((int)v, 32, 64));
  return v;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
  return wave_allreduce(v, [](uint32_t a, uint32_t b) { return a + b; });
}
__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
  return wave_allreduce(v, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  return wave_allreduce(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ uint32_t wave_and(uint32_t v) {
  return wave_allreduce(v, [](uint32_t a, uint32_t b) { return a & b; });
}
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
  return wave_allreduce(v, [](uint32_t a, uint32_t b) { return a | b; });
}
__device__ __forceinline__ int32_t wave_max_i(int32_t v) {
  return (int32_t)wave_allreduce((uint32_t)v, [](uint32_t a, uint32_t b) {
    return (int32_t)a > (int32_t)b ? a : b;
  });
}
__device__ __forceinline__ int32_t wave_min_i(int32_t v) {
  return (int32_t)wave_allreduce((uint32_t)v, [](uint32_t a, uint32_t b) {
    return (int32_t)a < (int32_t)b ? a : b;
  });
}

// Combination over the waves of a block of per-wave values stored at
// vals[0 .. nw) (nw <= 16): lane l reads vals[l % 16] (or the identity), and
// the 16 lanes of each row reduce by DPP; every lane gets the result.
template <typename F>
__device__ __forceinline__ uint32_t waves_combine(const uint32_t* vals, int nw, uint32_t identity,
                                                  F op) {
  const int i = threadIdx.x & 15;
  uint32_t v = i < nw ? vals[i] : identity;
  v = op(v, dpp_mov<0xB1>(v));
  v = op(v, dpp_mov<0x4E>(v));
  v = op(v, dpp_mov<0x141>(v));
  v = op(v, dpp_mov<0x140>(v));
  return v;
}

// inclusive prefix sum in lane order
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += dpp_mov<0x111>(v);        // row_shr:1 (lanes shifted in from outside the row add 0)
  v += dpp_mov<0x112>(v);        // row_shr:2
  v += dpp_mov<0x114>(v);        // row_shr:4
  v += dpp_mov<0x118>(v);        // row_shr:8
  v += dpp_mov<0x142, 0xA>(v);   // row_bcast:15 -> rows 1 and 3
  v += dpp_mov<0x143, 0xC>(v);   // row_bcast:31 -> rows 2 and 3
  return v;
}

// Reductions over the four 16-lane rows of a wave (lanes l, l^16, l^32,
// l^48): two register-to-register lane swaps (v_permlane16_swap pairs rows
// 0/1 and 2/3, v_permlane32_swap the two halves), no LDS round trip.  Every
// lane gets the result of its column.
template <typename F>
__device__ __forceinline__ float across_rows(float v, F op) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return op(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_across_rows(float v) {
  return across_rows(v, [](float x, float y) { return x + y; });
}
// max of two floats as one v_max_f32: in IEEE mode fmaxf first makes each
// operand that is not known to be canonical (a value moved between lanes)
// canonical, one more instruction each.  Not for NaN operands.
__device__ __forceinline__ float fmax_nc(float x, float y) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(x), "v"(y));
  return r;
}
__device__ __forceinline__ float max_across_rows(float v) {
  return across_rows(v, [](float x, float y) { return fmax_nc(x, y); });
}

}  // namespace csa2
