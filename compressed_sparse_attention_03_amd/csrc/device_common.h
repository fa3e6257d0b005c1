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

// bf16 bits -> E4M3FN code, round to nearest even, saturating to +-448
// (infinities included); NaN -> 0x7f.  Integer work on the bit fields.
__device__ __forceinline__ uint32_t bf16_to_e4m3(uint32_t h) {
  const uint32_t s = (h >> 8) & 0x80u;
  const uint32_t a = h & 0x7fffu;
  if (a > 0x7f80u) return 0x7fu;
  const int e = (int)(a >> 7) - 120;  // E4M3 biased exponent of the value
  if (e >= 1) {
    const uint32_t m = a & 0x7fu;     // 7 mantissa bits, keep the top 3
    uint32_t code = ((uint32_t)(e > 16 ? 16 : e) << 3) | (m >> 4);
    const uint32_t rem = m & 15u;
    if (rem > 8u || (rem == 8u && (code & 1u))) ++code;
    return s | (code > 0x7eu ? 0x7eu : code);
  }
  // below 2^-6: multiples of 2^-9 (8 rounds up to 2^-6, code 0x08)
  return s | (uint32_t)rintf(bf16_to_f32(a) * 512.0f);
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
