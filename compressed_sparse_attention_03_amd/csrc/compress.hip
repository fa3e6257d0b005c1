// compress.hip -- a1, the 2:1 Compressor (NVFP4 article, section 3.2):
// each pair of consecutive raw KV latents (tokens 2g, 2g+1) is pooled into one
// compressed latent with a softmax over the pair's per-channel gate logits,
// and written to the cache as bf16 or, quantised in the epilogue, as NVFP4
// (E2M1 codes in groups of 16 channels sharing one E4M3 scale, the same
// section).  Also here: the standalone NVFP4 quantiser and the decode step
// that carries the unfinished half of a pair in device state.
//
// HBM-bound streaming: per (group, channel) 8 bytes read (two bf16 tokens,
// two bf16 logits) and 2 (bf16) or 0.5625 (NVFP4) written.  No element is
// used twice, so there is nothing to stage in LDS; each thread moves 16-byte
// vectors and consecutive lanes cover consecutive bytes of a latent row, which
// keeps every load fully coalesced.
//
// Quantisation reading (the article names the format, not the encoder): the
// group scale is the E4M3 value nearest to amax/6 (6 being the largest E2M1
// magnitude), ties to even, saturating at 448; each element takes the E2M1
// value nearest to x/scale, ties to even, saturating at +-6, with x's sign; a
// group whose scale rounds to 0 stores all-zero codes.  Both roundings are
// decided exactly: amax/6 is one correctly rounded fp32 division, which
// cannot move a quotient onto or across an E4M3 rounding midpoint, and the
// element code compares |x| with the exact fp32 products midpoint * scale.
#include "device_common.h"
#include "launch.h"

namespace csa2 {

// The pooled value of one channel: softmax over the two gate logits, then
// the weighted sum of the two tokens.  Every cache writer calls this one
// function, so the bf16, NVFP4 and decode-step outputs agree bit for bit.
__device__ __forceinline__ float pool_pair(float a0, float a1, float z0, float z1) {
  const float m = fmaxf(z0, z1);
  const float e0 = expf(z0 - m), e1 = expf(z1 - m);
  // the fused multiply-add is written out so that no kernel's contraction
  // choice can change the bits
  return fmaf(e0, a0, e1 * a1) / (e0 + e1);
}

__global__ __launch_bounds__(256) void compress_kernel(
    const uint16_t* __restrict__ kv, int64_t kv_sb, const uint16_t* __restrict__ gate,
    int64_t g_sb, uint16_t* __restrict__ out, int64_t out_sb, int G) {
  // 64 threads per group row (8 channels each); 4 groups per 256-thread block.
  const int b = blockIdx.y;
  const int g = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (g >= G) return;
  const int c0 = (threadIdx.x & 63) * 8;
  const uint16_t* x0p = kv + b * kv_sb + (int64_t)(2 * g) * D + c0;
  const uint16_t* l0p = gate + b * g_sb + (int64_t)(2 * g) * D + c0;
  const u32x4 x0 = *reinterpret_cast<const u32x4*>(x0p);
  const u32x4 x1 = *reinterpret_cast<const u32x4*>(x0p + D);
  const u32x4 l0 = *reinterpret_cast<const u32x4*>(l0p);
  const u32x4 l1 = *reinterpret_cast<const u32x4*>(l0p + D);
  u32x4 y;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float r[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int sh = 16 * h;
      const float a0 = bf16_to_f32((x0[i] >> sh) & 0xffffu);
      const float a1 = bf16_to_f32((x1[i] >> sh) & 0xffffu);
      const float z0 = bf16_to_f32((l0[i] >> sh) & 0xffffu);
      const float z1 = bf16_to_f32((l1[i] >> sh) & 0xffffu);
      r[h] = pool_pair(a0, a1, z0, z1);
    }
    y[i] = pack_bf16x2(r[0], r[1]);
  }
  *reinterpret_cast<u32x4*>(out + b * out_sb + (int64_t)g * D + c0) = y;
}

hipError_t launch_compress(int B, int T, const void* kv, int64_t kv_sb, const void* gate,
                           int64_t g_sb, void* out, int64_t out_sb, hipStream_t s) {
  const int G = T / 2;
  dim3 grid((G + 3) / 4, B);
  hipLaunchKernelGGL(compress_kernel, grid, dim3(256), 0, s, (const uint16_t*)kv, kv_sb,
                     (const uint16_t*)gate, g_sb, (uint16_t*)out, out_sb, G);
  return hipGetLastError();
}


// ---- NVFP4 group quantiser ------------------------------------------------

// Non-negative finite fp32 -> nearest E4M3FN code, ties to even, saturating
// at 448 (0x7E).  Normal range: round the fp32 bit pattern to 3 mantissa bits
// (a carry moves into the exponent by itself) and rebias 127 -> 7; below
// 2^-6 the codes are the multiples of 2^-9 (code 8 is 2^-6 itself).
__device__ __forceinline__ uint32_t e4m3_nearest(float q) {
  if (q >= 448.0f) return 0x7eu;
  const uint32_t u = __float_as_uint(q);
  if (u >= 0x3c800000u) {  // q >= 2^-6
    const uint32_t r = (u + 0x7ffffu + ((u >> 20) & 1u)) >> 20;
    const uint32_t code = r - (120u << 3);
    return code > 0x7eu ? 0x7eu : code;
  }
  return (uint32_t)rintf(q * 512.0f);
}

// One group of 16 values -> its scale code and 16 E2M1 codes packed low
// nibble first (element 2i in bits 8i..8i+3 of the 64-bit word).
struct Fp4Group {
  u32x2 codes;
  uint32_t scale;
};

__device__ __forceinline__ Fp4Group quantise16(const float (&x)[16]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
  Fp4Group r;
  r.scale = e4m3_nearest(amax / 6.0f);
  r.codes = u32x2{0u, 0u};
  if (r.scale == 0u) return r;
  const float s = e4m3_to_f32(r.scale);
  // rounding midpoints between neighbouring E2M1 magnitudes, times the scale
  // (exact: at most 7 significant bits, far from fp32's range limits)
  const float t0 = 0.25f * s, t1 = 0.75f * s, t2 = 1.25f * s, t3 = 1.75f * s;
  const float t4 = 2.5f * s, t5 = 3.5f * s, t6 = 5.0f * s;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float a = fabsf(x[i]);
    // a tie goes to the magnitude with an even code: 0.25 -> 0, 0.75 -> 1,
    // 1.25 -> 1, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4
    const uint32_t mag = (uint32_t)(a > t0) + (uint32_t)(a >= t1) + (uint32_t)(a > t2) +
                         (uint32_t)(a >= t3) + (uint32_t)(a > t4) + (uint32_t)(a >= t5) +
                         (uint32_t)(a > t6);
    const uint32_t code = mag | (x[i] < 0.0f ? 8u : 0u);
    r.codes[i >> 3] |= code << (4 * (i & 7));
  }
  return r;
}

__device__ __forceinline__ void unpack_bf16x8(const u32x4& v, float* x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_to_f32(v[i] & 0xffffu);
    x[2 * i + 1] = bf16_to_f32(v[i] >> 16);
  }
}

// 16 pooled channels [c0, c0+16) of latent g from token rows t0 = 2g and
// t0 + 1 (row pointers at channel c0).
__device__ __forceinline__ void pool16(const uint16_t* x0p, const uint16_t* x1p,
                                       const uint16_t* l0p, const uint16_t* l1p, float (&y)[16]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float a0[8], a1[8], z0[8], z1[8];
    unpack_bf16x8(*reinterpret_cast<const u32x4*>(x0p + 8 * h), a0);
    unpack_bf16x8(*reinterpret_cast<const u32x4*>(x1p + 8 * h), a1);
    unpack_bf16x8(*reinterpret_cast<const u32x4*>(l0p + 8 * h), z0);
    unpack_bf16x8(*reinterpret_cast<const u32x4*>(l1p + 8 * h), z1);
#pragma unroll
    for (int i = 0; i < 8; ++i) y[8 * h + i] = pool_pair(a0[i], a1[i], z0[i], z1[i]);
  }
}

// Write 16 values of one cache row: bf16, or one NVFP4 group (8 code bytes
// at byte c0/2 of the 256-byte code row, the scale at byte c0/16 of the
// 32-byte scale row).
template <bool FP4>
__device__ __forceinline__ void store16(const float (&y)[16], void* row, uint8_t* srow, int c0) {
  if constexpr (FP4) {
    const Fp4Group q = quantise16(y);
    *reinterpret_cast<u32x2*>(static_cast<uint8_t*>(row) + c0 / 2) = q.codes;
    srow[c0 / 16] = (uint8_t)q.scale;
  } else {
    u32x4 lo, hi;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo[i] = pack_bf16x2(y[2 * i], y[2 * i + 1]);
      hi[i] = pack_bf16x2(y[8 + 2 * i], y[8 + 2 * i + 1]);
    }
    uint16_t* o = static_cast<uint16_t*>(row) + c0;
    *reinterpret_cast<u32x4*>(o) = lo;
    *reinterpret_cast<u32x4*>(o + 8) = hi;
  }
}

// Compressor with the NVFP4 epilogue: 32 lanes per latent (16 channels
// each), 8 latents per 256-thread block.  codes: [B][rows][256] bytes,
// scales [B][rows][32], batch stride out_sb rows for both.
__global__ __launch_bounds__(256) void compress_fp4_kernel(
    const uint16_t* __restrict__ kv, int64_t kv_sb, const uint16_t* __restrict__ gate,
    int64_t g_sb, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, int64_t out_sb,
    int G) {
  const int b = blockIdx.y;
  const int g = blockIdx.x * 8 + (threadIdx.x >> 5);
  if (g >= G) return;
  const int c0 = (threadIdx.x & 31) * 16;
  const int64_t x0 = b * kv_sb + (int64_t)(2 * g) * D + c0;
  const int64_t z0 = b * g_sb + (int64_t)(2 * g) * D + c0;
  float y[16];
  pool16(kv + x0, kv + x0 + D, gate + z0, gate + z0 + D, y);
  const int64_t row = b * out_sb + g;
  store16<true>(y, codes + row * (D / 2), scales + row * (D / 16), c0);
}

// One decode step of the compressor for B sequences, each at its own raw
// position pos[b] (negative: no token).  An even position parks the token
// (kv row, gate row) in state[b]; an odd position t pools the parked token
// with the new one into cache row t/2, written only if t/2 < n_cache.
// 32 lanes per sequence, 8 sequences per block.
template <bool FP4>
__global__ __launch_bounds__(256) void compress_step_kernel(
    int B, const uint16_t* __restrict__ kv, int64_t kv_sb, const uint16_t* __restrict__ gate,
    int64_t g_sb, const int64_t* __restrict__ pos, uint16_t* __restrict__ state,
    void* __restrict__ out, uint8_t* __restrict__ out_scale, int64_t out_sb, int64_t n_cache) {
  const int b = blockIdx.x * 8 + (threadIdx.x >> 5);
  if (b >= B) return;
  const int64_t t = pos[b];
  if (t < 0) return;
  const int c0 = (threadIdx.x & 31) * 16;
  const uint16_t* xn = kv + b * kv_sb + c0;
  const uint16_t* zn = gate + b * g_sb + c0;
  uint16_t* sx = state + (int64_t)b * 2 * D + c0;  // parked kv row, then gate row
  uint16_t* sz = sx + D;
  if ((t & 1) == 0) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      reinterpret_cast<u32x4*>(sx)[h] = reinterpret_cast<const u32x4*>(xn)[h];
      reinterpret_cast<u32x4*>(sz)[h] = reinterpret_cast<const u32x4*>(zn)[h];
    }
    return;
  }
  const int64_t g = t >> 1;
  if (g >= n_cache) return;
  float y[16];
  pool16(sx, xn, sz, zn, y);
  const int64_t row = b * out_sb + g;
  if constexpr (FP4)
    store16<true>(y, static_cast<uint8_t*>(out) + row * (D / 2), out_scale + row * (D / 16), c0);
  else
    store16<false>(y, static_cast<uint16_t*>(out) + row * D, nullptr, c0);
}

// Standalone quantiser: one thread per group of 16, consecutive threads on
// consecutive groups (rows of cols/16 groups laid end to end).
template <bool F32IN>
__global__ __launch_bounds__(256) void quant_fp4_kernel(const void* __restrict__ src,
                                                        int64_t groups, uint8_t* __restrict__ packed,
                                                        uint8_t* __restrict__ scales) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= groups) return;
  float x[16];
  if constexpr (F32IN) {
    const f32x4* p = static_cast<const f32x4*>(src) + 4 * i;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 v = p[j];
#pragma unroll
      for (int k = 0; k < 4; ++k) x[4 * j + k] = v[k];
    }
  } else {
    const u32x4* p = static_cast<const u32x4*>(src) + 2 * i;
    unpack_bf16x8(p[0], x);
    unpack_bf16x8(p[1], x + 8);
  }
  const Fp4Group q = quantise16(x);
  reinterpret_cast<u32x2*>(packed)[i] = q.codes;
  scales[i] = (uint8_t)q.scale;
}

hipError_t launch_compress_nvfp4(int B, int T, const void* kv, int64_t kv_sb, const void* gate,
                                 int64_t g_sb, uint8_t* codes, uint8_t* scales, int64_t out_sb,
                                 hipStream_t s) {
  const int G = T / 2;
  dim3 grid((G + 7) / 8, B);
  hipLaunchKernelGGL(compress_fp4_kernel, grid, dim3(256), 0, s, (const uint16_t*)kv, kv_sb,
                     (const uint16_t*)gate, g_sb, codes, scales, out_sb, G);
  return hipGetLastError();
}

hipError_t launch_compress_step(int B, const void* kv, int64_t kv_sb, const void* gate,
                                int64_t g_sb, const int64_t* pos, void* state, bool fp4,
                                void* out, uint8_t* out_scale, int64_t out_sb, int64_t n_cache,
                                hipStream_t s) {
  dim3 grid((B + 7) / 8);
  if (fp4)
    hipLaunchKernelGGL(compress_step_kernel<true>, grid, dim3(256), 0, s, B, (const uint16_t*)kv,
                       kv_sb, (const uint16_t*)gate, g_sb, pos, (uint16_t*)state, out, out_scale,
                       out_sb, n_cache);
  else
    hipLaunchKernelGGL(compress_step_kernel<false>, grid, dim3(256), 0, s, B, (const uint16_t*)kv,
                       kv_sb, (const uint16_t*)gate, g_sb, pos, (uint16_t*)state, out, out_scale,
                       out_sb, n_cache);
  return hipGetLastError();
}

hipError_t launch_quant_nvfp4(const void* src, bool f32_in, int64_t rows, int cols,
                              uint8_t* packed, uint8_t* scales, hipStream_t s) {
  const int64_t groups = rows * (cols / 16);
  dim3 grid((unsigned)((groups + 255) / 256));
  if (f32_in)
    hipLaunchKernelGGL(quant_fp4_kernel<true>, grid, dim3(256), 0, s, src, groups, packed, scales);
  else
    hipLaunchKernelGGL(quant_fp4_kernel<false>, grid, dim3(256), 0, s, src, groups, packed, scales);
  return hipGetLastError();
}

}  // namespace csa2
