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
// the weighted sum of the two tokens.  With two logits the softmax weight of
// token 0 is 1 / (1 + e^(z1 - z0)), so one exponential and one reciprocal
// suffice: y = a1 + w0 (a0 - a1).  The hardware exp2 and reciprocal (about
// one ulp each) keep the pooled value within a few fp32 ulps of
// max(|a0|, |a1|) of the exact one, and make the kernel streaming-bound
// rather than ALU-bound.  Every cache writer calls this one function, so the
// bf16, NVFP4 and decode-step outputs agree bit for bit.
__device__ __forceinline__ float pool_pair(float a0, float a1, float z0, float z1) {
  const float e = __builtin_amdgcn_exp2f((z1 - z0) * 1.4426950408889634f);
  const float w0 = __builtin_amdgcn_rcpf(1.0f + e);
  return fmaf(w0, a0 - a1, a1);
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

// Scale code of a group from the largest magnitude in it.
__device__ __forceinline__ uint32_t fp4_scale(float amax) { return e4m3_nearest(amax / 6.0f); }

// E2M1 codes of 8 values under scale code sc, element i in bits 4i..4i+3.
__device__ __forceinline__ uint32_t fp4_codes8(const float* x, uint32_t sc) {
  if (sc == 0u) return 0u;
  const float s = e4m3_to_f32(sc);
  // rounding midpoints between neighbouring E2M1 magnitudes, times the scale
  // (exact: at most 7 significant bits, far from fp32's range limits)
  const float t0 = 0.25f * s, t1 = 0.75f * s, t2 = 1.25f * s, t3 = 1.75f * s;
  const float t4 = 2.5f * s, t5 = 3.5f * s, t6 = 5.0f * s;
  uint32_t w = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float a = fabsf(x[i]);
    // binary search over the 7 midpoints; a tie goes to the magnitude with
    // an even code: 0.25 -> 0, 0.75 -> 1, 1.25 -> 1, 1.75 -> 2, 2.5 -> 2,
    // 3.5 -> 4, 5 -> 4 (hence >= at 0.75, 1.75, 3.5 and > elsewhere)
    const bool hi = a >= t3;
    const bool mid = a >= (hi ? t5 : t1);
    const bool lo = a > (hi ? (mid ? t6 : t4) : (mid ? t2 : t0));
    const uint32_t mag = (hi ? 4u : 0u) | (mid ? 2u : 0u) | (lo ? 1u : 0u);
    w |= (mag | (x[i] < 0.0f ? 8u : 0u)) << (4 * i);
  }
  return w;
}

// One group of 16 values -> its scale code and 16 codes packed low nibble
// first (element 2i in the low nibble of byte i).
struct Fp4Group {
  u32x2 codes;
  uint32_t scale;
};

__device__ __forceinline__ Fp4Group quantise16(const float (&x)[16]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
  Fp4Group r;
  r.scale = fp4_scale(amax);
  r.codes = u32x2{fp4_codes8(x, r.scale), fp4_codes8(x + 8, r.scale)};
  return r;
}

__device__ __forceinline__ void unpack_bf16x8(const u32x4& v, float* x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_to_f32(v[i] & 0xffffu);
    x[2 * i + 1] = bf16_to_f32(v[i] >> 16);
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

// The compressor over whole rows: one wave per latent row at a time, 8
// channels per lane, so every load instruction reads 1 KiB of one row
// contiguously (non-temporal: nothing is read twice).  Each wave takes two
// consecutive latents and issues all eight row loads before using any.
// FP4 = false: bf16 rows [B][rows][512] (each lane stores 16 bytes).
// FP4 = true: the NVFP4 epilogue -- the two lanes of a 16-channel group
// exchange their partial maxima by DPP, each stores its 8 codes (4 bytes)
// and the even lane the group's scale byte; codes [B][rows][256], scales
// [B][rows][32].  Batch stride out_sb: in elements for bf16 (any multiple of
// 8), in rows for NVFP4.
constexpr int CF_LAT_PER_WAVE = 2;

template <bool FP4>
__global__ __launch_bounds__(256) void compress_rows_kernel(
    const uint16_t* __restrict__ kv, int64_t kv_sb, const uint16_t* __restrict__ gate,
    int64_t g_sb, void* __restrict__ out, uint8_t* __restrict__ scales, int64_t out_sb, int G) {
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int g0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * CF_LAT_PER_WAVE;
  if (g0 >= G) return;  // whole wave
  const int c0 = lane * 8;
  u32x4 v[CF_LAT_PER_WAVE][4];
#pragma unroll
  for (int j = 0; j < CF_LAT_PER_WAVE; ++j) {
    if (g0 + j < G) {
      const u32x4* x = reinterpret_cast<const u32x4*>(kv + b * kv_sb + (int64_t)(2 * (g0 + j)) * D + c0);
      const u32x4* z = reinterpret_cast<const u32x4*>(gate + b * g_sb + (int64_t)(2 * (g0 + j)) * D + c0);
      v[j][0] = __builtin_nontemporal_load(x);
      v[j][1] = __builtin_nontemporal_load(x + D / 8);
      v[j][2] = __builtin_nontemporal_load(z);
      v[j][3] = __builtin_nontemporal_load(z + D / 8);
    }
  }
#pragma unroll
  for (int j = 0; j < CF_LAT_PER_WAVE; ++j) {
    if (g0 + j >= G) break;  // whole wave
    float a0[8], a1[8], z0[8], z1[8], y[8];
    unpack_bf16x8(v[j][0], a0);
    unpack_bf16x8(v[j][1], a1);
    unpack_bf16x8(v[j][2], z0);
    unpack_bf16x8(v[j][3], z1);
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = pool_pair(a0[i], a1[i], z0[i], z1[i]);
    if constexpr (FP4) {
      const int64_t row = b * out_sb + g0 + j;
      float am = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(y[i]));
      am = fmaxf(am, __uint_as_float(dpp_mov<0xB1>(__float_as_uint(am))));  // partner lane
      const uint32_t sc = fp4_scale(am);
      reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(out) + row * (D / 2))[lane] = fp4_codes8(y, sc);
      if ((lane & 1) == 0) scales[row * (D / 16) + (lane >> 1)] = (uint8_t)sc;
    } else {
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(y[2 * i], y[2 * i + 1]);
      reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + b * out_sb + (int64_t)(g0 + j) * D)[lane] = o;
    }
  }
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
  const int c0 = (threadIdx.x & 31) * 16;
  const u32x4* xn = reinterpret_cast<const u32x4*>(kv + b * kv_sb + c0);
  const u32x4* zn = reinterpret_cast<const u32x4*>(gate + b * g_sb + c0);
  u32x4* sx = reinterpret_cast<u32x4*>(state + (int64_t)b * 2 * D + c0);  // parked kv row
  u32x4* sz = sx + D / 8;                                                   // its gate row
  // the position, the new token and the parked one are fetched together
  const int64_t t = pos[b];
  u32x4 x[2][2], z[2][2];  // [parked, new][half]
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    x[0][h] = sx[h];
    z[0][h] = sz[h];
    x[1][h] = xn[h];
    z[1][h] = zn[h];
  }
  if (t < 0) return;
  if ((t & 1) == 0) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      sx[h] = x[1][h];
      sz[h] = z[1][h];
    }
    return;
  }
  const int64_t g = t >> 1;
  if (g >= n_cache) return;
  float y[16];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float a0[8], a1[8], z0[8], z1[8];
    unpack_bf16x8(x[0][h], a0);
    unpack_bf16x8(x[1][h], a1);
    unpack_bf16x8(z[0][h], z0);
    unpack_bf16x8(z[1][h], z1);
#pragma unroll
    for (int i = 0; i < 8; ++i) y[8 * h + i] = pool_pair(a0[i], a1[i], z0[i], z1[i]);
  }
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

static hipError_t launch_rows(bool fp4, int B, int T, const void* kv, int64_t kv_sb,
                              const void* gate, int64_t g_sb, void* out, uint8_t* scales,
                              int64_t out_sb, hipStream_t s) {
  const int G = T / 2;
  constexpr int per_block = 4 * CF_LAT_PER_WAVE;
  dim3 grid((G + per_block - 1) / per_block, B);
  if (fp4)
    hipLaunchKernelGGL(compress_rows_kernel<true>, grid, dim3(256), 0, s, (const uint16_t*)kv,
                       kv_sb, (const uint16_t*)gate, g_sb, out, scales, out_sb, G);
  else
    hipLaunchKernelGGL(compress_rows_kernel<false>, grid, dim3(256), 0, s, (const uint16_t*)kv,
                       kv_sb, (const uint16_t*)gate, g_sb, out, scales, out_sb, G);
  return hipGetLastError();
}

hipError_t launch_compress(int B, int T, const void* kv, int64_t kv_sb, const void* gate,
                           int64_t g_sb, void* out, int64_t out_sb, hipStream_t s) {
  return launch_rows(false, B, T, kv, kv_sb, gate, g_sb, out, nullptr, out_sb, s);
}

hipError_t launch_compress_nvfp4(int B, int T, const void* kv, int64_t kv_sb, const void* gate,
                                 int64_t g_sb, uint8_t* codes, uint8_t* scales, int64_t out_sb,
                                 hipStream_t s) {
  return launch_rows(true, B, T, kv, kv_sb, gate, g_sb, codes, scales, out_sb, s);
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
