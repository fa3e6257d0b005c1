// compress.hip -- a1, the 2:1 Compressor (NVFP4 article, section 3.2):
// each pair of consecutive raw KV latents (tokens 2g, 2g+1) is pooled into one
// compressed latent with a softmax over the pair's per-channel gate logits.
//
// HBM-bound streaming: per (group, channel) 8 bytes read (two bf16 tokens,
// two bf16 logits) and 2 written.  No element is used twice, so there is
// nothing to stage in LDS; each thread moves 16-byte vectors and a wave
// covers one full 1 KiB latent row per load, which keeps every load fully
// coalesced.
#include "device_common.h"
#include "launch.h"

namespace csa2 {

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
      const float m = fmaxf(z0, z1);
      const float e0 = expf(z0 - m), e1 = expf(z1 - m);
      r[h] = (e0 * a0 + e1 * a1) / (e0 + e1);
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

}  // namespace csa2
