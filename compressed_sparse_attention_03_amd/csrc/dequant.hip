// dequant.hip -- a7, standalone dequantisation of the low-precision caches
// (NVFP4 article, sections 3.1 and 3.2): FP8 E4M3 rows with an optional
// per-row fp32 scale, and NVFP4 rows (E2M1 codes times one E4M3 scale per 16
// elements).  The attention and indexer kernels decode the same formats
// in registers with the helpers of device_common.h; these kernels expose the
// decode on its own.
#include "device_common.h"
#include "launch.h"

namespace csa2 {

template <bool OUT_F32>
__global__ __launch_bounds__(256) void dequant_fp8_kernel(const uint8_t* __restrict__ src,
                                                          const float* __restrict__ row_scale,
                                                          int64_t rows, int cols,
                                                          void* __restrict__ dst) {
  const int64_t total = rows * (int64_t)cols;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / cols;
    float v = e4m3_to_f32(src[i]);
    if (row_scale) v *= row_scale[r];
    if (OUT_F32)
      static_cast<float*>(dst)[i] = v;
    else
      static_cast<uint16_t*>(dst)[i] = (uint16_t)f32_to_bf16(v);
  }
}

template <bool OUT_F32>
__global__ __launch_bounds__(256) void dequant_nvfp4_kernel(const uint8_t* __restrict__ packed,
                                                            const uint8_t* __restrict__ scales,
                                                            int64_t rows, int cols,
                                                            void* __restrict__ dst) {
  // one thread per packed byte (two elements)
  const int64_t total = rows * (int64_t)(cols / 2);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / (cols / 2);
    const int c = (int)(i - r * (cols / 2)) * 2;
    const uint32_t byte = packed[i];
    const float sc = e4m3_to_f32(scales[r * (cols / 16) + c / 16]);
    const float v0 = e2m1_to_f32(byte & 15u) * sc;
    const float v1 = e2m1_to_f32(byte >> 4) * sc;
    const int64_t o = r * cols + c;
    if (OUT_F32) {
      static_cast<float*>(dst)[o] = v0;
      static_cast<float*>(dst)[o + 1] = v1;
    } else {
      *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(dst) + o) = pack_bf16x2(v0, v1);
    }
  }
}

static unsigned grid_for(int64_t n) {
  int64_t g = (n + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (unsigned)g;
}

hipError_t launch_dequant_fp8(const uint8_t* src, const float* row_scale, int64_t rows, int cols,
                              void* dst, bool out_f32, hipStream_t s) {
  const unsigned g = grid_for(rows * (int64_t)cols);
  if (out_f32)
    hipLaunchKernelGGL(dequant_fp8_kernel<true>, dim3(g), dim3(256), 0, s, src, row_scale, rows,
                       cols, dst);
  else
    hipLaunchKernelGGL(dequant_fp8_kernel<false>, dim3(g), dim3(256), 0, s, src, row_scale, rows,
                       cols, dst);
  return hipGetLastError();
}

hipError_t launch_dequant_nvfp4(const uint8_t* packed, const uint8_t* scales, int64_t rows,
                                int cols, void* dst, bool out_f32, hipStream_t s) {
  const unsigned g = grid_for(rows * (int64_t)(cols / 2));
  if (out_f32)
    hipLaunchKernelGGL(dequant_nvfp4_kernel<true>, dim3(g), dim3(256), 0, s, packed, scales, rows,
                       cols, dst);
  else
    hipLaunchKernelGGL(dequant_nvfp4_kernel<false>, dim3(g), dim3(256), 0, s, packed, scales,
                       rows, cols, dst);
  return hipGetLastError();
}

}  // namespace csa2
