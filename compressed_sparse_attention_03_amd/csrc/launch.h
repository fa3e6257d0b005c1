// launch.h -- host-side launchers of the gfx950 kernels (internal to the
// library; the public entry points in csa2_api.cpp validate arguments and
// call these).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa2 {

hipError_t launch_compress(int B, int T, const void* kv, int64_t kv_sb, const void* gate,
                           int64_t g_sb, void* out, int64_t out_sb, hipStream_t s);

hipError_t launch_compress_nvfp4(int B, int T, const void* kv, int64_t kv_sb, const void* gate,
                                 int64_t g_sb, uint8_t* codes, uint8_t* scales, int64_t out_sb,
                                 hipStream_t s);
hipError_t launch_compress_step(int B, const void* kv, int64_t kv_sb, const void* gate,
                                int64_t g_sb, const int64_t* pos, void* state, bool fp4,
                                void* out, uint8_t* out_scale, int64_t out_sb, int64_t n_cache,
                                hipStream_t s);
hipError_t launch_quant_nvfp4(const void* src, bool f32_in, int64_t rows, int cols,
                              uint8_t* packed, uint8_t* scales, hipStream_t s);

enum { KEYS_BF16 = 0, KEYS_FP8 = 1, KEYS_MXFP4 = 2 };
hipError_t launch_index_scan(int B, int Tq, const void* q, const float* w, const void* k,
                             int k_fmt, const uint8_t* k_scale, int64_t k_sb, int64_t n_cache,
                             const int64_t* q_pos, float* scores, int64_t s_stride,
                             float* block_max, int64_t bm_stride, hipStream_t s);

hipError_t launch_index_cand(int B, int Tq, const void* q, const float* w, const void* k,
                             bool k_fp8, int64_t k_sb, int64_t n_cache, const int64_t* q_pos,
                             const int32_t* blocks, int K_b, float* scores, int32_t* ids,
                             int64_t s_stride, hipStream_t s);

hipError_t launch_gather_cand(int64_t R, const float* all, int64_t a_stride, int64_t n_cache,
                              const int64_t* q_pos, const int32_t* blocks, int K_b, float* scores,
                              int32_t* ids, int64_t s_stride, hipStream_t s);

size_t select_workspace_bytes(int64_t R, int64_t n, int64_t k);
hipError_t launch_select_topk(int R, int64_t n, const float* scores, int64_t s_stride,
                              const int32_t* ids, int64_t id_stride, const int32_t* forced,
                              int force_last, int k, int32_t* out, int64_t o_stride, void* ws,
                              hipStream_t s);
// candidate gather + position top-k in one pass (rows of 8 * K_b entries
// taking the register-row path only)
bool gather_select_supported(int64_t R, int64_t n);
hipError_t launch_gather_select(int R, const float* all, int64_t a_stride, int64_t n_cache,
                                const int64_t* q_pos, const int32_t* blocks, int K_b, int k,
                                int32_t* out, int64_t o_stride, hipStream_t s);

int attn_splits(int64_t R, int K, int W, int lat_fmt);
size_t attn_workspace_bytes(int64_t R, int K, int W);
size_t attn_workspace_bytes_fmt(int64_t R, int K, int W, int lat_fmt);
// the allocation-free variant's scratch: its size and, for the current
// device, its device address (looked up on first use, then cached)
constexpr size_t ATTN_SCRATCH_BYTES = size_t(32) << 20;
hipError_t attn_scratch(void** out);
hipError_t launch_sparse_attn(int B, int Tq, const void* q, int64_t q_sb, const void* lat,
                              int lat_fmt, const void* lat_scale, int64_t lat_sb, int64_t n_cache,
                              const int32_t* sel, int K, int64_t sel_sb, const void* win,
                              int win_fmt, const float* win_scale, int W, int W_cap,
                              int64_t win_sb, const int64_t* q_pos, const float* sink,
                              float scale, void* out, int64_t out_sb, float* lse, void* ws,
                              hipStream_t s);

hipError_t launch_dequant_fp8(const uint8_t* src, const float* row_scale, int64_t rows, int cols,
                              void* dst, bool out_f32, hipStream_t s);
hipError_t launch_dequant_nvfp4(const uint8_t* packed, const uint8_t* scales, int64_t rows,
                                int cols, void* dst, bool out_f32, hipStream_t s);

}  // namespace csa2
