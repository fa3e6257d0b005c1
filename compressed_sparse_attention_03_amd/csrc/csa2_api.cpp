// csa2_api.cpp -- the extern "C" entry points of libcsa2: host-side argument
// validation, then the kernel launchers.  Nothing is enqueued unless every
// check passes; no C++ exception crosses the ABI.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "../../include/csa2.h"
#include "launch.h"

namespace {

constexpr int64_t kMaxN = int64_t(1) << 24;
static_assert(csa2::ATTN_SCRATCH_BYTES == CSA2_ATTN_SCRATCH_BYTES,
              "the header states the scratch size of csa2_sparse_attn_noalloc");

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// [lo, hi) byte ranges overlap?
bool overlap(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
  const char* pa = static_cast<const char*>(a);
  const char* pb = static_cast<const char*>(b);
  return pa < pb + bbytes && pb < pa + abytes;
}

int launched(hipError_t e) { return e == hipSuccess ? CSA2_OK : CSA2_ELAUNCH; }

// Clear an error left behind by earlier, unrelated runtime calls so that a
// failure reported after our launches is our own.
void clear_stale_error() { (void)hipGetLastError(); }

}  // namespace

extern "C" {

const char* csa2_status_string(int status) {
  switch (status) {
    case CSA2_OK: return "ok";
    case CSA2_EINVAL: return "invalid argument (null pointer, size, stride or alignment)";
    case CSA2_EUNSUPPORTED: return "unsupported dtype or shape";
    case CSA2_ELAUNCH: return "kernel launch failed";
    case CSA2_EWORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

int csa2_version(void) { return (1 << 16) | 2; }

size_t csa2_workspace_bytes(int op, int64_t R, int64_t n, int64_t k) {
  if (R <= 0) return 0;
  if (op == CSA2_OP_SPARSE_ATTN) {
    if (n < 0 || n > 2048 || k < 1 || k > (int64_t(1) << 30)) return 0;
    return csa2::attn_workspace_bytes(R, (int)n, (int)k);
  }
  if (op == CSA2_OP_SELECT) {
    if (n < 1 || k < 1) return 0;
    return csa2::select_workspace_bytes(R, n, k);
  }
  return 0;
}

int csa2_compress(int B, int T, const void* kv, int64_t kv_sb, const void* gate, int64_t g_sb,
                  void* out, int64_t out_sb, hipStream_t stream) {
  if (B < 0 || T < 0 || (T & 1)) return CSA2_EINVAL;
  if (B == 0 || T == 0) return CSA2_OK;
  if (B > 65535) return CSA2_EUNSUPPORTED;
  if (!kv || !gate || !out) return CSA2_EINVAL;
  if (!aligned(kv, 16) || !aligned(gate, 16) || !aligned(out, 16)) return CSA2_EINVAL;
  const int64_t rowsz = (int64_t)T * CSA2_D, orow = (int64_t)(T / 2) * CSA2_D;
  if ((B > 1 && (kv_sb < rowsz || g_sb < rowsz || out_sb < orow)) || kv_sb % 8 || g_sb % 8 ||
      out_sb % 8 || kv_sb < 0 || g_sb < 0 || out_sb < 0)
    return CSA2_EINVAL;
  const int64_t kv_bytes = ((int64_t)(B - 1) * kv_sb + rowsz) * 2;
  const int64_t g_bytes = ((int64_t)(B - 1) * g_sb + rowsz) * 2;
  const int64_t o_bytes = ((int64_t)(B - 1) * out_sb + orow) * 2;
  if (overlap(out, o_bytes, kv, kv_bytes) || overlap(out, o_bytes, gate, g_bytes)) return CSA2_EINVAL;
  clear_stale_error();
  return launched(csa2::launch_compress(B, T, kv, kv_sb, gate, g_sb, out, out_sb, stream));
}

int csa2_compress_nvfp4(int B, int T, const void* kv, int64_t kv_sb, const void* gate,
                        int64_t g_sb, uint8_t* codes, uint8_t* scale_e4m3, int64_t out_sb,
                        hipStream_t stream) {
  if (B < 0 || T < 0 || (T & 1)) return CSA2_EINVAL;
  if (B == 0 || T == 0) return CSA2_OK;
  if (B > 65535) return CSA2_EUNSUPPORTED;
  if (!kv || !gate || !codes || !scale_e4m3) return CSA2_EINVAL;
  if (!aligned(kv, 16) || !aligned(gate, 16) || !aligned(codes, 8)) return CSA2_EINVAL;
  const int64_t rowsz = (int64_t)T * CSA2_D, G = T / 2;
  if ((B > 1 && (kv_sb < rowsz || g_sb < rowsz || out_sb < G)) || kv_sb % 8 || g_sb % 8 ||
      kv_sb < 0 || g_sb < 0 || out_sb < 0)
    return CSA2_EINVAL;
  const int64_t kv_bytes = ((int64_t)(B - 1) * kv_sb + rowsz) * 2;
  const int64_t g_bytes = ((int64_t)(B - 1) * g_sb + rowsz) * 2;
  const int64_t rows = (int64_t)(B - 1) * out_sb + G;
  const int64_t c_bytes = rows * (CSA2_D / 2), s_bytes = rows * (CSA2_D / 16);
  if (overlap(codes, c_bytes, kv, kv_bytes) || overlap(codes, c_bytes, gate, g_bytes) ||
      overlap(scale_e4m3, s_bytes, kv, kv_bytes) || overlap(scale_e4m3, s_bytes, gate, g_bytes) ||
      overlap(codes, c_bytes, scale_e4m3, s_bytes))
    return CSA2_EINVAL;
  clear_stale_error();
  return launched(csa2::launch_compress_nvfp4(B, T, kv, kv_sb, gate, g_sb, codes, scale_e4m3,
                                              out_sb, stream));
}

int csa2_compress_step(int B, const void* kv, int64_t kv_sb, const void* gate, int64_t g_sb,
                       const int64_t* pos, void* state, csa2_dtype out_dt, void* out,
                       uint8_t* out_scale, int64_t out_sb, int64_t n_cache, hipStream_t stream) {
  if (B < 0 || n_cache < 0) return CSA2_EINVAL;
  if (out_dt != CSA2_BF16 && out_dt != CSA2_NVFP4) return CSA2_EUNSUPPORTED;
  if (B == 0) return CSA2_OK;
  const bool fp4 = out_dt == CSA2_NVFP4;
  if (!kv || !gate || !pos || !state || !out || (fp4 && !out_scale)) return CSA2_EINVAL;
  if (!aligned(kv, 16) || !aligned(gate, 16) || !aligned(state, 16) || !aligned(pos, 8) ||
      !aligned(out, fp4 ? 8 : 16))
    return CSA2_EINVAL;
  if ((B > 1 && (kv_sb < CSA2_D || g_sb < CSA2_D || out_sb < n_cache)) || kv_sb % 8 ||
      g_sb % 8 || kv_sb < 0 || g_sb < 0 || out_sb < 0)
    return CSA2_EINVAL;
  const int64_t kv_bytes = ((int64_t)(B - 1) * kv_sb + CSA2_D) * 2;
  const int64_t g_bytes = ((int64_t)(B - 1) * g_sb + CSA2_D) * 2;
  const int64_t st_bytes = (int64_t)B * 2 * CSA2_D * 2;
  const int64_t rows = n_cache > 0 ? (int64_t)(B - 1) * out_sb + n_cache : 0;
  const int64_t o_bytes = rows * (fp4 ? CSA2_D / 2 : CSA2_D * 2);
  const int64_t s_bytes = fp4 ? rows * (CSA2_D / 16) : 0;
  if (overlap(state, st_bytes, kv, kv_bytes) || overlap(state, st_bytes, gate, g_bytes) ||
      overlap(out, o_bytes, kv, kv_bytes) || overlap(out, o_bytes, gate, g_bytes) ||
      overlap(out, o_bytes, state, st_bytes) ||
      (fp4 && (overlap(out_scale, s_bytes, kv, kv_bytes) ||
               overlap(out_scale, s_bytes, gate, g_bytes) ||
               overlap(out_scale, s_bytes, state, st_bytes) ||
               overlap(out_scale, s_bytes, out, o_bytes))))
    return CSA2_EINVAL;
  clear_stale_error();
  return launched(csa2::launch_compress_step(B, kv, kv_sb, gate, g_sb, pos, state, fp4, out,
                                             out_scale, out_sb, n_cache, stream));
}

int csa2_quant_nvfp4(const void* src, csa2_dtype src_dt, int64_t rows, int cols,
                     uint8_t* packed, uint8_t* scale_e4m3, hipStream_t stream) {
  if (rows < 0 || cols < 16 || cols % 16) return CSA2_EINVAL;
  if (src_dt != CSA2_BF16 && src_dt != CSA2_F32) return CSA2_EUNSUPPORTED;
  if (rows == 0) return CSA2_OK;
  if (!src || !packed || !scale_e4m3) return CSA2_EINVAL;
  if (!aligned(src, 16) || !aligned(packed, 8)) return CSA2_EINVAL;
  if (rows > (int64_t(1) << 40) / cols) return CSA2_EUNSUPPORTED;
  const int64_t n = rows * cols;
  const int64_t src_bytes = n * (src_dt == CSA2_F32 ? 4 : 2);
  if (overlap(packed, n / 2, src, src_bytes) || overlap(scale_e4m3, n / 16, src, src_bytes) ||
      overlap(packed, n / 2, scale_e4m3, n / 16))
    return CSA2_EINVAL;
  clear_stale_error();
  return launched(csa2::launch_quant_nvfp4(src, src_dt == CSA2_F32, rows, cols, packed,
                                           scale_e4m3, stream));
}

int csa2_index_scores(int mode, int B, int Tq, const void* q, csa2_dtype q_dt, const float* w,
                      const void* k, csa2_dtype k_dt, const uint8_t* k_scale, int64_t k_sb,
                      int64_t n_cache, const int64_t* q_pos, const int32_t* cand_blocks, int K_b,
                      float* scores, int64_t s_stride, int32_t* ids_out, float* block_max,
                      int64_t bm_stride, hipStream_t stream) {
  if (mode != CSA2_SCORES_SCAN && mode != CSA2_SCORES_CAND) return CSA2_EINVAL;
  if (B < 0 || Tq < 0 || n_cache < 0) return CSA2_EINVAL;
  if (q_dt != CSA2_BF16) return CSA2_EUNSUPPORTED;
  if (k_dt != CSA2_BF16 && k_dt != CSA2_FP8_E4M3 && k_dt != CSA2_MXFP4) return CSA2_EUNSUPPORTED;
  // MXFP4 keys: the many-query scan (prefill) only
  if (k_dt == CSA2_MXFP4 && (mode != CSA2_SCORES_SCAN || Tq < 64)) return CSA2_EUNSUPPORTED;
  if (n_cache > kMaxN * 8) return CSA2_EUNSUPPORTED;
  const int64_t R = (int64_t)B * Tq;
  if (R == 0) return CSA2_OK;
  if (!q || !w || !q_pos) return CSA2_EINVAL;
  if (!aligned(q, 16) || !aligned(w, 4)) return CSA2_EINVAL;
  const bool fp8 = k_dt == CSA2_FP8_E4M3, mx = k_dt == CSA2_MXFP4;
  // key row bytes: bf16 256, FP8 128, MXFP4 64 codes (+ 4 scale bytes apart)
  const int64_t row_units = mx ? CSA2_DI / 2 : CSA2_DI;
  if (n_cache > 0) {
    if (!k || !aligned(k, 16)) return CSA2_EINVAL;
    if (k_sb < 0 || (B > 1 && k_sb < n_cache * row_units) || (k_sb % (fp8 || mx ? 16 : 8)))
      return CSA2_EINVAL;
    if (mx && (!k_scale || !aligned(k_scale, 4))) return CSA2_EINVAL;
  }
  if (mode == CSA2_SCORES_SCAN) {
    if (!scores && !block_max) return CSA2_EINVAL;
    const int64_t nblk = (n_cache + CSA2_BLOCK - 1) / CSA2_BLOCK;
    if (scores && s_stride < n_cache) return CSA2_EINVAL;
    if (block_max && bm_stride < nblk) return CSA2_EINVAL;
    if (B > 65535 || (Tq + 3) / 4 > 65535) return CSA2_EUNSUPPORTED;
    if (n_cache == 0) return CSA2_OK;
    clear_stale_error();
    const int fmt = mx ? csa2::KEYS_MXFP4 : (fp8 ? csa2::KEYS_FP8 : csa2::KEYS_BF16);
    return launched(csa2::launch_index_scan(B, Tq, q, w, k, fmt, k_scale, k_sb, n_cache, q_pos,
                                            scores, s_stride, block_max, bm_stride, stream));
  }
  if (!cand_blocks || !scores || !ids_out || K_b < 1) return CSA2_EINVAL;
  if (K_b > kMaxN / CSA2_BLOCK) return CSA2_EUNSUPPORTED;
  if (s_stride < (int64_t)K_b * CSA2_BLOCK) return CSA2_EINVAL;
  if (R > 65535) return CSA2_EUNSUPPORTED;
  // n_cache == 0: nothing is visible, the kernel only writes absent entries
  // and never reads a key
  clear_stale_error();
  return launched(csa2::launch_index_cand(B, Tq, q, w, k, fp8, k_sb, n_cache, q_pos, cand_blocks,
                                          K_b, scores, ids_out, s_stride, stream));
}

int csa2_gather_scores(int B, int Tq, const float* all, int64_t a_stride, int64_t n_cache,
                       const int64_t* q_pos, const int32_t* cand_blocks, int K_b, float* scores,
                       int32_t* ids_out, int64_t s_stride, hipStream_t stream) {
  if (B < 0 || Tq < 0 || n_cache < 0) return CSA2_EINVAL;
  if (n_cache > kMaxN * 8) return CSA2_EUNSUPPORTED;
  const int64_t R = (int64_t)B * Tq;
  if (R == 0) return CSA2_OK;
  if (!q_pos || !cand_blocks || !scores || !ids_out || K_b < 1) return CSA2_EINVAL;
  if (K_b > kMaxN / CSA2_BLOCK) return CSA2_EUNSUPPORTED;
  if (R > 65535) return CSA2_EUNSUPPORTED;
  if (s_stride < (int64_t)K_b * CSA2_BLOCK || s_stride % 4) return CSA2_EINVAL;
  if (!aligned(scores, 16) || !aligned(ids_out, 16)) return CSA2_EINVAL;
  if (n_cache > 0 && (!all || !aligned(all, 16) || a_stride < n_cache || a_stride % 4))
    return CSA2_EINVAL;
  const int64_t o_bytes = ((R - 1) * s_stride + (int64_t)K_b * CSA2_BLOCK) * 4;
  if (overlap(scores, o_bytes, ids_out, o_bytes)) return CSA2_EINVAL;
  if (n_cache > 0) {
    const int64_t a_bytes = ((R - 1) * a_stride + n_cache) * 4;
    if (overlap(scores, o_bytes, all, a_bytes) || overlap(ids_out, o_bytes, all, a_bytes))
      return CSA2_EINVAL;
  }
  clear_stale_error();
  return launched(csa2::launch_gather_cand(R, all, a_stride, n_cache, q_pos, cand_blocks, K_b,
                                           scores, ids_out, s_stride, stream));
}

int csa2_gather_select(int B, int Tq, const float* all, int64_t a_stride, int64_t n_cache,
                       const int64_t* q_pos, const int32_t* cand_blocks, int K_b, int k,
                       int32_t* out, int64_t o_stride, hipStream_t stream) {
  if (B < 0 || Tq < 0 || n_cache < 0 || k < 1) return CSA2_EINVAL;
  if (n_cache > kMaxN * 8) return CSA2_EUNSUPPORTED;
  const int64_t R = (int64_t)B * Tq;
  if (R == 0) return CSA2_OK;
  if (!q_pos || !cand_blocks || !out || K_b < 1) return CSA2_EINVAL;
  if (K_b > kMaxN / CSA2_BLOCK || k > kMaxN) return CSA2_EUNSUPPORTED;
  if (R > INT32_MAX || !csa2::gather_select_supported(R, (int64_t)K_b * CSA2_BLOCK))
    return CSA2_EUNSUPPORTED;
  if (o_stride < k || !aligned(out, 4)) return CSA2_EINVAL;
  if (n_cache > 0 && (!all || !aligned(all, 4) || a_stride < n_cache)) return CSA2_EINVAL;
  if (n_cache > 0) {
    const int64_t a_bytes = ((R - 1) * a_stride + n_cache) * 4;
    const int64_t o_bytes = ((R - 1) * o_stride + k) * 4;
    if (overlap(out, o_bytes, all, a_bytes)) return CSA2_EINVAL;
  }
  clear_stale_error();
  return launched(csa2::launch_gather_select((int)R, all, a_stride, n_cache, q_pos, cand_blocks,
                                             K_b, k, out, o_stride, stream));
}

int csa2_select_topk(int R, int64_t n, const float* scores, int64_t s_stride, const int32_t* ids,
                     int64_t id_stride, const int32_t* forced, int force_last, int k, int32_t* out,
                     int64_t o_stride, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (R < 0 || n < 1 || k < 1) return CSA2_EINVAL;
  if (n > kMaxN || k > kMaxN) return CSA2_EUNSUPPORTED;
  if (R == 0) return CSA2_OK;
  if (!scores || !out) return CSA2_EINVAL;
  if (s_stride < n || o_stride < k) return CSA2_EINVAL;
  if (ids && id_stride < n) return CSA2_EINVAL;
  if (forced && force_last) return CSA2_EINVAL;
  if (!aligned(scores, 4) || !aligned(out, 4) || (ids && !aligned(ids, 4))) return CSA2_EINVAL;
  const size_t need = csa2::select_workspace_bytes(R, n, k);
  if (need > 0 && (!ws || ws_bytes < need || !aligned(ws, 64))) return CSA2_EWORKSPACE;
  clear_stale_error();
  return launched(csa2::launch_select_topk(R, n, scores, s_stride, ids, id_stride, forced,
                                           force_last ? 1 : 0, k, out, o_stride, ws, stream));
}

}  // extern "C"

namespace {

// Every argument check of the sparse attention calls except the scratch.
// CSA2_OK with R = 0 means there is nothing to do.
int check_sparse_attn(int B, int Tq, const void* q, int64_t q_sb, const void* lat,
                      csa2_dtype lat_dt, const void* lat_scale, int64_t lat_sb, int64_t n_cache,
                      const int32_t* sel, int K, int64_t sel_sb, const void* win,
                      csa2_dtype win_dt, const float* win_scale, int W, int W_cap, int64_t win_sb,
                      const int64_t* q_pos, const float* sink, void* out, int64_t out_sb,
                      float* lse) {
  if (B < 0 || Tq < 0 || K < 0 || W < 1 || W_cap < W || n_cache < 0) return CSA2_EINVAL;
  if (K > 2048) return CSA2_EUNSUPPORTED;
  if (lat_dt != CSA2_BF16 && lat_dt != CSA2_NVFP4) return CSA2_EUNSUPPORTED;
  if (win_dt != CSA2_BF16 && win_dt != CSA2_FP8_E4M3) return CSA2_EUNSUPPORTED;
  if (n_cache >= (int64_t(1) << 31)) return CSA2_EUNSUPPORTED;
  const int64_t R = (int64_t)B * Tq;
  if (R == 0) return CSA2_OK;
  if (R > 0x7fffffff) return CSA2_EUNSUPPORTED;
  if (!q || !win || !q_pos || !sink || !out) return CSA2_EINVAL;
  if (K > 0 && !sel) return CSA2_EINVAL;
  if (n_cache > 0 && !lat) return CSA2_EINVAL;
  if (lat_dt == CSA2_NVFP4 && n_cache > 0 && !lat_scale) return CSA2_EINVAL;
  if (win_dt == CSA2_FP8_E4M3 && !win_scale) return CSA2_EINVAL;
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(sink, 4) || (lse && !aligned(lse, 4)))
    return CSA2_EINVAL;
  if (lat && !aligned(lat, lat_dt == CSA2_BF16 ? 16 : 4)) return CSA2_EINVAL;
  if (!aligned(win, win_dt == CSA2_BF16 ? 16 : 8)) return CSA2_EINVAL;
  if (q_sb % 8 || q_sb < 0 || (B > 1 && q_sb < (int64_t)Tq * CSA2_HQ * CSA2_D)) return CSA2_EINVAL;
  if (out_sb % 8 || out_sb < (int64_t)CSA2_HQ * CSA2_D) return CSA2_EINVAL;
  if (K > 0 && sel_sb < K) return CSA2_EINVAL;
  if (lat_sb < 0 || (B > 1 && lat_sb < n_cache)) return CSA2_EINVAL;
  if (win_sb < 0 || (B > 1 && win_sb < W_cap)) return CSA2_EINVAL;
  return CSA2_OK;
}

}  // namespace

extern "C" {

int csa2_sparse_attn(int B, int Tq, const void* q, int64_t q_sb, const void* lat,
                     csa2_dtype lat_dt, const void* lat_scale, int64_t lat_sb, int64_t n_cache,
                     const int32_t* sel, int K, int64_t sel_sb, const void* win, csa2_dtype win_dt,
                     const float* win_scale, int W, int W_cap, int64_t win_sb,
                     const int64_t* q_pos, const float* sink, float scale, void* out,
                     int64_t out_sb, float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  const int st = check_sparse_attn(B, Tq, q, q_sb, lat, lat_dt, lat_scale, lat_sb, n_cache, sel,
                                   K, sel_sb, win, win_dt, win_scale, W, W_cap, win_sb, q_pos,
                                   sink, out, out_sb, lse);
  const int64_t R = (int64_t)B * Tq;
  if (st != CSA2_OK || R == 0) return st;
  const size_t need = csa2::attn_workspace_bytes(R, K, W);
  if (need > 0 && (!ws || ws_bytes < need || !aligned(ws, 16))) return CSA2_EWORKSPACE;
  clear_stale_error();
  const int lat_fmt = lat_dt == CSA2_NVFP4 ? 3 : 1;
  const int win_fmt = win_dt == CSA2_FP8_E4M3 ? 2 : 1;
  return launched(csa2::launch_sparse_attn(B, Tq, q, q_sb, lat, lat_fmt, lat_scale, lat_sb,
                                           n_cache, sel, K, sel_sb, win, win_fmt, win_scale, W,
                                           W_cap, win_sb, q_pos, sink, scale, out, out_sb, lse,
                                           ws, stream));
}

int csa2_sparse_attn_noalloc(int B, int Tq, const void* q, int64_t q_sb, const void* lat,
                             csa2_dtype lat_dt, const void* lat_scale, int64_t lat_sb,
                             int64_t n_cache, const int32_t* sel, int K, int64_t sel_sb,
                             const void* win, csa2_dtype win_dt, const float* win_scale, int W,
                             int W_cap, int64_t win_sb, const int64_t* q_pos, const float* sink,
                             float scale, void* out, int64_t out_sb, float* lse,
                             hipStream_t stream) {
  const int st = check_sparse_attn(B, Tq, q, q_sb, lat, lat_dt, lat_scale, lat_sb, n_cache, sel,
                                   K, sel_sb, win, win_dt, win_scale, W, W_cap, win_sb, q_pos,
                                   sink, out, out_sb, lse);
  const int64_t R = (int64_t)B * Tq;
  if (st != CSA2_OK || R == 0) return st;
  const int lat_fmt = lat_dt == CSA2_NVFP4 ? 3 : 1;
  const int win_fmt = win_dt == CSA2_FP8_E4M3 ? 2 : 1;
  // the same split policy as csa2_sparse_attn, so the results are the same
  // bits; the partials must fit the library's fixed scratch
  const size_t need = csa2::attn_workspace_bytes_fmt(R, K, W, lat_fmt);
  if (need > csa2::ATTN_SCRATCH_BYTES) return CSA2_EWORKSPACE;
  void* ws = nullptr;
  if (need > 0 && csa2::attn_scratch(&ws) != hipSuccess) return CSA2_ELAUNCH;
  clear_stale_error();
  return launched(csa2::launch_sparse_attn(B, Tq, q, q_sb, lat, lat_fmt, lat_scale, lat_sb,
                                           n_cache, sel, K, sel_sb, win, win_fmt, win_scale, W,
                                           W_cap, win_sb, q_pos, sink, scale, out, out_sb, lse,
                                           ws, stream));
}

int csa2_dequant_fp8(const uint8_t* src, const float* row_scale, int64_t rows, int cols,
                     void* dst, csa2_dtype dst_dt, hipStream_t stream) {
  if (rows < 0 || cols < 1) return CSA2_EINVAL;
  if (dst_dt != CSA2_BF16 && dst_dt != CSA2_F32) return CSA2_EUNSUPPORTED;
  if (rows == 0) return CSA2_OK;
  if (!src || !dst) return CSA2_EINVAL;
  if (!aligned(dst, dst_dt == CSA2_F32 ? 4 : 2)) return CSA2_EINVAL;
  clear_stale_error();
  return launched(csa2::launch_dequant_fp8(src, row_scale, rows, cols, dst, dst_dt == CSA2_F32,
                                           stream));
}

int csa2_dequant_nvfp4(const uint8_t* packed, const uint8_t* scale_e4m3, int64_t rows, int cols,
                       void* dst, csa2_dtype dst_dt, hipStream_t stream) {
  if (rows < 0 || cols < 16 || cols % 16) return CSA2_EINVAL;
  if (dst_dt != CSA2_BF16 && dst_dt != CSA2_F32) return CSA2_EUNSUPPORTED;
  if (rows == 0) return CSA2_OK;
  if (!packed || !scale_e4m3 || !dst) return CSA2_EINVAL;
  if (!aligned(dst, 4)) return CSA2_EINVAL;
  clear_stale_error();
  return launched(csa2::launch_dequant_nvfp4(packed, scale_e4m3, rows, cols, dst,
                                             dst_dt == CSA2_F32, stream));
}

}  // extern "C"
