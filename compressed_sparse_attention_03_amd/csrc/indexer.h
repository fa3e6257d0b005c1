// indexer.h -- device building blocks shared by the CSA2 indexer kernels
// (index_scan.hip, index_cand.hip): query / key MFMA operands and the fused
// contraction + ReLU . weight . head-sum epilogue over a tile of 16 keys,
// for the CSA2 indexer (NVFP4 article, section 3.3; oQ3e walkthrough,
// section 2.1):
//
//     score(p) = sum_{h < 32} w_h * max(0, q_h . k_p)        (q_h, k_p in R^128)
//
// as an MFMA contraction of the 32 index-query heads against 16 keys at a
// time, with ReLU, the per-head weight and the head sum fused into the
// epilogue, and (scan mode) the max over each block of 8 latents fused after
// that.
//
// Operand mapping (v_mfma_f32_16x16x32_bf16, wave64):
//   A (16 x 32) = 16 index heads x 32 feature dims, held in registers for the
//                 whole kernel (2 head halves x 4 feature chunks per query);
//   B (32 x 16) = 32 feature dims x 16 keys, loaded straight from HBM;
//   D (16 x 16) = head x key; lane l holds key l%16, heads 4(l/16) .. +3.
// A dot product does not care in which order its terms are summed, so the
// feature dims are assigned to MFMA k-slots in whatever order makes the key
// loads contiguous: lane group g = l/16 of chunk c carries dims 32c+8g..+7,
// i.e. bytes [64c + 16g, +16) of the 256-byte key row.  One load instruction
// then reads 64 contiguous bytes of each of 16 rows and 4 instructions read
// the whole 4 KiB tile exactly once.  The query operand uses the same
// assignment.  FP8 keys use v_mfma_f32_16x16x128_f8f6f4 directly on the
// stored E4M3 codes (one MFMA per head half covers all 128 dims; lane group g
// carries bytes [16g, +16) and [64 + 16g, +16)); the query is rounded to
// E4M3 once, in registers.
//
// With integer-valued q, k (|.| <= 3) and weights in multiples of 1/16 every
// partial sum is an exact fp32 integer multiple of 1/16 below 2^20, so the
// result equals the exact score bit for bit in any summation order.
#pragma once

#include <type_traits>

#include "device_common.h"

namespace csa2 {
namespace indexer {

constexpr int WAVES = 4;  // waves per 256-thread block



__device__ __forceinline__ int64_t n_visible(int64_t t, int64_t n_cache) {
  if (t < 0) return 0;
  const int64_t n = (t + 1) >> 1;
  return n < n_cache ? n : n_cache;
}

// ---- query operands -------------------------------------------------------
struct QBf16 {
  bf16x8 a[2][4];
  float w[2][4];
};

struct QFp8 {
  i32x8 a[2];
  float w[2][4];
};

__device__ __forceinline__ void load_weights(const float* w, float (&wl)[2][4], int g) {
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int i = 0; i < 4; ++i) wl[hh][i] = w[16 * hh + 4 * g + i];
}

__device__ __forceinline__ void load_query(const uint16_t* q, const float* w, QBf16& Q, int lane) {
  const int hl = lane & 15, g = lane >> 4;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      Q.a[hh][c] = *reinterpret_cast<const bf16x8*>(q + (16 * hh + hl) * DI + 32 * c + 8 * g);
  load_weights(w, Q.w, g);
}

// FP8 keys: the 32 x 128 query is rounded to E4M3 once per workgroup, each
// of the 256 threads converting 16 values into an LDS staging row, then every
// lane picks up its operand bytes (the same byte assignment as the keys).
// All threads of the block must call this.
__device__ __forceinline__ void load_query(const uint16_t* q, const float* w, QFp8& Q, int lane,
                                           uint8_t* stage /* 32*128 bytes of LDS */) {
  const int tid = threadIdx.x;
  {
    const int h = tid >> 3, d0 = (tid & 7) * 16;
    const u32x4 x0 = *reinterpret_cast<const u32x4*>(q + h * DI + d0);
    const u32x4 x1 = *reinterpret_cast<const u32x4*>(q + h * DI + d0 + 8);
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = i < 2 ? x0[2 * i] : x1[2 * i - 4];
      const uint32_t hi = i < 2 ? x0[2 * i + 1] : x1[2 * i - 3];
      o[i] = bf16x2_to_e4m3x2(lo) | (bf16x2_to_e4m3x2(hi) << 16);
    }
    __syncthreads();  // a previous user of the staging row is done
    *reinterpret_cast<u32x4*>(stage + h * DI + d0) = o;
    __syncthreads();
  }
  const int hl = lane & 15, g = lane >> 4;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const uint8_t* row = stage + (16 * hh + hl) * DI + 16 * g;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(row);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(row + 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      Q.a[hh][i] = (int)lo[i];
      Q.a[hh][4 + i] = (int)hi[i];
    }
  }
  load_weights(w, Q.w, g);
}

__device__ __forceinline__ void load_query(const uint16_t* q, const float* w, QBf16& Q, int lane,
                                           uint8_t*) {
  load_query(q, w, Q, lane);
}

// ---- key operands ---------------------------------------------------------
struct KBf16 {
  bf16x8 b[4];
};
struct KFp8 {
  i32x8 b;
};

// One key row straight into this lane's operand layout (the candidate
// gather; cached loads: in prefill the same blocks serve many queries).
__device__ __forceinline__ void load_key(const void* kbase, int64_t row, int g, KBf16& K) {
  const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(kbase) + row * DI + 8 * g);
#pragma unroll
  for (int c = 0; c < 4; ++c) K.b[c] = __builtin_bit_cast(bf16x8, p[4 * c]);
}

__device__ __forceinline__ void load_key(const void* kbase, int64_t row, int g, KFp8& K) {
  const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(kbase) + row * DI + 16 * g);
  const u32x4 lo = p[0];
  const u32x4 hi = p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    K.b[i] = (int)lo[i];
    K.b[4 + i] = (int)hi[i];
  }
}

__device__ __forceinline__ void zero_key(KBf16& K) {
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int j = 0; j < 8; ++j) K.b[c][j] = (__bf16)0.0f;
}
__device__ __forceinline__ void zero_key(KFp8& K) {
#pragma unroll
  for (int j = 0; j < 8; ++j) K.b[j] = 0;
}

template <typename KT>
__device__ __forceinline__ constexpr int64_t key_elem_bytes() {
  return std::is_same<KT, KFp8>::value ? 1 : 2;
}

// ReLU as an integer max on the fp32 bit pattern: every negative value
// (sign bit set) is a negative int32 and becomes +0, every non-negative one
// keeps its bits.  One v_max_i32, where fmaxf costs an extra canonicalising
// v_max_f32 per input in IEEE mode.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Max over each group of 8 consecutive lanes, by DPP within the lanes' row:
// three v_max_f32 whose first operand is the DPP-moved value (quad_perm
// [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror).  Written as asm because
// in IEEE mode the compiler does not fold a DPP move into fmaxf: it needs
// the moved value canonical and adds an instruction per step to make it so
// (three per step instead of one).  Each DPP read follows its source's VALU
// write by two wait states (s_nop 1).  Requires every lane of the wave
// active and no NaN inputs (scores are finite or -inf); max(-0, +0) = +0,
// which no maximum tells apart.
__device__ __forceinline__ float max_of_8_lanes(float m) {
  float r;
  asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\tv_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\tv_max_f32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf"
      : "=&v"(r)
      : "v"(m));
  return r;
}

// ---- the fused contraction + epilogue -------------------------------------
// Returns, in every lane, the score of key l%16 of the tile.
__device__ __forceinline__ float tile_score(const QBf16& Q, const KBf16& K) {
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Q.a[0][c], K.b[c], acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Q.a[1][c], K.b[c], acc1, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s = fmaf(Q.w[0][i], relu(acc0[i]), s);
    s = fmaf(Q.w[1][i], relu(acc1[i]), s);
  }
  return sum_across_rows(s);  // the four head groups of this key
}

__device__ __forceinline__ float tile_score(const QFp8& Q, const KFp8& K) {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  // format code 0 selects FP8 E4M3 for both operands; scale operands unused
  const f32x4 acc0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Q.a[0], K.b, z, 0, 0, 0, 0, 0, 0);
  const f32x4 acc1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Q.a[1], K.b, z, 0, 0, 0, 0, 0, 0);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s = fmaf(Q.w[0][i], relu(acc0[i]), s);
    s = fmaf(Q.w[1][i], relu(acc1[i]), s);
  }
  return sum_across_rows(s);  // the four head groups of this key
}

}  // namespace indexer
}  // namespace csa2
