// index_scores.hip -- a2 / a4, the CSA2 indexer (NVFP4 article, section 3.3;
// oQ3e walkthrough, section 2.1):
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
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace csa2 {

namespace {

constexpr int WAVES = 4;

struct ScanArgs {
  const uint16_t* q;
  const float* w;
  const void* k;
  int64_t k_sb;
  int64_t n_cache;
  const int64_t* q_pos;
  int Tq;
  float* scores;
  int64_t s_stride;
  float* block_max;
  int64_t bm_stride;
  int tiles_per_wave;
};

struct CandArgs {
  const uint16_t* q;
  const float* w;
  const void* k;
  int64_t k_sb;
  int64_t n_cache;
  const int64_t* q_pos;
  int Tq;
  const int32_t* blocks;
  int K_b;
  float* scores;
  int32_t* ids;
  int64_t s_stride;
  int pairs_per_wave;
};

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
      o[i] = bf16_to_e4m3(lo & 0xffffu) | (bf16_to_e4m3(lo >> 16) << 8) |
             (bf16_to_e4m3(hi & 0xffffu) << 16) | (bf16_to_e4m3(hi >> 16) << 24);
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

__device__ __forceinline__ void load_key(const void* kbase, int64_t row, int g, KBf16& K) {
  const uint16_t* p = static_cast<const uint16_t*>(kbase) + row * DI + 8 * g;
#pragma unroll
  for (int c = 0; c < 4; ++c) K.b[c] = *reinterpret_cast<const bf16x8*>(p + 32 * c);
}

__device__ __forceinline__ void load_key(const void* kbase, int64_t row, int g, KFp8& K) {
  const uint8_t* p = static_cast<const uint8_t*>(kbase) + row * DI + 16 * g;
  const u32x4 lo = *reinterpret_cast<const u32x4*>(p);
  const u32x4 hi = *reinterpret_cast<const u32x4*>(p + 64);
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
    s = fmaf(Q.w[0][i], fmaxf(acc0[i], 0.f), s);
    s = fmaf(Q.w[1][i], fmaxf(acc1[i], 0.f), s);
  }
  s += __shfl_xor(s, 16, 64);
  s += __shfl_xor(s, 32, 64);
  return s;
}

__device__ __forceinline__ float tile_score(const QFp8& Q, const KFp8& K) {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  // format code 0 selects FP8 E4M3 for both operands; scale operands unused
  const f32x4 acc0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Q.a[0], K.b, z, 0, 0, 0, 0, 0, 0);
  const f32x4 acc1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Q.a[1], K.b, z, 0, 0, 0, 0, 0, 0);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s = fmaf(Q.w[0][i], fmaxf(acc0[i], 0.f), s);
    s = fmaf(Q.w[1][i], fmaxf(acc1[i], 0.f), s);
  }
  s += __shfl_xor(s, 16, 64);
  s += __shfl_xor(s, 32, 64);
  return s;
}

// ---- scan: every latent, block max fused ------------------------------------
template <int QPB, typename QT, typename KT>
__global__ __launch_bounds__(256) void scan_kernel(ScanArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = blockIdx.y;
  const int j0 = blockIdx.z * QPB;
  const int nq = min(QPB, a.Tq - j0);
  const int g = lane >> 4, kl = lane & 15;
  const int64_t nblk = (a.n_cache + BLK - 1) / BLK;

  __shared__ __align__(16) uint8_t qstage[HI * DI];
  QT Q[QPB];
  int64_t nv[QPB];
  int64_t max_nv = 0;
#pragma unroll
  for (int qi = 0; qi < QPB; ++qi) {
    const int j = j0 + (qi < nq ? qi : 0);
    const int64_t r = (int64_t)b * a.Tq + j;
    load_query(a.q + r * (HI * DI), a.w + r * HI, Q[qi], lane, qstage);
    nv[qi] = qi < nq ? n_visible(a.q_pos[r], a.n_cache) : 0;
    max_nv = nv[qi] > max_nv ? nv[qi] : max_nv;
  }
  const void* kb = (const void*)((const char*)a.k + b * a.k_sb * key_elem_bytes<KT>());

  // A block owns WAVES * tiles_per_wave consecutive tiles; its waves take
  // them round-robin, so at any moment the block streams one contiguous
  // stretch of keys.
  const int64_t n_tiles = (a.n_cache + 15) / 16;
  const int64_t blk0 = (int64_t)blockIdx.x * WAVES * a.tiles_per_wave;
  int64_t t = blk0 + wave;
  const int64_t t_end = min(blk0 + (int64_t)WAVES * a.tiles_per_wave, n_tiles);
  if (t >= t_end) return;

  auto fetch = [&](int64_t tile, KT& K) {
    const int64_t row = tile * 16 + kl;
    if (tile * 16 < max_nv)
      load_key(kb, row < a.n_cache ? row : a.n_cache - 1, g, K);
    else
      zero_key(K);
  };
  auto process = [&](int64_t tile, const KT& K) {
    const int64_t p = tile * 16 + kl;
#pragma unroll
    for (int qi = 0; qi < QPB; ++qi) {
      if (qi >= nq) break;
      const int64_t r = (int64_t)b * a.Tq + j0 + qi;
      float s = -INFINITY;
      if (tile * 16 < nv[qi]) {
        s = tile_score(Q[qi], K);
        if (p >= nv[qi]) s = -INFINITY;
      }
      if (a.scores && g == 0 && p < a.n_cache) a.scores[r * a.s_stride + p] = s;
      if (a.block_max) {
        float m = s;
        m = fmaxf(m, __shfl_xor(m, 1, 64));
        m = fmaxf(m, __shfl_xor(m, 2, 64));
        m = fmaxf(m, __shfl_xor(m, 4, 64));
        const int64_t blk = p >> 3;
        if (g == 0 && (kl & 7) == 0 && blk < nblk) a.block_max[r * a.bm_stride + blk] = m;
      }
    }
  };
  // DEPTH tiles in flight per wave: the loads of a wave's next-but-one tile
  // are issued as soon as its current tile has been consumed
  constexpr int DEPTH = 2;
  KT buf[DEPTH];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d)
    if (t + d * WAVES < t_end) fetch(t + d * WAVES, buf[d]);
  for (; t < t_end; t += DEPTH * WAVES) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int64_t tt = t + d * WAVES;
      if (tt < t_end) {
        process(tt, buf[d]);
        if (tt + DEPTH * WAVES < t_end) fetch(tt + DEPTH * WAVES, buf[d]);
      }
    }
  }
}

// ---- candidates: the latents of the chosen blocks ---------------------------
// A tile is two candidate blocks (16 latents, two contiguous 2 KiB rows runs
// for bf16 keys).  A wave owns pairs_per_wave consecutive tiles and works on
// CB of them at a time: block ids first, then every key load of the batch,
// then the contractions, so the dependent id -> key -> MFMA latencies are paid
// once per batch instead of once per tile.
template <typename QT, typename KT>
__global__ __launch_bounds__(256) void cand_kernel(CandArgs a) {
  constexpr int CB = 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t r = blockIdx.y;
  const int b = (int)(r / a.Tq);
  const int g = lane >> 4, kl = lane & 15;
  __shared__ __align__(16) uint8_t qstage[HI * DI];
  QT Q;
  load_query(a.q + r * (HI * DI), a.w + r * HI, Q, lane, qstage);
  const int64_t nv = n_visible(a.q_pos[r], a.n_cache);
  const void* kb = (const void*)((const char*)a.k + b * a.k_sb * key_elem_bytes<KT>());
  const int n_pairs = (a.K_b + 1) / 2;
  const int pr0 = ((int)blockIdx.x * WAVES + wave) * a.pairs_per_wave;
  const int pr_end = min(pr0 + a.pairs_per_wave, n_pairs);
  const int32_t* brow = a.blocks + r * a.K_b;

  for (int pb = pr0; pb < pr_end; pb += CB) {
    int64_t key[CB];
    bool ok[CB];
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const int j = 2 * (pb + u) + (kl >> 3);
      const int32_t blk = (pb + u < pr_end && j < a.K_b) ? brow[j] : -1;
      key[u] = (int64_t)blk * BLK + (kl & 7);
      ok[u] = blk >= 0 && key[u] < nv;
    }
    KT K[CB];
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      if (ok[u])
        load_key(kb, key[u], g, K[u]);
      else
        zero_key(K[u]);
    }
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      if (pb + u >= pr_end) break;  // uniform
      const float s = tile_score(Q, K[u]);
      const int j = 2 * (pb + u) + (kl >> 3);
      if (g == 0 && j < a.K_b) {
        const int64_t col = r * a.s_stride + (int64_t)j * BLK + (kl & 7);
        a.scores[col] = ok[u] ? s : -INFINITY;
        a.ids[col] = ok[u] ? (int32_t)key[u] : -1;
      }
    }
  }
}

template <int QPB, bool FP8>
hipError_t launch_scan_t(const ScanArgs& a, int B, dim3 grid, hipStream_t s) {
  if (FP8)
    hipLaunchKernelGGL((scan_kernel<QPB, QFp8, KFp8>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((scan_kernel<QPB, QBf16, KBf16>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_index_scan(int B, int Tq, const void* q, const float* w, const void* k,
                             bool k_fp8, int64_t k_sb, int64_t n_cache, const int64_t* q_pos,
                             float* scores, int64_t s_stride, float* block_max,
                             int64_t bm_stride, hipStream_t s) {
  ScanArgs a{(const uint16_t*)q, w, k, k_sb, n_cache, q_pos, Tq,
             scores, s_stride, block_max, bm_stride, 1};
  const int qpb = Tq >= 4 ? 4 : (Tq >= 2 ? 2 : 1);
  const int64_t nz = (Tq + qpb - 1) / qpb;
  const int64_t n_tiles = (n_cache + 15) / 16;
  // at most 16 tiles per wave (a block streams 256 KiB of bf16 keys); fewer
  // when that would leave the chip short of blocks.  Measured on the 1M
  // decode scan: 16 tiles per wave with interleaved waves beat 8, 32 and 64.
  const int64_t target_waves = 4096;
  int64_t tpw = (n_tiles * B * nz + target_waves - 1) / target_waves;
  if (tpw < 1) tpw = 1;
  if (tpw > 16) tpw = 16;
  a.tiles_per_wave = (int)tpw;
  const int64_t per_block = tpw * WAVES;
  dim3 grid((unsigned)((n_tiles + per_block - 1) / per_block), (unsigned)B, (unsigned)nz);
  if (qpb == 4) return k_fp8 ? launch_scan_t<4, true>(a, B, grid, s) : launch_scan_t<4, false>(a, B, grid, s);
  if (qpb == 2) return k_fp8 ? launch_scan_t<2, true>(a, B, grid, s) : launch_scan_t<2, false>(a, B, grid, s);
  return k_fp8 ? launch_scan_t<1, true>(a, B, grid, s) : launch_scan_t<1, false>(a, B, grid, s);
}

hipError_t launch_index_cand(int B, int Tq, const void* q, const float* w, const void* k,
                             bool k_fp8, int64_t k_sb, int64_t n_cache, const int64_t* q_pos,
                             const int32_t* blocks, int K_b, float* scores, int32_t* ids,
                             int64_t s_stride, hipStream_t s) {
  CandArgs a{(const uint16_t*)q, w, k, k_sb, n_cache, q_pos, Tq, blocks, K_b,
             scores, ids, s_stride, 1};
  const int64_t R = (int64_t)B * Tq;
  const int n_pairs = (K_b + 1) / 2;
  // ~4096 waves over the chip, each taking whole batches of 4 tiles
  int64_t ppw = (n_pairs * R + 4095) / 4096;
  ppw = (ppw + 3) / 4 * 4;
  if (ppw < 4) ppw = 4;
  if (ppw > 16) ppw = 16;
  a.pairs_per_wave = (int)ppw;
  const int64_t per_block = ppw * WAVES;
  dim3 grid((unsigned)((n_pairs + per_block - 1) / per_block), (unsigned)R);
  if (k_fp8)
    hipLaunchKernelGGL((cand_kernel<QFp8, KFp8>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((cand_kernel<QBf16, KBf16>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace csa2
