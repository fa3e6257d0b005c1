// index_cand.hip -- a4, the current layer's indexer over the candidate
// latents (NVFP4 article, section 3.3): the 8 latents of each of the K_b
// chosen blocks are scored with the same fused MFMA contraction + ReLU .
// weight . head-sum epilogue as the scan (indexer.h).
#include "indexer.h"
#include "launch.h"

namespace csa2 {

namespace {

using namespace indexer;

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

}  // namespace

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


// ---- candidates from stored scan scores --------------------------------------
// With one indexer for both stages the candidates' scores are entries of the
// scan's score matrix: one thread per candidate block copies its 8 scores
// (two 16-byte loads, two 16-byte stores for scores and for ids), masking
// latents past the query's horizon exactly as the candidate kernel does.
// Consecutive threads take consecutive entries of the (ascending) block
// list, so neighbouring reads often share cache lines.
__global__ __launch_bounds__(256) void gather_cand_kernel(
    const float* __restrict__ all, int64_t a_stride, int64_t n_cache,
    const int64_t* __restrict__ q_pos, const int32_t* __restrict__ blocks, int K_b,
    float* __restrict__ scores, int32_t* __restrict__ ids, int64_t s_stride) {
  const int64_t r = blockIdx.y;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= K_b) return;
  const int64_t nv = indexer::n_visible(q_pos[r], n_cache);
  const int blk = blocks[r * K_b + j];
  const int64_t p0 = (int64_t)blk * BLK;
  float v[8];
  int id[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = -INFINITY;
    id[i] = -1;
  }
  if (blk >= 0 && p0 < nv) {
    const float* src = all + r * a_stride + p0;
    if (p0 + 8 <= nv) {
      const f32x4 lo = reinterpret_cast<const f32x4*>(src)[0];
      const f32x4 hi = reinterpret_cast<const f32x4*>(src)[1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[i] = lo[i];
        v[4 + i] = hi[i];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) id[i] = (int)(p0 + i);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (p0 + i < nv) {
          v[i] = src[i];
          id[i] = (int)(p0 + i);
        }
    }
  }
  f32x4* so = reinterpret_cast<f32x4*>(scores + r * s_stride + 8 * (int64_t)j);
  u32x4* io = reinterpret_cast<u32x4*>(ids + r * s_stride + 8 * (int64_t)j);
  so[0] = f32x4{v[0], v[1], v[2], v[3]};
  so[1] = f32x4{v[4], v[5], v[6], v[7]};
  io[0] = u32x4{(unsigned)id[0], (unsigned)id[1], (unsigned)id[2], (unsigned)id[3]};
  io[1] = u32x4{(unsigned)id[4], (unsigned)id[5], (unsigned)id[6], (unsigned)id[7]};
}

hipError_t launch_gather_cand(int64_t R, const float* all, int64_t a_stride, int64_t n_cache,
                              const int64_t* q_pos, const int32_t* blocks, int K_b, float* scores,
                              int32_t* ids, int64_t s_stride, hipStream_t s) {
  dim3 grid((unsigned)((K_b + 255) / 256), (unsigned)R);
  hipLaunchKernelGGL(gather_cand_kernel, grid, dim3(256), 0, s, all, a_stride, n_cache, q_pos,
                     blocks, K_b, scores, ids, s_stride);
  return hipGetLastError();
}

}  // namespace csa2
