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

}  // namespace csa2
