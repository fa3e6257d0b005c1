// index_scan.hip -- a2, the candidate-source indexer scan (NVFP4 article,
// section 3.3): every visible latent is scored,
//     score(p) = sum_{h < 32} w_h * max(0, q_h . k_p),
// and the maximum over each block of 8 latents is kept (a block is
// represented by its best in-block score).  Decode (few queries per
// sequence): keys streamed from HBM once per query group, MFMA operands and
// epilogue from indexer.h.  Several queries per sequence (speculative
// verification, prefill): see tile_scan_kernel.
#include "indexer.h"
#include "launch.h"

namespace csa2 {

namespace {

using namespace indexer;

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

// ---- scan: every latent, block max fused ------------------------------------
// Keys are read fully coalesced: a 16-key tile (4 KiB bf16, 2 KiB FP8) is
// loaded as 1 KiB contiguous per wave load, lane l taking 16-byte chunk
// l % C of tile row l / C + (64 / C) c (C = 16-byte chunks per row), the
// chunk index XOR-swizzled by the row; a per-wave LDS buffer then hands each
// lane its MFMA operand (key kl = l % 16: bf16 chunks g + 4c, FP8 chunks g
// and g + 4, g = l / 16).  The swizzle keeps the stores conflict free and the
// loads at most 2-way.
template <typename KT>
struct KRaw;
template <>
struct KRaw<KBf16> {
  static constexpr int ROW = DI * 2, LOADS = 4;
  u32x4 r[LOADS];
};
template <>
struct KRaw<KFp8> {
  static constexpr int ROW = DI, LOADS = 2;
  u32x4 r[LOADS];
};

template <typename KT>
__device__ __forceinline__ void load_key_coalesced(const void* kbase, int64_t tile, int64_t n_cache,
                                                   int lane, KRaw<KT>& R) {
  constexpr int ROW = KRaw<KT>::ROW, C = ROW / 16, RPL = 64 / C;  // chunks per row, rows per load
#pragma unroll
  for (int c = 0; c < KRaw<KT>::LOADS; ++c) {
    const int rl = lane / C + RPL * c;  // tile row
    int64_t row = tile * 16 + rl;
    row = row < n_cache ? row : n_cache - 1;
    const int chunk = (lane % C) ^ (rl % C);
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(kbase) + row * ROW) + chunk;
    R.r[c] = __builtin_nontemporal_load(p);
  }
}

// stage the tile into the wave's LDS buffer and read this lane's operand
__device__ __forceinline__ void relayout_key(const KRaw<KBf16>& R, uint8_t* kst, int lane, KBf16& K) {
#pragma unroll
  for (int c = 0; c < 4; ++c) *reinterpret_cast<u32x4*>(kst + 1024 * c + 16 * lane) = R.r[c];
  const int kl = lane & 15, g = lane >> 4;
#pragma unroll
  for (int c = 0; c < 4; ++c)
    K.b[c] = *reinterpret_cast<const bf16x8*>(kst + kl * 256 + (((g + 4 * c) ^ kl) << 4));
}

__device__ __forceinline__ void relayout_key(const KRaw<KFp8>& R, uint8_t* kst, int lane, KFp8& K) {
#pragma unroll
  for (int c = 0; c < 2; ++c) *reinterpret_cast<u32x4*>(kst + 1024 * c + 16 * lane) = R.r[c];
  const int kl = lane & 15, g = lane >> 4;
  const u32x4 lo = *reinterpret_cast<const u32x4*>(kst + kl * 128 + ((g ^ (kl & 7)) << 4));
  const u32x4 hi = *reinterpret_cast<const u32x4*>(kst + kl * 128 + (((g + 4) ^ (kl & 7)) << 4));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    K.b[i] = (int)lo[i];
    K.b[4 + i] = (int)hi[i];
  }
}

template <int QPB, typename QT, typename KT>
__global__ __launch_bounds__(256) void scan_kernel(ScanArgs a) {
  using KL = KRaw<KT>;  // what a fetch holds
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = blockIdx.y;
  const int j0 = blockIdx.z * QPB;
  const int nq = min(QPB, a.Tq - j0);
  const int g = lane >> 4, kl = lane & 15;
  const int64_t nblk = (a.n_cache + BLK - 1) / BLK;

  __shared__ __align__(16) uint8_t qstage[HI * DI];
  __shared__ __align__(16) uint8_t kstage[WAVES][16 * KRaw<KT>::ROW];
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

  // The first DEPTH tiles are fetched without waiting for the queries'
  // positions (any tile of the cache is readable; invisible keys are masked
  // when scored); later fetches skip tiles past every query's horizon.
  auto fetch = [&](int64_t tile, KL& K, int64_t horizon) {
    if (tile * 16 < horizon) load_key_coalesced<KT>(kb, tile, a.n_cache, lane, K);
  };
  auto process = [&](int64_t tile, const KL& KLd) {
    const int64_t p = tile * 16 + kl;
    KT K;
    // a tile past every query's horizon was not fetched and is not scored
    if (tile * 16 < max_nv) relayout_key(KLd, kstage[wave], lane, K);
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
  // DEPTH tiles in flight per wave: the loads of a wave's tile DEPTH ahead
  // are issued as soon as its current tile has been consumed
  // tiles in flight per wave: 3 for one query; with more queries the
  // registers of their operands leave room for 2
  constexpr int DEPTH = QPB == 1 ? 3 : 2;
  KL buf[DEPTH];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d)
    if (t + d * WAVES < t_end) fetch(t + d * WAVES, buf[d], a.n_cache);
  for (; t < t_end; t += DEPTH * WAVES) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int64_t tt = t + d * WAVES;
      if (tt < t_end) {
        process(tt, buf[d]);
        if (tt + DEPTH * WAVES < t_end) fetch(tt + DEPTH * WAVES, buf[d], max_nv);
      }
    }
  }
}

// ---- several queries per sequence: key tiles shared through LDS -------------
// A block = NW waves x QW queries = NW*QW consecutive queries of one
// sequence, over one key range.  32-key tiles (8 KiB of bf16 keys) are read
// coalesced by the whole block, DEPTH tiles ahead, into a double-buffered LDS
// tile that every wave uses for all of its queries: the keys cross HBM once
// per NW*QW queries.  v_mfma_f32_32x32x16_bf16: A = 32 heads x 16 dims of a
// query (registers, loaded once), B = 16 dims x 32 keys of the LDS tile,
// D = heads x keys; lane l holds key l%32 and heads 8(i/4) + 4(l/32) + i%4 of
// accumulator element i.  Epilogue per query and 32 keys: ReLU x w_h over the
// lane's 16 heads, one cross-half shuffle for the other 16, causal mask, max
// over each 8-key block.
// Prefill (thousands of queries, MFMA-bound): 8 waves x 2 queries, 8 key
// ranges with the range as the block id's low index, so that each XCD keeps
// "its" range resident in L2 while all query groups stream through it.
// Verification decode (a few queries per sequence, HBM-bound): 4 waves x 2
// queries, 3 tiles in flight, enough key ranges to fill the chip.
constexpr int TS_TILE = 32;              // keys per tile
constexpr int TS_LD = DI * 2 + 16;       // LDS bytes per key row (padded)

typedef __attribute__((ext_vector_type(16))) float f32x16;

template <int NW, int QW, int DEPTH>
__global__ __launch_bounds__(NW * 64, 1) void tile_scan_kernel(ScanArgs a, int64_t keys_per_chunk) {
  constexpr int NT = NW * 64;
  constexpr int NQ = NW * QW;                     // queries per block
  constexpr int LPT = TS_TILE * DI * 2 / 16 / NT;  // 16-byte loads per thread per tile
  static_assert(LPT >= 1 && LPT * NT * 16 == TS_TILE * DI * 2, "tile split");
  __shared__ __align__(16) uint8_t kt[2][TS_TILE * TS_LD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, kn = lane & 31;
  const int chunk = blockIdx.x;
  const int b = blockIdx.z;
  const int j0 = blockIdx.y * NQ + wave * QW;  // this wave's first query
  const int64_t k0 = (int64_t)chunk * keys_per_chunk;
  const int64_t k1 = min(a.n_cache, k0 + keys_per_chunk);
  const int64_t nblk = (a.n_cache + BLK - 1) / BLK;
  const uint16_t* kb = static_cast<const uint16_t*>(a.k) + b * a.k_sb;

  // query operands and per-lane head weights
  bf16x8 qa[QW][8];
  float wl[QW][16];
  int64_t nv[QW], rows[QW];
  bool qok[QW];
#pragma unroll
  for (int qi = 0; qi < QW; ++qi) {
    const int j = j0 + qi;
    qok[qi] = j < a.Tq;
    const int64_t r = (int64_t)b * a.Tq + (qok[qi] ? j : a.Tq - 1);
    rows[qi] = r;
    const uint16_t* qr = a.q + r * (HI * DI) + kn * DI + 8 * half;
#pragma unroll
    for (int c = 0; c < 8; ++c) qa[qi][c] = *reinterpret_cast<const bf16x8*>(qr + 16 * c);
#pragma unroll
    for (int i = 0; i < 16; ++i) wl[qi][i] = a.w[r * HI + 8 * (i >> 2) + 4 * half + (i & 3)];
    nv[qi] = qok[qi] ? n_visible(a.q_pos[r], a.n_cache) : 0;
  }
  // visible range of the whole block (queries are consecutive)
  int64_t nv_blk;
  {
    const int jl = min(a.Tq - 1, (int)blockIdx.y * NQ + NQ - 1);
    const int jf = min(a.Tq - 1, (int)blockIdx.y * NQ);
    nv_blk = max(n_visible(a.q_pos[(int64_t)b * a.Tq + jl], a.n_cache),
                 n_visible(a.q_pos[(int64_t)b * a.Tq + jf], a.n_cache));
  }
  // staging: load u of a tile -> (row (u NT + tid) / 16, 16-byte piece tid % 16)
  const int spiece = tid & 15;
  const int64_t kend = min(k1, max(k0, nv_blk));  // keys that need computing
  auto load_tile = [&](int64_t t0, u32x4 (&v)[LPT]) {
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int64_t row = t0 + (u * NT + tid) / 16;
      v[u] = (u32x4){0u, 0u, 0u, 0u};
      if (row < kend) v[u] = *reinterpret_cast<const u32x4*>(kb + row * DI + 8 * spiece);
    }
  };
  auto compute = [&](int64_t t0, const uint8_t* tile) {
    const int64_t p = t0 + kn;  // this lane's key
    bf16x8 kbop[8];
#pragma unroll
    for (int c = 0; c < 8; ++c)
      kbop[c] = *reinterpret_cast<const bf16x8*>(tile + kn * TS_LD + 32 * c + 16 * half);
#pragma unroll
    for (int qi = 0; qi < QW; ++qi) {
      if (!qok[qi]) continue;  // wave-uniform
      float s = -INFINITY;
      if (t0 < nv[qi]) {
        f32x16 acc = {};
#pragma unroll
        for (int c = 0; c < 8; ++c)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[qi][c], kbop[c], acc, 0, 0, 0);
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) sum = fmaf(wl[qi][i], fmaxf(acc[i], 0.f), sum);
        sum += __shfl_xor(sum, 32, 64);
        s = p < nv[qi] ? sum : -INFINITY;
      }
      if (a.scores && half == 0 && p < k1) a.scores[rows[qi] * a.s_stride + p] = s;
      if (a.block_max) {
        float m = s;
        m = fmaxf(m, __shfl_xor(m, 1, 64));
        m = fmaxf(m, __shfl_xor(m, 2, 64));
        m = fmaxf(m, __shfl_xor(m, 4, 64));
        const int64_t blk = p >> 3;
        if (half == 0 && (kn & 7) == 0 && blk < nblk && p < k1)
          a.block_max[rows[qi] * a.bm_stride + blk] = m;
      }
    }
  };
  // keys past every query's horizon: masked scores and block maxima only
  auto masked = [&](int64_t t0) {
    const int64_t p = t0 + kn;
#pragma unroll
    for (int qi = 0; qi < QW; ++qi) {
      if (!qok[qi]) continue;
      if (a.scores && half == 0 && p < k1) a.scores[rows[qi] * a.s_stride + p] = -INFINITY;
      const int64_t blk = p >> 3;
      if (a.block_max && half == 0 && (kn & 7) == 0 && blk < nblk && p < k1)
        a.block_max[rows[qi] * a.bm_stride + blk] = -INFINITY;
    }
  };

  u32x4 stage[DEPTH][LPT];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d)
    if (k0 + d * TS_TILE < kend) load_tile(k0 + d * TS_TILE, stage[d]);
  int buf = 0;
  int64_t t0 = k0;
  for (; t0 < kend; t0 += DEPTH * TS_TILE) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int64_t tt = t0 + d * TS_TILE;
      if (tt < kend) {  // block-uniform
#pragma unroll
        for (int u = 0; u < LPT; ++u) {
          const int row = (u * NT + tid) / 16;
          *reinterpret_cast<u32x4*>(&kt[buf][row * TS_LD + 16 * spiece]) = stage[d][u];
        }
        __syncthreads();
        if (tt + DEPTH * TS_TILE < kend) load_tile(tt + DEPTH * TS_TILE, stage[d]);
        compute(tt, kt[buf]);
        buf ^= 1;
      }
    }
  }
  // the tiles of the range that no query sees
  for (int64_t tt = max(k0, (kend + TS_TILE - 1) / TS_TILE * TS_TILE); tt < k1; tt += TS_TILE)
    masked(tt);
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
  if (!k_fp8 && Tq >= 64) {
    // many queries: MFMA-bound.  8 key ranges, tile-aligned (so block-aligned).
    constexpr int CH = 8;
    int64_t kpc = (n_cache + CH - 1) / CH;
    kpc = (kpc + TS_TILE - 1) / TS_TILE * TS_TILE;
    const unsigned nchunks = (unsigned)((n_cache + kpc - 1) / kpc);
    dim3 grid(nchunks, (unsigned)((Tq + 15) / 16), (unsigned)B);
    hipLaunchKernelGGL((tile_scan_kernel<8, 2, 1>), grid, dim3(512), 0, s, a, kpc);
    return hipGetLastError();
  }
  if (!k_fp8 && Tq >= 2) {
    // a few queries per sequence (speculative verification): HBM-bound, the
    // keys are read once per 8 queries; ranges of whole tiles, ~1024 blocks
    const int64_t groups = (Tq + 7) / 8;
    const int64_t n_tiles32 = (n_cache + TS_TILE - 1) / TS_TILE;
    int64_t ch = (1024 + B * groups - 1) / (B * groups);
    if (ch > n_tiles32) ch = n_tiles32;
    if (ch < 1) ch = 1;
    const int64_t kpc = (n_tiles32 + ch - 1) / ch * TS_TILE;
    const unsigned nchunks = (unsigned)((n_cache + kpc - 1) / kpc);
    dim3 grid(nchunks, (unsigned)groups, (unsigned)B);
    hipLaunchKernelGGL((tile_scan_kernel<8, 1, 6>), grid, dim3(512), 0, s, a, kpc);
    return hipGetLastError();
  }

  const int qpb = Tq >= 4 ? 4 : (Tq >= 2 ? 2 : 1);
  const int64_t nz = (Tq + qpb - 1) / qpb;
  const int64_t n_tiles = (n_cache + 15) / 16;
  // at most 32 tiles per wave (a block streams 512 KiB of bf16 keys); fewer
  // when that would leave the chip short of blocks.  Measured on the 1M
  // decode scan (3 tiles in flight per wave): 32 tiles per wave beat 8 to
  // 24 (per-block start-up) and 64 (2048 blocks balance the XCDs better).
  const int64_t target_waves = 8192;
  int64_t tpw = (n_tiles * B * nz + target_waves - 1) / target_waves;
  if (tpw < 1) tpw = 1;
  if (tpw > 32) tpw = 32;
  a.tiles_per_wave = (int)tpw;
  const int64_t per_block = tpw * WAVES;
  dim3 grid((unsigned)((n_tiles + per_block - 1) / per_block), (unsigned)B, (unsigned)nz);
  if (qpb == 4) return k_fp8 ? launch_scan_t<4, true>(a, B, grid, s) : launch_scan_t<4, false>(a, B, grid, s);
  if (qpb == 2) return k_fp8 ? launch_scan_t<2, true>(a, B, grid, s) : launch_scan_t<2, false>(a, B, grid, s);
  return k_fp8 ? launch_scan_t<1, true>(a, B, grid, s) : launch_scan_t<1, false>(a, B, grid, s);
}

}  // namespace csa2
