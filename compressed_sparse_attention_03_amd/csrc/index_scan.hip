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

constexpr int MAX_TPW = 32;  // tiles per wave of the decode scan (launcher's cap)

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
  const uint8_t* k_scale;  // MXFP4 keys: E8M0 scales [B][N][4], batch stride k_sb / 16
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

// A block's keys as one buffer resource: based at the block's first row and
// clipped to the cache, so a row at or past n_cache reads as zeros (its
// scores are masked like every invisible key's) and every offset is a small
// 32-bit value: a lane-constant part (row within the tile, swizzled chunk)
// and a wave-uniform part (the tile), which lives in a scalar register.
template <typename KT>
struct KeyRange {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t off[KRaw<KT>::LOADS];
};

constexpr int BUF_DWORD3 = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)

template <typename KT>
__device__ __forceinline__ KeyRange<KT> key_range(const void* kbase, int64_t row0, int64_t rows,
                                                  int lane) {
  constexpr int ROW = KRaw<KT>::ROW, C = ROW / 16, RPL = 64 / C;  // chunks per row, rows per load
  KeyRange<KT> kr;
  const uint8_t* base = static_cast<const uint8_t*>(kbase) + row0 * ROW;
  kr.rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0,
                                              (int)(rows * ROW), BUF_DWORD3);
#pragma unroll
  for (int c = 0; c < KRaw<KT>::LOADS; ++c) {
    const int rl = lane / C + RPL * c;  // tile row
    kr.off[c] = (uint32_t)(rl * ROW + (((lane % C) ^ (rl % C)) << 4));
  }
  return kr;
}

// tile_off: byte offset of the tile from the block's first row
template <typename KT>
__device__ __forceinline__ void load_key_coalesced(const KeyRange<KT>& kr, uint32_t tile_off,
                                                   KRaw<KT>& R) {
#pragma unroll
  for (int c = 0; c < KRaw<KT>::LOADS; ++c)
    R.r[c] = __builtin_amdgcn_raw_buffer_load_b128(kr.rsrc, kr.off[c], tile_off, 2 /* nt */);
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
  // the wave index through a scalar register: the compiler then keeps the
  // tile bookkeeping (indices, horizons, loop control) in scalar registers
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.y;
  const int j0 = blockIdx.z * QPB;
  const int nq = min(QPB, a.Tq - j0);
  const int g = lane >> 4, kl = lane & 15;
  const int64_t nblk = (a.n_cache + BLK - 1) / BLK;

  __shared__ __align__(16) uint8_t qstage[HI * DI];
  __shared__ __align__(16) uint8_t kstage[WAVES][16 * KRaw<KT>::ROW];
  // the block's block maxima, written out as one contiguous run at the end
  // (2 per tile, at most 32 tiles per wave)
  __shared__ float bmst[QPB][WAVES * MAX_TPW * 2];
  QT Q[QPB];
  int64_t nv[QPB];
  int64_t max_nv = 0;
#pragma unroll
  for (int qi = 0; qi < QPB; ++qi) {
    const int j = j0 + (qi < nq ? qi : 0);
    const int64_t r = (int64_t)b * a.Tq + j;
    load_query(a.q + r * (HI * DI), a.w + r * HI, Q[qi], lane, qstage);
    // the same in every lane: kept in scalar registers
    const int64_t v = qi < nq ? n_visible(a.q_pos[r], a.n_cache) : 0;
    nv[qi] = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(v >> 32)) << 32) |
                       (uint32_t)__builtin_amdgcn_readfirstlane((int)v));
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
  // a wave past the end of the block's stretch has no tile (it still joins
  // the final barrier)
  const int64_t row0 = blk0 * 16;
  const KeyRange<KT> kr = key_range<KT>(kb, row0, min(a.n_cache, t_end * 16) - row0, lane);

  // The first DEPTH tiles are fetched without waiting for the queries'
  // positions (any tile of the cache is readable; invisible keys are masked
  // when scored); later fetches skip tiles past every query's horizon.
  auto fetch = [&](int64_t tile, KL& K, int64_t horizon) {
    if (tile * 16 < horizon) load_key_coalesced<KT>(kr, (uint32_t)((tile - blk0) * 16 * KL::ROW), K);
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
        const float m = max_of_8_lanes(s);
        if (g == 0 && (kl & 7) == 0) bmst[qi][(tile - blk0) * 2 + (kl >> 3)] = m;
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
  if (a.block_max) {
    // every tile of [blk0, t_end) was processed by one of the waves
    __syncthreads();
    const int64_t nb = min(2 * (t_end - blk0), nblk - 2 * blk0);
#pragma unroll
    for (int qi = 0; qi < QPB; ++qi) {
      if (qi >= nq) break;
      float* dst = a.block_max + ((int64_t)b * a.Tq + j0 + qi) * a.bm_stride + 2 * blk0;
      for (int i = threadIdx.x; i < nb; i += WAVES * 64) dst[i] = bmst[qi][i];
    }
  }
}

// ---- several queries per sequence: key tiles shared through LDS -------------
// A block = NW waves x QW queries = NW*QW consecutive queries of one
// sequence, over one key range.  32-key tiles (8 KiB of bf16 keys, 4 KiB of
// FP8) are read coalesced by the whole block, DEPTH tiles ahead, into a
// double-buffered LDS tile that every wave uses for all of its queries: the
// keys cross HBM once per NW*QW queries.
// bf16 keys: v_mfma_f32_32x32x16_bf16, 8 per query and tile (K = 16 dims
// each); FP8 keys: v_mfma_f32_32x32x64_f8f6f4 on E4M3 codes, 2 per query and
// tile (the query rounded to E4M3 once, exact for the small integers index
// queries take).  A = 32 heads x K dims of a query (registers, loaded once),
// B = K dims x 32 keys from the LDS tile, D = heads x keys; lane l holds key
// l % 32 and heads 8(i/4) + 4(l/32) + i%4 of accumulator element i.  Lane
// half h = l / 32 supplies the same dims of A and B (the dot product does not
// care which dims a k-slot carries).
// Each wave issues the MFMAs of all its queries before their epilogues (the
// pipelined loop also issues the next tile's before this tile's epilogue),
// so no epilogue waits on the MFMA chain it follows; on one SIMD the MFMAs
// and the vector epilogue still mostly take turns.  Epilogue per query and
// 32 keys: ReLU x w_h over the
// lane's 16 heads, the other 16 from the partner half by one lane swap
// (v_permlane32_swap; with two queries one swap serves both, each half of
// the wave then finishing one query), causal mask, max over each 8-key block
// by three DPP steps.
// Prefill (thousands of queries, MFMA-bound): 4 waves x 2 queries, 8 key
// ranges (more when a range would reach 2^31 bytes) with the range as the
// block id's low index, so that each XCD keeps "its" range resident in L2
// while all query groups stream through it.  A few queries per sequence
// (speculative verification): verify_scan_kernel below.
constexpr int TS_TILE = 32;  // keys per tile

// MXFP4 index keys: E2M1 codes (dim 2i in the low nibble of byte i) and one
// E8M0 scale per 32 dims.  v_mfma_scale_f32_32x32x64_f8f6f4 with both
// operands in FP4: lane (row / column l % 32, half h) holds 32 values of
// one K-block of 32 and supplies that block's scale byte, so each lane's 32
// dims are exactly one MX block of its key (and of the query, whose scale is
// 1: the bf16 query is rounded to E2M1 once, exact for the small integers
// index queries take).
struct KMx4 {};

template <typename KT>
struct TileKeys;
template <>
struct TileKeys<KBf16> {
  static constexpr int ROWB = DI * 2;      // bytes per key row
  static constexpr int ESZ = 2;            // bytes per unit of the batch stride
  static constexpr int LD = ROWB + 16;     // LDS pitch (padded)
  typedef bf16x8 QOp[8];                   // a query's A operands (one per MFMA)
};
template <>
struct TileKeys<KFp8> {
  static constexpr int ROWB = DI;
  static constexpr int ESZ = 1;
  static constexpr int LD = ROWB + 16;
  typedef i32x8 QOp[2];
};
template <>
struct TileKeys<KMx4> {
  static constexpr int ROWB = DI / 2;
  static constexpr int ESZ = 1;
  static constexpr int LD = ROWB + 16;
  typedef i32x8 QOp[2];  // 4 of the 8 registers carry the 32 E2M1 codes
};

// this lane's A operands of query row r (32 heads x 128 dims)
__device__ __forceinline__ void tile_query(const uint16_t* q, int kn, int half, bf16x8 (&qa)[8]) {
  const uint16_t* qr = q + kn * DI + 8 * half;
#pragma unroll
  for (int c = 0; c < 8; ++c) qa[c] = *reinterpret_cast<const bf16x8*>(qr + 16 * c);
}
__device__ __forceinline__ void tile_query(const uint16_t* q, int kn, int half, i32x8 (&qa)[2]) {
  const uint16_t* qr = q + kn * DI + 32 * half;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const u32x4* p = reinterpret_cast<const u32x4*>(qr + 64 * c);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const u32x4 x = p[v];  // 8 bf16 -> 8 E4M3 codes = operand words 2v, 2v+1
      qa[c][2 * v] = (int)(bf16x2_to_e4m3x2(x[0]) | (bf16x2_to_e4m3x2(x[1]) << 16));
      qa[c][2 * v + 1] = (int)(bf16x2_to_e4m3x2(x[2]) | (bf16x2_to_e4m3x2(x[3]) << 16));
    }
  }
}

// this lane's B operands (key kn, the same dims as tile_query) from the tile
__device__ __forceinline__ void tile_key(const uint8_t* tile, int kn, int half, bf16x8 (&kb)[8]) {
  const uint8_t* row = tile + kn * TileKeys<KBf16>::LD + 16 * half;
#pragma unroll
  for (int c = 0; c < 8; ++c) kb[c] = *reinterpret_cast<const bf16x8*>(row + 32 * c);
}
__device__ __forceinline__ void tile_key(const uint8_t* tile, int kn, int half, i32x8 (&kb)[2]) {
  const uint8_t* row = tile + kn * TileKeys<KFp8>::LD + 32 * half;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(row + 64 * c);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(row + 64 * c + 16);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      kb[c][v] = (int)lo[v];
      kb[c][4 + v] = (int)hi[v];
    }
  }
}

// this lane's A operands for MXFP4 keys: dims 32(2c+h) .. +31 as E2M1 codes
__device__ __forceinline__ void tile_query_mx(const uint16_t* q, int kn, int half, i32x8 (&qa)[2]) {
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const u32x4* p = reinterpret_cast<const u32x4*>(q + kn * DI + 32 * (2 * c + half));
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      qa[c][v] = (int)bf16x8_to_e2m1x8(p[v]);  // 8 bf16 -> 8 codes = one operand word
      qa[c][4 + v] = 0;
    }
  }
}

// this lane's B operands and scale bytes for MXFP4 keys (key kn)
__device__ __forceinline__ void tile_key_mx(const uint8_t* tile, const uint32_t* scales, int kn,
                                            int half, i32x8 (&kb)[2], int (&ks)[2]) {
  const uint32_t sc = scales[kn];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(tile + kn * TileKeys<KMx4>::LD + 16 * (2 * c + half));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kb[c][i] = (int)v[i];
      kb[c][4 + i] = 0;
    }
    ks[c] = (int)((sc >> (8 * (2 * c + half))) & 0xffu);
  }
}

__device__ __forceinline__ f32x16 tile_mfma_mx(const i32x8 (&qa)[2], const i32x8 (&kb)[2],
                                               const int (&ks)[2]) {
  f32x16 acc = {};
  // format code 4 = FP4 E2M1 for both operands; the query's scale is 2^0
#pragma unroll
  for (int c = 0; c < 2; ++c)
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa[c], kb[c], acc, 4, 4, 0, 127, 0, ks[c]);
  return acc;
}

__device__ __forceinline__ f32x16 tile_mfma(const bf16x8 (&qa)[8], const bf16x8 (&kb)[8]) {
  f32x16 acc = {};
#pragma unroll
  for (int c = 0; c < 8; ++c) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[c], kb[c], acc, 0, 0, 0);
  return acc;
}
__device__ __forceinline__ f32x16 tile_mfma(const i32x8 (&qa)[2], const i32x8 (&kb)[2]) {
  f32x16 acc = {};
  // format code 0 = FP8 E4M3 for both operands; the scale operands are unused
#pragma unroll
  for (int c = 0; c < 2; ++c)
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa[c], kb[c], acc, 0, 0, 0, 0, 0, 0);
  return acc;
}

// The second launch bound is the minimum number of waves per SIMD.  A
// 4-wave block must leave room for at least two waves per SIMD (without it
// a bf16 block took 270 registers, one wave per SIMD); FP8 keys take three
// (168 registers, the tile loop free of spills: 1.66 -> 1.37 ms on an
// 8192-query prefill against two), MXFP4 keys four (128 registers; a fifth
// wave spills in the loop).
template <int NW, typename KT>
constexpr int tile_scan_min_waves() {
  static_assert(NW == 4, "4-wave blocks");
  return std::is_same<KT, KFp8>::value ? 3 : std::is_same<KT, KMx4>::value ? 4 : 2;
}

template <int NW, int QW, int DEPTH, bool PIPE, typename KT>
__global__ __launch_bounds__(NW * 64, (tile_scan_min_waves<NW, KT>())) void tile_scan_kernel(ScanArgs a, int64_t keys_per_chunk) {
  using TK = TileKeys<KT>;
  constexpr bool MX = std::is_same<KT, KMx4>::value;
  constexpr int NT = NW * 64;
  constexpr int NQ = NW * QW;                   // queries per block
  constexpr int PIECES = TS_TILE * TK::ROWB / 16;  // 16-byte pieces per tile
  constexpr int PPR = TK::ROWB / 16;            // pieces per row
  constexpr int LPT = (PIECES + NT - 1) / NT;   // pieces per thread
  // MXFP4: the tile's 32 scale words are loaded by the threads after the
  // code pieces (one 4-byte word per key)
  static_assert(!MX || (LPT == 1 && PIECES + TS_TILE <= NT), "scale loaders");
  __shared__ __align__(16) uint8_t kt[2][TS_TILE * TK::LD];
  __shared__ uint32_t kts[MX ? 2 : 1][MX ? TS_TILE : 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, kn = lane & 31;
  const int chunk = blockIdx.x;
  const int b = blockIdx.z;
  const int j0 = blockIdx.y * NQ + wave * QW;  // this wave's first query
  // key positions fit in 32 bits (the cache holds at most 2^27 latents)
  const int k0 = (int)(chunk * keys_per_chunk);
  const int k1 = (int)min(a.n_cache, (int64_t)k0 + keys_per_chunk);
  const uint8_t* kb = static_cast<const uint8_t*>(a.k) + b * a.k_sb * TK::ESZ;
  const uint32_t* ksb = MX ? reinterpret_cast<const uint32_t*>(a.k_scale + b * (a.k_sb / 16)) : nullptr;

  // query operands, per-lane head weights and output rows
  typename TK::QOp qa[QW];
  float wl[QW][16];
  int nv[QW];
  int64_t rows[QW];
  bool qok[QW];
  float* bm_row[QW];
#pragma unroll
  for (int qi = 0; qi < QW; ++qi) {
    const int j = j0 + qi;
    qok[qi] = j < a.Tq;
    const int64_t r = (int64_t)b * a.Tq + (qok[qi] ? j : a.Tq - 1);
    rows[qi] = r;
    if constexpr (MX)
      tile_query_mx(a.q + r * (HI * DI), kn, half, qa[qi]);
    else
      tile_query(a.q + r * (HI * DI), kn, half, qa[qi]);
#pragma unroll
    for (int i = 0; i < 16; ++i) wl[qi][i] = a.w[r * HI + 8 * (i >> 2) + 4 * half + (i & 3)];
    nv[qi] = qok[qi] ? (int)n_visible(a.q_pos[r], a.n_cache) : 0;
    // this lane's block maximum of a tile starting at key t0 (a multiple of
    // 32) is entry (t0 + kn) / 8 = t0 / 8 + kn / 8: the lane part is folded in
    bm_row[qi] = a.block_max ? a.block_max + r * a.bm_stride + (kn >> 3) : nullptr;
  }
  // visible range of the whole block: the widest of its queries' (any
  // order of positions)
  int64_t qp[NQ];  // NQ unconditional loads first, then their maximum
#pragma unroll
  for (int i = 0; i < NQ; ++i) qp[i] = a.q_pos[(int64_t)b * a.Tq + min((int)blockIdx.y * NQ + i, a.Tq - 1)];
  int nv_blk = 0;
#pragma unroll
  for (int i = 0; i < NQ; ++i) nv_blk = max(nv_blk, (int)n_visible(qp[i], a.n_cache));
  // staging: piece u*NT + tid of a tile -> row / PPR, 16-byte piece % PPR
  const int kend = min(k1, max(k0, nv_blk));  // keys that need computing
  // bf16 and MXFP4 keys: the block's key range [k0, k1) (and the MXFP4
  // scale words) as buffer resources, a load's offset a per-lane constant
  // plus the tile's offset in a scalar register, so the loop computes no
  // addresses (the launcher keeps a range below 2^31 bytes); rows past k1
  // read as zeros.  FP8 keys keep 64-bit addresses, rows past kend
  // repeating row kend - 1: measured faster for them (1.36-1.37 against
  // 1.40 ms on an 8192-query prefill), where the buffer loads gave bf16
  // 2.08-2.10 -> 2.05 ms, MXFP4 1.09 -> 1.08 ms and the verification scan
  // 300 -> 284-288 us.  Whatever a row past kend holds, every query of the
  // block masks it (p >= kend means p >= k1 or p >= every query's horizon).
  constexpr bool BUF = !std::is_same<KT, KFp8>::value;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(kb + (int64_t)k0 * TK::ROWB), (short)0, (k1 - k0) * TK::ROWB, BUF_DWORD3);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      MX ? const_cast<uint32_t*>(ksb + k0) : nullptr, (short)0, MX ? (k1 - k0) * 4 : 0, BUF_DWORD3);
  uint32_t voff[LPT];
#pragma unroll
  for (int u = 0; u < LPT; ++u) {
    const int pc = u * NT + tid;
    voff[u] = pc < PIECES ? (uint32_t)((pc / PPR) * TK::ROWB + 16 * (pc % PPR))
                          : (uint32_t)(4 * (pc - PIECES));
  }
  auto load_tile = [&](int t0, u32x4 (&v)[LPT]) {
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int pc = u * NT + tid;
      if constexpr (BUF) {
        if (pc < PIECES)
          v[u] = __builtin_amdgcn_raw_buffer_load_b128(krs, voff[u], (uint32_t)(t0 - k0) * TK::ROWB, 0);
        else if (MX && pc < PIECES + TS_TILE)  // one key's scale word
          v[u][0] = __builtin_amdgcn_raw_buffer_load_b32(srs, voff[u], (uint32_t)(t0 - k0) * 4u, 0);
      } else if (pc < PIECES) {
        const int row = min(t0 + pc / PPR, kend - 1);
        v[u] = *reinterpret_cast<const u32x4*>(kb + (int64_t)row * TK::ROWB + 16 * (pc % PPR));
      }
    }
  };
  // bi: the LDS tile buffer, a constant at every call site (stage i of the
  // pipelined loop and tile d of a trip of the other always use buffer i,
  // resp. d % 2), so no tile address is chosen at run time
  auto store_tile = [&](int bi, const u32x4 (&v)[LPT]) {
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int pc = u * NT + tid;
      if (pc < PIECES) *reinterpret_cast<u32x4*>(kt[bi] + (pc / PPR) * TK::LD + 16 * (pc % PPR)) = v[u];
      else if (MX && pc < PIECES + TS_TILE) kts[bi][pc - PIECES] = v[u][0];
    }
  };
  struct Accs {
    f32x16 v[QW];
  };
  // the MFMAs of all queries of the wave on one tile
  auto mma = [&](int bi, Accs& A) {
    const uint8_t* tile = kt[bi];
    typename TK::QOp kop;
    if constexpr (MX) {
      int ks[2];
      tile_key_mx(tile, kts[bi], kn, half, kop, ks);
#pragma unroll
      for (int qi = 0; qi < QW; ++qi) A.v[qi] = tile_mfma_mx(qa[qi], kop, ks);
    } else {
      tile_key(tile, kn, half, kop);
#pragma unroll
      for (int qi = 0; qi < QW; ++qi) A.v[qi] = tile_mfma(qa[qi], kop);
    }
  };
  // the epilogue of one tile: ReLU . w . head sum, causal mask, block max
  auto epi = [&](int t0, const Accs& A) {
    const int p = t0 + kn;  // this lane's key (non-negative: 32-bit unsigned offsets)
    const uint32_t pu = (uint32_t)p;
    auto finish = [&](float s, int nv_l, bool ok_l, int64_t row_l, float* bm_l) {
      s = p < nv_l ? s : -INFINITY;
      if (a.scores && ok_l && p < k1) a.scores[row_l * a.s_stride + pu] = s;
      if (a.block_max) {
        const float m = max_of_8_lanes(s);
        if (ok_l && (kn & 7) == 0 && p < k1) bm_l[(uint32_t)t0 >> 3] = m;
      }
    };
    if constexpr (QW % 2 == 0) {
      // queries in pairs: one lane swap leaves the full head sum of query
      // qp in lanes 0-31 and of query qp+1 in lanes 32-63, so the mask,
      // block max and stores run once for both
#pragma unroll
      for (int qp = 0; qp < QW; qp += 2) {
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          s0 = fmaf(wl[qp][i], relu(A.v[qp][i]), s0);
          s1 = fmaf(wl[qp + 1][i], relu(A.v[qp + 1][i]), s1);
        }
        // lanes 32-63 of s0 <-> lanes 0-31 of s1
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(s0), __float_as_uint(s1),
                                                         false, false);
        const float tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        finish(tot, half ? nv[qp + 1] : nv[qp], half ? qok[qp + 1] : qok[qp],
               half ? rows[qp + 1] : rows[qp], half ? bm_row[qp + 1] : bm_row[qp]);
      }
    } else {
#pragma unroll
      for (int qi = 0; qi < QW; ++qi) {
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) sum = fmaf(wl[qi][i], relu(A.v[qi][i]), sum);
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(sum), __float_as_uint(sum),
                                                         false, false);
        sum = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);  // both halves' heads
        finish(sum, nv[qi], qok[qi] && half == 0, rows[qi], bm_row[qi]);
      }
    }
  };
  auto compute = [&](int t0, int bi) {
    Accs A;
    mma(bi, A);
    epi(t0, A);
  };
  // keys past every query's horizon: masked scores and block maxima only
  auto masked = [&](int t0) {
    const int p = t0 + kn;
#pragma unroll
    for (int qi = 0; qi < QW; ++qi) {
      if (!qok[qi]) continue;
      if (a.scores && half == 0 && p < k1) a.scores[rows[qi] * a.s_stride + p] = -INFINITY;
      if (a.block_max && half == 0 && (kn & 7) == 0 && p < k1) bm_row[qi][(uint32_t)t0 >> 3] = -INFINITY;
    }
  };

  if constexpr (PIPE) {
    // software pipeline over tiles: the MFMAs of tile i+1 are issued before
    // the epilogue of tile i, so the matrix core and the vector ALU of a wave
    // work side by side; two tiles staged in registers (even / odd)
    static_assert(DEPTH == 2, "pipelined loop stages tiles in pairs");
    u32x4 stage[2][LPT];
    if (k0 < kend) load_tile(k0, stage[0]);
    if (k0 + TS_TILE < kend) load_tile(k0 + TS_TILE, stage[1]);
    auto step = [&](int tt, int bi, u32x4 (&st)[LPT], Accs& A) {
      store_tile(bi, st);
      __syncthreads();
      if (tt + 2 * TS_TILE < kend) load_tile(tt + 2 * TS_TILE, st);
      mma(bi, A);
    };
    Accs A0, A1;
    int tt = k0;
    if (tt < kend) {
      step(tt, 0, stage[0], A0);
      for (;;) {  // block-uniform trip count
        if (tt + TS_TILE >= kend) {
          epi(tt, A0);
          break;
        }
        step(tt + TS_TILE, 1, stage[1], A1);
        epi(tt, A0);
        tt += TS_TILE;
        if (tt + TS_TILE >= kend) {
          epi(tt, A1);
          break;
        }
        step(tt + TS_TILE, 0, stage[0], A0);
        epi(tt, A1);
        tt += TS_TILE;
      }
    }
  } else {
    // DEPTH tiles in flight: the loads of the tile DEPTH ahead are issued as
    // soon as the current tile is in LDS
    u32x4 stage[DEPTH][LPT];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
      if (k0 + d * TS_TILE < kend) load_tile(k0 + d * TS_TILE, stage[d]);
    static_assert(DEPTH % 2 == 0, "tile d of a trip uses LDS buffer d % 2");
    int t0 = k0;
    for (; t0 < kend; t0 += DEPTH * TS_TILE) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        const int tt = t0 + d * TS_TILE;
        if (tt < kend) {  // block-uniform
          store_tile(d % 2, stage[d]);
          __syncthreads();
          if (tt + DEPTH * TS_TILE < kend) load_tile(tt + DEPTH * TS_TILE, stage[d]);
          compute(tt, d % 2);
        }
      }
    }
  }
  // the tiles of the range that no query sees
  for (int tt = max(k0, (kend + TS_TILE - 1) / TS_TILE * TS_TILE); tt < k1; tt += TS_TILE)
    masked(tt);
}

// ---- speculative verification: (query, tile) units dealt over the waves ----
// A few queries per sequence (2-63 draft tokens), bf16 keys.  A block = 4
// waves over one key range and a group of up to 8 consecutive queries of one
// sequence.  Keys come in groups of VG_TILES = 4 tiles (128 keys, 32 KiB),
// fetched VERIFY_DEPTH groups ahead into registers (non-temporal raw buffer
// loads over the block's range, rows past it reading as zeros) and stored to
// one of two LDS group buffers: one barrier per group.  The 4n (query, tile) units of a group of
// n queries are dealt out evenly: wave w takes units wn .. wn + n - 1 in
// query-major order (unit u = query u / 4, tile u % 4), so every SIMD does n
// MFMA tiles and epilogues per group whatever n is (one wave per query slot,
// 8 slots, computes 3 empty slots for 5 queries).  Wave w meets queries
// floor(wn / 4) .. floor((wn + n - 1) / 4), at most two when n != 7: their
// operands and weights stay in registers.  Seven queries run as eight with
// the last slot empty.  MFMA and epilogue per unit as in tile_scan_kernel.
constexpr int VG_TILES = 4;
constexpr int VG_KEYS = VG_TILES * TS_TILE;  // keys per group
// Measured on the 1M verification workload (8 sequences x 5 queries, 1 GiB
// of keys): 2 groups in flight and ~512 blocks (two per CU, one round),
// 207-211 us; with cached instead of non-temporal loads 228-230 us (1 group
// in flight 232, 3 groups 229-234, 1024 / 2048 blocks 229-232 / 238); the
// 8-query-slot tile scan 275-285 us.  Not kept: the next unit's MFMAs issued
// before this unit's epilogue (242-245 us), two MFMA accumulation chains per
// unit (232-234), one LDS group buffer with three blocks per CU (232).
constexpr int VERIFY_DEPTH = 2;               // groups in flight per block

struct VerifyQuery {
  bf16x8 op[8];  // A operands: 32 heads x 128 dims
  float w[16];   // weights of this lane's 16 heads
  int nv;        // visible keys
  bool ok;       // a real query (not an empty slot)
  int64_t row;   // its row of the score and block-max outputs
};

__global__ __launch_bounds__(256, 2) void verify_scan_kernel(ScanArgs a, int64_t keys_per_chunk) {
  using TK = TileKeys<KBf16>;
  constexpr int NT = 256;
  constexpr int PPR = TK::ROWB / 16;                     // 16-byte pieces per key row
  constexpr int LPT = VG_KEYS * TK::ROWB / 16 / NT;      // pieces per thread and group
  static_assert(LPT * NT * 16 == VG_KEYS * TK::ROWB, "a group is whole pieces per thread");
  __shared__ __align__(16) uint8_t kt[2][VG_KEYS * TK::LD];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, kn = lane & 31;
  const int b = blockIdx.z;
  const int jg = blockIdx.y * 8;               // the group's first query
  const int nq = min(8, a.Tq - jg);            // its queries
  const int n = nq == 7 ? 8 : nq;              // its query slots
  const int u0 = wave * n;                     // this wave's first unit
  const int qa = u0 >> 2, qb = (u0 + n - 1) >> 2;
  const int na = min(n, 4 * (qa + 1) - u0);    // units of query slot qa
  const int k0 = (int)(blockIdx.x * keys_per_chunk);
  const int k1 = (int)min(a.n_cache, (int64_t)k0 + keys_per_chunk);
  const uint8_t* kb = static_cast<const uint8_t*>(a.k) + b * a.k_sb * TK::ESZ;

  auto setup = [&](int slot, VerifyQuery& Q) {
    Q.ok = slot < nq;
    const int64_t r = (int64_t)b * a.Tq + (Q.ok ? jg + slot : a.Tq - 1);
    Q.row = r;
    tile_query(a.q + r * (HI * DI), kn, half, Q.op);
#pragma unroll
    for (int i = 0; i < 16; ++i) Q.w[i] = a.w[r * HI + 8 * (i >> 2) + 4 * half + (i & 3)];
    Q.nv = Q.ok ? (int)n_visible(a.q_pos[r], a.n_cache) : 0;
  };
  VerifyQuery QA, QB;
  setup(qa, QA);
  setup(qb, QB);
  // keys that need computing: up to the widest horizon of the group's
  // queries (any order of positions)
  int64_t qp[8];  // 8 unconditional loads first, then their maximum
#pragma unroll
  for (int s = 0; s < 8; ++s) qp[s] = a.q_pos[(int64_t)b * a.Tq + jg + min(s, nq - 1)];
  int nv_blk = 0;
#pragma unroll
  for (int s = 0; s < 8; ++s) nv_blk = max(nv_blk, (int)n_visible(qp[s], a.n_cache));
  const int kend = min(k1, max(k0, nv_blk));

  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(kb + (int64_t)k0 * TK::ROWB), (short)0, (k1 - k0) * TK::ROWB, BUF_DWORD3);
  // piece u * NT + tid of a group is bytes 16 (u NT + tid) of its 128 rows
  auto load_group = [&](int g0, u32x4 (&v)[LPT]) {
#pragma unroll
    for (int u = 0; u < LPT; ++u)
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(krs, 16u * (uint32_t)tid,
                                                   (uint32_t)(g0 - k0) * TK::ROWB + 16u * NT * u,
                                                   2 /* nt: the keys are read once */);
  };
  auto store_group = [&](int bi, const u32x4 (&v)[LPT]) {
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int pc = u * NT + tid;
      *reinterpret_cast<u32x4*>(kt[bi] + (pc / PPR) * TK::LD + 16 * (pc % PPR)) = v[u];
    }
  };
  // one unit: tile t of the group at g0 for query Q
  auto unit = [&](int bi, int g0, int t, const VerifyQuery& Q) {
    bf16x8 kop[8];
    tile_key(kt[bi] + t * TS_TILE * TK::LD, kn, half, kop);
    const f32x16 acc = tile_mfma(Q.op, kop);
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) sum = fmaf(Q.w[i], relu(acc[i]), sum);
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(sum), __float_as_uint(sum), false, false);
    sum = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);  // both halves' heads
    const int t0 = g0 + TS_TILE * t;
    const int p = t0 + kn;
    const float s = p < Q.nv ? sum : -INFINITY;
    const bool st = Q.ok && half == 0 && p < k1;
    if (a.scores && st) a.scores[Q.row * a.s_stride + (uint32_t)p] = s;
    if (a.block_max) {
      const float m = max_of_8_lanes(s);
      if (st && (kn & 7) == 0) a.block_max[Q.row * a.bm_stride + ((uint32_t)p >> 3)] = m;
    }
  };
  auto group = [&](int bi, int g0) {
    for (int i = 0; i < na; ++i) unit(bi, g0, (u0 + i) & 3, QA);  // wave-uniform trip counts
    for (int i = na; i < n; ++i) unit(bi, g0, (u0 + i) & 3, QB);
  };

  // VERIFY_DEPTH groups in flight, staged in registers; the loop body is
  // unrolled so that every staging set and LDS buffer index is a constant
  constexpr int SD = VERIFY_DEPTH, UNR = SD % 2 ? 2 * SD : SD;
  u32x4 stage[SD][LPT];
#pragma unroll
  for (int d = 0; d < SD; ++d)
    if (k0 + d * VG_KEYS < kend) load_group(k0 + d * VG_KEYS, stage[d]);
  for (int g0 = k0; g0 < kend; g0 += UNR * VG_KEYS) {  // block-uniform
#pragma unroll
    for (int k = 0; k < UNR; ++k) {
      const int g = g0 + k * VG_KEYS;
      if (g >= kend) break;
      store_group(k % 2, stage[k % SD]);
      __syncthreads();
      if (g + SD * VG_KEYS < kend) load_group(g + SD * VG_KEYS, stage[k % SD]);
      group(k % 2, g);
    }
  }
  // the keys of the range that no query of the group sees
  const int mstart = kend > k0 ? k0 + (kend - k0 + VG_KEYS - 1) / VG_KEYS * VG_KEYS : k0;
  for (int slot = wave; slot < nq; slot += 4) {  // wave-uniform
    const int64_t r = (int64_t)b * a.Tq + jg + slot;
    if (a.scores)
      for (int p = mstart + lane; p < k1; p += 64) a.scores[r * a.s_stride + p] = -INFINITY;
    if (a.block_max)
      for (int blk = (mstart >> 3) + lane; blk < (k1 + 7) >> 3; blk += 64)
        a.block_max[r * a.bm_stride + blk] = -INFINITY;
  }
}

// Longest key range of one tile-scan block: its bytes stay below 2^31, the
// reach of the block's buffer resource (bf16 keys: 2^23 - 32 keys).
int64_t tile_scan_max_keys(int k_fmt) {
  const int64_t row = k_fmt == KEYS_MXFP4 ? 64 : k_fmt == KEYS_FP8 ? 128 : 256;
  return (INT32_MAX / row) / TS_TILE * TS_TILE;
}

// one launch of the tile scan: NW waves of QW queries per block
template <int NW, int QW, int DEPTH, bool PIPE, typename KT>
hipError_t launch_tile_scan(const ScanArgs& a, int64_t kpc, unsigned nchunks, int Tq, int B,
                            hipStream_t s) {
  constexpr int NQ = NW * QW;
  dim3 grid(nchunks, (unsigned)((Tq + NQ - 1) / NQ), (unsigned)B);
  hipLaunchKernelGGL((tile_scan_kernel<NW, QW, DEPTH, PIPE, KT>), grid, dim3(NW * 64), 0, s, a, kpc);
  return hipGetLastError();
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

constexpr int VERIFY_BLOCKS = 512;  // target blocks of a verification scan (two per CU)

hipError_t launch_index_scan(int B, int Tq, const void* q, const float* w, const void* k,
                             int k_fmt, const uint8_t* k_scale, int64_t k_sb, int64_t n_cache,
                             const int64_t* q_pos, float* scores, int64_t s_stride,
                             float* block_max, int64_t bm_stride, hipStream_t s) {
  ScanArgs a{(const uint16_t*)q, w, k, k_sb, n_cache, q_pos, Tq,
             scores, s_stride, block_max, bm_stride, 1, k_scale};
  const bool k_fp8 = k_fmt == KEYS_FP8;
  if (Tq >= 64) {
    // many queries: MFMA-bound.  8 key ranges, tile-aligned (so block-aligned).
    constexpr int CH = 8;
    int64_t kpc = (n_cache + CH - 1) / CH;
    kpc = (kpc + TS_TILE - 1) / TS_TILE * TS_TILE;
    kpc = min(kpc, tile_scan_max_keys(k_fmt));
    const unsigned nchunks = (unsigned)((n_cache + kpc - 1) / kpc);
    // 4-wave blocks of 2 queries per wave: two or more blocks per CU, so one
    // block's tile barrier is covered by another's work (8-wave blocks, one
    // per CU: bf16 2118-2145 -> 2079 us, FP8 1694-1708 -> 1639-1647).  The
    // MXFP4 scan, whose MFMAs are shortest, goes unpipelined: 128 VGPRs, four
    // waves per SIMD (1584-1592 -> 1105-1108 us; pipelined, three waves:
    // 1197-1200).  One query per wave doubles the LDS operand reads per MFMA
    // and loses (bf16 2425-2452).
    if (k_fmt == KEYS_MXFP4)
      return launch_tile_scan<4, 2, 2, false, KMx4>(a, kpc, nchunks, Tq, B, s);
    if (k_fp8) return launch_tile_scan<4, 2, 2, true, KFp8>(a, kpc, nchunks, Tq, B, s);
    return launch_tile_scan<4, 2, 2, true, KBf16>(a, kpc, nchunks, Tq, B, s);
  }
  if (k_fmt == KEYS_MXFP4) return hipErrorInvalidValue;  // rejected before launch
  if (!k_fp8 && Tq >= 2) {
    // a few queries per sequence (speculative verification): HBM-bound, the
    // keys are read once per 8 queries; ranges of whole 128-key groups,
    // ~VERIFY_BLOCKS blocks
    const int64_t groups = (Tq + 7) / 8;
    const int64_t n_groups = (n_cache + VG_KEYS - 1) / VG_KEYS;
    int64_t ch = (VERIFY_BLOCKS + B * groups - 1) / (B * groups);
    if (ch > n_groups) ch = n_groups;
    if (ch < 1) ch = 1;
    const int64_t kmax = (INT32_MAX / (DI * 2)) / VG_KEYS * VG_KEYS;  // range bytes < 2^31
    const int64_t kpc = min((n_groups + ch - 1) / ch * VG_KEYS, kmax);
    const unsigned nchunks = (unsigned)((n_cache + kpc - 1) / kpc);
    dim3 grid(nchunks, (unsigned)groups, (unsigned)B);
    hipLaunchKernelGGL(verify_scan_kernel, grid, dim3(256), 0, s, a, kpc);
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
  if (tpw > MAX_TPW) tpw = MAX_TPW;
  a.tiles_per_wave = (int)tpw;
  const int64_t per_block = tpw * WAVES;
  dim3 grid((unsigned)((n_tiles + per_block - 1) / per_block), (unsigned)B, (unsigned)nz);
  if (qpb == 4) return k_fp8 ? launch_scan_t<4, true>(a, B, grid, s) : launch_scan_t<4, false>(a, B, grid, s);
  if (qpb == 2) return k_fp8 ? launch_scan_t<2, true>(a, B, grid, s) : launch_scan_t<2, false>(a, B, grid, s);
  return k_fp8 ? launch_scan_t<1, true>(a, B, grid, s) : launch_scan_t<1, false>(a, B, grid, s);
}

}  // namespace csa2
