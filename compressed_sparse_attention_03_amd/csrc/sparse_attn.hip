// sparse_attn.hip -- a6, CSA2 sparse attention (NVFP4 article, sections 3,
// 3.1 and 3.4): for every query, the 64 heads attend over the selected
// compressed latents plus the raw sliding window, K = V = the 512-wide
// latent row, in one pass with an online softmax whose denominator also holds
// a learnable per-head sink logit.
//
// Work decomposition.  A query's rows come in tiles of 32: ceil(K/32) latent
// tiles (rows sel[i]) then ceil(W/32) window tiles (raw positions
// t-W+1 .. t), so a tile never mixes the two sources and its loads are
// straight-line code for one format.  A workgroup (4 waves) owns one query
// and a contiguous range of its tiles.  Few queries (decode) -> the tiles are
// split over several workgroups and a second kernel merges the partial (max,
// sum, numerator) triples; many queries (prefill) -> one workgroup per query,
// no merge.  Rows that do not exist (sel id < 0 or past the cache, a window
// position before 0, the padding of a partial tile) are masked: the
// register path loads row 0 of their source and zeroes it, the direct path
// loads a row of zeros kept in device memory.
//
// Per tile of 32 rows:
//   * every row is gathered from HBM once (1 KiB bf16, or 256 B NVFP4 codes +
//     32 B scales, or 512 B FP8 + a row scale), dequantised in registers to
//     bf16 (exact: E2M1 x E4M3 and E4M3 values are all bf16 values) and
//     stored to LDS once, row-major: the K operand is read from it directly
//     and the V operand through the LDS transpose read (ds_read_b64_tr_b16),
//     so the same bytes feed both contractions;
//   * wave w handles heads 16w..16w+15:
//       S^T = KV . Q^T  (v_mfma_f32_16x16x32_bf16, rows x heads, K = 512)
//     which leaves each lane with a single head (l%16) and 8 of the rows,
//     so the softmax statistics stay per lane; then
//       O^T += V^T . P^T (dims x heads, K = 32 rows)
//     whose B operand is exactly the P values the lane already holds.
//   * with rows loaded straight into LDS (bf16 caches, many tiles per
//     workgroup) PV is split by dims instead: each wave publishes its P^T
//     operand in LDS and computes O^T for dims 128w .. 128w+127 of all 64
//     heads, so each wave reads a quarter of the tile for PV.
// FP8 window rows keep their per-token scale out of the MFMA: it multiplies
// the logit of that row and its P weight.
#include <algorithm>
#include <atomic>

#include "device_common.h"
#include "launch.h"

namespace csa2 {

namespace {

constexpr int TILE = 32;            // rows per tile
// Row-major LDS tile: 528 bf16 per row (264 words, 8 mod 64 banks), which
// makes the PV transpose reads conflict-free (the 4 consecutive rows x 4
// half-pieces a 16-lane group reads land on 16 distinct bank pairs).
// Measured against 520, 536 and 552 (and 528 with a piece swizzle for the
// QK operand reads): 528 is fastest.
constexpr int KV_LD = D + 16;
constexpr int PART = D + 4;         // floats per (query, split, head) partial (16-B multiple)

enum { FMT_BF16 = 1, FMT_FP8 = 2, FMT_NVFP4 = 3 };

struct AttnArgs {
  const uint16_t* q;
  int64_t q_sb;
  int Tq;
  const void* lat;
  int lat_fmt;
  const uint8_t* lat_scale;
  int64_t lat_sb;
  int64_t n_cache;
  const int32_t* sel;
  int K;
  int64_t sel_sb;
  const void* win;
  int win_fmt;
  const float* win_scale;
  int W;
  int W_cap;
  int64_t win_sb;
  const int64_t* q_pos;
  const float* sink;
  float scale;
  uint16_t* out;
  int64_t out_sb;
  float* lse;
  float* part;       // [R][splits][64][PART] when splits > 1
  int splits;
  int tiles_lat;     // ceil(K / TILE), 0 when the cache is empty
  int tiles_win;     // ceil(W / TILE)
  int tiles_per_split;
};

constexpr int kMaxDevices = 64;
// The softmax runs in base 2: logits are pre-multiplied by log2(e) and the
// weights are exp2 of them (one v_exp_f32 each), which is the same
// distribution; the sink enters as sink * log2(e) and lse is converted back.
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float RESCALE_TAU = 11.5f;  // largest log2-weight above the reference point
constexpr int SEL_CAP = 2048;       // largest K: a split's sel entries are cached in LDS
constexpr int DIRECT_MIN_TILES = 10;  // tiles per workgroup from which bf16 rows go straight to LDS

// 8 bf16 of the PV contraction's A operand from two LDS transpose reads
// (4 values each) of the row-major tile.
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
__device__ __forceinline__ bf16x8 pv_operand(const uint16_t* lo, const uint16_t* hi) {
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)lo);
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)hi);
  const u32x2 a2 = __builtin_bit_cast(u32x2, a), b2 = __builtin_bit_cast(u32x2, b);
  return __builtin_bit_cast(bf16x8, (u32x4){a2[0], a2[1], b2[0], b2[1]});
}

// One 1 KiB row of zeros in device memory (zero-initialised, never
// written): the direct row loads read it for rows that do not exist, so that
// each row is one load without a branch.
__device__ __align__(1024) uint16_t zero_row[D];

// The tile buffers themselves are two static LDS arrays of the kernel (see
// the direct row loads); these are the per-tile row data and the Sel cache.
struct Smem {
  float rscale[2][TILE];
  int rvalid[2][TILE];
  uint32_t vmask[2][4];  // direct rows: per buffer and wave, bit x = row 8w + x exists
  int32_t selc[SEL_CAP];  // sel[lat_beg ..] of this workgroup's latent rows
};

// 8 consecutive dims [8p, 8p+8) of a row as bf16 bits, by source format.
// Every E2M1 x E4M3 product and every E4M3 value is exactly a bf16 value.
__device__ __forceinline__ u32x4 bf16_piece(const uint16_t* row, int p) {
  return *reinterpret_cast<const u32x4*>(row + 8 * p);
}

__device__ __forceinline__ u32x4 fp8_codes_to_bf16(uint32_t c0, uint32_t c1) {
  const u32x2 c = {c0, c1};
  u32x4 v;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t w = c[h];
      v[2 * h + i] = e4m3_to_bf16((w >> (16 * i)) & 0xffu) |
                     (e4m3_to_bf16((w >> (16 * i + 8)) & 0xffu) << 16);
    }
  return v;
}

// raw NVFP4 piece: 4 code bytes (8 nibbles) and the group's E4M3 scale byte
__device__ __forceinline__ u32x4 nvfp4_piece(uint32_t codes, uint32_t scale_byte) {
  const float s = e4m3_to_f32(scale_byte);
  u32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t byte = (codes >> (8 * i)) & 0xffu;
    v[i] = (__float_as_uint(e2m1_to_f32(byte & 15u) * s) >> 16) |
           (__float_as_uint(e2m1_to_f32(byte >> 4) * s) & 0xffff0000u);
  }
  return v;
}

// One wave per SIMD: a wave's 16 heads x 512 fp32 accumulators, its 16 query
// heads (QK operands) and the next tile's rows take the register file.
// DIRECT (bf16 latents and window only): rows move straight from memory
// into a double-buffered LDS tile instead of through registers.  The two
// buffers are separate static arrays and the tile loop alternates between
// them at compile time, so the compiler can see that the rows loading into
// one are not the rows read from the other and does not wait for the next
// tile's loads before the current tile's reads (with one indexed array it
// did).  What it saves (the staging registers, the masking and LDS stores,
// one barrier per tile) pays off when a workgroup walks many tiles
// (prefill, 20 per query: 1.38 -> 1.13 ms), not when it walks a few (the
// row addresses come from the Sel cache one scalar read at a time: 1M
// decode, 2 tiles: 18.4 -> 20.4 us; 128K and verification decodes, 5:
// 25.7 -> 30.2 and 29.0 -> 32.8 us), so the launcher picks by tiles per
// split.
template <int LF, int WF, bool DIRECT>
__global__ __launch_bounds__(256, 1) void sparse_attn_kernel(AttnArgs a) {
  static_assert(!DIRECT || (LF == FMT_BF16 && WF == FMT_BF16), "direct rows are bf16 rows");
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Smem& sm = *reinterpret_cast<Smem*>(smem_raw);
  // the tile, row-major: QK operand, and PV operand via transpose reads.
  // Two separate arrays, so that the compiler can tell that the rows being
  // loaded straight into one (direct path) are not the rows read from the
  // other; the register path uses the first only.
  __shared__ __align__(16) uint16_t kvA[TILE][KV_LD];
  __shared__ __align__(16) uint16_t kvB[TILE][KV_LD];
  // direct path only: each wave's PV weights (its PV B operand as the lanes
  // hold it), the per-head rescale factors and flags of the last tile, and
  // the per-head output factors
  __shared__ __align__(16) bf16x8 pxch[4][64];
  __shared__ float alpha_x[HQ];
  __shared__ __align__(16) int resc_x[4];
  __shared__ float fin_x[HQ];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane & 15, g = lane >> 4;
  const int64_t r = blockIdx.x;  // query row b*Tq + j
  const int split = blockIdx.y;
  const int b = (int)(r / a.Tq), j = (int)(r % a.Tq);
  const int64_t t = a.q_pos[r];
  const int32_t* selrow = a.sel + r * a.sel_sb;
  const int n_tiles = a.tiles_lat + a.tiles_win;
  const int tile_beg = split * a.tiles_per_split;
  const int tile_end = min(n_tiles, tile_beg + a.tiles_per_split);

  // this workgroup's sel entries, loaded once before anything else: the
  // row gathers of later tiles then need no dependent global load
  const int lat_beg = TILE * tile_beg;
  const int n_lat = max(0, min(TILE * min(tile_end, a.tiles_lat), a.K) - lat_beg);
  int32_t sv[SEL_CAP / 256];
#pragma unroll
  for (int m = 0; m < SEL_CAP / 256; ++m) {
    const int idx = tid + 256 * m;
    sv[m] = idx < n_lat ? selrow[lat_beg + idx] : -1;
  }

  // this wave's 16 heads of the query as QK operands, held in registers for
  // all tiles (lane: head 16w + l%16, dims 32c + 8g .. +7), loaded straight
  // from memory (every lane 16 contiguous bytes of one head)
  bf16x8 qreg[16];
  {
    const uint16_t* qh = a.q + (int64_t)b * a.q_sb + ((int64_t)j * HQ + 16 * wave + hl) * D + 8 * g;
#pragma unroll
    for (int c = 0; c < 16; ++c) qreg[c] = *reinterpret_cast<const bf16x8*>(qh + 32 * c);
  }

#pragma unroll
  for (int m = 0; m < SEL_CAP / 256; ++m)
    if (tid + 256 * m < n_lat) sm.selc[tid + 256 * m] = sv[m];
  __syncthreads();
  const float scale2 = a.scale * LOG2E;
  // first window slot: raw position t - W + 1 modulo W_cap (later rows of
  // the window follow it, wrapping once at most since W <= W_cap)
  const int64_t w0 = t - (a.W - 1);
  const int wslot0 = (int)(((w0 % a.W_cap) + a.W_cap) % a.W_cap);
  // direct rows: source base addresses, and the zero row that rows which do
  // not exist are loaded from (their weights are masked to 0 as well)
  const uint64_t lat_base = (uint64_t)(uintptr_t)a.lat;
  const uint64_t win_base = (uint64_t)(uintptr_t)a.win;
  const uint64_t zero_base = (uint64_t)(uintptr_t)zero_row;

  f32x4 o[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) o[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  bool seen = false;  // any valid row so far (wave-uniform)

  // staging map: lane -> row quad rq (rows 4rq..4rq+3) and pieces p0, p0+32;
  // four consecutive lanes take four consecutive pieces of the same rows
  // (64 contiguous bytes per row)
  const int rq = (lane >> 2) & 7;
  const int p0 = (lane & 3) + 4 * (lane >> 5) + 8 * wave;

  // A tile's rows are gathered into registers one tile ahead: the loads of
  // tile i+1 are in flight while tile i is computed from LDS.
  // A tile's raw bytes are gathered into registers one tile ahead: the
  // loads of tile i+1 are in flight while tile i is computed from LDS.
  // Nothing reads them before stage() (decode and masking happen there), so
  // issuing them never waits on memory.
  struct Staged {
    u32x4 v[2][4];  // bf16: 8 values; FP8: .xy = 8 codes; NVFP4: .x = codes, .y = scale byte
    float rs[4];    // window token scale (FP8)
    int ok[4];
    bool lat;       // latent tile (else window)
  } nxt;
  // tile tt: rows 4rq .. 4rq+3 of this lane, pieces p0 and p0 + 32
  auto gather = [&](int tt, Staged& st) {
    st.lat = tt < a.tiles_lat;
    if (st.lat) {
      int64_t row[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int i = TILE * tt + 4 * rq + x;
        const int32_t gidx = i < a.K ? sm.selc[i - lat_beg] : -1;
        st.ok[x] = gidx >= 0 && gidx < a.n_cache;
        row[x] = (int64_t)b * a.lat_sb + (st.ok[x] ? gidx : 0);
        st.rs[x] = 1.0f;
      }
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int p = p0 + 32 * pp;
          if (LF == FMT_NVFP4) {
            const uint8_t* codes = static_cast<const uint8_t*>(a.lat) + row[x] * (D / 2);
            st.v[pp][x][0] = *reinterpret_cast<const uint32_t*>(codes + 4 * p);
            st.v[pp][x][1] = a.lat_scale[row[x] * (D / 16) + (p >> 1)];
          } else {
            st.v[pp][x] = bf16_piece(static_cast<const uint16_t*>(a.lat) + row[x] * D, p);
          }
        }
    } else {
      int64_t slot[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int jw = TILE * (tt - a.tiles_lat) + 4 * rq + x;
        st.ok[x] = jw < a.W && w0 + jw >= 0;
        int sl = wslot0 + jw;
        sl = sl >= a.W_cap ? sl - a.W_cap : sl;
        slot[x] = (int64_t)b * a.win_sb + (st.ok[x] ? sl : 0);
        st.rs[x] = WF == FMT_FP8 ? a.win_scale[slot[x]] : 1.0f;
      }
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int p = p0 + 32 * pp;
          if (WF == FMT_FP8) {
            const u32x2 c = *reinterpret_cast<const u32x2*>(
                static_cast<const uint8_t*>(a.win) + slot[x] * D + 8 * p);
            st.v[pp][x][0] = c[0];
            st.v[pp][x][1] = c[1];
          } else {
            st.v[pp][x] = bf16_piece(static_cast<const uint16_t*>(a.win) + slot[x] * D, p);
          }
        }
    }
  };
  // decode to bf16, zero the rows that do not exist
  auto decoded = [&](const Staged& st, int pp, int x) -> u32x4 {
    u32x4 v = st.v[pp][x];
    if (st.lat && LF == FMT_NVFP4) v = nvfp4_piece(v[0], v[1]);
    if (!st.lat && WF == FMT_FP8) v = fp8_codes_to_bf16(v[0], v[1]);
    return st.ok[x] ? v : (u32x4){0u, 0u, 0u, 0u};
  };
  auto stage = [&](const Staged& st) {
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      const int p = p0 + 32 * pp;
#pragma unroll
      for (int x = 0; x < 4; ++x)
        *reinterpret_cast<u32x4*>(&kvA[4 * rq + x][8 * p]) = decoded(st, pp, x);
    }
    if (wave == 0 && lane < 32 && (lane & 3) == 0) {  // one lane per row quad (rq = 0..7)
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        sm.rscale[0][4 * rq + x] = st.ok[x] ? st.rs[x] : 1.0f;
        sm.rvalid[0][4 * rq + x] = st.ok[x];
      }
    }
  };
  // bf16 caches: wave w moves rows 8w .. 8w+7 of tile tt straight from
  // memory into LDS buffer buf, one global_load_lds_dwordx4 per row (lane l
  // carries bytes 16l .. 16l+15 of the 1 KiB row, measured), with no
  // register staging; rows that do not exist are read from a row of zeros.
  // A row's source is the same for the whole wave (scalar registers).
  auto gather_direct = [&](int tt, uint16_t (*kvd)[KV_LD], int buf) {
    // lane x < 8 finds row 8w + x's source (one LDS read of the Sel cache
    // for the wave's 8 rows) and its full address -- the zero row when the
    // row does not exist, so every row is one load with no branch; the
    // addresses reach the scalar unit by v_readlane, so the row loads go
    // out back to back
    const bool lat_tile = tt < a.tiles_lat;
    const int rl0 = (TILE / 4) * wave + (lane & 7);
    bool okl;
    uint64_t raddr;
    if (lat_tile) {
      const int i = TILE * tt + rl0;
      const int32_t gidx = i < a.K ? sm.selc[i - lat_beg] : -1;
      okl = gidx >= 0 && gidx < a.n_cache;
      raddr = lat_base + (uint64_t)(b * a.lat_sb + (okl ? gidx : 0)) * (D * 2);
    } else {
      const int jw = TILE * (tt - a.tiles_lat) + rl0;
      okl = jw < a.W && w0 + jw >= 0;
      int sl = wslot0 + jw;
      sl = sl >= a.W_cap ? sl - a.W_cap : sl;
      raddr = win_base + (uint64_t)(b * a.win_sb + (okl ? sl : 0)) * (D * 2);
    }
    raddr = okl ? raddr : zero_base;
    const uint32_t mask = (uint32_t)__ballot(okl) & 0xffu;
    const uint32_t a_lo = (uint32_t)raddr, a_hi = (uint32_t)(raddr >> 32);
#pragma unroll
    for (int x = 0; x < TILE / 4; ++x) {
      // readlane returns a signed int: both halves go through uint32_t so
      // that the low half is zero-extended, not sign-extended into the high
      const uint64_t ra = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)a_lo, x) |
                          ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)a_hi, x) << 32);
      // Issued from asm: the compiler models this load as a pending flat LDS
      // access and would then force every LDS wait of the tile's QK^T to
      // zero; the loop waits for it explicitly (vmcnt(0), then a barrier).
      // The row address was just written to scalar registers by v_readlane,
      // and a memory instruction that reads them needs 5 wait states after
      // that write: s_mov + s_nop 4 give 6.
      const uint32_t ldsa = (uint32_t)(uintptr_t)&kvd[(TILE / 4) * wave + x][0];
      asm volatile(
          "s_mov_b32 m0, %0\n\t"
          "s_nop 4\n\t"
          "global_load_lds_dwordx4 %1, %2"
          :
          : "s"(ldsa), "v"(16u * (uint32_t)lane), "s"(ra)
          : "memory", "m0");
    }
    if (lane == 0) sm.vmask[buf][wave] = mask;
  };

  // PV operand addresses: ds_read_b64_tr_b16 works on 16-lane groups, lane
  // 4a + b of a group receiving, as its value j, element b of the four
  // 16-bit values addressed by lane 4j + a.  Lane (group g, 4j + a) therefore
  // addresses dims 16T + 4a .. +3 of row 4g + j (k-slots 0-3) and of row
  // 16 + 4g + j (k-slots 4-7), and every lane gets its dim's 8 rows.
  const int trj = (lane & 15) >> 2, tra = lane & 3;

  // one tile from LDS (kv, and its rows' scales and validity)
  auto tile_body = [&](const uint16_t (*kv)[KV_LD], const float* rscale, const int* rvalid,
                       int buf) {
    // direct rows (bf16, unit row scales): one validity word per tile
    uint32_t vm = 0;
    if constexpr (DIRECT)
      vm = sm.vmask[buf][0] | (sm.vmask[buf][1] << 8) | (sm.vmask[buf][2] << 16) |
           (sm.vmask[buf][3] << 24);
    const uint16_t* tr_lo = &kv[4 * g + trj][4 * tra];
    const uint16_t* tr_hi = &kv[16 + 4 * g + trj][4 * tra];

    // S^T = KV . Q^T for rows [16st, 16st+16): the two row halves are
    // independent accumulation chains; their K operands are read in pairs
    f32x4 s[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int c = 0; c < 16; c += 2) {
      bf16x8 kop[2][2];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int u = 0; u < 2; ++u)
          kop[st][u] = *reinterpret_cast<const bf16x8*>(&kv[16 * st + hl][32 * (c + u) + 8 * g]);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int st = 0; st < 2; ++st)
          s[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[st][u], qreg[c + u], s[st], 0, 0, 0);
    }
    // logits of rows 16st + 4g + i for head l%16
    float lg[2][4], rs[2][4];
    float mt = -INFINITY;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * st + 4 * g + i;
        if constexpr (DIRECT) {
          rs[st][i] = 1.0f;
          lg[st][i] = (vm >> row) & 1u ? s[st][i] * scale2 : -INFINITY;
        } else {
          rs[st][i] = rscale[row];
          lg[st][i] = rvalid[row] ? s[st][i] * scale2 * rs[st][i] : -INFINITY;
        }
        mt = fmaxf(mt, lg[st][i]);
      }
    mt = max_across_rows(mt);
    // row validity does not depend on the head, and the 64 lanes together
    // hold all 32 rows: the ballot is the same answer for the whole wave
    if constexpr (DIRECT) {
      seen |= vm != 0u;
    } else {
      bool mine = false;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) mine |= rvalid[16 * st + 4 * g + i] != 0;
      seen |= __ballot(mine) != 0;
    }
    if (!seen) return;
    // Lazy rescaling: m_run is a reference point, not necessarily the
    // running max; it moves only when a logit exceeds it by more than
    // RESCALE_TAU, so the weights stay below e^RESCALE_TAU and the
    // accumulators are rescaled rarely (never when the head had no row yet,
    // its accumulators being zero).  The sums are the same, each term
    // relative to the final reference.
    const bool grow = mt > m_run + RESCALE_TAU;
    const bool scale_acc = grow && m_run != -INFINITY;
    if (__ballot(scale_acc) != 0) {
      const float alpha = scale_acc ? __builtin_amdgcn_exp2f(m_run - mt) : 1.0f;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 32; ++i) o[i] *= alpha;
    }
    if (grow) m_run = mt;
    float psum = 0.f;
    bf16x8 pop;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(lg[st][i] - m_run);
        psum += p;
        pop[4 * st + i] = (__bf16)(p * rs[st][i]);
      }
    l_run += psum;
    // O^T += V^T . P^T ; A lane: dim 16T + l%16, k-slots = rows 4g..4g+3, 16+4g..16+4g+3,
    // read from the row-major tile by two LDS transpose reads (tr_lo, tr_hi);
    // operands read 4 MFMAs ahead so that LDS latency overlaps the MFMAs
#pragma unroll
    for (int T0 = 0; T0 < 32; T0 += 4) {
      bf16x8 vop[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) vop[u] = pv_operand(tr_lo + 16 * (T0 + u), tr_hi + 16 * (T0 + u));
#pragma unroll
      for (int u = 0; u < 4; ++u)
        o[T0 + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[u], pop, o[T0 + u], 0, 0, 0);
    }
  };

  // Direct path, PV split by dims: wave w still forms S^T and the softmax
  // weights of its 16 heads, publishes the weights (its PV B operand) in
  // LDS, and after one barrier computes O^T for dims 128w .. 128w+127 of all
  // 64 heads.  Each wave then reads a quarter of the tile through the
  // transpose reads instead of all of it: a workgroup reads 176 KB of LDS
  // per tile instead of 256.  o[4T + hb] is dims 128w + 16T + (rows of the
  // C layout) of heads 16hb + l%16.  The barrier only waits for LDS: the
  // next tile's row loads stay in flight across it.
  auto tile_body_ds = [&](const uint16_t (*kv)[KV_LD], int buf) {
    const uint32_t vm = sm.vmask[buf][0] | (sm.vmask[buf][1] << 8) |
                        (sm.vmask[buf][2] << 16) | (sm.vmask[buf][3] << 24);
    // vm is the same word in every wave, so this exit is workgroup-uniform
    seen |= vm != 0u;
    if (!seen) return;
    f32x4 s[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    // operands of chunk c + 1 are read before the MFMAs of chunk c
    bf16x8 kop[2][2];
#pragma unroll
    for (int st = 0; st < 2; ++st)
      kop[0][st] = *reinterpret_cast<const bf16x8*>(&kv[16 * st + hl][8 * g]);
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      if (c + 1 < 16) {
#pragma unroll
        for (int st = 0; st < 2; ++st)
          kop[(c + 1) & 1][st] =
              *reinterpret_cast<const bf16x8*>(&kv[16 * st + hl][32 * (c + 1) + 8 * g]);
      }
#pragma unroll
      for (int st = 0; st < 2; ++st)
        s[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[c & 1][st], qreg[c], s[st], 0, 0, 0);
    }
    float lg[2][4];
    float mt = -INFINITY;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * st + 4 * g + i;
        lg[st][i] = (vm >> row) & 1u ? s[st][i] * scale2 : -INFINITY;
        mt = fmaxf(mt, lg[st][i]);
      }
    mt = max_across_rows(mt);
    // lazy reference point as in the register path; the factor reaches the
    // other waves (which hold these heads' other dims) through LDS
    const bool grow = mt > m_run + RESCALE_TAU;
    const bool scale_acc = grow && m_run != -INFINITY;
    const float alpha = scale_acc ? __builtin_amdgcn_exp2f(m_run - mt) : 1.0f;
    const bool any = __ballot(scale_acc) != 0;
    if (any) l_run *= alpha;
    if (grow) m_run = mt;
    float psum = 0.f;
    bf16x8 pop;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pw = __builtin_amdgcn_exp2f(lg[st][i] - m_run);
        psum += pw;
        pop[4 * st + i] = (__bf16)pw;
      }
    l_run += psum;
    pxch[wave][lane] = pop;
    if (lane < 16) alpha_x[16 * wave + lane] = alpha;
    if (lane == 0) resc_x[wave] = any ? 1 : 0;
    // LDS-only barrier: wait for this wave's LDS writes, not for its
    // in-flight row loads (a __syncthreads would wait for those too)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt untouched
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const int4 rf = *reinterpret_cast<const int4*>(resc_x);
    if ((rf.x | rf.y | rf.z | rf.w) != 0) {
      const int rfa[4] = {rf.x, rf.y, rf.z, rf.w};
#pragma unroll
      for (int hb = 0; hb < 4; ++hb)
        if (rfa[hb]) {
          const float f = alpha_x[16 * hb + hl];
#pragma unroll
          for (int T = 0; T < 8; ++T) o[4 * T + hb] *= f;
        }
    }
    bf16x8 pb[4];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) pb[hb] = pxch[hb][lane];
    const uint16_t* tr_lo = &kv[4 * g + trj][4 * tra + 128 * wave];
    const uint16_t* tr_hi = &kv[16 + 4 * g + trj][4 * tra + 128 * wave];
#pragma unroll
    for (int T0 = 0; T0 < 8; T0 += 2) {
      bf16x8 vop[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) vop[u] = pv_operand(tr_lo + 16 * (T0 + u), tr_hi + 16 * (T0 + u));
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
          o[4 * (T0 + u) + hb] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[u], pb[hb], o[4 * (T0 + u) + hb], 0, 0, 0);
    }
  };

  if constexpr (DIRECT) {
    // two tiles per trip, one per buffer: each half reads a buffer that is
    // known at compile time while the next tile's rows load into the other
    if (tile_beg < tile_end) gather_direct(tile_beg, kvA, 0);
    for (int tt = tile_beg; tt < tile_end; tt += 2) {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's rows of tile tt are in
      __syncthreads();  // every wave's rows are in; kvB's readers (tile tt-1) are done
      if (tt + 1 < tile_end) gather_direct(tt + 1, kvB, 1);
      tile_body_ds(kvA, 0);
      if (tt + 1 >= tile_end) break;
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();  // tile tt+1 is in; kvA's readers (tile tt) are done
      if (tt + 2 < tile_end) gather_direct(tt + 2, kvA, 0);
      tile_body_ds(kvB, 1);
    }
  } else {
    if (tile_beg < tile_end) gather(tile_beg, nxt);
    for (int tt = tile_beg; tt < tile_end; ++tt) {
      __syncthreads();  // previous tile fully consumed
      stage(nxt);
      __syncthreads();
      if (tt + 1 < tile_end) gather(tt + 1, nxt);
      tile_body(kvA, sm.rscale[0], sm.rvalid[0], 0);
    }
  }

  // full row sum for this head (each lane group held a quarter of the rows)
  l_run = sum_across_rows(l_run);
  const int h = 16 * wave + hl;
  if constexpr (DIRECT) {
    // this wave holds dims 128w .. 128w+127 of every head; the reference
    // and sum of heads 16w .. 16w+15
    if (a.splits > 1) {
      float* pq = a.part + (r * a.splits + split) * HQ * PART;
#pragma unroll
      for (int hb = 0; hb < 4; ++hb)
#pragma unroll
        for (int T = 0; T < 8; ++T)
          *reinterpret_cast<f32x4*>(pq + (16 * hb + hl) * PART + 128 * wave + 16 * T + 4 * g) =
              o[4 * T + hb];
      if (g == 0) {
        pq[h * PART + D] = m_run;
        pq[h * PART + D + 1] = l_run;
      }
      return;
    }
    const float sk = a.sink[h] * LOG2E;
    const float M = fmaxf(m_run, sk);
    const float em = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - M);
    const float Z = l_run * em + __builtin_amdgcn_exp2f(sk - M);
    if (g == 0) fin_x[h] = em / Z;
    if (a.lse && g == 0) a.lse[r * HQ + h] = (M + __log2f(Z)) * LN2;
    __syncthreads();
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      const float f = fin_x[16 * hb + hl];
      uint16_t* orow = a.out + r * a.out_sb + (int64_t)(16 * hb + hl) * D + 128 * wave;
#pragma unroll
      for (int T = 0; T < 8; ++T) {
        u32x2 pk;
        pk[0] = pack_bf16x2(o[4 * T + hb][0] * f, o[4 * T + hb][1] * f);
        pk[1] = pack_bf16x2(o[4 * T + hb][2] * f, o[4 * T + hb][3] * f);
        *reinterpret_cast<u32x2*>(orow + 16 * T + 4 * g) = pk;
      }
    }
    return;
  }
  if (a.splits > 1) {
    float* pp = a.part + ((r * a.splits + split) * HQ + h) * PART;
#pragma unroll
    for (int T = 0; T < 32; ++T) *reinterpret_cast<f32x4*>(pp + 16 * T + 4 * g) = o[T];
    if (g == 0) {
      pp[D] = m_run;
      pp[D + 1] = l_run;
    }
    return;
  }
  const float sk = a.sink[h] * LOG2E;
  const float M = fmaxf(m_run, sk);
  const float em = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - M);
  const float Z = l_run * em + __builtin_amdgcn_exp2f(sk - M);
  const float f = em / Z;
  uint16_t* orow = a.out + r * a.out_sb + (int64_t)h * D;
#pragma unroll
  for (int T = 0; T < 32; ++T) {
    u32x2 pk;
    pk[0] = pack_bf16x2(o[T][0] * f, o[T][1] * f);
    pk[1] = pack_bf16x2(o[T][2] * f, o[T][3] * f);
    *reinterpret_cast<u32x2*>(orow + 16 * T + 4 * g) = pk;
  }
  if (a.lse && g == 0) a.lse[r * HQ + h] = (M + __log2f(Z)) * LN2;
}

// merge the split partials of one query: grid (R, 16), 256 threads =
// 4 heads x 64 threads x 8 dims.  The (reference, sum) pairs of all splits
// are read first, then the numerators in batches of MERGE_BATCH splits whose
// loads are all issued before any is used.
constexpr int MAX_SPLITS = 32;
constexpr int MERGE_BATCH = 8;
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  const int64_t r = blockIdx.x;
  const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int d0 = (threadIdx.x & 63) * 8;
  const float sk = a.sink[h] * LOG2E;  // the partials' references are base 2
  const float* part = a.part + (r * a.splits * HQ + h) * PART;  // split s at + s * HQ * PART
  float ms[MAX_SPLITS], ls[MAX_SPLITS];
#pragma unroll
  for (int s = 0; s < MAX_SPLITS; ++s) {
    ms[s] = -INFINITY;
    ls[s] = 0.f;
    if (s < a.splits) {
      ms[s] = part[(int64_t)s * HQ * PART + D];
      ls[s] = part[(int64_t)s * HQ * PART + D + 1];
    }
  }
  float M = sk;
#pragma unroll
  for (int s = 0; s < MAX_SPLITS; ++s) M = fmaxf(M, ms[s]);
  float Z = __builtin_amdgcn_exp2f(sk - M);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s0 = 0; s0 < MAX_SPLITS; s0 += MERGE_BATCH) {
    if (s0 >= a.splits) break;
    f32x4 x0[MERGE_BATCH], x1[MERGE_BATCH];
#pragma unroll
    for (int u = 0; u < MERGE_BATCH; ++u) {
      x0[u] = (f32x4){0.f, 0.f, 0.f, 0.f};
      x1[u] = x0[u];
      if (s0 + u < a.splits) {
        const float* pp = part + (int64_t)(s0 + u) * HQ * PART + d0;
        x0[u] = *reinterpret_cast<const f32x4*>(pp);
        x1[u] = *reinterpret_cast<const f32x4*>(pp + 4);
      }
    }
#pragma unroll
    for (int u = 0; u < MERGE_BATCH; ++u) {
      const int s = s0 + u;
      const float e = ms[s] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms[s] - M);
      Z += ls[s] * e;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i] += x0[u][i] * e;
        acc[4 + i] += x1[u][i] * e;
      }
    }
  }
  const float inv = 1.0f / Z;
  u32x4 pk;
#pragma unroll
  for (int i = 0; i < 4; ++i) pk[i] = pack_bf16x2(acc[2 * i] * inv, acc[2 * i + 1] * inv);
  *reinterpret_cast<u32x4*>(a.out + r * a.out_sb + (int64_t)h * D + d0) = pk;
  if (a.lse && (threadIdx.x & 63) == 0) a.lse[r * HQ + h] = (M + __log2f(Z)) * LN2;
}

}  // namespace

// Tiles of one query: latent tiles then window tiles (never mixed).
static int attn_tiles(int K, int W) { return (K + TILE - 1) / TILE + (W + TILE - 1) / TILE; }

// Tiles handled by one workgroup: many query rows -> one workgroup per
// query (no merge); few -> split the tiles so that roughly TARGET
// workgroups run, down to one tile each (each split costs a 128 KiB fp32
// partial that the merge reads back, but a workgroup's gathers all start at
// once, and one gather round is 2-4 us of latency on random latent rows).
// Measured: bf16 latents are fastest at ~128 workgroups (1M decode, 8
// queries: 10 splits of 2 tiles beat 20 of 1, 7 of 3 and 5 of 4; 40
// queries: 4 splits beat 7 and 2),
// NVFP4 latents, whose rows cost more to decode, at ~256.
static int attn_tiles_per_split(int64_t R, int K, int W, int lat_fmt) {
  const int tiles = attn_tiles(K, W);
  if (R >= 192 || tiles <= 1) return tiles > 0 ? tiles : 1;
  const int64_t target = lat_fmt == FMT_NVFP4 ? 256 : 128;
  const int64_t want = (target + R - 1) / R;  // splits wanted per query
  int tps = (int)((tiles + want - 1) / want);
  if (tps < 1) tps = 1;
  if ((tiles + tps - 1) / tps > MAX_SPLITS) tps = (tiles + MAX_SPLITS - 1) / MAX_SPLITS;
  return tps;
}

int attn_splits(int64_t R, int K, int W, int lat_fmt) {
  const int tiles = attn_tiles(K, W);
  const int tps = attn_tiles_per_split(R, K, W, lat_fmt);
  const int s = (tiles + tps - 1) / tps;
  return s < 1 ? 1 : s;
}

// split partials of one call in a given latent format (0 when unsplit)
size_t attn_workspace_bytes_fmt(int64_t R, int K, int W, int lat_fmt) {
  const int s = attn_splits(R, K, W, lat_fmt);
  if (s <= 1) return 0;
  return (size_t)R * s * HQ * PART * sizeof(float);
}

// the larger of the two formats' needs: the workspace query has no format
size_t attn_workspace_bytes(int64_t R, int K, int W) {
  return std::max(attn_workspace_bytes_fmt(R, K, W, FMT_BF16),
                  attn_workspace_bytes_fmt(R, K, W, FMT_NVFP4));
}

// Scratch of the allocation-free entry point: a fixed array in device
// memory that every GPU the library runs on holds until the process ends.
// In host code the array's name is only a stand-in (passing it to a kernel
// would fault): its device address is looked up once per device with
// hipGetSymbolAddress and that address is what kernels receive.
static __device__ __align__(256) unsigned char scratch[ATTN_SCRATCH_BYTES];
static std::atomic<void*> scratch_addr[kMaxDevices];

hipError_t attn_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // with this device current: each device has its own copy of the array
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    scratch_addr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

hipError_t launch_sparse_attn(int B, int Tq, const void* q, int64_t q_sb, const void* lat,
                              int lat_fmt, const void* lat_scale, int64_t lat_sb, int64_t n_cache,
                              const int32_t* sel, int K, int64_t sel_sb, const void* win,
                              int win_fmt, const float* win_scale, int W, int W_cap,
                              int64_t win_sb, const int64_t* q_pos, const float* sink,
                              float scale, void* out, int64_t out_sb, float* lse, void* ws,
                              hipStream_t s) {
  const int64_t R = (int64_t)B * Tq;
  const int splits = attn_splits(R, K, W, lat_fmt);
  const int tiles_per_split = attn_tiles_per_split(R, K, W, lat_fmt);
  // with an empty cache no latent row exists: its tiles are dropped (they
  // would only be masked rows, and the cache pointer may be null)
  const int tiles_lat = n_cache > 0 ? (K + TILE - 1) / TILE : 0;
  const int tiles_win = (W + TILE - 1) / TILE;
  AttnArgs a{(const uint16_t*)q, q_sb, Tq, lat, lat_fmt, (const uint8_t*)lat_scale, lat_sb,
             n_cache, sel, K, sel_sb, win, win_fmt, win_scale, W, W_cap, win_sb, q_pos, sink,
             scale, (uint16_t*)out, out_sb, lse, (float*)ws, splits, tiles_lat, tiles_win,
             tiles_per_split};
  // the dynamic LDS limit is raised once per device and kernel
  static std::atomic<int> attr_set[kMaxDevices];
  int dev = 0;
  hipError_t e0 = hipGetDevice(&dev);
  if (e0 != hipSuccess) return e0;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  const void* kernels[5] = {(const void*)sparse_attn_kernel<FMT_BF16, FMT_BF16, true>,
                            (const void*)sparse_attn_kernel<FMT_BF16, FMT_BF16, false>,
                            (const void*)sparse_attn_kernel<FMT_BF16, FMT_FP8, false>,
                            (const void*)sparse_attn_kernel<FMT_NVFP4, FMT_BF16, false>,
                            (const void*)sparse_attn_kernel<FMT_NVFP4, FMT_FP8, false>};
  if (!attr_set[dev].load(std::memory_order_acquire)) {
    for (const void* k : kernels) {
      e0 = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(Smem));
      if (e0 != hipSuccess) return e0;
    }
    attr_set[dev].store(1, std::memory_order_release);
  }
  const dim3 grid((unsigned)R, (unsigned)splits), block(256);
  const bool lat4 = lat_fmt == FMT_NVFP4, win8 = win_fmt == FMT_FP8;
  if (!lat4 && !win8 && tiles_per_split >= DIRECT_MIN_TILES)
    hipLaunchKernelGGL((sparse_attn_kernel<FMT_BF16, FMT_BF16, true>), grid, block, sizeof(Smem), s, a);
  else if (!lat4 && !win8)
    hipLaunchKernelGGL((sparse_attn_kernel<FMT_BF16, FMT_BF16, false>), grid, block, sizeof(Smem), s, a);
  else if (!lat4)
    hipLaunchKernelGGL((sparse_attn_kernel<FMT_BF16, FMT_FP8, false>), grid, block, sizeof(Smem), s, a);
  else if (!win8)
    hipLaunchKernelGGL((sparse_attn_kernel<FMT_NVFP4, FMT_BF16, false>), grid, block, sizeof(Smem), s, a);
  else
    hipLaunchKernelGGL((sparse_attn_kernel<FMT_NVFP4, FMT_FP8, false>), grid, block, sizeof(Smem), s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)R, HQ / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace csa2
