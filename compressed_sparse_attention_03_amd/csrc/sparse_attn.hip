// sparse_attn.hip -- a6, CSA2 sparse attention (NVFP4 article, sections 3,
// 3.1 and 3.4): for every query, the 64 heads attend over the selected
// compressed latents plus the raw sliding window, K = V = the 512-wide
// latent row, in one pass with an online softmax whose denominator also holds
// a learnable per-head sink logit.
//
// Work decomposition.  A workgroup (4 waves) owns one query and a contiguous
// range of its row list (i < K: latent sel[i]; K <= i < K+W: window positions
// t-W+1 .. t).  Few queries (decode) -> the row list is split over several
// workgroups and a second kernel merges the partial (max, sum, numerator)
// triples; many queries (prefill) -> one workgroup per query, no merge.
//
// Per tile of 32 rows:
//   * every row is gathered from HBM once (1 KiB bf16, or 256 B NVFP4 codes +
//     32 B scales, or 512 B FP8 + a row scale), dequantised in registers to
//     bf16 (exact: E2M1 x E4M3 and E4M3 values are all bf16 values) and
//     stored to LDS twice: row-major (the K operand) and transposed (the V
//     operand), so the same bytes feed both contractions;
//   * wave w handles heads 16w..16w+15:
//       S^T = KV . Q^T  (v_mfma_f32_16x16x32_bf16, rows x heads, K = 512)
//     which leaves each lane with a single head (l%16) and 8 of the rows,
//     so the softmax statistics stay per lane; then
//       O^T += V^T . P^T (dims x heads, K = 32 rows)
//     whose B operand is exactly the P values the lane already holds.
// FP8 window rows keep their per-token scale out of the MFMA: it multiplies
// the logit of that row and its P weight.
#include "device_common.h"
#include "launch.h"

namespace csa2 {

namespace {

constexpr int TILE = 32;            // rows per tile
constexpr int KV_LD = D + 8;        // bf16 per row-major LDS row (1040 B)
constexpr int VT_LD = TILE + 4;     // bf16 per transposed LDS row (72 B)
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
  int rows_per_split;
};

struct Smem {
  uint16_t kv[TILE][KV_LD];
  uint16_t vt[D][VT_LD];
  float rscale[TILE];
  int rvalid[TILE];
};

struct RowSrc {
  const void* base;  // row start (codes)
  const uint8_t* sc; // NVFP4 group scales of the row
  float rscale;      // FP8 window token scale, else 1
  int fmt;           // 0 = no row
};

__device__ __forceinline__ RowSrc row_source(const AttnArgs& a, int b, int64_t t,
                                             const int32_t* selrow, int i, int row_end) {
  RowSrc r{nullptr, nullptr, 1.0f, 0};
  if (i >= row_end) return r;
  if (i < a.K) {
    const int32_t gidx = selrow[i];
    if (gidx < 0 || gidx >= a.n_cache) return r;
    const int64_t row = (int64_t)b * a.lat_sb + gidx;
    if (a.lat_fmt == FMT_NVFP4) {
      r.base = static_cast<const uint8_t*>(a.lat) + row * (D / 2);
      r.sc = a.lat_scale + row * (D / 16);
    } else {
      r.base = static_cast<const uint16_t*>(a.lat) + row * D;
    }
    r.fmt = a.lat_fmt;
    return r;
  }
  const int64_t pos = t - (a.W - 1) + (i - a.K);
  if (pos < 0) return r;
  const int64_t slot = (int64_t)b * a.win_sb + pos % a.W_cap;
  if (a.win_fmt == FMT_FP8) {
    r.base = static_cast<const uint8_t*>(a.win) + slot * D;
    r.rscale = a.win_scale[slot];
  } else {
    r.base = static_cast<const uint16_t*>(a.win) + slot * D;
  }
  r.fmt = a.win_fmt;
  return r;
}

// 8 consecutive dims [8p, 8p+8) of a row as bf16 bits (scale of FP8 rows not applied)
__device__ __forceinline__ u32x4 load_piece(const RowSrc& r, int p) {
  u32x4 v = {0u, 0u, 0u, 0u};
  if (r.fmt == FMT_BF16) {
    v = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(r.base) + 8 * p);
  } else if (r.fmt == FMT_FP8) {
    const u32x2 c = *reinterpret_cast<const u32x2*>(static_cast<const uint8_t*>(r.base) + 8 * p);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t w = c[h];
        v[2 * h + i] = e4m3_to_bf16((w >> (16 * i)) & 0xffu) |
                       (e4m3_to_bf16((w >> (16 * i + 8)) & 0xffu) << 16);
      }
  } else if (r.fmt == FMT_NVFP4) {
    const uint32_t c = *reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(r.base) + 4 * p);
    const float s = e4m3_to_f32(r.sc[p >> 1]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t byte = (c >> (8 * i)) & 0xffu;
      // products of an E2M1 value and an E4M3 scale are exact in bf16
      v[i] = (__float_as_uint(e2m1_to_f32(byte & 15u) * s) >> 16) |
             (__float_as_uint(e2m1_to_f32(byte >> 4) * s) & 0xffff0000u);
    }
  }
  return v;
}

// One wave per SIMD: the 64 heads x 512 fp32 accumulators, the query
// operand and the next tile's rows take more than half of the register file.
__global__ __launch_bounds__(256, 1) void sparse_attn_kernel(AttnArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Smem& sm = *reinterpret_cast<Smem*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane & 15, g = lane >> 4;
  const int64_t r = blockIdx.x;  // query row b*Tq + j
  const int split = blockIdx.y;
  const int b = (int)(r / a.Tq), j = (int)(r % a.Tq);
  const int64_t t = a.q_pos[r];
  const int32_t* selrow = a.sel + r * a.sel_sb;
  const int n_rows = a.K + a.W;
  const int row_beg = split * a.rows_per_split;
  const int row_end = min(n_rows, row_beg + a.rows_per_split);

  // Q^T operand of this wave's 16 heads: lane holds head 16w + l%16,
  // dims 32c + 8g .. +7 for c = 0..15
  const uint16_t* qrow = a.q + (int64_t)b * a.q_sb + ((int64_t)j * HQ + 16 * wave + hl) * D;
  bf16x8 qop[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) qop[c] = *reinterpret_cast<const bf16x8*>(qrow + 32 * c + 8 * g);

  f32x4 o[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) o[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  bool seen = false;  // any valid row so far (wave-uniform)

  // staging map: lane -> row quad rq (rows 4rq..4rq+3) and pieces p0, p0+32
  const int rq = lane & 7;
  const int p0 = (lane >> 3) + 8 * wave;

  // A tile's rows are gathered into registers one tile ahead: the loads of
  // tile i+1 are in flight while tile i is computed from LDS.
  struct Staged {
    u32x4 v[2][4];
    float rs[4];
    int ok[4];
  } nxt;
  auto gather = [&](int i0, Staged& st) {
    RowSrc src[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) src[x] = row_source(a, b, t, selrow, i0 + 4 * rq + x, row_end);
#pragma unroll
    for (int pp = 0; pp < 2; ++pp)
#pragma unroll
      for (int x = 0; x < 4; ++x) st.v[pp][x] = load_piece(src[x], p0 + 32 * pp);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      st.rs[x] = src[x].rscale;
      st.ok[x] = src[x].fmt != 0;
    }
  };
  auto stage = [&](const Staged& st) {
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      const int p = p0 + 32 * pp;
#pragma unroll
      for (int x = 0; x < 4; ++x) *reinterpret_cast<u32x4*>(&sm.kv[4 * rq + x][8 * p]) = st.v[pp][x];
      // transpose: dim 8p+d gets the four rows' values side by side
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const int w32 = d >> 1, sh = 16 * (d & 1);
        u32x2 pr;
        pr[0] = ((st.v[pp][0][w32] >> sh) & 0xffffu) | (((st.v[pp][1][w32] >> sh) & 0xffffu) << 16);
        pr[1] = ((st.v[pp][2][w32] >> sh) & 0xffffu) | (((st.v[pp][3][w32] >> sh) & 0xffffu) << 16);
        *reinterpret_cast<u32x2*>(&sm.vt[8 * p + d][4 * rq]) = pr;
      }
    }
    if (wave == 0 && (lane >> 3) == 0) {
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        sm.rscale[4 * rq + x] = st.rs[x];
        sm.rvalid[4 * rq + x] = st.ok[x];
      }
    }
  };

  if (row_beg < row_end) gather(row_beg, nxt);
  for (int i0 = row_beg; i0 < row_end; i0 += TILE) {
    __syncthreads();  // previous tile fully consumed
    stage(nxt);
    __syncthreads();
    if (i0 + TILE < row_end) gather(i0 + TILE, nxt);

    // S^T = KV . Q^T for rows [16st, 16st+16)
    f32x4 s[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const bf16x8 kop = *reinterpret_cast<const bf16x8*>(&sm.kv[16 * st + hl][32 * c + 8 * g]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[c], acc, 0, 0, 0);
      }
      s[st] = acc;
    }
    // logits of rows 16st + 4g + i for head l%16
    float lg[2][4], rs[2][4];
    float mt = -INFINITY;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * st + 4 * g + i;
        rs[st][i] = sm.rscale[row];
        lg[st][i] = sm.rvalid[row] ? s[st][i] * a.scale * rs[st][i] : -INFINITY;
        mt = fmaxf(mt, lg[st][i]);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    // row validity does not depend on the head, and the 64 lanes together
    // hold all 32 rows: the ballot is the same answer for the whole wave
    bool mine = false;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) mine |= sm.rvalid[16 * st + 4 * g + i] != 0;
    seen |= __ballot(mine) != 0;
    if (!seen) continue;
    const float m_new = fmaxf(m_run, mt);
    const float alpha = m_run == -INFINITY ? 0.f : expf(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
    bf16x8 pop;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = expf(lg[st][i] - m_new);
        psum += p;
        pop[4 * st + i] = (__bf16)(p * rs[st][i]);
      }
    l_run = l_run * alpha + psum;
    if (alpha != 1.0f) {
#pragma unroll
      for (int i = 0; i < 32; ++i) o[i] *= alpha;
    }
    // O^T += V^T . P^T ; A lane: dim 16T + l%16, k-slots = rows 4g..4g+3, 16+4g..16+4g+3
#pragma unroll
    for (int T = 0; T < 32; ++T) {
      const u32x2 lo = *reinterpret_cast<const u32x2*>(&sm.vt[16 * T + hl][4 * g]);
      const u32x2 hi = *reinterpret_cast<const u32x2*>(&sm.vt[16 * T + hl][16 + 4 * g]);
      const u32x4 vv = {lo[0], lo[1], hi[0], hi[1]};
      const bf16x8 vop = __builtin_bit_cast(bf16x8, vv);
      o[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop, o[T], 0, 0, 0);
    }
  }

  // full row sum for this head (each lane group held a quarter of the rows)
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  const int h = 16 * wave + hl;
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
  const float sk = a.sink[h];
  const float M = fmaxf(m_run, sk);
  const float em = m_run == -INFINITY ? 0.f : expf(m_run - M);
  const float Z = l_run * em + expf(sk - M);
  const float f = em / Z;
  uint16_t* orow = a.out + r * a.out_sb + (int64_t)h * D;
#pragma unroll
  for (int T = 0; T < 32; ++T) {
    u32x2 pk;
    pk[0] = pack_bf16x2(o[T][0] * f, o[T][1] * f);
    pk[1] = pack_bf16x2(o[T][2] * f, o[T][3] * f);
    *reinterpret_cast<u32x2*>(orow + 16 * T + 4 * g) = pk;
  }
  if (a.lse && g == 0) a.lse[r * HQ + h] = M + logf(Z);
}

// merge the split partials of one query: grid (R, 16), 256 threads =
// 4 heads x 64 threads x 8 dims.  All of a thread's partial loads are issued
// before any is used (splits are at most MAX_SPLITS).
constexpr int MAX_SPLITS = 16;
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  const int64_t r = blockIdx.x;
  const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int d0 = (threadIdx.x & 63) * 8;
  const float sk = a.sink[h];
  float ms[MAX_SPLITS], ls[MAX_SPLITS];
  f32x4 x0[MAX_SPLITS], x1[MAX_SPLITS];
#pragma unroll
  for (int s = 0; s < MAX_SPLITS; ++s) {
    if (s < a.splits) {
      const float* pp = a.part + ((r * a.splits + s) * HQ + h) * PART;
      ms[s] = pp[D];
      ls[s] = pp[D + 1];
      x0[s] = *reinterpret_cast<const f32x4*>(pp + d0);
      x1[s] = *reinterpret_cast<const f32x4*>(pp + d0 + 4);
    } else {
      ms[s] = -INFINITY;
      ls[s] = 0.f;
      x0[s] = (f32x4){0.f, 0.f, 0.f, 0.f};
      x1[s] = x0[s];
    }
  }
  float M = sk;
#pragma unroll
  for (int s = 0; s < MAX_SPLITS; ++s) M = fmaxf(M, ms[s]);
  float Z = expf(sk - M);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < MAX_SPLITS; ++s) {
    const float e = ms[s] == -INFINITY ? 0.f : expf(ms[s] - M);
    Z += ls[s] * e;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[i] += x0[s][i] * e;
      acc[4 + i] += x1[s][i] * e;
    }
  }
  const float inv = 1.0f / Z;
  u32x4 pk;
#pragma unroll
  for (int i = 0; i < 4; ++i) pk[i] = pack_bf16x2(acc[2 * i] * inv, acc[2 * i + 1] * inv);
  *reinterpret_cast<u32x4*>(a.out + r * a.out_sb + (int64_t)h * D + d0) = pk;
  if (a.lse && (threadIdx.x & 63) == 0) a.lse[r * HQ + h] = M + logf(Z);
}

}  // namespace

// Tiles of 32 rows handled by one workgroup: many query rows -> one
// workgroup per query (no merge); few -> split the row list so that roughly
// 256+ workgroups run, at least 2 tiles each (each split costs a 128 KiB
// fp32 partial that the merge reads back).
static int attn_tiles_per_split(int64_t R, int n_rows) {
  const int tiles = (n_rows + TILE - 1) / TILE;
  if (R >= 192 || tiles <= 2) return tiles > 0 ? tiles : 1;
  const int64_t want = (256 + R - 1) / R;  // splits wanted per query
  int tps = (int)((tiles + want - 1) / want);
  if (tps < 2) tps = 2;
  if ((tiles + tps - 1) / tps > MAX_SPLITS) tps = (tiles + MAX_SPLITS - 1) / MAX_SPLITS;
  return tps;
}

int attn_splits(int64_t R, int n_rows) {
  const int tiles = (n_rows + TILE - 1) / TILE;
  const int tps = attn_tiles_per_split(R, n_rows);
  const int s = (tiles + tps - 1) / tps;
  return s < 1 ? 1 : s;
}

size_t attn_workspace_bytes(int64_t R, int n_rows) {
  const int s = attn_splits(R, n_rows);
  if (s <= 1) return 0;
  return (size_t)R * s * HQ * PART * sizeof(float);
}

hipError_t launch_sparse_attn(int B, int Tq, const void* q, int64_t q_sb, const void* lat,
                              int lat_fmt, const void* lat_scale, int64_t lat_sb, int64_t n_cache,
                              const int32_t* sel, int K, int64_t sel_sb, const void* win,
                              int win_fmt, const float* win_scale, int W, int W_cap,
                              int64_t win_sb, const int64_t* q_pos, const float* sink,
                              float scale, void* out, int64_t out_sb, float* lse, void* ws,
                              hipStream_t s) {
  const int64_t R = (int64_t)B * Tq;
  const int n_rows = K + W;
  const int splits = attn_splits(R, n_rows);
  const int tiles_per_split = attn_tiles_per_split(R, n_rows);
  AttnArgs a{(const uint16_t*)q, q_sb, Tq, lat, lat_fmt, (const uint8_t*)lat_scale, lat_sb,
             n_cache, sel, K, sel_sb, win, win_fmt, win_scale, W, W_cap, win_sb, q_pos, sink,
             scale, (uint16_t*)out, out_sb, lse, (float*)ws, splits, tiles_per_split * TILE};
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)sparse_attn_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(Smem));
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(sparse_attn_kernel, dim3((unsigned)R, (unsigned)splits), dim3(256),
                     sizeof(Smem), s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)R, HQ / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace csa2
