// select_topk.hip -- a3 / a5, the two top-k stages of CSA2 selection (NVFP4
// article, section 3.3): block level (top-K_b blocks by their in-block
// maximum, the newest block always kept) and position level (top-K latents
// of the candidate blocks).
//
// One 1024-thread workgroup per row:
//   1. a stats pass turns every score into an order-preserving uint32 key
//      (larger score -> larger key; invalid entries -> 0), counts the valid
//      entries, finds the forced entry and the min / max key;
//   2. radix select finds the k-th largest key T among the non-forced valid
//      entries, 8 bits per pass, starting below the bits every key shares
//      (the common prefix of min and max), so integer-valued scores usually
//      finish in 2-3 passes.  Histograms live in LDS; each wave first adds its
//      most common digit with one atomic (ballot + popcount), which removes
//      the same-address atomic pile-up of concentrated score ranges;
//   3. an ordered compaction keeps every key > T, the first (k - #(> T))
//      keys == T in column order (ties -> smaller id, as ids increase with
//      the column), and the forced entry, and writes their ids ascending.
// Everything is integer work: the result is deterministic and bit-exact.
#include "device_common.h"
#include "launch.h"

namespace csa2 {

namespace {

constexpr int THREADS = 1024;
constexpr int NWAVES = THREADS / 64;

struct SelArgs {
  const float* scores;
  int64_t s_stride;
  const int32_t* ids;
  int64_t id_stride;
  const int32_t* forced;
  int force_last;
  int64_t n;
  int k;
  int32_t* out;
  int64_t o_stride;
};

__device__ __forceinline__ uint32_t order_key(float s) {
  const uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct Elem {
  uint32_t key;  // 0 = invalid
  int32_t id;
};

__device__ __forceinline__ Elem load_elem(const SelArgs& a, int64_t row, int64_t j) {
  const float s = a.scores[row * a.s_stride + j];
  const int32_t id = a.ids ? a.ids[row * a.id_stride + j] : (int32_t)j;
  Elem e;
  e.id = id;
  const bool ok = id >= 0 && !(s != s) && s != -INFINITY;
  e.key = ok ? order_key(s) : 0u;
  return e;
}

struct Shared {
  uint32_t hist[256];
  uint32_t wred[NWAVES * 4];
  uint32_t scan[NWAVES];
  uint32_t bcast[8];
};

// exclusive block scan of one uint32 per thread
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, Shared& sh, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh.scan[wave] = x;
  __syncthreads();
  uint32_t wpre = 0, tot = 0;
  for (int i = 0; i < NWAVES; ++i) {
    const uint32_t t = sh.scan[i];
    if (i < wave) wpre += t;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return wpre + x - v;
}

}  // namespace

__global__ __launch_bounds__(THREADS) void select_topk_kernel(SelArgs a) {
  __shared__ Shared sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const int64_t n = a.n;
  const int32_t fid = a.forced ? a.forced[row] : -1;

  // ---- 1. stats ------------------------------------------------------------
  uint32_t cnt = 0, kmin = 0xffffffffu, kmax = 0u;
  int64_t fcol = -1;  // forced column candidate (max over lanes)
  for (int64_t j = tid; j < n; j += THREADS) {
    const Elem e = load_elem(a, row, j);
    if (e.key) {
      ++cnt;
      kmin = min(kmin, e.key);
      kmax = max(kmax, e.key);
      if (a.force_last) fcol = j;  // increasing j: the last one wins
      else if (fid >= 0 && e.id == fid && fcol < 0) fcol = j;
    }
  }
  // block reductions: sum cnt, min kmin, max kmax, forced column
  {
    int fc = (int)fcol;  // n <= 2^24
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      cnt += __shfl_xor(cnt, o, 64);
      kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o, 64));
      kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
      const int other = __shfl_xor(fc, o, 64);
      if (a.force_last) fc = max(fc, other);
      else fc = (fc < 0) ? other : (other < 0 ? fc : min(fc, other));
    }
    if (lane == 0) {
      sh.wred[wave * 4 + 0] = cnt;
      sh.wred[wave * 4 + 1] = kmin;
      sh.wred[wave * 4 + 2] = kmax;
      sh.wred[wave * 4 + 3] = (uint32_t)fc;
    }
    __syncthreads();
    cnt = 0;
    kmin = 0xffffffffu;
    kmax = 0;
    fc = -1;
    for (int i = 0; i < NWAVES; ++i) {
      cnt += sh.wred[i * 4 + 0];
      kmin = min(kmin, sh.wred[i * 4 + 1]);
      kmax = max(kmax, sh.wred[i * 4 + 2]);
      const int other = (int)sh.wred[i * 4 + 3];
      if (a.force_last) fc = max(fc, other);
      else fc = (fc < 0) ? other : (other < 0 ? fc : min(fc, other));
    }
    fcol = fc;
    __syncthreads();
  }
  const int have_forced = fcol >= 0 ? 1 : 0;
  const uint32_t k_rem = (uint32_t)(a.k - have_forced);
  const uint32_t n_rest = cnt - (uint32_t)have_forced;

  // ---- 2. threshold key T and how many keys == T to take ------------------
  uint32_t T = 0, take_eq = 0;  // T = 0: every valid entry is kept
  if (k_rem == 0) {
    T = 0xffffffffu;  // above every valid key: only the forced entry stays
  } else if (n_rest > k_rem) {
    uint32_t prefix = 0, remaining = k_rem;
    int hi = (kmin == kmax) ? 0 : 32 - __clz(kmin ^ kmax);
    prefix = hi >= 32 ? 0u : (kmax & ~((1u << hi) - 1u));
    while (hi > 0) {
      const int lo = hi > 8 ? hi - 8 : 0;
      const uint32_t dmask = (1u << (hi - lo)) - 1u;
      for (int i = tid; i < 256; i += THREADS) sh.hist[i] = 0;
      __syncthreads();
      for (int64_t base = 0; base < n; base += THREADS) {
        const int64_t j = base + tid;
        bool act = false;
        uint32_t d = 0;
        if (j < n && j != fcol) {
          const Elem e = load_elem(a, row, j);
          const bool match = hi >= 32 ? true : ((e.key >> hi) == (prefix >> hi));
          act = e.key != 0 && match;
          d = (e.key >> lo) & dmask;
        }
        const uint64_t am = __ballot(act);
        if (am) {
          const int leader = __ffsll((unsigned long long)am) - 1;
          const uint32_t ld = (uint32_t)__shfl((int)d, leader, 64);
          const uint64_t same = __ballot(act && d == ld);
          if (lane == leader) atomicAdd(&sh.hist[ld], (uint32_t)__popcll(same));
          if (act && d != ld) atomicAdd(&sh.hist[d], 1u);
        }
      }
      __syncthreads();
      if (wave == 0) {
        uint32_t c[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) c[i] = sh.hist[4 * lane + i];
        const uint32_t tot = c[0] + c[1] + c[2] + c[3];
        uint32_t suf = tot;  // sum over lanes >= this lane
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const uint32_t y = __shfl_down(suf, o, 64);
          if (lane + o < 64) suf += y;
        }
        const uint32_t above = suf - tot;
        if (above < remaining && remaining <= suf) {
          uint32_t acc = above;
          for (int i = 3; i >= 0; --i) {
            if (acc + c[i] >= remaining) {
              sh.bcast[0] = 4u * lane + i;
              sh.bcast[1] = acc;
              break;
            }
            acc += c[i];
          }
        }
      }
      __syncthreads();
      const uint32_t dsel = sh.bcast[0];
      remaining -= sh.bcast[1];
      prefix |= dsel << lo;
      hi = lo;
      __syncthreads();
    }
    T = prefix;
    take_eq = remaining;
  }

  // ---- 3. ordered compaction ---------------------------------------------
  const int64_t chunk = (n + THREADS - 1) / THREADS;
  const int64_t c0 = (int64_t)tid * chunk;
  const int64_t c1 = min(n, c0 + chunk);
  uint32_t n_eq = 0, n_gt = 0, n_f = 0;
  for (int64_t j = c0; j < c1; ++j) {
    if (j == fcol) {
      n_f = 1;
      continue;
    }
    const uint32_t key = load_elem(a, row, j).key;
    if (key == 0) continue;
    n_gt += key > T;
    n_eq += key == T;
  }
  uint32_t tot;
  const uint32_t eq_before = block_exclusive_scan(n_eq, sh, &tot);
  const uint32_t take_here =
      take_eq > eq_before ? min(take_eq - eq_before, n_eq) : 0u;
  uint32_t n_sel_total;
  uint32_t off = block_exclusive_scan(n_gt + take_here + n_f, sh, &n_sel_total);
  int32_t* orow = a.out + row * a.o_stride;
  uint32_t eq_seen = 0;
  for (int64_t j = c0; j < c1; ++j) {
    const Elem e = load_elem(a, row, j);
    bool keep;
    if (j == fcol) {
      keep = true;
    } else if (e.key == 0) {
      keep = false;
    } else if (e.key > T) {
      keep = true;
    } else if (e.key == T) {
      keep = eq_seen < take_here;
      ++eq_seen;
    } else {
      keep = false;
    }
    if (keep && off < (uint32_t)a.k) orow[off++] = e.id;
  }
  for (int64_t j = (int64_t)n_sel_total + tid; j < a.k; j += THREADS) orow[j] = -1;
}

hipError_t launch_select_topk(int R, int64_t n, const float* scores, int64_t s_stride,
                              const int32_t* ids, int64_t id_stride, const int32_t* forced,
                              int force_last, int k, int32_t* out, int64_t o_stride,
                              hipStream_t s) {
  SelArgs a{scores, s_stride, ids, id_stride, forced, force_last, n, k, out, o_stride};
  hipLaunchKernelGGL(select_topk_kernel, dim3((unsigned)R), dim3(THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace csa2
