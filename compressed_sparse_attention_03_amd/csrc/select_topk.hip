// select_topk.hip -- a3 / a5, the two top-k stages of CSA2 selection (NVFP4
// article, section 3.3): block level (top-K_b blocks by their in-block
// maximum, the newest block always kept) and position level (top-K latents
// of the candidate blocks).  Ranking key: (score descending, id ascending).
//
// Scores become order-preserving uint32 keys (larger score -> larger key;
// invalid entries -> 0).  One workgroup of 1024 threads owns a row.
//
// Sampled path (8192 <= n <= 2^18, k <= 2048: both decode stages).  A
// histogram of 2048 keys spread evenly over the row brackets the k-th key
// with a wide margin (4 sigma of the sample rank + 16).  ONE coalesced pass
// over the row then splits it into "certainly in" (key above the bracket,
// column list) and "candidate" (key inside the bracket, (key, column) list);
// everything else is out.  If #in <= k <= #in + #candidates the answer is
// the "in" list plus the best candidates, found by an exact radix select on
// the unique (key, ~column) composites; the chosen columns are marked in a
// bitmap and read back in column order.  Otherwise (ties spanning the
// bracket, fewer valid entries than k) the row falls back to the exact radix
// path, so the result never depends on the sample.  Few rows: the pass is
// spread over many workgroups (bracket / classify / finish kernels).
//
// Radix path (any n, k).  A stats pass finds the valid count, the forced
// entry and the min / max key; radix select finds the k-th largest key T,
// 8 bits per pass below the bits all keys share; histograms live in LDS and
// each wave first adds its most common digit with one atomic (ballot +
// popcount); an ordered compaction keeps keys > T and the first keys == T in
// column order.
//
// Ties go to the smaller column, which is the smaller id because ids grow
// with the column (documented precondition).  Everything is integer work:
// results are deterministic and bit-exact.
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

// Exact radix select of one row straight from global memory (any n, any k).
__device__ void radix_select_row(const SelArgs& a, int64_t row, Shared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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


constexpr int SAMPLE = 2048;          // sampled keys per row
constexpr int NBIN = 1024;            // sample histogram bins
constexpr int CAND_CAP = 8192;        // candidate list capacity per row
constexpr int CAND_PT = CAND_CAP / THREADS;
constexpr int KFAST = 2048;           // largest k of the sampled paths
constexpr int64_t MAX_N_FAST = 1 << 18;  // longest row of the sampled paths (bitmap)

// Per-row state of the split path (lives in the caller's workspace).
struct RowState {
  uint32_t A, Bt;          // in: key > A; candidate: Bt <= key <= A
  int32_t fcol;            // forced column known before the pass (force_last)
  int32_t fcol_found;      // forced column found during the pass (forced id)
  uint32_t n_in, n_cand;
  uint32_t pad[10];
};

struct SampleSmem {
  uint32_t hist[NBIN];
  uint32_t b1, b2;
};

struct FinishSmem {
  uint32_t bitmap[MAX_N_FAST / 32];
  uint32_t hist[256];
  uint32_t bc[4];
};

// Wave-aggregated append of the flagged lanes to a list (LDS or global);
// entries past cap are dropped, the counter still counts them.
template <typename T>
__device__ __forceinline__ void wave_append(bool flag, T value, T* list, uint32_t* counter,
                                            uint32_t cap) {
  const int lane = threadIdx.x & 63;
  const uint64_t m = __ballot(flag);
  if (!m) return;
  const int leader = __ffsll((unsigned long long)m) - 1;
  uint32_t base = 0;
  if (lane == leader) base = atomicAdd(counter, (uint32_t)__popcll(m));
  base = (uint32_t)__shfl((int)base, leader, 64);
  if (flag) {
    const uint32_t pos = base + (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
    if (pos < cap) list[pos] = value;
  }
}

// Column of the last valid entry of the row (-1 if none), scanning back
// from the end one block-wide chunk at a time.  1024 threads.
__device__ int32_t last_valid_column(const SelArgs& a, int64_t row, Shared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t n = a.n;
  for (int64_t base = ((n - 1) / THREADS) * THREADS; base >= 0; base -= THREADS) {
    const int64_t j = base + tid;
    const bool v = j < n && load_elem(a, row, j).key != 0;
    const uint64_t m = __ballot(v);
    if (lane == 0)
      sh.wred[wave] = m ? (uint32_t)(64 * wave + 63 - __clzll((unsigned long long)m)) : 0xffffffffu;
    __syncthreads();
    int32_t best = -1;
    for (int i = 0; i < NWAVES; ++i)
      if (sh.wred[i] != 0xffffffffu) best = max(best, (int32_t)(base + sh.wred[i]));
    __syncthreads();
    if (best >= 0) return best;
  }
  return -1;
}

// Bracket [Bt, A] around the k-th key of the row from SAMPLE keys spread
// evenly over it (forced entry excluded): a NBIN-bin histogram of the sample
// over [min, max] with power-of-two bin width locates the sample ranks
// r -/+ delta (r = expected rank of the k-th key, delta = 4 sqrt(r) + 16); the
// bracket is made of whole bins, so it is approximate by design -- the exact
// answer comes later and a bracket that misses is detected and handled.
// 1024 threads.
__device__ void sample_bracket(const SelArgs& a, int64_t row, int32_t fcol, int32_t fid,
                               SampleSmem& ss, Shared& sh, uint32_t* A, uint32_t* Bt) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t n = a.n;
  uint32_t v[SAMPLE / THREADS];
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int i = 0; i < SAMPLE / THREADS; ++i) {
    const int64_t j = (int64_t)(tid + i * THREADS) * n / SAMPLE;
    const Elem e = load_elem(a, row, j);
    const bool forced = (j == fcol) || (fid >= 0 && e.id == fid);
    v[i] = forced ? 0u : e.key;
    if (v[i]) {
      kmin = min(kmin, v[i]);
      kmax = max(kmax, v[i]);
    }
  }
  for (int i = tid; i < NBIN; i += THREADS) ss.hist[i] = 0;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o, 64));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
  }
  if (lane == 0) {
    sh.wred[wave * 4 + 1] = kmin;
    sh.wred[wave * 4 + 2] = kmax;
  }
  __syncthreads();
  kmin = 0xffffffffu;
  kmax = 0u;
  for (int i = 0; i < NWAVES; ++i) {
    kmin = min(kmin, sh.wred[i * 4 + 1]);
    kmax = max(kmax, sh.wred[i * 4 + 2]);
  }
  const int have_forced_guess = (fcol >= 0 || fid >= 0) ? 1 : 0;
  const float r = (float)(a.k - have_forced_guess) * (float)SAMPLE / (float)n;
  const float delta = 4.0f * sqrtf(r) + 16.0f;
  const int r_hi = (int)floorf(r - delta);
  const int r_lo = (int)ceilf(r + delta);
  if (kmax == 0u) {  // no valid sample
    *A = 0xffffffffu;
    *Bt = 1u;
    __syncthreads();
    return;
  }
  const uint32_t range = kmax - kmin;
  const int w = range < (uint32_t)NBIN ? 0 : (32 - __clz(range)) - 10;  // range >> w < NBIN
#pragma unroll
  for (int i = 0; i < SAMPLE / THREADS; ++i)
    if (v[i]) atomicAdd(&ss.hist[(v[i] - kmin) >> w], 1u);
  if (tid == 0) {
    ss.b1 = 0xffffffffu;
    ss.b2 = 0xffffffffu;
  }
  __syncthreads();
  // thread t owns bin NBIN-1-t: an exclusive prefix over t counts the
  // samples in higher bins
  const int bin = NBIN - 1 - tid;
  const uint32_t cnt = tid < NBIN ? ss.hist[bin] : 0u;
  uint32_t tot;
  const uint32_t above = block_exclusive_scan(cnt, sh, &tot);
  if (tid < NBIN && cnt) {
    if (r_hi >= 0 && above <= (uint32_t)r_hi && (uint32_t)r_hi < above + cnt) ss.b1 = bin;
    if (above <= (uint32_t)r_lo && (uint32_t)r_lo < above + cnt) ss.b2 = bin;
  }
  __syncthreads();
  const uint32_t b1 = ss.b1, b2 = ss.b2;
  // in: whole bins above b1; candidates: bins b2 .. b1
  if (r_hi < 0 || b1 == 0xffffffffu) {
    *A = 0xffffffffu;
  } else {
    const uint64_t edge = (uint64_t)kmin + ((uint64_t)(b1 + 1) << w);  // first key above bin b1
    *A = edge > 0xffffffffull ? 0xffffffffu : (uint32_t)(edge - 1);
  }
  *Bt = (b2 == 0xffffffffu) ? 1u : max(1u, kmin + (b2 << w));
  __syncthreads();
}

// Classify entries [j0, j1) of a row (stride = blockDim.x) into the in and
// candidate lists.  Loads are issued PRE rounds at a time before any of them
// is classified, so their latencies overlap.
__device__ void classify_range(const SelArgs& a, int64_t row, int64_t j0, int64_t j1, uint32_t A,
                               uint32_t Bt, int32_t fcol, int32_t fid, int32_t* in_list,
                               uint32_t* n_in, uint32_t in_cap, uint64_t* cand, uint32_t* n_cand,
                               uint32_t cand_cap, int32_t* fcol_found) {
  constexpr int PRE = 8;
  const int64_t step = blockDim.x;
  for (int64_t base = j0; base < j1; base += PRE * step) {
    Elem e[PRE];
#pragma unroll
    for (int u = 0; u < PRE; ++u) {
      const int64_t j = base + u * step + threadIdx.x;
      e[u].key = 0;
      e[u].id = -1;
      if (j < j1) e[u] = load_elem(a, row, j);
    }
#pragma unroll
    for (int u = 0; u < PRE; ++u) {
      const int64_t j = base + u * step + threadIdx.x;
      uint32_t key = e[u].key;
      if (j < j1) {
        if (j == fcol) {
          key = 0;
        } else if (fid >= 0 && e[u].id == fid && key != 0) {
          atomicMin(fcol_found, (int32_t)j);
          key = 0;
        }
      }
      const bool isin = key > A;
      const bool iscand = !isin && key >= Bt && key != 0;
      wave_append<int32_t>(isin, (int32_t)j, in_list, n_in, in_cap);
      wave_append<uint64_t>(iscand, ((uint64_t)key << 32) | (uint64_t)(0xffffffffu - (uint32_t)j),
                            cand, n_cand, cand_cap);
    }
  }
}

// k-th largest (k >= 1) of the distinct nonzero uint64 values held by the
// block (CAND_PT per thread): radix select, 8 bits per pass below the bits
// all values share.  A pass whose chosen digit bin holds exactly the number
// still wanted ends the search early.  Result: v is among the k largest iff
// (v >> *lo) >= (*T >> *lo).  1024 threads.
__device__ void kth_largest_u64(const uint64_t (&v)[CAND_PT], uint32_t k, FinishSmem& fs,
                                Shared& sh, uint64_t* T, int* lo_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint64_t vmin = ~0ull, vmax = 0ull;
#pragma unroll
  for (int i = 0; i < CAND_PT; ++i)
    if (v[i]) {
      vmin = v[i] < vmin ? v[i] : vmin;
      vmax = v[i] > vmax ? v[i] : vmax;
    }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint64_t a = __shfl_xor(vmin, o, 64), b = __shfl_xor(vmax, o, 64);
    vmin = a < vmin ? a : vmin;
    vmax = b > vmax ? b : vmax;
  }
  __shared__ uint64_t red[2 * NWAVES];
  if (lane == 0) {
    red[wave] = vmin;
    red[NWAVES + wave] = vmax;
  }
  __syncthreads();
  vmin = ~0ull;
  vmax = 0ull;
  for (int i = 0; i < NWAVES; ++i) {
    vmin = red[i] < vmin ? red[i] : vmin;
    vmax = red[NWAVES + i] > vmax ? red[NWAVES + i] : vmax;
  }
  int hi = vmin == vmax ? 0 : 64 - __clzll((unsigned long long)(vmin ^ vmax));
  uint64_t prefix = hi >= 64 ? 0ull : (vmax & ~((1ull << hi) - 1ull));
  uint32_t remaining = k;
  while (hi > 0) {
    const int lo = hi > 8 ? hi - 8 : 0;
    const uint32_t dmask = (1u << (hi - lo)) - 1u;
    for (int i = tid; i < 256; i += THREADS) fs.hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < CAND_PT; ++i) {
      const bool match = v[i] && (hi >= 64 || (v[i] >> hi) == (prefix >> hi));
      if (match) atomicAdd(&fs.hist[(uint32_t)(v[i] >> lo) & dmask], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      uint32_t c[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) c[i] = fs.hist[4 * lane + i];
      const uint32_t tot = c[0] + c[1] + c[2] + c[3];
      uint32_t suf = tot;
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
            fs.bc[0] = 4u * lane + i;
            fs.bc[1] = acc;
            fs.bc[2] = c[i];
            break;
          }
          acc += c[i];
        }
      }
    }
    __syncthreads();
    const uint32_t dsel = fs.bc[0], cabove = fs.bc[1], cbin = fs.bc[2];
    __syncthreads();
    remaining -= cabove;
    prefix |= (uint64_t)dsel << lo;
    hi = lo;
    if (remaining == cbin) break;  // the whole bin is wanted
  }
  *T = prefix;
  *lo_out = hi;
}

// From the in list and the candidate list to the k ids, ascending.  Returns
// false (nothing written) when the bracket did not hold.  The chosen
// columns are marked in an LDS bitmap and read back in column order.
// 1024 threads.
__device__ bool finish_from_lists(const SelArgs& a, int64_t row, int32_t fcol, uint32_t n_in,
                                  uint32_t n_cand, const int32_t* in_list,
                                  const uint64_t* cand_src, FinishSmem& fs, Shared& sh) {
  const int tid = threadIdx.x;
  const int have_forced = fcol >= 0 ? 1 : 0;
  const uint32_t k_rem = (uint32_t)(a.k - have_forced);
  if (n_in > k_rem || n_in + n_cand < k_rem || n_cand > CAND_CAP || a.n > MAX_N_FAST) return false;
  const uint32_t m = k_rem - n_in;
  uint64_t v[CAND_PT];
#pragma unroll
  for (int i = 0; i < CAND_PT; ++i) {
    const uint32_t idx = tid + i * THREADS;
    v[i] = idx < n_cand ? cand_src[idx] : 0ull;
  }
  uint64_t T = ~0ull;
  int lo = 0;
  if (m > 0) kth_largest_u64(v, m, fs, sh, &T, &lo);
  const int64_t n = a.n;
  const int words = (int)((n + 31) / 32);
  for (int i = tid; i < words; i += THREADS) fs.bitmap[i] = 0u;
  __syncthreads();
  for (uint32_t i = tid; i < n_in; i += THREADS) {
    const uint32_t c = (uint32_t)in_list[i];
    atomicOr(&fs.bitmap[c >> 5], 1u << (c & 31));
  }
  if (m > 0) {
#pragma unroll
    for (int i = 0; i < CAND_PT; ++i)
      if (v[i] && (v[i] >> lo) >= (T >> lo)) {
        const uint32_t c = 0xffffffffu - (uint32_t)(v[i] & 0xffffffffull);
        atomicOr(&fs.bitmap[c >> 5], 1u << (c & 31));
      }
  }
  if (tid == 0 && have_forced) atomicOr(&fs.bitmap[fcol >> 5], 1u << (fcol & 31));
  __syncthreads();
  // ordered read-back: thread t owns a contiguous run of words
  const int wpt = (words + THREADS - 1) / THREADS;
  const int w0 = tid * wpt, w1 = min(words, w0 + wpt);
  uint32_t cnt = 0;
  for (int wi = w0; wi < w1; ++wi) cnt += __popc(fs.bitmap[wi]);
  uint32_t total;
  uint32_t pos = block_exclusive_scan(cnt, sh, &total);
  int32_t* orow = a.out + row * a.o_stride;
  for (int wi = w0; wi < w1; ++wi) {
    uint32_t bits = fs.bitmap[wi];
    while (bits) {
      const int b = __ffs(bits) - 1;
      bits &= bits - 1u;
      const int64_t c = (int64_t)wi * 32 + b;
      if (pos < (uint32_t)a.k) orow[pos] = a.ids ? a.ids[row * a.id_stride + c] : (int32_t)c;
      ++pos;
    }
  }
  for (int i = (int)total + tid; i < a.k; i += THREADS) orow[i] = -1;
  return true;
}

// ---- many rows: one workgroup per row --------------------------------------
struct RowSmem {
  Shared sh;
  SampleSmem ss;
  FinishSmem fs;
  uint64_t cand[CAND_CAP];
  int32_t in_list[KFAST];
  uint32_t n_in, n_cand;
  int32_t fcol_found;
};

__global__ __launch_bounds__(THREADS) void select_topk_kernel(SelArgs a, int try_sampled) {
  __shared__ RowSmem sm;
  const int64_t row = blockIdx.x;
  if (try_sampled) {
    const int32_t fid = a.forced ? a.forced[row] : -1;
    int32_t fcol = a.force_last ? last_valid_column(a, row, sm.sh) : -1;
    uint32_t A, Bt;
    if (threadIdx.x == 0) {
      sm.n_in = 0;
      sm.n_cand = 0;
      sm.fcol_found = 0x7fffffff;
    }
    sample_bracket(a, row, fcol, fid, sm.ss, sm.sh, &A, &Bt);
    classify_range(a, row, 0, a.n, A, Bt, fcol, fid, sm.in_list, &sm.n_in, KFAST, sm.cand,
                   &sm.n_cand, CAND_CAP, &sm.fcol_found);
    __syncthreads();
    if (fid >= 0) fcol = sm.fcol_found == 0x7fffffff ? -1 : sm.fcol_found;
    if (finish_from_lists(a, row, fcol, sm.n_in, sm.n_cand, sm.in_list, sm.cand, sm.fs, sm.sh))
      return;
    __syncthreads();
  }
  radix_select_row(a, row, sm.sh);
}

// ---- few rows: the pass over the row is split over many workgroups ----------
// K0: forced column, sample, bracket; resets the row's counters.
__global__ __launch_bounds__(THREADS) void select_bracket_kernel(SelArgs a, RowState* st) {
  __shared__ Shared sh;
  __shared__ SampleSmem ss;
  const int64_t row = blockIdx.x;
  const int32_t fid = a.forced ? a.forced[row] : -1;
  const int32_t fcol = a.force_last ? last_valid_column(a, row, sh) : -1;
  uint32_t A, Bt;
  sample_bracket(a, row, fcol, fid, ss, sh, &A, &Bt);
  if (threadIdx.x == 0) {
    RowState& s = st[row];
    s.A = A;
    s.Bt = Bt;
    s.fcol = fcol;
    s.fcol_found = 0x7fffffff;
    s.n_in = 0;
    s.n_cand = 0;
  }
}

// K1: grid (chunks, rows), 256 threads, CHUNK entries per workgroup.  The
// workgroup collects its in / candidate entries in LDS, then reserves room
// in the row's global lists with one atomic per list and copies them out.
constexpr int CLS_THREADS = 256;
constexpr int CHUNK = 2048;

__global__ __launch_bounds__(CLS_THREADS) void select_classify_kernel(SelArgs a, RowState* st,
                                                                      int32_t* in_lists,
                                                                      uint64_t* cand_lists) {
  __shared__ int32_t l_in[CHUNK];
  __shared__ uint64_t l_cand[CHUNK];
  __shared__ uint32_t l_n_in, l_n_cand, g_in, g_cand;
  __shared__ int32_t l_fcol;
  const int64_t row = blockIdx.y;
  const int64_t j0 = (int64_t)blockIdx.x * CHUNK;
  const int64_t j1 = min(a.n, j0 + CHUNK);
  RowState& s = st[row];
  const int32_t fid = a.forced ? a.forced[row] : -1;
  if (threadIdx.x == 0) {
    l_n_in = 0;
    l_n_cand = 0;
    l_fcol = 0x7fffffff;
  }
  __syncthreads();
  classify_range(a, row, j0, j1, s.A, s.Bt, s.fcol, fid, l_in, &l_n_in, CHUNK, l_cand, &l_n_cand,
                 CHUNK, &l_fcol);
  __syncthreads();
  if (threadIdx.x == 0) {
    g_in = l_n_in ? atomicAdd(&s.n_in, l_n_in) : 0u;
    g_cand = l_n_cand ? atomicAdd(&s.n_cand, l_n_cand) : 0u;
    if (l_fcol != 0x7fffffff) atomicMin(&s.fcol_found, l_fcol);
  }
  __syncthreads();
  int32_t* gin = in_lists + row * KFAST;
  uint64_t* gcand = cand_lists + row * CAND_CAP;
  for (uint32_t i = threadIdx.x; i < l_n_in; i += CLS_THREADS)
    if (g_in + i < KFAST) gin[g_in + i] = l_in[i];
  for (uint32_t i = threadIdx.x; i < l_n_cand; i += CLS_THREADS)
    if (g_cand + i < CAND_CAP) gcand[g_cand + i] = l_cand[i];
}

// K2: exact order among the candidates and the ascending id list.
__global__ __launch_bounds__(THREADS) void select_finish_kernel(SelArgs a, const RowState* st,
                                                                const int32_t* in_lists,
                                                                const uint64_t* cand_lists) {
  __shared__ FinishSmem fs;
  __shared__ Shared sh;
  const int64_t row = blockIdx.x;
  const RowState& s = st[row];
  int32_t fcol = s.fcol;
  if (a.forced) fcol = s.fcol_found == 0x7fffffff ? -1 : s.fcol_found;
  if (finish_from_lists(a, row, fcol, s.n_in, s.n_cand, in_lists + row * KFAST,
                        cand_lists + row * CAND_CAP, fs, sh))
    return;
  __syncthreads();
  radix_select_row(a, row, sh);
}

bool sampled_ok(int64_t n, int k) { return n >= 4 * SAMPLE && n <= MAX_N_FAST && k <= KFAST; }
bool split_path(int64_t R, int64_t n, int k) { return R < 256 && sampled_ok(n, k); }

}  // namespace

size_t select_workspace_bytes(int64_t R, int64_t n, int64_t k) {
  if (!split_path(R, n, (int)k)) return 0;
  return (size_t)R * (sizeof(RowState) + KFAST * sizeof(int32_t) + CAND_CAP * sizeof(uint64_t));
}

hipError_t launch_select_topk(int R, int64_t n, const float* scores, int64_t s_stride,
                              const int32_t* ids, int64_t id_stride, const int32_t* forced,
                              int force_last, int k, int32_t* out, int64_t o_stride, void* ws,
                              hipStream_t s) {
  SelArgs a{scores, s_stride, ids, id_stride, forced, force_last, n, k, out, o_stride};
  if (split_path(R, n, k)) {
    RowState* st = static_cast<RowState*>(ws);
    int32_t* in_lists = reinterpret_cast<int32_t*>(st + R);
    uint64_t* cand_lists = reinterpret_cast<uint64_t*>(in_lists + (int64_t)R * KFAST);
    hipLaunchKernelGGL(select_bracket_kernel, dim3((unsigned)R), dim3(THREADS), 0, s, a, st);
    hipLaunchKernelGGL(select_classify_kernel, dim3((unsigned)((n + CHUNK - 1) / CHUNK), (unsigned)R),
                       dim3(CLS_THREADS), 0, s, a, st, in_lists, cand_lists);
    hipLaunchKernelGGL(select_finish_kernel, dim3((unsigned)R), dim3(THREADS), 0, s, a, st,
                       in_lists, cand_lists);
    return hipGetLastError();
  }
  const int try_sampled = sampled_ok(n, k) ? 1 : 0;
  hipLaunchKernelGGL(select_topk_kernel, dim3((unsigned)R), dim3(THREADS), 0, s, a, try_sampled);
  return hipGetLastError();
}

}  // namespace csa2
