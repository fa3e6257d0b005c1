// select_topk.hip -- a3 / a5, the two top-k stages of CSA2 selection (NVFP4
// article, section 3.3): block level (top-K_b blocks by their in-block
// maximum, the newest block always kept) and position level (top-K latents
// of the candidate blocks).  Ranking key: (score descending, id ascending).
//
// Scores become order-preserving uint32 keys (larger score -> larger key;
// invalid entries -> 0).  A row is owned by one workgroup, except on the
// split sampled path below.
//
// Sampled path (8192 <= n <= 2^17, k <= 2048: the decode block stage).  A
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
// Radix rows (>= 1024 rows of <= 16,384 entries: the chunked prefill, a
// 256/512-thread workgroup per row, several per CU; fewer rows of 8K-16K
// entries: 1024 threads, one row per CU): exact radix threshold over the
// bits the row's keys differ in, column bitmaps by ballot, one block scan
// for the ordered output (select_many_kernel).
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

// Candidates gathered on the fly (one indexer for both stages): entry j of
// row r is latent p = 8 * blocks[r][j / 8] + j % 8 of the scan's score
// matrix, valid when the block id is >= 0 and p < n_vis(q_pos[r]); its id is
// p.  Used by the register-row kernel only.
struct GatherSrc {
  const float* all;  // [R][a_stride] scan scores
  int64_t a_stride;
  const int32_t* blocks;  // [R][K_b], ascending, -1 padded
  int K_b;
  const int64_t* q_pos;  // [R]
  int64_t n_cache;
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
  uint32_t wred_x[NWAVES];
  uint32_t bcast[8];
};

// exclusive block scan of one uint32 per thread (any block size <= 1024):
// DPP scan inside each wave, then the 16 lanes of a row scan the wave totals
// and each wave picks its prefix with readlane.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, Shared& sh, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = (int)(blockDim.x >> 6);
  const uint32_t x = wave_incl_scan(v);
  if (lane == 63) sh.scan[wave] = x;
  __syncthreads();
  const int i = lane & 15;
  uint32_t t = i < nw ? sh.scan[i] : 0u;
  t += dpp_mov<0x111>(t);  // row_shr:1
  t += dpp_mov<0x112>(t);  // row_shr:2
  t += dpp_mov<0x114>(t);  // row_shr:4
  t += dpp_mov<0x118>(t);  // row_shr:8
  const uint32_t through_me = (uint32_t)__builtin_amdgcn_readlane((int)t, wave);
  const uint32_t mine = (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
  *total = (uint32_t)__builtin_amdgcn_readlane((int)t, nw - 1);
  __syncthreads();  // sh.scan may be rewritten by the next scan
  return through_me - mine + x - v;
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
constexpr int64_t MAX_N_FAST = 1 << 17;  // longest row of the sampled paths (bitmaps)
constexpr int KBIN = 4096;               // radix digit bins of the candidate select (12 bits)

struct SampleSmem {
  uint32_t hist[NBIN];
  uint32_t o1[4], o2[4];  // bins of the two bracket ranks (wave_find_bin)
};

struct ThreshSmem {
  uint32_t hist[2][KBIN];  // radix digit bins, one buffer per pass parity
  uint32_t bc[4];
};

// Statistics of a candidate set: AND and OR of the keys (their common bits),
// smallest and largest key, count; and the count of keys above the set.
struct CandStats {
  uint32_t kand, kor, kmin, kmax, count, above;
};

// Wave 0 scans NB bins from the top (bin NB-1 first), NB / 64 per lane:
// finds the bin holding the `want`-th entry (want >= 1) and returns, through
// out[0..2], the bin, the count in higher bins and the bin's count.  Only
// wave 0 may call this; nothing is written if want exceeds the total.  Kept
// out of line: inlined into the 1024-thread kernels it made the register
// allocator spill.  Its pointers are typed as LDS pointers, so that the
// out-of-line body reads the histogram with LDS instructions rather than
// generic (flat) loads.
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) const uint32_t lds_cu32;
template <int NB>
__device__ __noinline__ void wave_find_bin_lds(lds_cu32* hist, uint32_t want, lds_u32* out) {
  constexpr int PL = NB / 64, NG = PL / 4;  // bins per lane, groups of 4 per lane
  const int lane = threadIdx.x & 63;
  lds_cu32* mine = hist + NB - PL * (lane + 1);  // this lane's bins, ascending
  uint32_t gsum[NG];
  uint32_t tot = 0;
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const u32x4 x = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(mine + 4 * gi);
    gsum[gi] = x[0] + x[1] + x[2] + x[3];
    tot += gsum[gi];
  }
  const uint32_t incl = wave_incl_scan(tot);  // over lanes (lane 0 = highest bins)
  uint32_t above = incl - tot;
  if (above < want && want <= incl) {  // one lane: its group, then the bin
    int gsel = 0;
    uint32_t gabove = above;
#pragma unroll
    for (int gi = NG - 1; gi >= 0; --gi) {
      if (above < want && want <= above + gsum[gi]) {
        gsel = gi;
        gabove = above;
      }
      above += gsum[gi];
    }
    const u32x4 x = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(mine + 4 * gsel);
    above = gabove;
#pragma unroll
    for (int j = 3; j >= 0; --j) {
      if (above < want && want <= above + x[j]) {
        out[0] = (uint32_t)(NB - PL * (lane + 1) + 4 * gsel + j);
        out[1] = above;
        out[2] = x[j];
      }
      above += x[j];
    }
  }
}

// Call sites pass their (LDS) histogram and result arrays through this.
template <int NB>
__device__ __forceinline__ void wave_find_bin(const uint32_t* hist, uint32_t want, uint32_t* out) {
  wave_find_bin_lds<NB>((lds_cu32*)hist, want, (lds_u32*)out);
}

struct FinishSmem {
  uint32_t bitmap[MAX_N_FAST / 32];  // chosen columns
  uint32_t tiemap[MAX_N_FAST / 32];  // columns tied at the threshold key
  ThreshSmem ts;
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
// from the end one block-wide chunk at a time.  Any block size <= 1024.
__device__ int32_t last_valid_column(const SelArgs& a, int64_t row, Shared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nt = (int)blockDim.x, nw = nt >> 6;
  const int64_t n = a.n;
  for (int64_t base = ((n - 1) / nt) * nt; base >= 0; base -= nt) {
    const int64_t j = base + tid;
    const bool v = j < n && load_elem(a, row, j).key != 0;
    const uint64_t m = __ballot(v);
    if (lane == 0)
      sh.wred[wave] = m ? (uint32_t)(64 * wave + 63 - __clzll((unsigned long long)m)) : 0xffffffffu;
    __syncthreads();
    int32_t best = -1;
    for (int i = 0; i < nw; ++i)
      if (sh.wred[i] != 0xffffffffu) best = max(best, (int32_t)(base + sh.wred[i]));
    __syncthreads();
    if (best >= 0) return best;
  }
  return -1;
}

// The SAMPLE sampled entries of a row, SAMPLE / NT per thread (thread t
// holds samples t, t + NT, ...): 64 runs of 32 consecutive entries, run s
// starting at entry floor(s n / 64), so that a wave's loads touch two cache
// lines and every column is sampled with probability SAMPLE / n (n >= 2048).
template <int NT>
__device__ __forceinline__ void load_sample(const SelArgs& a, int64_t row, Elem (&e)[SAMPLE / NT],
                                            int64_t (&j)[SAMPLE / NT]) {
#pragma unroll
  for (int i = 0; i < SAMPLE / NT; ++i) {
    const int s = threadIdx.x + i * NT;
    j[i] = (int64_t)(s >> 5) * a.n / 64 + (s & 31);
    e[i] = load_elem(a, row, j[i]);
  }
}

// Bracket [Bt, A] around the k-th key of the row from SAMPLE keys spread
// evenly over it (forced entry excluded): a NBIN-bin histogram of the sample
// over [min, max] with power-of-two bin width locates the sample ranks
// r -/+ delta (r = expected rank of the k-th key, delta = 4 sqrt(r) + 16); the
// bracket is made of whole bins, so it is approximate by design -- the exact
// answer comes later and a bracket that misses is detected and handled.
// Block of NT threads; the result depends only on the row, not on NT.
// Core of the bracket: SPT sampled keys per thread (0 = absent) and r, the
// expected sample rank of the wanted key.
template <int NT, int SPT>
__device__ void bracket_core(const uint32_t (&v)[SPT], float r, SampleSmem& ss, Shared& sh,
                             uint32_t* A, uint32_t* Bt) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    if (v[i]) {
      kmin = min(kmin, v[i]);
      kmax = max(kmax, v[i]);
    }
  }
  for (int i = tid; i < NBIN; i += NT) ss.hist[i] = 0;
  kmin = wave_min(kmin);
  kmax = wave_max(kmax);
  if (lane == 0) {
    sh.wred[1 * NWAVES + wave] = kmin;
    sh.wred[2 * NWAVES + wave] = kmax;
  }
  __syncthreads();
  kmin = waves_combine(sh.wred + 1 * NWAVES, NT / 64, 0xffffffffu, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
  kmax = waves_combine(sh.wred + 2 * NWAVES, NT / 64, 0u, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
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
  for (int i = 0; i < SPT; ++i)
    if (v[i]) atomicAdd(&ss.hist[(v[i] - kmin) >> w], 1u);
  if (tid == 0) {
    ss.o1[0] = 0xffffffffu;
    ss.o2[0] = 0xffffffffu;
  }
  __syncthreads();
  // wave 0 locates the bins of sample ranks r_hi and r_lo (0-based, from the
  // top); a rank beyond the sample leaves its bin unset
  if (wave == 0) {
    if (r_hi >= 0) wave_find_bin<NBIN>(ss.hist, (uint32_t)r_hi + 1u, ss.o1);
    wave_find_bin<NBIN>(ss.hist, (uint32_t)r_lo + 1u, ss.o2);
  }
  __syncthreads();
  const uint32_t b1 = ss.o1[0], b2 = ss.o2[0];
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

template <int NT>
__device__ void bracket_from_sample(const SelArgs& a, const Elem (&e)[SAMPLE / NT],
                                    const int64_t (&js)[SAMPLE / NT], int32_t fcol, int32_t fid,
                                    SampleSmem& ss, Shared& sh, uint32_t* A, uint32_t* Bt) {
  constexpr int SPT = SAMPLE / NT;  // samples per thread
  uint32_t v[SPT];
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const bool forced = (js[i] == fcol) || (fid >= 0 && e[i].id == fid);
    v[i] = forced ? 0u : e[i].key;
  }
  // each column is sampled with probability SAMPLE / n; invalid entries rank
  // below every valid one, so the k-th key sits near sample rank k SAMPLE / n
  const int have_forced_guess = (fcol >= 0 || fid >= 0) ? 1 : 0;
  const float r = (float)(a.k - have_forced_guess) * (float)SAMPLE / (float)a.n;
  bracket_core<NT, SPT>(v, r, ss, sh, A, Bt);
}

// Bracket [Bt, A] around the k-th key of the row (see bracket_from_sample).
template <int NT>
__device__ void sample_bracket(const SelArgs& a, int64_t row, int32_t fcol, int32_t fid,
                               SampleSmem& ss, Shared& sh, uint32_t* A, uint32_t* Bt) {
  Elem e[SAMPLE / NT];
  int64_t js[SAMPLE / NT];
  load_sample<NT>(a, row, e, js);
  bracket_from_sample<NT>(a, e, js, fcol, fid, ss, sh, A, Bt);
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

// Threshold on the candidate KEYS such that the m best candidates are: every
// key above it, plus -- when the threshold key itself is shared by more
// candidates than still wanted -- the `need` smallest columns among those
// tied at it.  Low bits that every candidate key has in common are dropped
// (integer-valued scores leave the low mantissa bits constant) and the
// smallest key is subtracted, d = (key >> tz) - base, so the digits cover
// only the spread of the candidates; then 12-bit radix digits of d from the
// top, a digit bin that holds exactly the number still wanted ending the
// search.  Candidate order: see th_cmp.  P values per thread; the key of
// value x is x >> SHIFT, and it is a candidate iff lo_key <= key <= hi_key
// (lo_key >= 1).  1024 threads.
struct KeyThreshold {
  uint32_t D;     // digits of d chosen so far (bits >= lo)
  uint32_t base;  // smallest candidate key >> tz
  int lo, tz;
  bool take_all;  // every candidate in the threshold bin is taken
  uint32_t need;  // else: how many of them, in column order
};

// +1: candidate above the threshold bin (chosen); 0: in it; -1: below.
__device__ __forceinline__ int th_cmp(const KeyThreshold& th, uint32_t key) {
  const uint32_t d = ((key >> th.tz) - th.base) >> th.lo;
  const uint32_t D = th.D >> th.lo;
  return d > D ? 1 : (d == D ? 0 : -1);
}

// Candidate statistics over P values per thread (key = value >> SHIFT,
// candidate iff lo_key <= key <= hi_key), reduced over the block.
template <int P, int SHIFT, typename T>
__device__ CandStats cand_stats(const T (&vals)[P], uint32_t lo_key, uint32_t hi_key, Shared& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  CandStats st{0xffffffffu, 0u, 0xffffffffu, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const uint32_t k = (uint32_t)(vals[i] >> SHIFT);
    if (k >= lo_key && k <= hi_key) {
      st.kand &= k;
      st.kor |= k;
      st.kmin = min(st.kmin, k);
      st.kmax = max(st.kmax, k);
      ++st.count;
    }
    st.above += k > hi_key;
  }
  st.kand = wave_and(st.kand);
  st.kor = wave_or(st.kor);
  st.kmin = wave_min(st.kmin);
  st.kmax = wave_max(st.kmax);
  st.count = wave_sum(st.count);
  st.above = wave_sum(st.above);
  __syncthreads();  // earlier readers of sh.wred are done
  if (lane == 0) {
    sh.wred[0 * NWAVES + wave] = st.kand;
    sh.wred[1 * NWAVES + wave] = st.kor;
    sh.wred[2 * NWAVES + wave] = st.kmin;
    sh.wred[3 * NWAVES + wave] = st.kmax;
    sh.scan[wave] = st.count;
    sh.wred_x[wave] = st.above;
  }
  __syncthreads();
  const int nw = (int)(blockDim.x >> 6);
  CandStats t;
  t.kand = waves_combine(sh.wred + 0 * NWAVES, nw, 0xffffffffu, [](uint32_t a, uint32_t b) { return a & b; });
  t.kor = waves_combine(sh.wred + 1 * NWAVES, nw, 0u, [](uint32_t a, uint32_t b) { return a | b; });
  t.kmin = waves_combine(sh.wred + 2 * NWAVES, nw, 0xffffffffu, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
  t.kmax = waves_combine(sh.wred + 3 * NWAVES, nw, 0u, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
  t.count = waves_combine(sh.scan, nw, 0u, [](uint32_t a, uint32_t b) { return a + b; });
  t.above = waves_combine(sh.wred_x, nw, 0u, [](uint32_t a, uint32_t b) { return a + b; });
  return t;
}

// Threshold over the candidates (see above).  `st` are their statistics
// (cand_stats).  Per radix pass: the block adds its digits into one
// histogram buffer, wave 0 scans it while the other waves clear the other
// buffer, two barriers in all.  1024 threads.
template <int P, int SHIFT, typename T>
__device__ KeyThreshold key_threshold(const T (&vals)[P], uint32_t lo_key, uint32_t hi_key,
                                      uint32_t m, const CandStats& st, ThreshSmem& fs) {
  const int tid = threadIdx.x, wave = tid >> 6;
  KeyThreshold th;
  const uint32_t varying = st.kand ^ st.kor;  // bits that differ between some keys
  th.tz = varying ? __ffs(varying) - 1 : 0;
  th.base = st.kmin >> th.tz;
  const uint32_t spread = (st.kmax >> th.tz) - th.base;  // d in [0, spread]
  int hi = spread ? 32 - __clz(spread) : 0;              // d < 2^hi
  uint32_t prefix = 0u;
  uint32_t remaining = m, cbin = st.count;  // spread 0: one key shared by all
  th.take_all = false;
  th.lo = 0;
  int cur = 0;
  if (hi > 0) {
    for (int i = tid; i < KBIN; i += THREADS) fs.hist[0][i] = 0;
    __syncthreads();
  }
  while (hi > 0) {
    const int lo = hi > 12 ? hi - 12 : 0;
    const uint32_t dmask = (1u << (hi - lo)) - 1u;
    uint32_t* h = fs.hist[cur];
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const uint32_t k = (uint32_t)(vals[i] >> SHIFT);
      if (k < lo_key || k > hi_key) continue;
      const uint32_t d = (k >> th.tz) - th.base;
      if (hi >= 32 || (d >> hi) == (prefix >> hi)) atomicAdd(&h[(d >> lo) & dmask], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      wave_find_bin<KBIN>(h, remaining, fs.bc);
    } else {
      uint32_t* other = fs.hist[cur ^ 1];
      for (int i = tid - 64; i < KBIN; i += THREADS - 64) other[i] = 0;
    }
    __syncthreads();
    const uint32_t dsel = fs.bc[0];
    remaining -= fs.bc[1];
    cbin = fs.bc[2];
    prefix |= dsel << lo;
    hi = lo;
    th.lo = lo;
    cur ^= 1;
    if (remaining == cbin) break;
  }
  th.D = prefix;
  th.take_all = remaining == cbin;
  th.need = remaining;
  // the next use of fs.bc (another pass, another row) comes after a barrier
  // of the caller or of the next key_threshold's first pass
  return th;
}

// Ordered read-back of the chosen bitmap (words of 32 columns, column order):
// unless th.take_all, the first th.need columns of the tie bitmap join the
// chosen ones; the ids of the chosen columns are written in column order and
// the row is padded with -1 up to k.  1024 threads.
__device__ __forceinline__ void read_back(const SelArgs& a, int64_t row, const KeyThreshold& th, int words,
                          uint32_t* bitmap, const uint32_t* tiemap, Shared& sh,
                          const GatherSrc* gs = nullptr) {
  const int tid = threadIdx.x;
  // thread t owns a contiguous run of words
  const int wpt = (words + THREADS - 1) / THREADS;
  const int w0 = tid * wpt, w1 = min(words, w0 + wpt);
  uint32_t nt = 0;
  if (!th.take_all)
    for (int wi = w0; wi < w1; ++wi) nt += __popc(tiemap[wi]);
  uint32_t tot_t = 0;
  uint32_t tie_rank = th.take_all ? 0u : block_exclusive_scan(nt, sh, &tot_t);
  // keep the ties with rank < need: fold them into the chosen bitmap words
  uint32_t cnt = 0;
  for (int wi = w0; wi < w1; ++wi) {
    uint32_t word = bitmap[wi];
    if (!th.take_all) {
      uint32_t tb = tiemap[wi];
      while (tb) {
        const uint32_t bit = tb & (0u - tb);
        tb &= tb - 1u;
        if (tie_rank < th.need) word |= bit;
        ++tie_rank;
      }
      bitmap[wi] = word;
    }
    cnt += __popc(word);
  }
  uint32_t total;
  uint32_t pos = block_exclusive_scan(cnt, sh, &total);
  int32_t* orow = a.out + row * a.o_stride;
  for (int wi = w0; wi < w1; ++wi) {
    uint32_t bits = bitmap[wi];
    while (bits) {
      const int b = __ffs(bits) - 1;
      bits &= bits - 1u;
      const int64_t c = (int64_t)wi * 32 + b;
      if (pos < (uint32_t)a.k)
        orow[pos] = gs ? gs->blocks[row * gs->K_b + (c >> 3)] * BLK + (int32_t)(c & 7)
                       : (a.ids ? a.ids[row * a.id_stride + c] : (int32_t)c);
      ++pos;
    }
  }
  for (int i = (int)total + tid; i < a.k; i += THREADS) orow[i] = -1;
}

// From the "in" columns and the candidate composites (held in registers,
// CAND_PT per thread, 0 = empty) to the k ids, ascending.  The chosen
// columns are marked in an LDS bitmap, candidates tied at the threshold key
// in a second one, and both are read back in column order, keeping the
// first `need` tied columns.  The caller has checked the bracket
// (n_in + m == k_rem, n_cand <= CAND_CAP).  1024 threads.
__device__ void finish_core(const SelArgs& a, int64_t row, int32_t fcol, uint32_t n_in,
                            const int32_t* in_list, uint32_t m, const uint32_t (&ckey)[CAND_PT],
                            const uint32_t (&ccol)[CAND_PT], FinishSmem& fs, Shared& sh) {
  const int tid = threadIdx.x;
  KeyThreshold th{0u, 0u, 0, 0, true, 0u};
  if (m > 0) {
    const CandStats st = cand_stats<CAND_PT, 0>(ckey, 1u, 0xffffffffu, sh);
    th = key_threshold<CAND_PT, 0>(ckey, 1u, 0xffffffffu, m, st, fs.ts);
  }
  const int64_t n = a.n;
  const int words = (int)((n + 31) / 32);
  for (int i = tid; i < words; i += THREADS) {
    fs.bitmap[i] = 0u;
    fs.tiemap[i] = 0u;
  }
  __syncthreads();
  for (uint32_t i = tid; i < n_in; i += THREADS) {
    const uint32_t c = (uint32_t)in_list[i];
    atomicOr(&fs.bitmap[c >> 5], 1u << (c & 31));
  }
  if (m > 0) {
#pragma unroll
    for (int i = 0; i < CAND_PT; ++i) {
      if (!ckey[i]) continue;
      const int cmp = th_cmp(th, ckey[i]);
      const uint32_t c = ccol[i];
      if (cmp > 0 || (cmp == 0 && th.take_all))
        atomicOr(&fs.bitmap[c >> 5], 1u << (c & 31));
      else if (cmp == 0)
        atomicOr(&fs.tiemap[c >> 5], 1u << (c & 31));
    }
  }
  if (tid == 0 && fcol >= 0) atomicOr(&fs.bitmap[fcol >> 5], 1u << (fcol & 31));
  __syncthreads();
  read_back(a, row, th, words, fs.bitmap, fs.tiemap, sh);
}

// Lists in one place (LDS): check the bracket, then finish.  Returns false
// (nothing written) when the bracket did not hold.
__device__ bool finish_from_lists(const SelArgs& a, int64_t row, int32_t fcol, uint32_t n_in,
                                  uint32_t n_cand, const int32_t* in_list,
                                  const uint64_t* cand_src, FinishSmem& fs, Shared& sh) {
  const int tid = threadIdx.x;
  const uint32_t k_rem = (uint32_t)(a.k - (fcol >= 0 ? 1 : 0));
  if (n_in > k_rem || n_in + n_cand < k_rem || n_cand > CAND_CAP || a.n > MAX_N_FAST) return false;
  uint32_t ckey[CAND_PT], ccol[CAND_PT];
#pragma unroll
  for (int i = 0; i < CAND_PT; ++i) {
    const uint32_t idx = tid + i * THREADS;
    const uint64_t v = idx < n_cand ? cand_src[idx] : 0ull;
    ckey[i] = (uint32_t)(v >> 32);
    ccol[i] = 0xffffffffu - (uint32_t)v;
  }
  finish_core(a, row, fcol, n_in, in_list, k_rem - n_in, ckey, ccol, fs, sh);
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
    sample_bracket<THREADS>(a, row, fcol, fid, sm.ss, sm.sh, &A, &Bt);
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
// K1 (grid chunks x rows, 256 threads): every block recomputes the row's
// forced column and bracket from the same sample -- identical integer work,
// so all blocks of a row agree -- and classifies its CH entries straight
// into its own slot (no atomics across blocks).  K2 (one 1024-thread block
// per row) gathers the slots and finishes.
constexpr int CLS_THREADS = 256;
// Entries per K1 block: 1024 for few rows (more blocks over the chip),
// 2048 once there are more than 16 rows.  Measured on the 1M block stages
// (classify + finish, µs): 8 rows 22.5 -> 20.5 with 1024; 32 rows 26.5
// against 27.1, 40 rows 28.2 against 31.2 with 1024 (2048 kept there);
// 4096: 26.6 / 29.8 / 30.6.
constexpr int CHUNK_FEW = 1024, CHUNK_MANY = 2048;
inline int64_t split_chunk(int64_t R) { return R <= 16 ? CHUNK_FEW : CHUNK_MANY; }
constexpr int SLOT = 512;  // per-chunk capacity of each list
constexpr int MAX_CHUNKS = (int)(MAX_N_FAST / CHUNK_FEW);

struct Slot {
  uint32_t n_in, n_cand;  // may exceed SLOT: the slot then overflowed
  int32_t fcol;           // forced column known before the pass (force_last)
  int32_t fcol_found;     // forced column found in this chunk (forced id)
  uint32_t pad[4];
  int32_t in[SLOT];
  uint64_t cand[SLOT];
};

template <int CH>
__global__ __launch_bounds__(CLS_THREADS) void select_classify_kernel(SelArgs a, Slot* slots,
                                                                      int nchunks) {
  constexpr int CPT = CH / CLS_THREADS;  // chunk entries per thread
  __shared__ Shared sh;
  __shared__ SampleSmem ss;
  __shared__ uint32_t l_n_in, l_n_cand;
  __shared__ int32_t l_fcol;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.y;
  const int chunk = blockIdx.x;
  const int64_t n = a.n;
  const int64_t j0 = (int64_t)chunk * CH;
  const int64_t j1 = min(n, j0 + CH);
  const int32_t fid = a.forced ? a.forced[row] : -1;
  if (tid == 0) {
    l_n_in = 0;
    l_n_cand = 0;
    l_fcol = 0x7fffffff;
  }
  // every load of the block is issued before any of them is used: this
  // chunk, the row sample and the row's last CLS_THREADS entries
  Elem ce[CPT];
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int64_t j = j0 + u * CLS_THREADS + tid;
    ce[u].key = 0;
    ce[u].id = -1;
    if (j < j1) ce[u] = load_elem(a, row, j);
  }
  Elem se[SAMPLE / CLS_THREADS];
  int64_t sj[SAMPLE / CLS_THREADS];
  load_sample<CLS_THREADS>(a, row, se, sj);
  const int64_t tail0 = ((n - 1) / CLS_THREADS) * CLS_THREADS;
  const bool tail_valid = a.force_last && tail0 + tid < n && load_elem(a, row, tail0 + tid).key != 0;
  int32_t fcol = -1;
  if (a.force_last) {
    const uint64_t m = __ballot(tail_valid);
    if (lane == 0)
      sh.wred[wave] = m ? (uint32_t)(64 * wave + 63 - __clzll((unsigned long long)m)) : 0xffffffffu;
    __syncthreads();
    for (int i = 0; i < CLS_THREADS / 64; ++i)
      if (sh.wred[i] != 0xffffffffu) fcol = max(fcol, (int32_t)(tail0 + sh.wred[i]));
    __syncthreads();
    if (fcol < 0) fcol = last_valid_column(a, row, sh);  // the row ends in invalid entries
  }
  uint32_t A, Bt;
  bracket_from_sample<CLS_THREADS>(a, se, sj, fcol, fid, ss, sh, &A, &Bt);
  Slot& sl = slots[row * nchunks + chunk];
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int64_t j = j0 + u * CLS_THREADS + tid;
    uint32_t key = ce[u].key;
    if (j < j1) {
      if (j == fcol) {
        key = 0;
      } else if (fid >= 0 && ce[u].id == fid && key != 0) {
        atomicMin(&l_fcol, (int32_t)j);
        key = 0;
      }
    }
    const bool isin = key > A;
    const bool iscand = !isin && key >= Bt && key != 0;
    wave_append<int32_t>(isin, (int32_t)j, sl.in, &l_n_in, SLOT);
    wave_append<uint64_t>(iscand, ((uint64_t)key << 32) | (uint64_t)(0xffffffffu - (uint32_t)j),
                          sl.cand, &l_n_cand, SLOT);
  }
  __syncthreads();
  if (tid == 0) {
    sl.n_in = l_n_in;
    sl.n_cand = l_n_cand;
    sl.fcol = fcol;
    sl.fcol_found = l_fcol;
  }
}

__global__ __launch_bounds__(THREADS) void select_finish_kernel(SelArgs a, const Slot* slots,
                                                                int nchunks) {
  __shared__ FinishSmem fs;
  __shared__ Shared sh;
  __shared__ uint32_t p_in[MAX_CHUNKS + 1], p_cand[MAX_CHUNKS + 1];
  __shared__ int32_t in_flat[KFAST];
  __shared__ int32_t s_ff;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const Slot* sr = slots + row * nchunks;
  uint32_t ni = 0, nc = 0;
  int over = 0;
  if (tid == 0) s_ff = 0x7fffffff;
  if (tid < nchunks) {
    ni = sr[tid].n_in;
    nc = sr[tid].n_cand;
    over = (ni > SLOT || nc > SLOT) ? 1 : 0;
  }
  uint32_t tot_in, tot_cand;
  const uint32_t b_in = block_exclusive_scan(ni, sh, &tot_in);
  const uint32_t b_cand = block_exclusive_scan(nc, sh, &tot_cand);
  if (tid < nchunks) {
    p_in[tid] = b_in;
    p_cand[tid] = b_cand;
    if (a.forced) atomicMin(&s_ff, sr[tid].fcol_found);
  }
  if (tid == 0) {
    p_in[nchunks] = tot_in;
    p_cand[nchunks] = tot_cand;
  }
  const int any_over = __syncthreads_or(over);
  int32_t fcol = a.force_last ? sr[0].fcol : -1;
  if (a.forced) fcol = s_ff == 0x7fffffff ? -1 : s_ff;
  const uint32_t k_rem = (uint32_t)(a.k - (fcol >= 0 ? 1 : 0));
  if (any_over || tot_in > k_rem || tot_in + tot_cand < k_rem || tot_cand > CAND_CAP) {
    radix_select_row(a, row, sh);
    return;
  }
  // chunk holding flat entry i of a list with prefix array p (last chunk
  // whose prefix is <= i; chunk counts may be 0)
  auto chunk_of = [&](const uint32_t* p, uint32_t i) {
    int lo = 0, hi = nchunks - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p[mid] <= i) lo = mid;
      else hi = mid - 1;
    }
    return lo;
  };
  for (uint32_t i = tid; i < tot_in; i += THREADS) {
    const int c = chunk_of(p_in, i);
    in_flat[i] = sr[c].in[i - p_in[c]];
  }
  uint32_t ckey[CAND_PT], ccol[CAND_PT];
#pragma unroll
  for (int q = 0; q < CAND_PT; ++q) {
    const uint32_t i = tid + q * THREADS;
    uint64_t v = 0ull;
    if (i < tot_cand) {
      const int c = chunk_of(p_cand, i);
      v = sr[c].cand[i - p_cand[c]];
    }
    ckey[q] = (uint32_t)(v >> 32);
    ccol[q] = 0xffffffffu - (uint32_t)v;
  }
  __syncthreads();
  finish_core(a, row, fcol, tot_in, in_flat, k_rem - tot_in, ckey, ccol, fs, sh);
}

// ---- rows of up to 1024 * E entries, held in registers ----------------------
// One 1024-thread workgroup per row.  Entry j of the row is element j / 1024
// of thread j % 1024, so the 32 columns of a bitmap word sit in 32
// consecutive lanes of one wave and one ballot writes them (no atomics, no
// clearing).  The row is read from memory once; everything after that works
// on registers and LDS:
//  1. keys, valid count and forced column (last valid entry, or the first
//     valid entry holding the forced id) by block reductions; the forced key
//     is set aside (0) and k_rem = k - 1 others are wanted;
//  2. E > 8: a bracket [Bt, A] from 2048 of the register keys, as in the
//     sampled paths; "in" = key > A, candidates = Bt <= key <= A, both
//     counted by one block scan.  When the bracket holds and the candidates
//     fit ROW_LIST, they are compacted into an LDS list of (key, column)
//     composites, two per thread at most, and steps 3-4 work on the list;
//     when the counts show that it missed, every valid entry is a candidate
//     instead (in registers), so the result never depends on the sample.
//     E = 8: all are candidates;
//  3. the exact key threshold over the candidates (radix on the list, or on
//     the registers);
//  4. ballots into the chosen and tie bitmaps (list candidates: bit sets),
//     ordered read-back.
constexpr int ROW_LIST = 2048;  // compacted candidate capacity of the register-row path

template <int E>
struct RowsSmem {
  Shared sh;
  SampleSmem ss;
  ThreshSmem ts;
  uint64_t bitmap[E * 16];  // 64 columns per entry: the two words of one ballot
  uint64_t tiemap[E * 16];
  uint64_t list[E > 8 ? ROW_LIST : 1];  // (key << 32) | ~column of each candidate
};

template <int E, bool IDS>
__device__ __forceinline__ void load_row_keys(const SelArgs& a, int64_t row, int32_t fid,
                                              uint32_t (&key)[E], int32_t* last_valid,
                                              int32_t* first_fid, uint32_t* n_valid) {
  const int tid = threadIdx.x;
  const int n = (int)a.n;
  const float* srow = a.scores + row * a.s_stride;
  const int32_t* irow = IDS ? a.ids + row * a.id_stride : nullptr;
  // with ids, 16 entries at a time so that ids and scores are not all live
  constexpr int G = (IDS && E > 16) ? 16 : E;
  static_assert(E % G == 0, "whole batches");
  int32_t lv = -1, ff = 0x7fffffff;
  uint32_t nv = 0;
#pragma unroll
  for (int g = 0; g < E; g += G) {
    float sc[G];
    int32_t id[G];
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int j = (g + u) * THREADS + tid;
      sc[u] = j < n ? srow[j] : -INFINITY;
      id[u] = IDS ? (j < n ? irow[j] : -1) : j;
    }
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int j = (g + u) * THREADS + tid;
      const bool ok = id[u] >= 0 && !(sc[u] != sc[u]) && sc[u] != -INFINITY;
      key[g + u] = ok ? order_key(sc[u]) : 0u;
      if (ok) {
        lv = j;  // j grows with g + u
        ++nv;
        if (fid >= 0 && id[u] == fid) ff = min(ff, j);
      }
    }
  }
  *last_valid = lv;
  *first_fid = ff;
  *n_valid = nv;
}

// The row's keys from the scan's score matrix through its block list (see
// GatherSrc): the block ids first, then the scores of the visible latents,
// 16 entries at a time.  No forced entry in this mode.
template <int E>
__device__ __forceinline__ void load_row_keys_gather(const SelArgs& a, const GatherSrc& gs,
                                                     int64_t row, uint32_t (&key)[E],
                                                     int32_t* last_valid, uint32_t* n_valid) {
  const int tid = threadIdx.x;
  const int n = (int)a.n;
  const int64_t t = gs.q_pos[row];
  const int64_t nvis = t < 0 ? 0 : min((t + 1) >> 1, gs.n_cache);
  const int32_t* brow = gs.blocks + row * gs.K_b;
  const float* srow = gs.all + row * gs.a_stride;
  constexpr int G = E > 16 ? 16 : E;
  static_assert(E % G == 0, "whole batches");
  int32_t lv = -1;
  uint32_t nv = 0;
#pragma unroll
  for (int g = 0; g < E; g += G) {
    int64_t p[G];
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int j = (g + u) * THREADS + tid;
      const int32_t blk = j < n ? brow[j >> 3] : -1;
      p[u] = blk >= 0 ? (int64_t)blk * BLK + (j & 7) : -1;
    }
    float sc[G];
#pragma unroll
    for (int u = 0; u < G; ++u) sc[u] = (p[u] >= 0 && p[u] < nvis) ? srow[p[u]] : -INFINITY;
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int j = (g + u) * THREADS + tid;
      const bool ok = !(sc[u] != sc[u]) && sc[u] != -INFINITY;
      key[g + u] = ok ? order_key(sc[u]) : 0u;
      if (ok) {
        lv = j;
        ++nv;
      }
    }
  }
  *last_valid = lv;
  *n_valid = nv;
}

template <int E, bool GATHER>
__global__ __launch_bounds__(THREADS) void select_rows_kernel(SelArgs a, GatherSrc gs) {
  __shared__ RowsSmem<E> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const int32_t fid = a.forced ? a.forced[row] : -1;

  // ---- 1 -------------------------------------------------------------------
  uint32_t key[E];
  int32_t lv, ff = 0x7fffffff;
  uint32_t nv;
  if (GATHER) load_row_keys_gather<E>(a, gs, row, key, &lv, &nv);
  else if (a.ids) load_row_keys<E, true>(a, row, fid, key, &lv, &ff, &nv);
  else load_row_keys<E, false>(a, row, fid, key, &lv, &ff, &nv);
  lv = wave_max_i(lv);
  ff = wave_min_i(ff);
  nv = wave_sum(nv);
  if (lane == 0) {
    sm.sh.wred[0 * NWAVES + wave] = (uint32_t)lv;
    sm.sh.wred[1 * NWAVES + wave] = (uint32_t)ff;
    sm.sh.wred[2 * NWAVES + wave] = nv;
  }
  __syncthreads();
  lv = (int32_t)waves_combine(sm.sh.wred + 0 * NWAVES, NWAVES, 0xffffffffu, [](uint32_t a, uint32_t b) {
    return (int32_t)a > (int32_t)b ? a : b;
  });
  ff = (int32_t)waves_combine(sm.sh.wred + 1 * NWAVES, NWAVES, 0x7fffffffu, [](uint32_t a, uint32_t b) {
    return (int32_t)a < (int32_t)b ? a : b;
  });
  nv = waves_combine(sm.sh.wred + 2 * NWAVES, NWAVES, 0u, [](uint32_t a, uint32_t b) { return a + b; });
  __syncthreads();
  int32_t fcol = -1;
  if (a.force_last) fcol = lv;
  else if (fid >= 0 && ff != 0x7fffffff) fcol = ff;
  if (fcol >= 0) {
#pragma unroll
    for (int i = 0; i < E; ++i)
      if (i * THREADS + tid == fcol) key[i] = 0u;
  }
  const uint32_t k_rem = (uint32_t)a.k - (fcol >= 0 ? 1u : 0u);
  const uint32_t n_rest = nv - (fcol >= 0 ? 1u : 0u);

  // ---- 2 -------------------------------------------------------------------
  uint32_t A = 0u, Bt = 1u, m = 0u;  // A = 0: every valid key is in
  CandStats st{0u, 0u, 0u, 0u, 0u, 0u};
  bool have_st = false;
  int listed = 0;            // candidates compacted into sm.list (block-uniform)
  uint32_t n_list = 0;
  if (n_rest > k_rem) {
    A = 0xffffffffu;  // nothing in, every valid key a candidate
    m = k_rem;
    if (E > 8) {
      // 2048 samples: thread t takes elements (h * 1024 + t) * E / 2048, h = 0, 1
      uint32_t v[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int want = (h * THREADS + tid) * E / (2 * THREADS);
        v[h] = 0u;
#pragma unroll
        for (int i = 0; i < E; ++i)
          if (i == want) v[h] = key[i];
      }
      // every column of [0, 1024 E) is sampled with probability 2 / E
      uint32_t A2, B2;
      bracket_core<THREADS, 2>(v, (float)k_rem * 2.0f / (float)E, sm.ss, sm.sh, &A2, &B2);
      // keys above the bracket and inside it, counted by one scan of both
      // (packed: 16 bits each, totals at most 16384 below 2^16)
      uint32_t c_in = 0, c_cand = 0;
#pragma unroll
      for (int i = 0; i < E; ++i) {
        c_in += key[i] > A2 ? 1u : 0u;
        c_cand += (key[i] >= B2 && key[i] <= A2) ? 1u : 0u;
      }
      uint32_t tot;
      const uint32_t before = block_exclusive_scan((c_in << 16) | c_cand, sm.sh, &tot);
      const uint32_t n_in = tot >> 16, n_cand = tot & 0xffffu;
      if (n_in <= k_rem && k_rem <= n_in + n_cand) {
        A = A2;
        Bt = B2;
        m = k_rem - n_in;
        if (n_cand <= (uint32_t)ROW_LIST) {
          listed = 1;
          n_list = n_cand;
          uint32_t pos = before & 0xffffu;
#pragma unroll
          for (int i = 0; i < E; ++i)
            if (key[i] >= B2 && key[i] <= A2)
              sm.list[pos++] = ((uint64_t)key[i] << 32) | (uint64_t)(0xffffffffu - (uint32_t)(i * THREADS + tid));
        } else {
          st = cand_stats<E, 0>(key, Bt, A, sm.sh);
          have_st = true;
        }
      }
    }
    if (!listed && !have_st && m > 0) st = cand_stats<E, 0>(key, Bt, A, sm.sh);
  }

  // ---- 3 -------------------------------------------------------------------
  KeyThreshold th{0u, 0u, 0, 0, true, 0u};
  constexpr int LP = ROW_LIST / THREADS;  // list entries per thread
  uint32_t lkey[LP], lcol[LP];
#pragma unroll
  for (int u = 0; u < LP; ++u) {
    lkey[u] = 0u;
    lcol[u] = 0u;
  }
  if (listed) {
    __syncthreads();  // the list is written
#pragma unroll
    for (int u = 0; u < LP; ++u) {
      const uint32_t idx = tid + u * THREADS;
      const uint64_t c = idx < n_list ? sm.list[idx] : 0ull;
      lkey[u] = (uint32_t)(c >> 32);
      lcol[u] = 0xffffffffu - (uint32_t)c;
    }
    if (m > 0) {
      const CandStats ls = cand_stats<LP, 0>(lkey, 1u, 0xffffffffu, sm.sh);
      th = key_threshold<LP, 0>(lkey, 1u, 0xffffffffu, m, ls, sm.ts);
    }
  } else if (m > 0) {
    th = key_threshold<E, 0>(key, Bt, A, m, st, sm.ts);
  }

  // ---- 4 -------------------------------------------------------------------
  // lane i of each wave keeps the ballots of element i: one store per lane.
  // Listed candidates are not in the ballots (their key <= A); they are set
  // in the bitmaps afterwards.
  uint64_t my_cb = 0ull, my_tb = 0ull;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const uint32_t k = key[i];
    bool chosen = k > A || i * THREADS + tid == fcol;
    bool tie = false;
    if (!listed && m > 0 && k >= Bt && k <= A) {
      const int cmp = th_cmp(th, k);
      chosen = chosen || cmp > 0 || (cmp == 0 && th.take_all);
      tie = cmp == 0 && !th.take_all;
    }
    const uint64_t cb = __ballot(chosen), tb = __ballot(tie);
    if (lane == i) {
      my_cb = cb;
      my_tb = tb;
    }
  }
  if (lane < E) {
    sm.bitmap[lane * NWAVES + wave] = my_cb;
    sm.tiemap[lane * NWAVES + wave] = my_tb;
  }
  if (listed && m > 0) {
    __syncthreads();  // ballot words stored
    uint32_t* bm32 = reinterpret_cast<uint32_t*>(sm.bitmap);
    uint32_t* tm32 = reinterpret_cast<uint32_t*>(sm.tiemap);
#pragma unroll
    for (int u = 0; u < LP; ++u) {
      if (!lkey[u]) continue;
      const int cmp = th_cmp(th, lkey[u]);
      const uint32_t c = lcol[u];
      if (cmp > 0 || (cmp == 0 && th.take_all)) atomicOr(&bm32[c >> 5], 1u << (c & 31));
      else if (cmp == 0) atomicOr(&tm32[c >> 5], 1u << (c & 31));
    }
  }
  __syncthreads();
  read_back(a, row, th, (int)((a.n + 31) / 32), reinterpret_cast<uint32_t*>(sm.bitmap),
            reinterpret_cast<const uint32_t*>(sm.tiemap), sm.sh, GATHER ? &gs : nullptr);
}


// ---- radix rows: one 256-, 512- or 1024-thread workgroup per row -----------
// For thousands of rows (the chunked prefill's two stages, 8192 rows) the
// register-row kernel's latency chain (16 waves, a dozen barrier-separated
// phases per row) leaves the CUs waiting; a smaller workgroup per row lets
// several rows share a CU and keeps the instruction count per entry low.
// With 1024 threads it also serves few rows of 8K-16K entries (the decodes'
// position stage), one row per CU, where it beats the sampled bracket:
//  1. the row in registers, entry c = e * MT + t of thread t (coalesced; in
//     gather mode the block list is staged in LDS first, so all score loads
//     of the row go out in one round through a buffer resource);
//  2. the k-th key exactly by radix over the bits in which the valid keys
//     differ (AND / OR of the keys first), 11-bit digits counted in an LDS
//     histogram: with integer-valued scores ~16 bits differ, two passes;
//  3. one ballot per (entry, wave) writes the "above" and "tied" bits of 64
//     consecutive columns; each thread then owns one 64-column word, one
//     block scan of the packed (above, tied) counts gives its output offset
//     and how many ties precede it, and it writes its chosen ids in column
//     order (ties go to the smaller columns).
constexpr int MBIN = 2048;                   // radix digit bins (11 bits)
constexpr int SEL_BUF_DWORD3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9 family)

template <int MT, int E, bool GATHER>
struct ManySmem {
  Shared sh;
  uint32_t hist[MBIN];
  uint64_t above[E * (MT / 64)];  // word e * NW + wave: columns e * MT + 64 * wave + [0, 64)
  uint64_t tied[E * (MT / 64)];
  uint32_t fb[4];                 // wave_find_bin result
  int32_t blk[GATHER ? E * MT / BLK : 1];  // the row's block list (gather mode)
};

// Minimum waves per SIMD (the launch bound's second argument): the gather
// of 16K candidates per row (E = 32, 512 threads) asks for three
// workgroups per CU (80 registers, a 16-byte spill) instead of the two its
// 98 registers allowed -- more rows' score loads in flight: 296 -> 272 us
// on an 8192-row prefill stage.  The other shapes already fit.
template <int MT, int E, bool GATHER>
constexpr int many_min_waves() {
  return (GATHER && MT == 512 && E >= 32) ? 6 : 1;
}

template <int MT, int E, bool GATHER, bool IDS>
__global__ __launch_bounds__(MT, (many_min_waves<MT, E, GATHER>())) void select_many_kernel(SelArgs a, GatherSrc gs) {
  __shared__ ManySmem<MT, E, GATHER> sm;
  constexpr int NW = MT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const int n = (int)a.n;
  const int32_t fid = (!GATHER && a.forced) ? a.forced[row] : -1;

  // ---- 1: keys --------------------------------------------------------------
  uint32_t key[E];
  int32_t lv = -1, ff = 0x7fffffff;
  uint32_t nv = 0;
  if (GATHER) {
    // the block list to LDS first, so that every score load of the row is
    // issued in one round (positions from LDS, no dependent global loads)
    const int64_t t = gs.q_pos[row];
    const int32_t nvis = (int32_t)(t < 0 ? 0 : min((t + 1) >> 1, gs.n_cache));
    const int32_t* brow = gs.blocks + row * gs.K_b;
    const float* srow = gs.all + row * gs.a_stride;
    const int nb = (n + BLK - 1) / BLK;  // <= K_b
    // padded with -1 to the slot count, so that every slot reads its block
    // id unconditionally (the reads then go out together)
    for (int i = tid; i < E * MT / BLK; i += MT) sm.blk[i] = i < nb ? brow[i] : -1;
    __syncthreads();
    // the row's visible scores as one buffer resource: 32-bit lane offsets
    // (one register per load instead of a 64-bit address), clipped to n_vis
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(srow), (short)0, (int)(nvis * 4), SEL_BUF_DWORD3);
    static_assert(E <= 32, "one 32-bit mask of the thread's entries");
    uint32_t okm = 0u;  // entry e visible: bit e (one register, not E flags)
    // any caller block id is safe: an id above nvis / 8 (negative ones
    // included, as unsigned) fails the first test, and below it the
    // position fits 32 bits
    const uint32_t nvb = (uint32_t)nvis >> 3;
    static_assert(MT % BLK == 0, "slot c = e * MT + tid: block e * MT / BLK + tid / BLK");
#pragma unroll
    for (int e = 0; e < E; ++e) {
      // slot c = e * MT + tid (c >= n reads a padding -1): one LDS address
      // per thread, the entry in the immediate offset
      const uint32_t blk = (uint32_t)sm.blk[e * (MT / BLK) + (tid >> 3)];
      const uint32_t pos = blk * (uint32_t)BLK + (uint32_t)(tid & 7);
      const bool ok = blk <= nvb && pos < (uint32_t)nvis;
      key[e] = __builtin_amdgcn_raw_buffer_load_b32(rs, ok ? pos << 2 : 0u, 0, 0);
      okm |= (uint32_t)ok << e;
    }
    // branch-free (a branch per entry made the compiler copy the whole key
    // array around each one): a select per entry for the key (the order key
    // as sign-dependent bit flips), the valid entries as one mask whose top
    // bit and popcount give the last valid column and the count
    uint32_t vm = 0u;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t u = key[e];
      const bool ok = ((okm >> e) & 1u) && u != 0xff800000u && (u & 0x7fffffffu) <= 0x7f800000u;
      key[e] = ok ? u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u) : 0u;
      vm |= (uint32_t)ok << e;
    }
    lv = vm ? (31 - __clz((int)vm)) * MT + tid : -1;  // columns grow with e
    nv = (uint32_t)__popc(vm);
  } else {
    const float* srow = a.scores + row * a.s_stride;
    const int32_t* irow = IDS ? a.ids + row * a.id_stride : nullptr;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(srow), (short)0, n * 4, SEL_BUF_DWORD3);
    // (without ids the row's own scores stand in, never read)
    const __amdgpu_buffer_rsrc_t ri = __builtin_amdgcn_make_buffer_rsrc(
        IDS ? (void*)const_cast<int32_t*>(irow) : (void*)const_cast<float*>(srow), (short)0, n * 4,
        SEL_BUF_DWORD3);
    // entries in batches of G (the last batch may be partial: E % G != 0)
    constexpr int G = (IDS && E > 16) ? 16 : E;
    static_assert(E <= 32, "one 32-bit mask of the thread's entries");
    uint32_t vm = 0u;  // entry e valid: bit e
#pragma unroll
    for (int g = 0; g < E; g += G) {
      float sc[G];
      int32_t id[G];
#pragma unroll
      for (int u = 0; u < G; ++u) {
        if (g + u >= E) break;  // compile-time after unrolling
        const int c = (g + u) * MT + tid;
        const uint32_t off = (uint32_t)c << 2;  // past the row: reads as 0, masked here
        const float v = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
        sc[u] = c < n ? v : -INFINITY;
        if (IDS) {
          const int32_t x = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(ri, off, 0, 0);
          id[u] = c < n ? x : -1;
        } else {
          id[u] = c;
        }
      }
#pragma unroll
      for (int u = 0; u < G; ++u) {
        if (g + u >= E) break;
        const int c = (g + u) * MT + tid;
        const bool ok = id[u] >= 0 && !(sc[u] != sc[u]) && sc[u] != -INFINITY;
        const uint32_t su = __float_as_uint(sc[u]);
        key[g + u] = ok ? su ^ ((uint32_t)((int32_t)su >> 31) | 0x80000000u) : 0u;  // order_key
        vm |= (uint32_t)ok << (g + u);
        // the forced id's first column, under a block-uniform branch (with
        // ids while the batch's ids are live)
        if (IDS && fid >= 0) ff = (ok && id[u] == fid && c < ff) ? c : ff;
      }
    }
    // without ids the forced id is its own column
    if (!IDS && fid >= 0) {
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (e * MT + tid == fid && ((vm >> e) & 1u)) ff = fid;
    }
    lv = vm ? (31 - __clz((int)vm)) * MT + tid : -1;  // columns grow with the entry
    nv = (uint32_t)__popc(vm);
  }
  lv = wave_max_i(lv);
  ff = wave_min_i(ff);
  nv = wave_sum(nv);
  if (lane == 0) {
    sm.sh.wred[0 * NW + wave] = (uint32_t)lv;
    sm.sh.wred[1 * NW + wave] = (uint32_t)ff;
    sm.sh.wred[2 * NW + wave] = nv;
  }
  __syncthreads();
  lv = (int32_t)waves_combine(sm.sh.wred + 0 * NW, NW, 0xffffffffu, [](uint32_t x, uint32_t y) {
    return (int32_t)x > (int32_t)y ? x : y;
  });
  ff = (int32_t)waves_combine(sm.sh.wred + 1 * NW, NW, 0x7fffffffu, [](uint32_t x, uint32_t y) {
    return (int32_t)x < (int32_t)y ? x : y;
  });
  nv = waves_combine(sm.sh.wred + 2 * NW, NW, 0u, [](uint32_t x, uint32_t y) { return x + y; });
  int32_t fcol = -1;
  if (a.force_last) fcol = lv;
  else if (fid >= 0 && ff != 0x7fffffff) fcol = ff;
  // the forced entry leaves the ranking and comes back as an "above" bit;
  // it is entry f_e (the same for the whole block) of lane f_lane
  const int f_e = fcol >= 0 ? fcol / MT : -1;
  const bool f_lane = fcol >= 0 && fcol % MT == tid;
#pragma unroll
  for (int e = 0; e < E; ++e) key[e] = (e == f_e && f_lane) ? 0u : key[e];
  const uint32_t k_rem = (uint32_t)a.k - (fcol >= 0 ? 1u : 0u);
  const uint32_t n_rest = nv - (fcol >= 0 ? 1u : 0u);

  // ---- 2: threshold key T and the number of ties at T to take --------------
  uint32_t T = 0u, need = 0u;  // T = 0, need = 0: every valid key (key > 0)
  if (n_rest > k_rem && k_rem == 0u) {
    T = 0xffffffffu;  // above every key: only the forced entry
  } else if (n_rest > k_rem) {
    uint32_t kand = 0xffffffffu, kor = 0u;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (key[e] != 0u) {
        kand &= key[e];
        kor |= key[e];
      }
    kand = wave_and(kand);
    kor = wave_or(kor);
    __syncthreads();  // wred reused
    if (lane == 0) {
      sm.sh.wred[0 * NW + wave] = kand;
      sm.sh.wred[1 * NW + wave] = kor;
    }
    __syncthreads();
    kand = waves_combine(sm.sh.wred + 0 * NW, NW, 0xffffffffu, [](uint32_t x, uint32_t y) { return x & y; });
    kor = waves_combine(sm.sh.wred + 1 * NW, NW, 0u, [](uint32_t x, uint32_t y) { return x | y; });
    const uint32_t diff = kand ^ kor;
    if (diff == 0u) {  // every valid key equal
      T = kand;
      need = k_rem;
    } else {
      const int hb = 31 - __clz(diff), lb = __ffs(diff) - 1;
      uint32_t prefix = hb == 31 ? 0u : (kand & ~((2u << hb) - 1u));
      uint32_t rem = k_rem;
      int hi = hb, lo;
      while (true) {
        lo = hi - 10 > 0 ? hi - 10 : 0;
        const uint32_t dmask = (2u << (hi - lo)) - 1u;  // hi - lo <= 10
        for (int i = tid; i < MBIN; i += MT) sm.hist[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const bool match = key[e] != 0u && (hi == 31 || (key[e] >> (hi + 1)) == (prefix >> (hi + 1)));
          if (match) atomicAdd(&sm.hist[(key[e] >> lo) & dmask], 1u);
        }
        __syncthreads();
        if (wave == 0) wave_find_bin<MBIN>(sm.hist, rem, sm.fb);
        __syncthreads();
        const uint32_t d = sm.fb[0], above = sm.fb[1];
        prefix |= d << lo;
        rem -= above;
        if (lo <= lb) break;
        hi = lo - 1;
      }
      // bits below the last digit are the same in every valid key
      prefix |= kand & ((1u << lo) - 1u);
      T = prefix;
      need = rem;
    }
  }

  // ---- 3: column bitmaps, ordered output -------------------------------------
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool up = key[e] > T || (e == f_e && f_lane);
    const bool tie = need > 0u && key[e] == T;
    const uint64_t mu = __ballot(up), mt = __ballot(tie);
    if (lane == 0) {
      sm.above[e * NW + wave] = mu;
      sm.tied[e * NW + wave] = mt;
    }
  }
  __syncthreads();
  const int nwords = (n + 63) >> 6;  // <= E * NW = MT * E / 64
  static_assert(E * NW <= MT, "one bitmap word per thread");
  const int w = tid;
  uint64_t mu = 0ull, mt = 0ull;
  if (w < nwords) {
    mu = sm.above[w];
    mt = sm.tied[w];
  }
  const uint32_t cu = (uint32_t)__popcll(mu), ct = (uint32_t)__popcll(mt);
  uint32_t tot;
  const uint32_t before = block_exclusive_scan((cu << 16) | ct, sm.sh, &tot);
  const uint32_t t_before = before & 0xffffu;
  uint32_t take = need > t_before ? need - t_before : 0u;
  uint64_t chosen = mu;
  for (uint64_t m = mt; m && take; --take) {
    const uint64_t low = m & (~m + 1ull);  // lowest set bit: smallest tied column
    chosen |= low;
    m ^= low;
  }
  uint32_t pos = (before >> 16) + (t_before < need ? t_before : need);
  int32_t* orow = a.out + row * a.o_stride;
  if (chosen) {
    const int32_t* irow = IDS ? a.ids + row * a.id_stride : nullptr;
    for (uint64_t m = chosen; m; m &= m - 1ull) {
      const int b = __ffsll((unsigned long long)m) - 1;
      const int word_col = 64 * (w & (NW - 1)) + MT * (w / NW);  // first column of word w
      const int c = word_col + b;
      int32_t id;
      if (GATHER) id = sm.blk[c >> 3] * BLK + (c & 7);
      else if (IDS) id = irow[c];
      else id = c;
      if (pos < (uint32_t)a.k) orow[pos] = id;  // never more than k (bounds guard)
      ++pos;
    }
  }
  const uint32_t total = (tot >> 16) + ((tot & 0xffffu) < need ? (tot & 0xffffu) : need);
  for (int j = (int)total + tid; j < a.k; j += MT) orow[j] = -1;
}

template <int MT, int E, bool GATHER, bool IDS>
void launch_many_cfg(int R, const SelArgs& a, const GatherSrc& gs, hipStream_t s) {
  hipLaunchKernelGGL((select_many_kernel<MT, E, GATHER, IDS>), dim3((unsigned)R), dim3(MT), 0, s, a, gs);
}

// (threads, entries per thread) by row length on the many-rows path.  Measured
// on the 8192-row prefill stages: 512 threads beat 256 (fewer entries per
// thread, 4 workgroups per CU at n = 4608, 2 at n = 16,384) and 1024.  The
// kernel is vector-instruction bound there and its per-entry work runs for
// every slot, so a row fills its slots exactly where it can: the 4608-entry
// block stage takes 512 x 9 (128.6-129.1 -> 114-117 us against 512 x 12;
// 256 x 18: 125-126 us).
template <bool GATHER, bool IDS>
void launch_many(int R, int64_t n, const SelArgs& a, const GatherSrc& gs, hipStream_t s) {
  if (n <= 2048) launch_many_cfg<256, 8, GATHER, IDS>(R, a, gs, s);
  else if (n <= 4096) launch_many_cfg<256, 16, GATHER, IDS>(R, a, gs, s);
  else if (n <= 4608) launch_many_cfg<512, 9, GATHER, IDS>(R, a, gs, s);
  else if (n <= 6144) launch_many_cfg<512, 12, GATHER, IDS>(R, a, gs, s);
  else if (n <= 8192) launch_many_cfg<512, 16, GATHER, IDS>(R, a, gs, s);
  else if (n <= 12288) launch_many_cfg<512, 24, GATHER, IDS>(R, a, gs, s);
  else launch_many_cfg<512, 32, GATHER, IDS>(R, a, gs, s);
}

// Rows enough to give every CU several workgroups of the many-rows kernel.
constexpr int MANY_ROWS = 1024;
bool many_path(int64_t R, int64_t n) { return R >= MANY_ROWS && n <= 16384; }
// Few rows of 4K-16K entries (the decode's position stage, 16,384
// candidates per query; the 128K decode's block stage, 8192 blocks): the
// same kernel with 1024 threads per row, one row per CU, beats the
// register-row kernel's sampled bracket (8 rows of 16,384: 19.0 -> 16.4 us;
// 32 rows of 8192: 13.4 -> 9.4 us); at 65,536 entries (the 1M block stage)
// it loses to the split classify / finish pair (39.5 vs 24.8 us).
bool wide_path(int64_t R, int64_t n) { return R < MANY_ROWS && n > 4096 && n <= 16384; }

// Path choice.  One CU works through a register-held row at a few entries
// per lane-cycle, so a row of more than 16K entries is faster spread over
// many workgroups (split path) when there are too few rows to fill the chip.
bool sampled_ok(int64_t n, int k) { return n >= 4 * SAMPLE && n <= MAX_N_FAST && k <= KFAST; }
bool rows_path(int64_t R, int64_t n) { return n <= 16 * THREADS || (R >= 256 && n <= 32 * THREADS); }
bool split_path(int64_t R, int64_t n, int k) {
  return !rows_path(R, n) && R < 256 && sampled_ok(n, k);
}

}  // namespace

size_t select_workspace_bytes(int64_t R, int64_t n, int64_t k) {
  if (!split_path(R, n, (int)k)) return 0;
  const int64_t ch = split_chunk(R);
  const int64_t nchunks = (n + ch - 1) / ch;
  return (size_t)(R * nchunks) * sizeof(Slot);
}

bool gather_select_supported(int64_t R, int64_t n) { return rows_path(R, n); }

hipError_t launch_gather_select(int R, const float* all, int64_t a_stride, int64_t n_cache,
                                const int64_t* q_pos, const int32_t* blocks, int K_b, int k,
                                int32_t* out, int64_t o_stride, hipStream_t s) {
  const int64_t n = (int64_t)K_b * BLK;
  if (!rows_path(R, n)) return hipErrorInvalidValue;  // rejected before launch
  SelArgs a{nullptr, 0, nullptr, 0, nullptr, 0, n, k, out, o_stride};
  const GatherSrc gs{all, a_stride, blocks, K_b, q_pos, n_cache};
  if (many_path(R, n)) {
    launch_many<true, false>(R, n, a, gs, s);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)R), block(THREADS);
  if (n <= 8 * THREADS) hipLaunchKernelGGL((select_rows_kernel<8, true>), grid, block, 0, s, a, gs);
  else if (n <= 16 * THREADS) hipLaunchKernelGGL((select_rows_kernel<16, true>), grid, block, 0, s, a, gs);
  else hipLaunchKernelGGL((select_rows_kernel<32, true>), grid, block, 0, s, a, gs);
  return hipGetLastError();
}

hipError_t launch_select_topk(int R, int64_t n, const float* scores, int64_t s_stride,
                              const int32_t* ids, int64_t id_stride, const int32_t* forced,
                              int force_last, int k, int32_t* out, int64_t o_stride, void* ws,
                              hipStream_t s) {
  SelArgs a{scores, s_stride, ids, id_stride, forced, force_last, n, k, out, o_stride};
  if (wide_path(R, n)) {
    const GatherSrc none{};
    if (n <= 8192) {
      if (ids) launch_many_cfg<1024, 8, false, true>(R, a, none, s);
      else launch_many_cfg<1024, 8, false, false>(R, a, none, s);
    } else {
      if (ids) launch_many_cfg<1024, 16, false, true>(R, a, none, s);
      else launch_many_cfg<1024, 16, false, false>(R, a, none, s);
    }
    return hipGetLastError();
  }
  if (many_path(R, n)) {
    const GatherSrc none{};
    if (ids) launch_many<false, true>(R, n, a, none, s);
    else launch_many<false, false>(R, n, a, none, s);
    return hipGetLastError();
  }
  if (rows_path(R, n)) {
    const dim3 grid((unsigned)R), block(THREADS);
    const GatherSrc none{};
    if (n <= 8 * THREADS) hipLaunchKernelGGL((select_rows_kernel<8, false>), grid, block, 0, s, a, none);
    else if (n <= 16 * THREADS) hipLaunchKernelGGL((select_rows_kernel<16, false>), grid, block, 0, s, a, none);
    else hipLaunchKernelGGL((select_rows_kernel<32, false>), grid, block, 0, s, a, none);
    return hipGetLastError();
  }
  if (split_path(R, n, k)) {
    const int64_t ch = split_chunk(R);
    const int nchunks = (int)((n + ch - 1) / ch);
    Slot* slots = static_cast<Slot*>(ws);
    if (ch == CHUNK_FEW)
      hipLaunchKernelGGL(select_classify_kernel<CHUNK_FEW>, dim3((unsigned)nchunks, (unsigned)R),
                         dim3(CLS_THREADS), 0, s, a, slots, nchunks);
    else
      hipLaunchKernelGGL(select_classify_kernel<CHUNK_MANY>, dim3((unsigned)nchunks, (unsigned)R),
                         dim3(CLS_THREADS), 0, s, a, slots, nchunks);
    hipLaunchKernelGGL(select_finish_kernel, dim3((unsigned)R), dim3(THREADS), 0, s, a, slots,
                       nchunks);
    return hipGetLastError();
  }
  const int try_sampled = sampled_ok(n, k) ? 1 : 0;
  hipLaunchKernelGGL(select_topk_kernel, dim3((unsigned)R), dim3(THREADS), 0, s, a, try_sampled);
  return hipGetLastError();
}

}  // namespace csa2
