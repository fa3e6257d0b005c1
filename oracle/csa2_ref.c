/*
 * csa2_ref.c -- plain CPU oracle for the CSA2 hot path (test infrastructure
 * only; see csa2_ref.h for the contract, the sources and the readings).
 *
 * Written for obviousness, not speed: every step follows the method's
 * definition directly, in IEEE double, with library sorting (qsort) as the
 * only primitive.  OpenMP only spreads independent rows / positions over
 * host cores; it never changes what is summed or in which order a single
 * result is formed.
 */
#include "csa2_ref.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

/* Threads of the OpenMP regions below (only independent rows / positions
 * are spread over them): the count the next region uses, and setting it. */
int csa2ref_threads(void) { return omp_get_max_threads(); }
void csa2ref_set_threads(int n) {
  if (n > 0) omp_set_num_threads(n);
}

/* ===================================================================== */
/* Element decoders, written from the format definitions.                */
/* ===================================================================== */

/* bfloat16: the upper 16 bits of an IEEE-754 binary32 word. */
double csa2ref_bf16(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* OCP 8-bit E4M3FN: sign, 4 exponent bits (bias 7), 3 mantissa bits.
 * Exponent field 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; there is no
 * infinity, so the largest finite magnitude is 1.75 * 2^8 = 448.  The cache
 * format named by the NVFP4 article (section 3.2, E4M3 group scale; section
 * 3.1, FP8 window) is this one. */
double csa2ref_e4m3(uint8_t bits) {
  int s = (bits >> 7) & 1;
  int e = (bits >> 3) & 15;
  int m = bits & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    mag = ldexp((double)m / 8.0, -6);
  else
    mag = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -mag : mag;
}

/* OCP 4-bit E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit; exponent
 * field 0 is subnormal (m * 0.5).  Magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6. */
double csa2ref_e2m1(uint8_t nibble) {
  int s = (nibble >> 3) & 1;
  int e = (nibble >> 1) & 3;
  int m = nibble & 1;
  double mag;
  if (e == 0)
    mag = 0.5 * (double)m;
  else
    mag = ldexp(1.0 + 0.5 * (double)m, e - 1);
  return s ? -mag : mag;
}

/* OCP MX E8M0 scale: 2^(e-127) for e < 255; 0xFF is NaN.  The format of
 * the per-32 scales of MXFP4 (the NVFP4 article's section 4 names MXFP4 as
 * E2M1 values with one UE8M0 scale per 32 elements). */
double csa2ref_e8m0(uint8_t bits) {
  if (bits == 0xFF) return NAN;
  return ldexp(1.0, (int)bits - 127);
}

/* Round a double to the nearest bfloat16 (8 significant bits, binary32
 * exponent range), ties to even, by scaling to the value's quantum and
 * rounding with nearbyint() under the default round-to-nearest-even mode. */
uint16_t csa2ref_round_bf16(double x) {
  double a, quantum, r;
  int e, unb;
  float f;
  uint32_t u;
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  if (isnan(x)) return 0x7FC0;
  a = fabs(x);
  if (a == 0.0) return sign;
  if (isinf(a)) return (uint16_t)(sign | 0x7F80);
  frexp(a, &e);  /* a in [2^(e-1), 2^e) */
  unb = e - 1;
  if (unb < -126) unb = -126; /* subnormal range shares the quantum 2^-133 */
  quantum = ldexp(1.0, unb - 7);
  r = nearbyint(a / quantum) * quantum;
  if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80);
  f = (float)r; /* exact: r has at most 8 significant bits */
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(sign | (u >> 16));
}

/* ===================================================================== */
/* Visibility.                                                           */
/* ===================================================================== */

/* Latent g pools raw tokens 2g, 2g+1 and exists once token 2g+1 has been
 * seen (the Compressor emits one latent per completed pair; the article's
 * section 3.2 keeps the unfinished half in state).  A query at raw position
 * t therefore sees latents g < (t+1)/2, capped by what the cache holds. */
int64_t csa2ref_n_vis(int64_t t, int64_t n_cache) {
  int64_t n;
  if (t < 0) return 0;
  n = (t + 1) / 2;
  return n < n_cache ? n : n_cache;
}

/* The block holding the newest visible latent (section 3.3 keeps it). */
int64_t csa2ref_newest_block(int64_t t, int64_t n_cache) {
  int64_t nv = csa2ref_n_vis(t, n_cache);
  if (nv <= 0) return -1;
  return (nv + CSA2REF_BLK - 1) / CSA2REF_BLK - 1;
}

/* ===================================================================== */
/* a1: Compressor -- softmax over the two tokens of a group, per channel,  */
/* then the gate-weighted sum (NVFP4 article, section 3.2).                */
/* ===================================================================== */
void csa2ref_compress(int B, int T, const uint16_t *kv, int64_t kv_sb,
                      const uint16_t *gate, int64_t g_sb, uint16_t *out,
                      int64_t out_sb, double *out_f64) {
  int G = T / 2;
  for (int b = 0; b < B; ++b) {
#pragma omp parallel for schedule(static)
    for (int g = 0; g < G; ++g) {
      for (int c = 0; c < CSA2REF_D; ++c) {
        double x0 = csa2ref_bf16(kv[b * kv_sb + (int64_t)(2 * g) * CSA2REF_D + c]);
        double x1 = csa2ref_bf16(kv[b * kv_sb + (int64_t)(2 * g + 1) * CSA2REF_D + c]);
        double l0 = csa2ref_bf16(gate[b * g_sb + (int64_t)(2 * g) * CSA2REF_D + c]);
        double l1 = csa2ref_bf16(gate[b * g_sb + (int64_t)(2 * g + 1) * CSA2REF_D + c]);
        double m = l0 > l1 ? l0 : l1;
        double e0 = exp(l0 - m), e1 = exp(l1 - m);
        double y = (e0 * x0 + e1 * x1) / (e0 + e1);
        out[b * out_sb + (int64_t)g * CSA2REF_D + c] = csa2ref_round_bf16(y);
        if (out_f64) out_f64[((int64_t)b * G + g) * CSA2REF_D + c] = y;
      }
    }
  }
}

/* ===================================================================== */
/* Indexer score of one latent: sum over the 32 index heads of            */
/* w_h * ReLU(q_h . k)  (section 3.3 of the NVFP4 article: ReLU, then a    */
/* per-head weight, summed over heads).                                   */
/* ===================================================================== */
static void decode_key_row(const void *k, int k_fmt, int64_t row, double *dst) {
  if (k_fmt == CSA2REF_BF16) {
    const uint16_t *p = (const uint16_t *)k + row * CSA2REF_DI;
    for (int d = 0; d < CSA2REF_DI; ++d) dst[d] = csa2ref_bf16(p[d]);
  } else if (k_fmt == CSA2REF_MXFP4) {
    /* the oracle's packed row: 64 code bytes (dim 2i in the low nibble of
     * byte i) then the 4 E8M0 scales of dims 0-31, 32-63, 64-95, 96-127 */
    const uint8_t *p = (const uint8_t *)k + row * CSA2REF_MXFP4_ROW;
    for (int d = 0; d < CSA2REF_DI; ++d) {
      uint8_t byte = p[d / 2];
      uint8_t nib = (d & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
      dst[d] = csa2ref_e2m1(nib) * csa2ref_e8m0(p[64 + d / 32]);
    }
  } else {
    const uint8_t *p = (const uint8_t *)k + row * CSA2REF_DI;
    for (int d = 0; d < CSA2REF_DI; ++d) dst[d] = csa2ref_e4m3(p[d]);
  }
}

static double index_score(const double *qd /*[32][128]*/, const float *w,
                          const double *kd /*[128]*/) {
  double s = 0.0;
  for (int h = 0; h < CSA2REF_HI; ++h) {
    double dot = 0.0;
    for (int d = 0; d < CSA2REF_DI; ++d) dot += qd[h * CSA2REF_DI + d] * kd[d];
    s += (double)w[h] * (dot > 0.0 ? dot : 0.0);
  }
  return s;
}

/* The index query in the key's number format.  The NVFP4 article (section
 * 3.3) runs the indexer on FP4-quantised index queries; the pages do not say
 * how a query meets a key of another format.  Reading: the query is rounded
 * to the format of the keys it is scored against -- E4M3 keys: the nearest
 * E4M3 value; MXFP4 keys: the nearest E2M1 value (unit block scale) -- and
 * stays bf16 for bf16 keys.  Both roundings are nearest, ties to the even
 * code, saturating at the largest finite magnitude (448 / 6), the sign taken
 * from x < 0.  The search runs over every finite code in double. */
uint8_t csa2ref_round_e4m3(double x) {
  double a = fabs(x), best_d = INFINITY;
  uint8_t best = 0;
  if (isnan(x)) return 0x7F;
  /* at or past the largest finite value: saturate (for huge |x| the two
   * largest candidates' distances would round to the same double) */
  if (a >= 448.0) return (uint8_t)(0x7E | (x < 0.0 ? 0x80 : 0));
  for (int c = 0; c <= 0x7E; ++c) { /* every finite non-negative code */
    double d = fabs(csa2ref_e4m3((uint8_t)c) - a);
    if (d < best_d || (d == best_d && (c & 1) == 0)) {
      best = (uint8_t)c;
      best_d = d;
    }
  }
  return (uint8_t)(best | (x < 0.0 ? 0x80 : 0));
}

uint8_t csa2ref_round_e2m1(double x) {
  double a = fabs(x), best_d = INFINITY;
  uint8_t best = 0;
  if (a >= 6.0) return (uint8_t)(7 | (x < 0.0 ? 8 : 0)); /* saturate, as above */
  for (int c = 0; c < 8; ++c) { /* the eight magnitudes */
    double d = fabs(csa2ref_e2m1((uint8_t)c) - a);
    if (d < best_d || (d == best_d && (c & 1) == 0)) {
      best = (uint8_t)c;
      best_d = d;
    }
  }
  return (uint8_t)(best | (x < 0.0 ? 8 : 0));
}

static void decode_index_query(const uint16_t *q, int k_fmt, double *qd) {
  for (int i = 0; i < CSA2REF_HI * CSA2REF_DI; ++i) {
    double x = csa2ref_bf16(q[i]);
    if (k_fmt == CSA2REF_E4M3)
      x = csa2ref_e4m3(csa2ref_round_e4m3(x));
    else if (k_fmt == CSA2REF_MXFP4)
      x = csa2ref_e2m1(csa2ref_round_e2m1(x));
    qd[i] = x;
  }
}

/* ===================================================================== */
/* a2: score every visible latent; block score = max over the block's     */
/* visible latents (section 3.3: a block is represented by its best       */
/* in-block score).                                                       */
/* ===================================================================== */
void csa2ref_scan(int B, int Tq, const uint16_t *q, const float *w,
                  const void *k, int k_fmt, int64_t k_sb, int64_t n_cache,
                  const int64_t *q_pos, double *scores, int64_t s_stride,
                  double *block_max, int64_t bm_stride) {
  int64_t nblk = (n_cache + CSA2REF_BLK - 1) / CSA2REF_BLK;
  double *tmp = (double *)malloc(sizeof(double) * (size_t)(n_cache > 0 ? n_cache : 1));
  double *qd = (double *)malloc(sizeof(double) * CSA2REF_HI * CSA2REF_DI);
  for (int r = 0; r < B * Tq; ++r) {
    int b = r / Tq;
    int64_t nv = csa2ref_n_vis(q_pos[r], n_cache);
    const float *wr = w + (int64_t)r * CSA2REF_HI;
    const void *kb = (k_fmt == CSA2REF_BF16)
                         ? (const void *)((const uint16_t *)k + b * k_sb)
                         : (const void *)((const uint8_t *)k + b * k_sb); /* bytes */
    decode_index_query(q + (int64_t)r * CSA2REF_HI * CSA2REF_DI, k_fmt, qd);
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < n_cache; ++p) {
      double kd[CSA2REF_DI];
      if (p < nv) {
        decode_key_row(kb, k_fmt, p, kd);
        tmp[p] = index_score(qd, wr, kd);
      } else {
        tmp[p] = -INFINITY;
      }
    }
    if (scores)
      for (int64_t p = 0; p < n_cache; ++p) scores[r * s_stride + p] = tmp[p];
    if (block_max) {
      for (int64_t bl = 0; bl < nblk; ++bl) {
        double m = -INFINITY;
        for (int i = 0; i < CSA2REF_BLK; ++i) {
          int64_t p = bl * CSA2REF_BLK + i;
          if (p < nv && tmp[p] > m) m = tmp[p];
        }
        block_max[r * bm_stride + bl] = m;
      }
    }
  }
  free(qd);
  free(tmp);
}

/* ===================================================================== */
/* a3 / a5: top-k by (score descending, id ascending).                    */
/* ===================================================================== */
typedef struct {
  double s;
  int32_t id;
} entry_t;

static int by_key(const void *pa, const void *pb) {
  const entry_t *a = (const entry_t *)pa, *b = (const entry_t *)pb;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  return (a->id > b->id) - (a->id < b->id);
}

static int by_int(const void *pa, const void *pb) {
  int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
  return (a > b) - (a < b);
}

void csa2ref_select(int R, int64_t n, const double *scores, int64_t s_stride,
                    const int32_t *ids, int64_t id_stride,
                    const int32_t *forced, int k, int32_t *out,
                    int64_t o_stride) {
#pragma omp parallel for schedule(dynamic)
  for (int r = 0; r < R; ++r) {
    entry_t *e = (entry_t *)malloc(sizeof(entry_t) * (size_t)(n > 0 ? n : 1));
    int32_t *pick = (int32_t *)malloc(sizeof(int32_t) * (size_t)(k > 0 ? k : 1));
    int64_t cnt = 0;
    int have_forced = 0, npick = 0;
    int32_t f = forced ? forced[r] : -1;
    for (int64_t j = 0; j < n; ++j) {
      double s = scores[r * s_stride + j];
      int32_t id = ids ? ids[r * id_stride + j] : (int32_t)j;
      if (id < 0 || isnan(s) || s == -INFINITY) continue;
      if (f >= 0 && id == f) {
        have_forced = 1; /* kept regardless of its score */
        continue;
      }
      e[cnt].s = s;
      e[cnt].id = id;
      ++cnt;
    }
    qsort(e, (size_t)cnt, sizeof(entry_t), by_key);
    if (have_forced && k > 0) pick[npick++] = f;
    for (int64_t j = 0; j < cnt && npick < k; ++j) pick[npick++] = e[j].id;
    qsort(pick, (size_t)npick, sizeof(int32_t), by_int);
    for (int j = 0; j < k; ++j) out[r * o_stride + j] = j < npick ? pick[j] : -1;
    free(pick);
    free(e);
  }
}

/* ===================================================================== */
/* a4: the current layer's indexer over the latents of the chosen blocks. */
/* ===================================================================== */
void csa2ref_cand(int B, int Tq, const uint16_t *q, const float *w,
                  const void *k, int k_fmt, int64_t k_sb, int64_t n_cache,
                  const int64_t *q_pos, const int32_t *blocks, int K_b,
                  double *scores, int32_t *ids, int64_t stride) {
#pragma omp parallel for schedule(dynamic)
  for (int r = 0; r < B * Tq; ++r) {
    int b = r / Tq;
    double *qd = (double *)malloc(sizeof(double) * CSA2REF_HI * CSA2REF_DI);
    double kd[CSA2REF_DI];
    int64_t nv = csa2ref_n_vis(q_pos[r], n_cache);
    const void *kb = (k_fmt == CSA2REF_BF16)
                         ? (const void *)((const uint16_t *)k + b * k_sb)
                         : (const void *)((const uint8_t *)k + b * k_sb); /* bytes */
    decode_index_query(q + (int64_t)r * CSA2REF_HI * CSA2REF_DI, k_fmt, qd);
    for (int j = 0; j < K_b; ++j) {
      int32_t blk = blocks[(int64_t)r * K_b + j];
      for (int i = 0; i < CSA2REF_BLK; ++i) {
        int64_t col = r * stride + (int64_t)j * CSA2REF_BLK + i;
        int64_t g = (int64_t)blk * CSA2REF_BLK + i;
        if (blk >= 0 && g < nv) {
          decode_key_row(kb, k_fmt, g, kd);
          scores[col] = index_score(qd, w + (int64_t)r * CSA2REF_HI, kd);
          ids[col] = (int32_t)g;
        } else {
          scores[col] = -INFINITY;
          ids[col] = -1;
        }
      }
    }
    free(qd);
  }
}

/* ===================================================================== */
/* a6: attention of 64 heads over Sel (compressed latents) and the raw     */
/* window (NVFP4 article, section 3 and 3.4), K = V = the latent row, plus */
/* a per-head sink logit that only enlarges the softmax denominator.      */
/* ===================================================================== */
static void decode_latent_row(const void *lat, int lat_fmt,
                              const uint8_t *lat_scale, int64_t row,
                              double *dst) {
  if (lat_fmt == CSA2REF_BF16) {
    const uint16_t *p = (const uint16_t *)lat + row * CSA2REF_D;
    for (int c = 0; c < CSA2REF_D; ++c) dst[c] = csa2ref_bf16(p[c]);
  } else { /* NVFP4: value = E2M1 code * E4M3 scale of its 16-element group */
    const uint8_t *p = (const uint8_t *)lat + row * (CSA2REF_D / 2);
    const uint8_t *sc = lat_scale + row * (CSA2REF_D / 16);
    for (int c = 0; c < CSA2REF_D; ++c) {
      uint8_t byte = p[c / 2];
      uint8_t nib = (c & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
      dst[c] = csa2ref_e2m1(nib) * csa2ref_e4m3(sc[c / 16]);
    }
  }
}

static void decode_window_row(const void *win, int win_fmt,
                              const float *win_scale, int64_t slot,
                              double *dst) {
  if (win_fmt == CSA2REF_BF16) {
    const uint16_t *p = (const uint16_t *)win + slot * CSA2REF_D;
    for (int c = 0; c < CSA2REF_D; ++c) dst[c] = csa2ref_bf16(p[c]);
  } else { /* FP8 E4M3 with one f32 scale per token */
    const uint8_t *p = (const uint8_t *)win + slot * CSA2REF_D;
    double s = (double)win_scale[slot];
    for (int c = 0; c < CSA2REF_D; ++c) dst[c] = csa2ref_e4m3(p[c]) * s;
  }
}

void csa2ref_attn(int B, int Tq, const uint16_t *q, int64_t q_sb,
                  const void *lat, int lat_fmt, const uint8_t *lat_scale,
                  int64_t lat_sb, int64_t n_cache, const int32_t *sel, int K,
                  int64_t sel_sb, const void *win, int win_fmt,
                  const float *win_scale, int W, int W_cap, int64_t win_sb,
                  const int64_t *q_pos, const float *sink, double scale,
                  double *out, double *lse) {
#pragma omp parallel for schedule(dynamic)
  for (int r = 0; r < B * Tq; ++r) {
    int b = r / Tq, tq = r % Tq;
    int64_t t = q_pos[r];
    int64_t w0 = t - W + 1 < 0 ? 0 : t - W + 1;
    int nrow_max = K + W;
    double *kv = (double *)malloc(sizeof(double) * (size_t)nrow_max * CSA2REF_D);
    double *lg = (double *)malloc(sizeof(double) * (size_t)nrow_max);
    double qd[CSA2REF_D];
    int nrow = 0;
    /* source 2: the selected compressed latents */
    for (int j = 0; j < K; ++j) {
      int32_t g = sel[(int64_t)r * sel_sb + j];
      if (g < 0 || g >= n_cache) continue;
      if (lat_fmt == CSA2REF_BF16)
        decode_latent_row((const uint16_t *)lat + b * lat_sb * CSA2REF_D, lat_fmt,
                          NULL, g, kv + (int64_t)nrow * CSA2REF_D);
      else
        decode_latent_row((const uint8_t *)lat + b * lat_sb * (CSA2REF_D / 2), lat_fmt,
                          lat_scale + b * lat_sb * (CSA2REF_D / 16), g,
                          kv + (int64_t)nrow * CSA2REF_D);
      ++nrow;
    }
    /* source 1: the raw sliding window, positions w0 .. t */
    for (int64_t p = w0; p <= t; ++p) {
      int64_t slot = p % W_cap;
      if (win_fmt == CSA2REF_BF16)
        decode_window_row((const uint16_t *)win + b * win_sb * CSA2REF_D, win_fmt,
                          NULL, slot, kv + (int64_t)nrow * CSA2REF_D);
      else
        decode_window_row((const uint8_t *)win + b * win_sb * CSA2REF_D, win_fmt,
                          win_scale + b * win_sb, slot, kv + (int64_t)nrow * CSA2REF_D);
      ++nrow;
    }
    for (int h = 0; h < CSA2REF_HQ; ++h) {
      const uint16_t *qh = q + b * q_sb + ((int64_t)tq * CSA2REF_HQ + h) * CSA2REF_D;
      double m = (double)sink[h], z, *o;
      for (int c = 0; c < CSA2REF_D; ++c) qd[c] = csa2ref_bf16(qh[c]);
      for (int i = 0; i < nrow; ++i) {
        double dot = 0.0;
        for (int c = 0; c < CSA2REF_D; ++c) dot += qd[c] * kv[(int64_t)i * CSA2REF_D + c];
        lg[i] = dot * scale;
        if (lg[i] > m) m = lg[i];
      }
      z = exp((double)sink[h] - m);
      for (int i = 0; i < nrow; ++i) z += exp(lg[i] - m);
      o = out + ((int64_t)r * CSA2REF_HQ + h) * CSA2REF_D;
      for (int c = 0; c < CSA2REF_D; ++c) o[c] = 0.0;
      for (int i = 0; i < nrow; ++i) {
        double p = exp(lg[i] - m) / z;
        for (int c = 0; c < CSA2REF_D; ++c) o[c] += p * kv[(int64_t)i * CSA2REF_D + c];
      }
      if (lse) lse[(int64_t)r * CSA2REF_HQ + h] = m + log(z);
    }
    free(lg);
    free(kv);
  }
}

/* ===================================================================== */
/* a7: standalone dequantisation.                                         */
/* ===================================================================== */
void csa2ref_dequant_fp8(const uint8_t *src, const float *row_scale,
                         int64_t rows, int cols, double *dst) {
  for (int64_t r = 0; r < rows; ++r) {
    double s = row_scale ? (double)row_scale[r] : 1.0;
    for (int c = 0; c < cols; ++c)
      dst[r * cols + c] = csa2ref_e4m3(src[r * cols + c]) * s;
  }
}

void csa2ref_dequant_nvfp4(const uint8_t *packed, const uint8_t *scales,
                           int64_t rows, int cols, double *dst) {
  for (int64_t r = 0; r < rows; ++r)
    for (int c = 0; c < cols; ++c) {
      uint8_t byte = packed[r * (cols / 2) + c / 2];
      uint8_t nib = (c & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
      dst[r * cols + c] = csa2ref_e2m1(nib) * csa2ref_e4m3(scales[r * (cols / 16) + c / 16]);
    }
}

/* ===================================================================== */
/* f1: NVFP4 quantisation of compressed latents (NVFP4 article, section   */
/* 3.2: the cache holds E2M1 values in groups of 16 sharing one E4M3      */
/* scale).  The article names the format, not the encoder; the reading    */
/* taken here is the plain one:                                           */
/*   scale  = the E4M3 value nearest to amax/6 (6 = largest E2M1          */
/*            magnitude), ties to the even code, saturating at 448;       */
/*   code_i = the E2M1 value nearest to x_i / scale, ties to the even     */
/*            code, saturating at +-6, sign taken from x_i;               */
/*   a group whose scale rounds to 0 stores scale 0 and all-zero codes.   */
/* "Nearest" is decided on the exact real quotients: both quotients are   */
/* formed in double, whose rounding cannot move a quotient of an fp32     */
/* numerator by an E4M3 / E2M1 value onto or across a rounding midpoint   */
/* (a midpoint has at most 5 significant bits, the exact quotient either  */
/* equals it or differs from it by far more than 2^-53 relative).  The    */
/* search is a brute-force scan over every finite code.                   */
/* ===================================================================== */
uint8_t csa2ref_quant_scale_e4m3(float amax) {
  double target = (double)amax / 6.0;
  uint8_t best = 0;
  double best_d = INFINITY;
  for (int c = 0; c <= 0x7E; ++c) { /* every finite non-negative code */
    double d = fabs(csa2ref_e4m3((uint8_t)c) - target);
    if (d < best_d || (d == best_d && (c & 1) == 0)) {
      best = (uint8_t)c;
      best_d = d;
    }
  }
  return best;
}

uint8_t csa2ref_quant_e2m1(float x, uint8_t scale_code) {
  double s = csa2ref_e4m3(scale_code);
  double target, best_d = INFINITY;
  uint8_t best = 0;
  if (s == 0.0) return 0;
  target = fabs((double)x) / s;
  /* saturate at 6 first: for a huge quotient the distances to 4 and 6 would
   * round to the same double and the tie rule would pick 4 */
  if (target >= 6.0) return (uint8_t)(7 | (x < 0.0f ? 8 : 0));
  for (int c = 0; c < 8; ++c) { /* the eight magnitudes */
    double d = fabs(csa2ref_e2m1((uint8_t)c) - target);
    if (d < best_d || (d == best_d && (c & 1) == 0)) {
      best = (uint8_t)c;
      best_d = d;
    }
  }
  return (uint8_t)(best | (x < 0.0f ? 8 : 0));
}

void csa2ref_quant_nvfp4(const float *src, int64_t rows, int cols,
                         uint8_t *packed, uint8_t *scales) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int g = 0; g < cols / 16; ++g) {
      const float *x = src + r * cols + 16 * g;
      float amax = 0.0f;
      uint8_t sc;
      for (int i = 0; i < 16; ++i)
        if (fabsf(x[i]) > amax) amax = fabsf(x[i]);
      sc = csa2ref_quant_scale_e4m3(amax);
      scales[r * (cols / 16) + g] = sc;
      for (int i = 0; i < 16; i += 2) {
        uint8_t lo = csa2ref_quant_e2m1(x[i], sc);
        uint8_t hi = csa2ref_quant_e2m1(x[i + 1], sc);
        packed[r * (cols / 2) + (16 * g + i) / 2] = (uint8_t)(lo | (hi << 4));
      }
    }
  }
}
