/*
 * csa2_ref.h -- plain CPU oracle for the CSA2 (Compressed Sparse Attention 2)
 * decode / prefill hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or
 * call this library: only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark use it.  It shares no code, header, table or helper with
 * the HIP library.
 *
 * Sources (web pages; cited by page title and section):
 *   [NVFP4]  "DeepSeek-V4.1-Flash-NVFP4" article (lpnh.cn/news/2752702):
 *            section 3 (two KV sources, 128 + 512 = 640 positions),
 *            3.1 (128-token sliding window ring), 3.2 (2:1 softmax-gated
 *            Compressor, NVFP4 cache with 16-element groups and E4M3 scale),
 *            3.3 (block-level top-2048 over blocks of 8 scored by their
 *            in-block maximum with the newest block always kept; 32-head
 *            ReLU + per-head weighted indexer keeping the top 512 positions),
 *            3.4 (one-pass gather + online-softmax sparse attention with a
 *            learnable per-head attention sink).
 *   [OQ3E]   "CSA2 sparse attention, 384-expert MoE and 1M context in
 *            DeepSeek-V4.1-Flash-1017-oQ3e-ngram-mtp" (nxmr.cn/news/161930):
 *            section 2.1 (index_n_heads 32, index_head_dim 128,
 *            index_topk 512, candidate_block_size 8, candidate_topk_blocks
 *            2048, sliding_window 128), section 1 (64 Q heads, 1 KV head).
 *
 * Every floating-point quantity is computed in IEEE double.  All arrays are
 * host memory in the same logical layouts the device library uses; strides
 * are in elements, innermost dimension contiguous.
 *
 * Readings of points the pages leave open:
 *   - latent g pools raw tokens 2g and 2g+1; a query at raw position t sees
 *     latent g iff 2g+1 <= t, i.e. n_vis(t) = min(N, (t+1)/2);
 *   - block b holds latents [8b, 8b+8); its score is the max over its
 *     visible latents; the newest block is ceil(n_vis/8)-1;
 *   - ties in every top-k are broken by the smaller id;
 *   - the window holds raw positions max(0, t-W+1) .. t (the query's own
 *     token included), stored at slot (pos mod W_cap);
 *   - selected latents and window rows are both attended (no dedup);
 *   - K = V = the 512-wide latent; logits scaled by `scale`; the sink is a
 *     per-head logit that enters only the softmax denominator.
 */
#ifndef CSA2_REF_H
#define CSA2_REF_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage formats understood by the oracle's decoders. */
#define CSA2REF_BF16 1  /* bfloat16 bytes                                  */
#define CSA2REF_E4M3 2  /* OCP FP8 E4M3FN bytes                            */
#define CSA2REF_NVFP4 3 /* E2M1 nibbles + one E4M3 scale per 16 elements   */
#define CSA2REF_F32 4
#define CSA2REF_MXFP4 5 /* index keys: E2M1 codes + one E8M0 scale per 32  */
#define CSA2REF_MXFP4_ROW 68 /* oracle key row: 64 code bytes, 4 scales  */

#define CSA2REF_D 512   /* latent width (one shared KV head)               */
#define CSA2REF_HQ 64   /* query heads                                     */
#define CSA2REF_HI 32   /* index heads                                     */
#define CSA2REF_DI 128  /* index head width                                */
#define CSA2REF_BLK 8   /* candidate block size (latents)                  */

/* ---- threads: OpenMP spreads independent rows / positions only ------ */
int csa2ref_threads(void);        /* threads the next parallel region uses */
void csa2ref_set_threads(int n);  /* n > 0                                 */

/* ---- element decoders (format definitions, no tables) ---------------- */
double csa2ref_bf16(uint16_t bits);
double csa2ref_e4m3(uint8_t bits);   /* NaN for S.1111.111                */
double csa2ref_e2m1(uint8_t nibble); /* low 4 bits used                   */
double csa2ref_e8m0(uint8_t bits);   /* 2^(bits-127); NaN for 0xFF        */
uint16_t csa2ref_round_bf16(double x); /* round-to-nearest-even to bf16   */

/* ---- the index query in the key's format ----------------------------- */
/* Nearest E4M3 code / E2M1 nibble to x, ties to the even code, saturating
 * at 448 / 6, sign bit from x < 0 (E4M3: NaN gives 0x7F).  The indexer
 * rounds the bf16 index query this way before scoring it against E4M3 or
 * MXFP4 keys (reading of the NVFP4 article, section 3.3: FP4 index
 * queries); bf16 keys meet the bf16 query unrounded.                      */
uint8_t csa2ref_round_e4m3(double x);
uint8_t csa2ref_round_e2m1(double x);

/* ---- visibility helpers -------------------------------------------- */
int64_t csa2ref_n_vis(int64_t t, int64_t n_cache);
int64_t csa2ref_newest_block(int64_t t, int64_t n_cache); /* -1 if none */

/* ---- a1: 2:1 softmax-gated pooling ---------------------------------- */
/* kv, gate: bf16 [B][T][512] (batch strides kv_sb, g_sb elements), T even.
 * out: bf16 [B][T/2][512] (batch stride out_sb), rounded to nearest even;
 * out_f64 (optional, may be NULL): the same values before rounding,
 * [B][T/2][512] densely packed.                                           */
void csa2ref_compress(int B, int T, const uint16_t *kv, int64_t kv_sb,
                      const uint16_t *gate, int64_t g_sb, uint16_t *out,
                      int64_t out_sb, double *out_f64);

/* ---- a2: index scores over all visible latents + block max ---------- */
/* q: bf16 [B][Tq][32][128], rounded to the key format first (see
 * csa2ref_round_e4m3 / _e2m1); w: f32 [B][Tq][32]; q_pos: [B][Tq].
 * scores (optional): [B*Tq][s_stride], -inf for invisible positions.
 * block_max (optional): [B*Tq][bm_stride], -inf for invisible blocks.     */
/* Index keys k: [B][N][128] in k_fmt (CSA2REF_BF16, CSA2REF_E4M3 or
 * CSA2REF_MXFP4 as packed 68-byte rows), batch stride k_sb elements (bytes
 * for the byte formats). */
void csa2ref_scan(int B, int Tq, const uint16_t *q, const float *w,
                  const void *k, int k_fmt, int64_t k_sb, int64_t n_cache,
                  const int64_t *q_pos, double *scores, int64_t s_stride,
                  double *block_max, int64_t bm_stride);

/* ---- a3 / a5: top-k by (score desc, id asc) -------------------------- */
/* Row r: entries j < n with ids[r][j] >= 0 (ids NULL: id = j) and a score
 * that is not -inf or NaN are valid.  forced (optional): per-row id that is
 * always kept (ignored when < 0 or not a valid entry of the row).  The
 * result lists the chosen ids ascending, padded with -1 to k.             */
void csa2ref_select(int R, int64_t n, const double *scores, int64_t s_stride,
                    const int32_t *ids, int64_t id_stride,
                    const int32_t *forced, int k, int32_t *out,
                    int64_t o_stride);

/* ---- a4: indexer scores over the candidate blocks -------------------- */
/* q, w, k as for csa2ref_scan (the query rounded to the key format).
 * blocks: [B*Tq][K_b] block ids (-1 = none).  Output column j*8+i is the
 * latent 8*blocks[j]+i when that latent is visible, else id -1 and score
 * -inf.                                                                   */
void csa2ref_cand(int B, int Tq, const uint16_t *q, const float *w,
                  const void *k, int k_fmt, int64_t k_sb, int64_t n_cache,
                  const int64_t *q_pos, const int32_t *blocks, int K_b,
                  double *scores, int32_t *ids, int64_t stride);

/* ---- a6: sparse attention over Sel + window, with sink --------------- */
/* q: bf16 [B][Tq][64][512] (batch stride q_sb elements).
 * lat: compressed latent cache [B][n_cache][row] in lat_fmt:
 *      BF16 row = 512 bf16; NVFP4 row = 256 bytes (element 2i in the low
 *      nibble of byte i) with lat_scale [B][n_cache][32] E4M3 bytes;
 *      lat_sb = batch stride in rows.
 * sel: int32 [B*Tq][sel_sb] of which the first K are used; -1 = empty.
 * win: window source [B][W_cap][512] in win_fmt (BF16, or E4M3 with a
 *      per-slot f32 scale win_scale [B][W_cap]); batch stride win_sb rows.
 * out: [B*Tq][64][512] double; lse (optional): [B*Tq][64].                */
void csa2ref_attn(int B, int Tq, const uint16_t *q, int64_t q_sb,
                  const void *lat, int lat_fmt, const uint8_t *lat_scale,
                  int64_t lat_sb, int64_t n_cache, const int32_t *sel, int K,
                  int64_t sel_sb, const void *win, int win_fmt,
                  const float *win_scale, int W, int W_cap, int64_t win_sb,
                  const int64_t *q_pos, const float *sink, double scale,
                  double *out, double *lse);

/* ---- a7: standalone dequantisation --------------------------------- */
void csa2ref_dequant_fp8(const uint8_t *src, const float *row_scale,
                         int64_t rows, int cols, double *dst);
void csa2ref_dequant_nvfp4(const uint8_t *packed, const uint8_t *scales,
                           int64_t rows, int cols, double *dst);


/* ---- f1: NVFP4 quantisation (the inverse of csa2ref_dequant_nvfp4) ---- */
/* scale code: nearest E4M3 to amax/6, ties to even, saturating at 448.
 * element code: nearest E2M1 to x/scale (sign from x), ties to even,
 * saturating at 6; scale 0 gives code 0.  src f32 [rows][cols], cols % 16
 * == 0; packed [rows][cols/2] (element 2i in the low nibble of byte i),
 * scales [rows][cols/16].                                                */
uint8_t csa2ref_quant_scale_e4m3(float amax);
uint8_t csa2ref_quant_e2m1(float x, uint8_t scale_code);
void csa2ref_quant_nvfp4(const float *src, int64_t rows, int cols,
                         uint8_t *packed, uint8_t *scales);

#ifdef __cplusplus
}
#endif
#endif
