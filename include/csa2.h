/*
 * csa2.h -- C ABI of the CSA2 (Compressed Sparse Attention 2) hot path for
 * AMD Instinct MI355X (gfx950).
 *
 * The method (sources cited by page title and section):
 *   [NVFP4]  "DeepSeek-V4.1-Flash-NVFP4" article, lpnh.cn/news/2752702:
 *            section 3 (two KV sources per query: a 128-token raw window and
 *            512 selected compressed positions, 640 rows in one sparse
 *            attention call), 3.1 (sliding-window ring), 3.2 (2:1 Compressor
 *            with softmax gating; NVFP4 cache, 16-element groups with an E4M3
 *            scale), 3.3 (block-level top-2048 over blocks of 8 compressed
 *            positions scored by their in-block maximum, newest block always
 *            kept; a 32-head indexer with ReLU and per-head weights keeping
 *            the top 512 positions), 3.4 (one-pass gather + online softmax
 *            with a learnable attention sink).
 *   [OQ3E]   "CSA2 sparse attention, 384-expert MoE and 1M context in
 *            DeepSeek-V4.1-Flash-1017-oQ3e-ngram-mtp", nxmr.cn/news/161930:
 *            section 1 (64 query heads, one latent KV head), section 2.1
 *            (index_n_heads 32, index_head_dim 128, index_topk 512,
 *            candidate_block_size 8, candidate_topk_blocks 2048,
 *            sliding_window 128).
 *
 * Conventions shared by every call
 *   - Tensor arguments are DEVICE pointers owned by the caller.  The library
 *     keeps no pointer after a call returns and allocates no device memory;
 *     scratch space, where a call needs it, is passed in by the caller
 *     (csa2_sparse_attn_noalloc instead uses a fixed scratch array the
 *     library holds on each device).
 *   - Calls enqueue work on the given HIP stream and return without waiting.
 *     The only state the library keeps is per device and written once,
 *     atomically: a flag recording that the attention kernels' dynamic-LDS
 *     limit has been raised, and the device address of the scratch array of
 *     csa2_sparse_attn_noalloc.  Calls may be made from several threads at
 *     once on different streams (csa2_sparse_attn_noalloc: see there).
 *   - Strides are in elements of the tensor's own storage type (bytes for
 *     FP8 / NVFP4 data); the innermost dimension is contiguous.
 *   - Every call returns a csa2_status.  Arguments are validated on the host
 *     before anything is enqueued; a call that returns an error has enqueued
 *     nothing and written nothing.  Conditions only visible on the device
 *     (contents of index arrays) are documented preconditions; a violation
 *     gives unspecified results inside the documented output buffers, never
 *     an access outside the buffers described here.
 *   - Shapes fixed by the method: latent width D = 512, query heads HQ = 64,
 *     index heads HI = 32, index width DI = 128, block size 8, compression
 *     ratio 2.  Anything else is CSA2_EUNSUPPORTED.
 *   - Positions: latent g pools raw tokens 2g and 2g+1; a query at raw
 *     position t sees latents g < n_vis(t) = min(n_cache, (t+1)/2).
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA2_D 512
#define CSA2_HQ 64
#define CSA2_HI 32
#define CSA2_DI 128
#define CSA2_BLOCK 8

typedef enum csa2_dtype {
  CSA2_BF16 = 1,     /* bfloat16                                           */
  CSA2_FP8_E4M3 = 2, /* OCP FP8 E4M3FN (bias 7, max 448, S.1111.111 = NaN) */
  CSA2_NVFP4 = 3,    /* E2M1 codes, 2 per byte (element 2i in the low      */
                     /* nibble of byte i), one E4M3 scale per 16 elements  */
  CSA2_F32 = 4,
  CSA2_MXFP4 = 5     /* index keys: E2M1 codes, 2 per byte (dim 2i in the  */
                     /* low nibble of byte i), one E8M0 scale per 32 dims  */
} csa2_dtype;

typedef enum csa2_status {
  CSA2_OK = 0,
  CSA2_EINVAL = -1,       /* null pointer, bad size or stride             */
  CSA2_EUNSUPPORTED = -2, /* dtype / shape combination not implemented    */
  CSA2_ELAUNCH = -3,      /* the HIP runtime refused a kernel launch      */
  CSA2_EWORKSPACE = -4    /* workspace missing or smaller than required   */
} csa2_status;

/* Static description of a status code (never NULL). */
const char *csa2_status_string(int status);

/* Library version, (major << 16) | minor. */
int csa2_version(void);

/* ------------------------------------------------------------------------
 * a1. Compressor: 2:1 softmax-gated pooling  ([NVFP4] section 3.2).
 *
 * For each sequence b, group g < T/2 and channel c:
 *   out[b][g][c] = sum_{i=0,1} softmax_i(gate[b][2g+i][c]) * kv[b][2g+i][c]
 * (softmax over the two tokens of the group, independently per channel),
 * computed in fp32 and rounded to nearest-even bf16.
 *   kv, gate : bf16 [B][T][512], batch strides kv_sb, g_sb (elements)
 *   out      : bf16 [B][T/2][512], batch stride out_sb; may point into a
 *              latent cache.  Must not overlap kv or gate.
 * T must be even (the token of an unfinished group stays with the caller,
 * who keeps it as the compressor's state until its partner arrives); the
 * first token of the input sits at an even raw position.  T = 0 or B = 0 is
 * a no-op.
 * ---------------------------------------------------------------------- */
int csa2_compress(int B, int T, const void *kv, int64_t kv_sb,
                  const void *gate, int64_t g_sb, void *out, int64_t out_sb,
                  hipStream_t stream);

/* ------------------------------------------------------------------------
 * f1. Compressor writing the NVFP4 cache  ([NVFP4] section 3.2: the
 * compressed KV is stored as E2M1 values in groups of 16 sharing one E4M3
 * scale; during decode the unfinished half of a token pair waits in the
 * compressor's state).
 *
 * Quantisation of a group of 16 values x (the section names the format, not
 * the encoder; this is the plain reading):
 *   scale   = the E4M3 value nearest to max|x| / 6, ties to the even code,
 *             saturating at 448 (6 is the largest E2M1 magnitude);
 *   code[i] = the E2M1 value nearest to x[i] / scale, ties to the even
 *             code, saturating at +-6, sign bit from x[i] (x < 0);
 *   a group whose scale is 0 stores all-zero codes.
 * Both roundings are decided on the exact quotients.  csa2_dequant_nvfp4 is
 * the inverse; a group of representable values (x = e2m1 * s with some
 * |x| = 6 s) survives the round trip exactly.
 *
 * csa2_compress_nvfp4: the pooling of csa2_compress, kept in fp32 (not
 *   rounded to bf16) and quantised in the same kernel.
 *   kv, gate   : as for csa2_compress (T even, T = 0 or B = 0 is a no-op)
 *   codes      : [B][rows][256] bytes, element 2i in the low nibble of byte
 *                i; row g of sequence b at (b*out_sb + g)*256; 8-byte aligned
 *   scale_e4m3 : [B][rows][32] bytes at (b*out_sb + g)*32
 *   out_sb     : batch stride in ROWS (>= T/2 when B > 1), the layout
 *                csa2_sparse_attn reads (lat, lat_scale, lat_sb).
 *   Outputs must not overlap the inputs or each other.
 *
 * csa2_compress_step: one decode step for B sequences, each at its own raw
 *   position pos[b] (device int64 [B]; negative = no token this step).
 *   kv, gate : bf16 [B][512] with batch strides kv_sb, g_sb (elements)
 *   state    : bf16 [B][2][512], device memory the caller allocates and
 *              keeps between calls: the parked kv row, then its gate row
 *   An even position t stores the token in state[b].  An odd position t
 *   pools state[b] (token t-1) with the new token into cache row t/2 of
 *   sequence b, which is written only if t/2 < n_cache (no error otherwise:
 *   positions live on the device).  out_dt CSA2_BF16: out bf16 [B][rows][512]
 *   (16-byte aligned), out_scale unused; CSA2_NVFP4: out = codes,
 *   out_scale = scales, as for csa2_compress_nvfp4.  out_sb in rows
 *   (>= n_cache when B > 1).  The written row is bit-identical to what
 *   csa2_compress / csa2_compress_nvfp4 write for the same two tokens, so a
 *   prefill of even length followed by decode steps fills the cache as one
 *   batch call would.  A token at an odd position needs its partner parked
 *   by an earlier step (or written into state by the caller).
 *
 * csa2_quant_nvfp4: the quantiser alone.  src [rows][cols] in src_dt
 *   (CSA2_BF16 or CSA2_F32), 16-byte aligned, cols % 16 == 0; packed
 *   [rows][cols/2] (8-byte aligned), scale_e4m3 [rows][cols/16].
 * ---------------------------------------------------------------------- */
int csa2_compress_nvfp4(int B, int T, const void *kv, int64_t kv_sb,
                        const void *gate, int64_t g_sb, uint8_t *codes,
                        uint8_t *scale_e4m3, int64_t out_sb,
                        hipStream_t stream);
int csa2_compress_step(int B, const void *kv, int64_t kv_sb, const void *gate,
                       int64_t g_sb, const int64_t *pos, void *state,
                       csa2_dtype out_dt, void *out, uint8_t *out_scale,
                       int64_t out_sb, int64_t n_cache, hipStream_t stream);
int csa2_quant_nvfp4(const void *src, csa2_dtype src_dt, int64_t rows,
                     int cols, uint8_t *packed, uint8_t *scale_e4m3,
                     hipStream_t stream);

/* ------------------------------------------------------------------------
 * a2 / a4. Indexer scores  ([NVFP4] section 3.3; [OQ3E] section 2.1).
 *
 *   score(p) = sum_{h<32} w[h] * max(0, q[h] . k[p])
 *
 * Row r = b*Tq + j is the query (b, j) at raw position q_pos[b][j].
 *   q     : bf16 [B][Tq][32][128] (q_dt must be CSA2_BF16).  The query
 *           meets the keys in their format ([NVFP4] section 3.3 runs the
 *           indexer on FP4 index queries): with CSA2_FP8_E4M3 keys every
 *           query value is first rounded to the nearest E4M3 value (ties to
 *           even, saturating at +-448), with CSA2_MXFP4 keys to the nearest
 *           E2M1 value (ties to even, saturating at +-6); bf16 keys use it as
 *           is.  Small integers are exact in every format.
 *   w     : f32  [B][Tq][32] per-query, per-head weights
 *   k     : [B][n_cache][128] in k_dt (CSA2_BF16 or CSA2_FP8_E4M3), batch
 *           stride k_sb elements; or CSA2_MXFP4 ([NVFP4] section 3.3 keeps
 *           the index keys in FP4; section 4 describes MXFP4): k holds the
 *           E2M1 codes [B][n_cache][64] bytes, batch stride k_sb bytes
 *           (a multiple of 16), and k_scale the E8M0 scales
 *           [B][n_cache][4] (dims 0-31, 32-63, 64-95, 96-127), batch stride
 *           k_sb/16 bytes, 4-byte aligned (the query rounded to E2M1, as
 *           above).  MXFP4 keys
 *           are supported by the many-query scan (SCAN mode, Tq >= 64, the
 *           chunked prefill) and return CSA2_EUNSUPPORTED elsewhere.
 *   k_scale : MXFP4 only, else ignored (may be NULL)
 *   q_pos : int64 [B][Tq]
 *
 * mode CSA2_SCORES_SCAN: every latent p < n_cache is scored;
 *   scores    (optional, may be NULL): f32 [B*Tq][s_stride >= n_cache],
 *             -inf where p >= n_vis(t)
 *   block_max (optional): f32 [B*Tq][bm_stride >= ceil(n_cache/8)], the max
 *             of the block's visible scores, -inf for blocks with none
 *   cand_blocks, K_b, ids_out are ignored.  At least one output is needed.
 * mode CSA2_SCORES_CAND: only the latents of the chosen blocks are scored;
 *   cand_blocks : int32 [B*Tq][K_b] block ids, -1 = none; an id at or
 *             past ceil(n_cache/8) names latents that are not visible
 *             (score -inf, id -1; nothing past the cache is read).
 *   scores    : f32 [B*Tq][s_stride >= 8*K_b]; column 8j+i scores latent
 *             8*cand_blocks[j]+i;
 *   ids_out   : int32 [B*Tq][s_stride], that latent's index, or -1 (score
 *             -inf) when the block id is -1 or the latent is not visible.
 *   block_max, bm_stride are ignored.
 * With integer-valued q, k (|q|,|k| <= 3) and weights that are multiples of
 * 1/16 every score is exact in fp32, whatever the summation order.  For other
 * queries each head's dot product is exact whenever its terms fit fp32 (E4M3
 * or E2M1 query against E4M3 or MXFP4 keys of moderate size), and the
 * weighted sum of the 32 non-negative head terms is rounded in fp32.
 * ---------------------------------------------------------------------- */
#define CSA2_SCORES_SCAN 0
#define CSA2_SCORES_CAND 1
int csa2_index_scores(int mode, int B, int Tq, const void *q, csa2_dtype q_dt,
                      const float *w, const void *k, csa2_dtype k_dt,
                      const uint8_t *k_scale, int64_t k_sb, int64_t n_cache,
                      const int64_t *q_pos,
                      const int32_t *cand_blocks, int K_b, float *scores,
                      int64_t s_stride, int32_t *ids_out, float *block_max,
                      int64_t bm_stride, hipStream_t stream);

/* ------------------------------------------------------------------------
 * a4 from stored scores ([NVFP4] section 3.3: the candidate-source indexer
 * scores every position and the current layer's indexer re-scores the
 * candidates; where one indexer serves both stages, as in the chunked
 * prefill, the candidates' scores are entries of the scan's score matrix).
 * Gathers them instead of recomputing; the output is exactly that of
 * csa2_index_scores(CSA2_SCORES_CAND) for the same (q, w, k):
 *   all        : f32 [B*Tq][a_stride >= n_cache], the SCAN scores; 16-byte
 *                aligned, a_stride % 4 == 0
 *   q_pos      : int64 [B][Tq];  cand_blocks, K_b : as for CAND
 *   scores     : f32 [B*Tq][s_stride >= 8*K_b], column 8j+i = latent
 *                8*cand_blocks[j]+i, -inf when the block id is -1 or the
 *                latent is not visible (n_vis of the query's position)
 *   ids_out    : int32, same shape, that latent's index or -1
 *   scores and ids_out 16-byte aligned, s_stride % 4 == 0, no overlap.
 * Block ids at or past ceil(n_cache/8) count as not visible (never read).
 * ---------------------------------------------------------------------- */
int csa2_gather_scores(int B, int Tq, const float *all, int64_t a_stride,
                       int64_t n_cache, const int64_t *q_pos,
                       const int32_t *cand_blocks, int K_b, float *scores,
                       int32_t *ids_out, int64_t s_stride,
                       hipStream_t stream);

/* ------------------------------------------------------------------------
 * a4 from stored scores and a5 in one pass ([NVFP4] section 3.3, as for
 * csa2_gather_scores): the position top-k of the candidates gathered from
 * the scan's score matrix, without materialising the candidate scores.
 * The result equals
 *   csa2_gather_scores(B, Tq, all, a_stride, n_cache, q_pos, cand_blocks,
 *                      K_b, scores, ids, ...)
 *   csa2_select_topk(B*Tq, 8*K_b, scores, .., ids, .., NULL, 0, k, out, ..)
 * bit for bit: out int32 [B*Tq][o_stride >= k], the kept latent indices in
 * ascending order, then -1.  all, q_pos, cand_blocks as for
 * csa2_gather_scores (all 4-byte aligned here); out must not overlap all.
 * Supported when a row of 8*K_b candidates is held in registers by one
 * workgroup: 8*K_b <= 16384, or up to 32768 with B*Tq >= 256; else
 * CSA2_EUNSUPPORTED (use the two calls above).  Block ids at or past
 * ceil(n_cache/8) count as not visible (never read).  Precondition: a row's
 * valid block ids ascending.
 * ---------------------------------------------------------------------- */
int csa2_gather_select(int B, int Tq, const float *all, int64_t a_stride,
                       int64_t n_cache, const int64_t *q_pos,
                       const int32_t *cand_blocks, int K_b, int k, int32_t *out,
                       int64_t o_stride, hipStream_t stream);

/* ------------------------------------------------------------------------
 * a3 / a5. Top-k selection  ([NVFP4] section 3.3).
 *
 * Per row r < R over entries j < n: an entry is valid when its id is >= 0
 * (ids == NULL means id = j) and its score is neither -inf nor NaN.  The
 * result keeps the k valid entries with the largest scores, ties going to
 * the smaller id; if fewer than k are valid, all of them.  A forced id is
 * always kept, taking the place of the weakest pick:
 *   forced     (optional) int32 [R]: id to keep in row r (-1 = none; an id
 *              that is not a valid entry of the row is ignored);
 *   force_last nonzero: additionally keep the valid entry with the largest
 *              column index (for block scores this is the newest visible
 *              block).  forced and force_last are mutually exclusive.
 * out: int32 [R][o_stride >= k]: the kept ids in ascending order, then -1.
 * Precondition when ids != NULL: the ids of a row's valid entries increase
 * with the column index (true for the CAND output of csa2_index_scores when
 * its block list is ascending, as this call produces it).
 * ws / ws_bytes: scratch, size from csa2_workspace_bytes(CSA2_OP_SELECT..),
 * may be NULL when that size is 0.  1 <= n <= 2^24, 1 <= k <= 2^24 (k > n
 * simply keeps every valid entry and pads).
 * ---------------------------------------------------------------------- */
int csa2_select_topk(int R, int64_t n, const float *scores, int64_t s_stride,
                     const int32_t *ids, int64_t id_stride,
                     const int32_t *forced, int force_last, int k,
                     int32_t *out, int64_t o_stride, void *ws,
                     size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * a6. Sparse attention over the selected latents and the raw window, with a
 * per-head sink ([NVFP4] sections 3, 3.1, 3.4).
 *
 * For query row r = b*Tq + j at raw position t = q_pos[b][j], head h < 64:
 *   rows    = { lat[b][sel[r][i]] : i < K, sel[r][i] >= 0 }
 *           + { win[b][p mod W_cap] : max(0, t-W+1) <= p <= t }
 *   l_i     = scale * (q[b][j][h] . row_i)          (K = V = the row)
 *   out     = sum_i e^{l_i} row_i / (e^{sink[h]} + sum_i e^{l_i})
 *   lse     = log(e^{sink[h]} + sum_i e^{l_i})
 * computed with an online softmax in fp32, bf16 MFMA products, bf16 out.
 *   q        : bf16 [B][Tq][64][512], batch stride q_sb elements
 *   lat      : latent cache [B][n_cache][row] in lat_dt (CSA2_BF16: 512
 *              bf16 per row; CSA2_NVFP4: 256 bytes per row), batch stride
 *              lat_sb ROWS (>= n_cache)
 *   lat_scale: CSA2_NVFP4 only, E4M3 bytes [B][n_cache][32] with the same
 *              batch stride lat_sb rows; NULL otherwise
 *   sel      : int32 [B*Tq][sel_sb], first K used (-1 = empty).
 *              Precondition: every id is -1 or < n_cache.
 *   win      : window source [B][W_cap][512] in win_dt (CSA2_BF16, or
 *              CSA2_FP8_E4M3 with win_scale f32 [B][W_cap] per slot), batch
 *              stride win_sb ROWS (>= W_cap) for both win and win_scale.  Precondition: slot p mod W_cap holds
 *              raw position p for every window position of every query of
 *              the sequence (W_cap >= W + spread of the row's q_pos).
 *   sink     : f32 [64];  scale: logit scale (1/sqrt(512) in the configs)
 *   out      : bf16 [B*Tq][64][512], 16-byte aligned, row stride out_sb
 *              (elements, a multiple of 8)
 *   lse      : optional f32 [B*Tq][64]
 *   ws       : scratch of csa2_workspace_bytes(CSA2_OP_SPARSE_ATTN, ...)
 * 0 <= K <= 2048, 1 <= W <= W_cap.
 * ---------------------------------------------------------------------- */
int csa2_sparse_attn(int B, int Tq, const void *q, int64_t q_sb,
                     const void *lat, csa2_dtype lat_dt, const void *lat_scale,
                     int64_t lat_sb, int64_t n_cache, const int32_t *sel,
                     int K, int64_t sel_sb, const void *win,
                     csa2_dtype win_dt, const float *win_scale, int W,
                     int W_cap, int64_t win_sb, const int64_t *q_pos,
                     const float *sink, float scale, void *out,
                     int64_t out_sb, float *lse, void *ws, size_t ws_bytes,
                     hipStream_t stream);

/* ------------------------------------------------------------------------
 * csa2_sparse_attn without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Arguments, results and preconditions are
 * those of csa2_sparse_attn (the same kernels and the same split of a
 * query's rows over workgroups, so the same bits).  Where csa2_sparse_attn
 * would use the caller's workspace, this call uses a scratch array of
 * CSA2_ATTN_SCRATCH_BYTES that the library holds in the memory of every GPU
 * it runs on until the process ends; its device address is looked up on the
 * first call on a device that needs it.  The call allocates nothing.
 *   - Returns CSA2_EWORKSPACE, having enqueued nothing, when the call's split
 *     partials would exceed the scratch (csa2_workspace_bytes(
 *     CSA2_OP_SPARSE_ATTN, B*Tq, K, W) bounds them: e.g. 32 NVFP4 queries of
 *     512 + 128 rows need 29.6 MB, 40 need 37 MB and are refused).  Calls
 *     of 192 or more queries, and bf16 calls of 128 to 191, need none.
 *   - Every call on a GPU shares that GPU's one scratch array and leaves its
 *     partials there: calls that overlap in time on one GPU (different
 *     streams, or different threads) race and must be serialised by the
 *     caller.  Nothing in the scratch needs to start at zero.
 * ---------------------------------------------------------------------- */
#define CSA2_ATTN_SCRATCH_BYTES (32u << 20)
int csa2_sparse_attn_noalloc(int B, int Tq, const void *q, int64_t q_sb,
                             const void *lat, csa2_dtype lat_dt,
                             const void *lat_scale, int64_t lat_sb,
                             int64_t n_cache, const int32_t *sel, int K,
                             int64_t sel_sb, const void *win,
                             csa2_dtype win_dt, const float *win_scale, int W,
                             int W_cap, int64_t win_sb, const int64_t *q_pos,
                             const float *sink, float scale, void *out,
                             int64_t out_sb, float *lse, hipStream_t stream);

/* ------------------------------------------------------------------------
 * a7. Standalone dequantisation ([NVFP4] sections 3.1, 3.2).
 *   fp8   : src E4M3 [rows][cols], optional f32 row_scale [rows] (NULL = 1)
 *   nvfp4 : packed [rows][cols/2] (element 2i low nibble of byte i),
 *           scale_e4m3 [rows][cols/16]; cols % 16 == 0
 *   dst   : [rows][cols] in dst_dt (CSA2_BF16 or CSA2_F32)
 * ---------------------------------------------------------------------- */
int csa2_dequant_fp8(const uint8_t *src, const float *row_scale, int64_t rows,
                     int cols, void *dst, csa2_dtype dst_dt,
                     hipStream_t stream);
int csa2_dequant_nvfp4(const uint8_t *packed, const uint8_t *scale_e4m3,
                       int64_t rows, int cols, void *dst, csa2_dtype dst_dt,
                       hipStream_t stream);

/* ------------------------------------------------------------------------
 * Scratch sizes.  op = CSA2_OP_SELECT: (R = rows, n = entries per row, k).
 * op = CSA2_OP_SPARSE_ATTN: (R = B*Tq, n = K, k = W).  Returns bytes (0 when
 * the call needs no scratch for that shape).
 * ---------------------------------------------------------------------- */
#define CSA2_OP_SELECT 1
#define CSA2_OP_SPARSE_ATTN 2
size_t csa2_workspace_bytes(int op, int64_t R, int64_t n, int64_t k);

#ifdef __cplusplus
}
#endif
#endif /* CSA2_H */
