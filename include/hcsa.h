/*
 * hcsa.h -- C ABI of libhcsa, the hybrid compressed attention (CSA + HCA) of DeepSeek-V4
 * on AMD Instinct MI355X (gfx950).
 *
 * Method (web pages on the DeepSeek-V4 release):
 *   Lighthouse, "deep deepseek v4 release", section 八 item 3: CSA pools the KV of every
 *   m = 4 tokens into one entry, a Lightning Indexer keeps the top-k compressed entries
 *   (1024 Pro / 512 Flash) for sparse attention, and a sliding-window branch of
 *   n_win = 128 raw tokens restores local detail; HCA pools every m' = 128 tokens into
 *   one entry and attends densely over all of them.
 *   Same page, item 7: the indexer keeps its own compressed keys.
 *   9fzt.com digest, item 4: FP4 on the indexer's QK path; FP32 index scores compressed
 *   to BF16 for the top-k selector.
 *   tulong.co Q&A, 技术架构创新 item 1: every 4 tokens -> one block, every 128 -> one entry.
 *
 * Readings where the pages are silent (the library implements exactly these):
 *   - pooling: y[j] = sum_i alpha_i x[j*r + i], alpha = softmax(omega), omega [r] shared
 *     by every block, sequence and channel; the T mod r tail is not pooled.
 *   - indexer score: s_j = sum_g w_g * max(0, q_g . k_j), fp32 accumulate, optionally
 *     rounded to bf16 (nearest-even); -0 is stored as +0.
 *   - top-k: the min(k, n) largest scores, ties to the lowest index, output ascending,
 *     padded with -1.
 *   - CSA attention: one softmax over [selected entries] ++ [raw window tokens
 *     max(0, p-n_win+1) .. p]; HCA attention: one softmax over all visible entries.
 *   - visibility: entry j of a stream with ratio r is visible to the token at position p
 *     iff (j+1)*r <= p+1.  Query i of sequence b sits at position pos0 + i, or at
 *     seq_pos[b] + i when the call is given seq_pos (ragged batches: each sequence at its
 *     own length).
 *   - one KV head shared by all query heads (MQA); logits are scale * q.k, with scale
 *     positive and finite (the attention calls reject other values with HCSA_EINVAL).
 *   - MXFP4: OCP MX e2m1 elements with one e8m0 scale per 32 elements, scale exponent
 *     floor(log2 amax) - 2 (clamped to [-127, 127]; amax = 0 gives -127), elements
 *     rounded to nearest-even on the e2m1 grid and saturated at +-6.  Two elements per
 *     byte, element 2i in the low nibble.  Scale byte = exponent + 127.
 *
 * Conventions for every call:
 *   - All data pointers are device pointers owned by the caller; the library never
 *     allocates device memory.  Calls that need scratch take (workspace, ws_bytes) and a
 *     matching *_workspace_size() query; workspace must be 256-byte aligned.
 *   - Tensors are row-major with contiguous rows; "bstride" is the distance between
 *     sequences, in elements for F32/BF16 tensors and in bytes for MXFP4 tensors.
 *   - Data pointers must be 16-byte aligned and bstrides must keep that alignment.
 *   - Every call validates its arguments on the host before any launch and returns
 *     HCSA_OK (0) or a negative code; hcsa_last_error() gives a message (thread-local).
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = default stream) and
 *     never synchronizes.  Outputs are defined once the stream reaches the call.
 *   - Calls that share a workspace on different streams race.
 *   - seq_pos (the calls that take pos0): NULL, or a device array of B int64 positions,
 *     8-byte aligned, each >= 0, giving the position of query 0 of each sequence; pos0 is
 *     then unused.  Its values sit in device memory and are not validated on the host.
 *   - pages (the calls that read or write caches): NULL for contiguous caches, or a paged
 *     layout (hcsa_pages below).
 */
#ifndef HCSA_H
#define HCSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *hcsa_stream; /* hipStream_t */

/*
 * Cache layout [the heterogeneous KV cache: paged compressed caches in 128-token blocks,
 * lcm(m, m') = lcm(4, 128), and a fixed-size state cache for the sliding window and the
 * tokens not yet pooled: Lighthouse section 八 item 7].
 *
 * block_table (NULL: caches contiguous, bstride arguments apply): positions
 * [128*blk, 128*blk + 128) of sequence b live in page block_table[b*table_stride + blk] of
 * every cache tensor.  A tensor pooled at ratio r (r divides 128) holds 128/r rows per page:
 * its pointer is then a page pool [pages][128/r][row] (raw tokens: 128 rows per page, CSA
 * entries and indexer keys 32, HCA entries 1) and its bstride argument is ignored.  The table
 * is device memory (int32, 4-byte aligned), must cover every block holding a position a call
 * touches, and is not validated on the host.
 *
 * raw_ring (0: raw tokens laid out like the caches): a power of two in [128, 2^30].  Raw
 * tokens (x of the pooling jobs, k_raw/v_raw of CSA attention) are then a ring of raw_ring
 * rows per sequence, [B][raw_ring][row] with the call's raw bstride: position t sits in row
 * t mod raw_ring.  The caller keeps the last raw_ring tokens of every sequence there; a call
 * may touch only those (a decode step needs the window and the tokens since the last
 * completed 128-token block).
 */
typedef struct hcsa_pages {
  const int32_t *block_table;
  int64_t table_stride;
  int64_t raw_ring;
} hcsa_pages;

/*
 * Element types.  HCSA_MXFP4_FP8 is accepted only as the key type of the indexer calls: the
 * keys are stored exactly as HCSA_MXFP4 (same codes, same scales), and the scan widens the
 * e2m1 codes to e4m3 and runs the FP8 matrix-core instruction with the same block scales
 * [9fzt.com digest item 4: FP4 dequantized to FP8 without loss, reusing an FP8 path;
 * tulong.co 技术架构创新 item 2: FP4+FP8 mixed precision].  Every e2m1 value is exact in
 * e4m3, so the scores equal those of HCSA_MXFP4 keys.
 */
enum hcsa_dtype { HCSA_F32 = 0, HCSA_BF16 = 1, HCSA_MXFP4 = 2, HCSA_MXFP4_FP8 = 3 };

enum hcsa_status {
  HCSA_OK = 0,
  HCSA_EINVAL = -1,     /* bad size, pointer or combination of arguments */
  HCSA_EDTYPE = -2,     /* unsupported dtype for this call */
  HCSA_EALIGN = -3,     /* pointer or stride not 16-byte aligned */
  HCSA_EWORKSPACE = -4, /* workspace missing, misaligned or too small */
  HCSA_EHIP = -5        /* a HIP launch failed; message has hipGetErrorString */
};

/* Library version (major*10000 + minor*100 + patch). */
int hcsa_version(void);

/* Message of the last non-zero status returned on this thread ("" if none). */
const char *hcsa_last_error(void);

/*
 * Kernel timing for benchmarks and profiling: the next indexer-score kernel launched by
 * this thread (hcsa_csa_index_scores or hcsa_csa_index_topk) records start_event and stop_event
 * (hipEvent_t, timing enabled) as part of its own dispatch, so their elapsed time is the
 * kernel's execution alone.  NULL, NULL cancels.  Not for use under graph capture.
 */
int hcsa_time_next_indexer(void *start_event, void *stop_event);

/*
 * Split count of the attention calls made later on this thread, for tuning and for checking
 * that results do not depend on it: 0 (the default) lets each call choose; n in [1, 1024]
 * asks the split-K kernels (bf16, 16 heads x 128; the query-by-query decode forms of
 * hcsa_csa_sparse_attn, hcsa_hca_dense_attn and hcsa_csa_hca_attn) for n splits of each
 * query's key list, as far as their 4096-key blocks allow; other forms are unaffected.
 * The workspace sizes reported afterwards follow the same choice.  The split results are
 * combined exactly (log-sum-exp merge), so outputs agree across split counts up to the
 * rounding of fp32 sums [Lighthouse section 八 item 3: one softmax over the key list].
 */
int hcsa_set_attn_splits(int splits);

/*
 * Block pooling (CSA m = 4, HCA m' = 128, indexer keys m = 4)
 * [Lighthouse section 八 item 3; tulong.co 技术架构创新 item 1].
 *
 * x      [B][T][D] F32 or BF16; sequence b starts at x + b*x_bstride (elements).
 * omega  [ratio] F32 pooling logits; alpha = softmax(omega) is computed on the device.
 * y      F32/BF16: [B][T/ratio][D], sequence stride y_bstride elements.
 *        MXFP4: packed codes [B][T/ratio][D/2] bytes, sequence stride y_bstride bytes,
 *        and y_scales [B][T/ratio][D/32] e8m0 bytes, stride ys_bstride bytes.
 * Writes floor(T/ratio) rows per sequence; accumulates in fp32 and rounds once.
 * Limits: 1 <= ratio <= 1024, D % 8 == 0, D <= 2048 (MXFP4: D % 32 == 0); T >= 0, B >= 1.
 */
int hcsa_compress_kv(const void *x, int x_dtype, int64_t x_bstride, int B, int T, int D,
                     const float *omega, int ratio, void *y, int y_dtype, int64_t y_bstride,
                     uint8_t *y_scales, int64_t ys_bstride, hcsa_stream stream);

/*
 * Several pooling jobs of one batch in a single launch (for instance the CSA K, V and
 * indexer-key blocks and the HCA K and V blocks that one decode token completes).  Each job
 * has the meaning and limits of hcsa_compress_kv (x has its own T; jobs share B).  The
 * call validates every job first and launches nothing if any is invalid.  Outputs of
 * different jobs must not overlap.  With a block table, x and y (and y_scales) are page
 * pools, ratio divides 128, and a job pools the tokens [pos0, pos0 + T) of every sequence
 * into its entries pos0/ratio .. (pos0 + T)/ratio - 1 (pos0 a multiple of ratio).  With a
 * raw-token ring, x is the ring (x_bstride apart, raw_ring rows per sequence), ratio divides
 * 128, T <= raw_ring and the job pools the tokens [pos0, pos0 + T) from it, into y's rows
 * from the first (contiguous y) or into the pages of those entries (paged y).
 */
#define HCSA_MAX_POOL_JOBS 8
typedef struct hcsa_pool_job {
  const void *x;
  int x_dtype;
  int64_t x_bstride;
  int T, D;
  const float *omega;
  int ratio;
  void *y;
  int y_dtype;
  int64_t y_bstride;
  uint8_t *y_scales;
  int64_t ys_bstride;
  int64_t pos0;        /* paged or ring form: position of the first token (a multiple of ratio) */
} hcsa_pool_job;
int hcsa_compress_kv_batched(const hcsa_pool_job *jobs, int n_jobs, int B,
                             const hcsa_pages *pages, hcsa_stream stream);

/*
 * MXFP4 quantization of rows [rows][D] (F32 or BF16) into packed codes [rows][D/2] and
 * e8m0 scales [rows][D/32] [9fzt.com digest item 4: FP4 on the indexer QK path].
 * D % 32 == 0.
 */
int hcsa_mxfp4_quantize(const void *x, int x_dtype, int64_t rows, int D, uint8_t *packed,
                        uint8_t *scales, hcsa_stream stream);

/*
 * Top-k selector over score rows [Lighthouse section 八 item 3: the indexer keeps the
 * top-k compressed blocks; 9fzt.com digest item 4: BF16 scores for the selector].
 *
 * scores  [B*Nq][row_stride] F32 or BF16; row r = b*Nq + i belongs to the token at
 *         position p = pos0 + i (or seq_pos[b] + i), which sees n = min(N, (p+1)/ratio)
 *         entries; only scores[r][0..n) are read.
 * idx     [B*Nq][k] int32 output: the min(k, n) entries with the largest scores (ties to
 *         the lowest index) in ascending order, then -1.  Bit-exact and deterministic.
 * Limits: 1 <= k <= 4096, 1 <= N <= 2^25, row_stride >= N, ratio >= 1, pos0 >= 0.
 * Workspace: caller-owned device memory of hcsa_topk_workspace_size bytes, 256-byte
 * aligned, fully rewritten by each call (no state is kept between calls).  The size is 0
 * (workspace may be NULL) when at least 64 rows of at most 131072 scores are resolved one
 * block per row with on-chip state only; otherwise it holds per-row candidate lists of
 * about 8 KB per 8192 entries.  Scoring and selection as two calls (hcsa_csa_index_scores,
 * then hcsa_topk on its scores) give the result of hcsa_csa_index_topk.
 */
size_t hcsa_topk_workspace_size(int score_dtype, int B, int Nq, int N, int k);
int hcsa_topk(const void *scores, int score_dtype, int64_t row_stride, int B, int Nq, int N,
              int ratio, int64_t pos0, const int64_t *seq_pos, int k, int32_t *idx,
              void *workspace, size_t ws_bytes, hcsa_stream stream);

/*
 * Lightning indexer + top-k [Lighthouse section 八 items 3 and 7; 9fzt.com digest item 4].
 *
 * q_idx   [B][Nq][H_I][d_I] F32 or BF16 indexer queries.
 * w_idx   [B][Nq][H_I] F32 head weights.
 * k_idx   compressed indexer keys of every sequence: F32/BF16 [B][N][d_I] (bstride in
 *         elements) or MXFP4 packed [B][N][d_I/2] (bstride in bytes) with k_scales
 *         [B][N][d_I/32] (ks_bstride bytes).  With MXFP4 keys the queries are quantized
 *         to MXFP4 (per head vector) inside the call and the dot products are exact.
 *         k_dtype MXFP4 runs the scan on e2m1 operands, MXFP4_FP8 on the same codes
 *         widened to e4m3 (same scores).
 * Scores s_j = sum_g w_g max(0, q_g . k_j) for the visible j (see hcsa_topk), rounded to
 * score_dtype, then top-k as in hcsa_topk.
 * scores_out  optional [B*Nq][N] score_dtype copy of the scores (NULL to skip).
 * Without a copy, MXFP4 keys, BF16 scores and a few long rows (the decode case: fewer than
 * 64 rows, or rows of more than 131072 entries), the scores are never stored: a floor per
 * row is set from 4096 scored samples, the key scan keeps the keys scoring at or above it
 * in per-chunk candidate lists, and the exact threshold is found among them; a row whose
 * lists hold fewer than k or too many candidates is rescanned into the workspace and
 * selected over all its scores.  The selection is the same as with a copy.
 * workspace   hcsa_csa_index_topk_workspace_size(B, Nq, N, k, score_dtype) bytes (covers
 *             every key dtype), 256-byte aligned; its contents need not be initialized.
 * Limits: H_I in {1, 2, 4, 8, 16}; d_I in {32, 64, 128} (F32 keys: {32, 64});
 *         q dtype F32 with F32 keys, BF16 with BF16 keys, F32 or BF16 with MXFP4 keys.
 */
size_t hcsa_csa_index_topk_workspace_size(int B, int Nq, int N, int k, int score_dtype);
int hcsa_csa_index_topk(const void *q_idx, int q_dtype, const float *w_idx, const void *k_idx,
                        int k_dtype, int64_t k_bstride, const uint8_t *k_scales,
                        int64_t ks_bstride, int B, int Nq, int H_I, int d_I, int N, int ratio,
                        int64_t pos0, const int64_t *seq_pos, const hcsa_pages *pages, int k,
                        int score_dtype, int32_t *topk_idx, void *scores_out, void *workspace,
                        size_t ws_bytes, hcsa_stream stream);

/*
 * Pooling on append + indexer + top-k: hcsa_compress_kv_batched(jobs, n_jobs, B, pages)
 * then hcsa_csa_index_topk(...) with the same arguments, as one call with the same results
 * [Lighthouse section 八 items 3 and 7: the tokens of a step complete the blocks the step's
 * indexer then scans].  Every job and argument is validated before anything is launched.
 * When the selection runs without a score array (see hcsa_csa_index_topk), the pooling
 * blocks share the launch of the per-row floors, whose samples then read only the entries
 * completed before each sequence's first query token: the jobs must not rewrite those.
 * workspace as for hcsa_csa_index_topk.
 */
int hcsa_csa_pool_index_topk(const hcsa_pool_job *jobs, int n_jobs, const void *q_idx,
                             int q_dtype, const float *w_idx, const void *k_idx, int k_dtype,
                             int64_t k_bstride, const uint8_t *k_scales, int64_t ks_bstride,
                             int B, int Nq, int H_I, int d_I, int N, int ratio, int64_t pos0,
                             const int64_t *seq_pos, const hcsa_pages *pages, int k,
                             int score_dtype, int32_t *topk_idx, void *scores_out,
                             void *workspace, size_t ws_bytes, hcsa_stream stream);

/*
 * Lightning-indexer scores only (the first half of hcsa_csa_index_topk; same arguments
 * and limits): scores [B*Nq][N] in score_dtype, entries at or past the visible count of a
 * row are left untouched.  No workspace.
 */
int hcsa_csa_index_scores(const void *q_idx, int q_dtype, const float *w_idx,
                          const void *k_idx, int k_dtype, int64_t k_bstride,
                          const uint8_t *k_scales, int64_t ks_bstride, int B, int Nq, int H_I,
                          int d_I, int N, int ratio, int64_t pos0, const int64_t *seq_pos,
                          const hcsa_pages *pages, int score_dtype, void *scores,
                          hcsa_stream stream);

/*
 * CSA sparse attention [Lighthouse section 八 item 3]: for each query token (position
 * p = pos0 + i, or seq_pos[b] + i) and head, one softmax over the selected compressed
 * entries (topk_idx, entries outside [0, n_c(p)) are skipped) followed by the raw window
 * tokens max(0, p-n_win+1) .. p.
 *
 * q       [B][Nq][H][d]; kc, vc [B][N][d] (c_bstride elements); topk_idx [B][Nq][k].
 * k_raw, v_raw [B][T_raw][d] (raw_bstride elements); row t holds position raw_pos0 + t.
 *         Every window position of every query must lie in [raw_pos0, raw_pos0 + T_raw)
 *         (checked on the host when seq_pos and pages are NULL; the caller's guarantee
 *         otherwise).  With a block table, k_raw/v_raw are raw-token page pools and
 *         raw_pos0 is 0.  With a raw-token ring, they are the ring (T_raw == raw_ring,
 *         raw_pos0 == 0, n_win + Nq - 1 <= raw_ring) holding every window position.
 * out     [B][Nq][H][d] F32, lse [B][Nq][H] F32 (natural log; -inf and o = 0 when no key).
 * kv_dtype F32 or BF16 (q has the same dtype).  ratio is the CSA pooling ratio.
 * Limits: 1 <= H <= 64, d % 8 == 0, 8 <= d <= 256, H*d <= 4096, 0 <= k <= 4096,
 *         0 <= n_win <= 4096.
 */
size_t hcsa_csa_sparse_attn_workspace_size(int B, int Nq, int H, int d, int k, int n_win);
int hcsa_csa_sparse_attn(const void *q, const void *kc, const void *vc, int64_t c_bstride,
                         int N, const int32_t *topk_idx, int k, const void *k_raw,
                         const void *v_raw, int64_t raw_bstride, int64_t T_raw,
                         int64_t raw_pos0, int n_win, int ratio, int64_t pos0,
                         const int64_t *seq_pos, const hcsa_pages *pages, int kv_dtype, int B,
                         int Nq, int H, int d, float scale, float *out, float *lse,
                         void *workspace, size_t ws_bytes, hcsa_stream stream);

/*
 * HCA dense attention [Lighthouse section 八 item 3; tulong.co 技术架构创新 item 1]:
 * for each query token (position p = pos0 + i, or seq_pos[b] + i) and head, one softmax
 * over every visible entry j < min(N, (p+1)/ratio) of kh/vh [B][N][d] (h_bstride
 * elements).
 * Same q/out/lse layout and limits as hcsa_csa_sparse_attn.
 */
size_t hcsa_hca_dense_attn_workspace_size(int B, int Nq, int H, int d, int N);
int hcsa_hca_dense_attn(const void *q, const void *kh, const void *vh, int64_t h_bstride,
                        int N, int ratio, int64_t pos0, const int64_t *seq_pos,
                        const hcsa_pages *pages, int kv_dtype, int B, int Nq, int H, int d,
                        float scale, float *out, float *lse, void *workspace, size_t ws_bytes,
                        hcsa_stream stream);

/*
 * CSA sparse attention and HCA dense attention of the same query tokens in one call
 * [Lighthouse section 八 item 3: CSA and HCA layers over the same tokens]: the arguments of
 * hcsa_csa_sparse_attn (kc ... ratio, out_c, lse_c) and of hcsa_hca_dense_attn (kh, vh,
 * h_bstride, N_h, ratio_h, out_h, lse_h), sharing q, positions, pages, dtype, shapes and
 * scale; same results as the two calls.  For one-token decode in bf16 with 16 heads x 128,
 * both attentions run as one launch (their blocks side by side) and their split merges as
 * one more; other shapes run the two calls' kernels in turn.
 * workspace: at least hcsa_csa_hca_attn_workspace_size(B, Nq, H, d, k, n_win, N_h) bytes.
 */
size_t hcsa_csa_hca_attn_workspace_size(int B, int Nq, int H, int d, int k, int n_win, int N_h);
int hcsa_csa_hca_attn(const void *q, const void *kc, const void *vc, int64_t c_bstride, int N,
                      const int32_t *topk_idx, int k, const void *k_raw, const void *v_raw,
                      int64_t raw_bstride, int64_t T_raw, int64_t raw_pos0, int n_win,
                      int ratio, const void *kh, const void *vh, int64_t h_bstride, int N_h,
                      int ratio_h, int64_t pos0, const int64_t *seq_pos,
                      const hcsa_pages *pages, int kv_dtype, int B, int Nq, int H, int d,
                      float scale, float *out_c, float *lse_c, float *out_h, float *lse_h,
                      void *workspace, size_t ws_bytes, hcsa_stream stream);

/*
 * One decode step of a CSA layer and an HCA layer [Lighthouse section 八 items 3 and 7: the
 * tokens of a step complete the blocks its indexer scans; CSA and HCA layers over the same
 * tokens]: hcsa_csa_pool_index_topk(jobs, ..., scores_out = NULL) followed by
 * hcsa_csa_hca_attn(...) with the same arguments, as one call.  The indexer shares N and
 * ratio with CSA (one indexer key per CSA entry).
 *
 * For one query token per sequence with MXFP4 keys (fp4 operands), bf16 queries and scores,
 * the selection without a score array, bf16 16 x 128 attention and k + n_win <= 4096 (caches
 * contiguous or paged, raw tokens in rows or a ring, one position for all sequences or
 * per-sequence positions), the step runs in four launches: the per-row selection floors
 * beside the pooling; the key scan; two blocks per row each resolving the row's top-k and
 * then attending over half of its CSA key list, beside the HCA splits on the other compute
 * units; the merge of the CSA and HCA splits.  The pooled caches and the selection equal those of the two calls bit for bit; the
 * attention outputs are split differently and agree with theirs up to the rounding of the
 * split sums (the softmax probabilities enter P.V as bf16, rounded relative to each split's
 * running maximum).  Other shapes run the two calls' kernels in turn, with their results.
 *
 * workspace: hcsa_decode_step_workspace_size(B, Nq, N, k, score_dtype, H, d, n_win, N_h)
 * bytes, 256-byte aligned; its contents need not be initialized.
 */
size_t hcsa_decode_step_workspace_size(int B, int Nq, int N, int k, int score_dtype, int H,
                                       int d, int n_win, int N_h);
int hcsa_decode_step(const hcsa_pool_job *jobs, int n_jobs, const void *q_idx, int q_dtype,
                     const float *w_idx, const void *k_idx, int k_dtype, int64_t k_bstride,
                     const uint8_t *k_scales, int64_t ks_bstride, int H_I, int d_I,
                     int score_dtype, int32_t *topk_idx, const void *q, const void *kc,
                     const void *vc, int64_t c_bstride, int N, int k, const void *k_raw,
                     const void *v_raw, int64_t raw_bstride, int64_t T_raw, int64_t raw_pos0,
                     int n_win, int ratio, const void *kh, const void *vh, int64_t h_bstride,
                     int N_h, int ratio_h, int64_t pos0, const int64_t *seq_pos,
                     const hcsa_pages *pages, int kv_dtype, int B, int Nq, int H, int d,
                     float scale, float *out_c, float *lse_c, float *out_h, float *lse_h,
                     void *workspace, size_t ws_bytes, hcsa_stream stream);

/*
 * hcsa_decode_step without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  The step's workspace is a scratch array of HCSA_DECODE_STEP_SCRATCH_BYTES in
 * the library's own device memory: one copy on each GPU the call runs on, reserved when the
 * library's code is loaded there and held until the process ends.  Nothing is allocated by
 * the call.  Arguments, results and errors are those of hcsa_decode_step; a step whose
 * hcsa_decode_step_workspace_size exceeds the scratch (a batch of 32 sequences at
 * 1 048 576 tokens needs about 85 MiB) is rejected with HCSA_EWORKSPACE before any launch.
 * All calls on one GPU share its scratch: calls that overlap on one GPU (other streams,
 * other host threads) race and give wrong results; serialize them.  The scratch needs no
 * clearing between calls (the step initializes what it reads).
 */
#define HCSA_DECODE_STEP_SCRATCH_BYTES ((size_t)128 << 20)
int hcsa_decode_step_noalloc(const hcsa_pool_job *jobs, int n_jobs, const void *q_idx,
                             int q_dtype, const float *w_idx, const void *k_idx, int k_dtype,
                             int64_t k_bstride, const uint8_t *k_scales, int64_t ks_bstride,
                             int H_I, int d_I, int score_dtype, int32_t *topk_idx,
                             const void *q, const void *kc, const void *vc, int64_t c_bstride,
                             int N, int k, const void *k_raw, const void *v_raw,
                             int64_t raw_bstride, int64_t T_raw, int64_t raw_pos0, int n_win,
                             int ratio, const void *kh, const void *vh, int64_t h_bstride,
                             int N_h, int ratio_h, int64_t pos0, const int64_t *seq_pos,
                             const hcsa_pages *pages, int kv_dtype, int B, int Nq, int H,
                             int d, float scale, float *out_c, float *lse_c, float *out_h,
                             float *lse_h, hcsa_stream stream);

/*
 * Backward (training) [Lighthouse section 八 item 2: the sparse attention is trained from
 * the 64K stage of the length curriculum; item 3 for the attention itself].  Gradients of
 * the loss sum(dout * out) + sum(dlse * lse) of the forward call with the same arguments;
 * the top-k selection is held fixed, a rounding to the cache type passes gradients
 * unchanged.  Caches are contiguous (no pages, no raw-token ring).
 *
 * out, lse   the forward's outputs [B][Nq][H][d], [B][Nq][H] (F32).
 * dout       [B][Nq][H][d] F32; dlse [B][Nq][H] F32 or NULL (no gradient on lse).
 * dq         [B][Nq][H][d] F32, written.
 * CSA: dkc, dvc [B][N][d] F32 (dc_bstride elements), the selected entries' gradients, and
 *      dk_raw, dv_raw [B][T_raw][d] F32 (draw_bstride), the window rows' gradients, are
 *      accumulated (+=): they may be shared with other calls, and start from the caller's
 *      values (zero them first for a fresh gradient).
 * HCA: dkh, dvh [B][N][d] F32 (dh_bstride), accumulated.
 * The accumulations use floating-point atomics: their order, and the last bits of the
 * accumulated gradients, can differ between runs; dq is deterministic.
 * Limits: the forward's, and H <= 64/c with c = 1, 2, 4 for d <= 64, 128, 256 (H counted
 * rounded up to 4, 16, 32 or 64).  Workspace: hcsa_csa_sparse_attn_bwd_workspace_size
 * (the call's B, Nq, H, d, kv_dtype, N and k) or hcsa_hca_dense_attn_bwd_workspace_size
 * bytes, 256-byte aligned (zero bytes, and NULL allowed, except for bf16 16 x 128 with 16
 * or more query tokens, where the keys shared by consecutive tokens -- HCA entries, CSA
 * window rows -- get their gradients key-major, one block per 16 keys and 128 tokens, and
 * the CSA selected entries key-major by tiles of 128 entries: each row's selections are
 * sorted by tile, the pairs' probabilities and dS are kept in the workspace (64 bytes per
 * selected pair: about B * Nq * k * 64 bytes in all), and each tile's gradients are summed
 * over 4096 tokens before they are added; with a NULL workspace all of them stay
 * query-major).
 */
size_t hcsa_csa_sparse_attn_bwd_workspace_size(int B, int Nq, int H, int d, int kv_dtype,
                                               int N, int k);
int hcsa_csa_sparse_attn_bwd(const void *q, const void *kc, const void *vc, int64_t c_bstride,
                             int N, const int32_t *topk_idx, int k, const void *k_raw,
                             const void *v_raw, int64_t raw_bstride, int64_t T_raw,
                             int64_t raw_pos0, int n_win, int ratio, int64_t pos0,
                             const int64_t *seq_pos, int kv_dtype, int B, int Nq, int H, int d,
                             float scale, const float *out, const float *lse,
                             const float *dout, const float *dlse, float *dq, float *dkc,
                             float *dvc, int64_t dc_bstride, float *dk_raw, float *dv_raw,
                             int64_t draw_bstride, void *workspace, size_t ws_bytes,
                             hcsa_stream stream);
size_t hcsa_hca_dense_attn_bwd_workspace_size(int B, int Nq, int H, int d, int kv_dtype);
int hcsa_hca_dense_attn_bwd(const void *q, const void *kh, const void *vh, int64_t h_bstride,
                            int N, int ratio, int64_t pos0, const int64_t *seq_pos,
                            int kv_dtype, int B, int Nq, int H, int d, float scale,
                            const float *out, const float *lse, const float *dout,
                            const float *dlse, float *dq, float *dkh, float *dvh,
                            int64_t dh_bstride, void *workspace, size_t ws_bytes,
                            hcsa_stream stream);

/*
 * Backward of hcsa_compress_kv (same x, omega, ratio, B, T, D) [Lighthouse section 八 items 2
 * and 3]: given dy [B][T/ratio][D] F32 (dy_bstride elements), accumulates dx [B][T][D] F32
 * (dx_bstride; token j*ratio + i gets alpha_i dy_j, the unpooled tail nothing) and, when
 * domega is not NULL, domega [ratio] F32 (the softmax's derivative: alpha_k (g_k -
 * sum_i alpha_i g_i) with g_i = sum over sequences and entries of dy_j . x_{j*ratio+i}).
 * The sums run in a fixed order (deterministic).  workspace: at least
 * hcsa_compress_kv_bwd_workspace_size(B, T, ratio) bytes, 256-byte aligned.
 */
size_t hcsa_compress_kv_bwd_workspace_size(int B, int T, int ratio);
int hcsa_compress_kv_bwd(const void *x, int x_dtype, int64_t x_bstride, int B, int T, int D,
                         const float *omega, int ratio, const float *dy, int64_t dy_bstride,
                         float *dx, int64_t dx_bstride, float *domega, void *workspace,
                         size_t ws_bytes, hcsa_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* HCSA_H */
