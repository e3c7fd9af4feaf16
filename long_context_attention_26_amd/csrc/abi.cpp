// C ABI of libhcsa: argument validation on the host, then asynchronous launches on the
// caller's stream.  No call allocates device memory or synchronizes.
#include <cmath>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <initializer_list>
#include <string>

#include "internal.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return HCSA_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(HCSA_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

int elem_size(int dt) { return dt == HCSA_F32 ? 4 : 2; }

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return HCSA_OK;
  if (ws == nullptr || ws_bytes < need)
    return fail(HCSA_EWORKSPACE, "workspace of %zu bytes needed, %zu given%s", need, ws_bytes,
                ws == nullptr ? " (null)" : "");
  if (!aligned256(ws)) return fail(HCSA_EWORKSPACE, "workspace must be 256-byte aligned");
  return HCSA_OK;
}

// Common checks of the attention calls (q/out/lse shape and dtype).
int check_attn_common(const void* q, int kv_dtype, int B, int Nq, int H, int d, float scale,
                      const float* out, const float* lse, int ratio, int64_t pos0) {
  if (kv_dtype != HCSA_F32 && kv_dtype != HCSA_BF16)
    return fail(HCSA_EDTYPE, "kv_dtype must be F32 or BF16");
  if (B < 1 || Nq < 1) return fail(HCSA_EINVAL, "B and Nq must be >= 1");
  if (static_cast<int64_t>(B) * Nq > 65535) return fail(HCSA_EINVAL, "B*Nq must be <= 65535");
  if (H < 1 || H > 64) return fail(HCSA_EINVAL, "H must be in [1, 64]");
  if (d < 8 || d > 256 || d % 8 != 0) return fail(HCSA_EINVAL, "d must be a multiple of 8 in [8, 256]");
  if (H * d > 4096) return fail(HCSA_EINVAL, "H*d must be <= 4096");
  if (!(scale > 0.0f) || !std::isfinite(scale))
    return fail(HCSA_EINVAL, "scale must be positive and finite");
  if (ratio < 1) return fail(HCSA_EINVAL, "ratio must be >= 1");
  if (pos0 < 0) return fail(HCSA_EINVAL, "pos0 must be >= 0");
  if (!q || !out || !lse) return fail(HCSA_EINVAL, "q, out and lse must be non-null");
  if (!aligned16(q) || !aligned16(out) || !aligned16(lse))
    return fail(HCSA_EALIGN, "q, out and lse must be 16-byte aligned");
  return HCSA_OK;
}

// Cache layout: a block table (device int32, 4-byte aligned) and its row stride, or none
// (contiguous caches); every pooling ratio of a paged call must divide the 128-token page.
// raw_ring: 0, or a power of two in [128, 2^30] (raw tokens in a ring of that many rows).
int check_pages(const hcsa_pages* pages, std::initializer_list<int> ratios) {
  if (!pages) return HCSA_OK;
  if (pages->raw_ring != 0 &&
      (pages->raw_ring < 128 || pages->raw_ring > (1LL << 30) ||
       !is_pow2(static_cast<int>(pages->raw_ring))))
    return fail(HCSA_EINVAL, "pages->raw_ring must be 0 or a power of two in [128, 2^30]");
  if (!pages->block_table) return HCSA_OK;
  if (reinterpret_cast<uintptr_t>(pages->block_table) % 4 != 0)
    return fail(HCSA_EALIGN, "pages->block_table must be 4-byte aligned");
  if (pages->table_stride < 1) return fail(HCSA_EINVAL, "pages->table_stride must be >= 1");
  for (int r : ratios)
    if (r < 1 || 128 % r != 0) return fail(HCSA_EINVAL, "paged caches need ratios dividing 128 (got %d)", r);
  return HCSA_OK;
}
const int32_t* page_table(const hcsa_pages* pages) { return pages ? pages->block_table : nullptr; }
int64_t page_stride(const hcsa_pages* pages) { return pages ? pages->table_stride : 0; }
bool is_paged(const hcsa_pages* pages) { return pages && pages->block_table; }
int64_t raw_ring(const hcsa_pages* pages) { return pages ? pages->raw_ring : 0; }

}  // namespace

namespace hcsa {

int abi_fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

}  // namespace hcsa

extern "C" {

int hcsa_version(void) { return 100; }

int hcsa_time_next_indexer(void* start_event, void* stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr))
    return fail(HCSA_EINVAL, "give both events or neither");
  hcsa::time_next_indexer(static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event));
  return ok();
}

int hcsa_set_attn_splits(int splits) {
  if (splits < 0 || splits > 1024) return fail(HCSA_EINVAL, "splits must be in [0, 1024]");
  hcsa::set_attn_splits(splits);
  return ok();
}

const char* hcsa_last_error(void) { return g_err.c_str(); }

static int check_compress(const void* x, int x_dtype, int64_t x_bstride, int T, int64_t x_rows,
                          int Bx, int By, int D, const float* omega, int ratio, void* y,
                          int y_dtype, int64_t y_bstride, uint8_t* y_scales,
                          int64_t ys_bstride);

int hcsa_compress_kv(const void* x, int x_dtype, int64_t x_bstride, int B, int T, int D,
                     const float* omega, int ratio, void* y, int y_dtype, int64_t y_bstride,
                     uint8_t* y_scales, int64_t ys_bstride, hcsa_stream stream) {
  const int rc = check_compress(x, x_dtype, x_bstride, T, T, B, B, D, omega, ratio, y, y_dtype,
                                y_bstride, y_scales, ys_bstride);
  if (rc) return rc;
  if (T / ratio == 0) return ok();
  return hip_status(hcsa::launch_compress(x, x_dtype, x_bstride, B, T, D, omega, ratio, y,
                                          y_dtype, y_bstride, y_scales, ys_bstride,
                                          static_cast<hipStream_t>(stream)),
                    "hcsa_compress_kv");
}

static int check_pool_jobs(const hcsa_pool_job* jobs, int n_jobs, int B,
                           const hcsa_pages* pages) {
  if (n_jobs < 0 || n_jobs > HCSA_MAX_POOL_JOBS)
    return fail(HCSA_EINVAL, "n_jobs must be in [0, %d]", HCSA_MAX_POOL_JOBS);
  if (n_jobs > 0 && !jobs) return fail(HCSA_EINVAL, "jobs must be non-null");
  int rc = check_pages(pages, {});
  if (rc) return rc;
  const bool paged = is_paged(pages);
  const int64_t ring = raw_ring(pages);
  for (int i = 0; i < n_jobs; ++i) {
    const hcsa_pool_job& q = jobs[i];
    // strides of page pools are unused; a ring's sequences are x_bstride apart and hold
    // `ring` rows each
    rc = check_compress(q.x, q.x_dtype, q.x_bstride, q.T, ring ? ring : q.T,
                        ring || !paged ? B : 1, paged ? 1 : B, q.D, q.omega, q.ratio,
                        q.y, q.y_dtype, q.y_bstride, q.y_scales, q.ys_bstride);
    if (!rc && (paged || ring)) {
      rc = check_pages(pages, {q.ratio});
      if (!rc && (q.ratio > 128 || 128 % q.ratio != 0))
        rc = fail(HCSA_EINVAL, "ratio must divide 128");
      if (!rc && (q.pos0 < 0 || q.pos0 % q.ratio != 0))
        rc = fail(HCSA_EINVAL, "pos0 must be a non-negative multiple of ratio");
      if (!rc && ring && q.T > ring)
        rc = fail(HCSA_EINVAL, "T (%d) exceeds the raw-token ring (%lld rows)", q.T,
                  static_cast<long long>(ring));
    }
    if (rc) return fail(rc, "job %d: %s", i, g_err.c_str());
  }
  return HCSA_OK;
}

int hcsa_compress_kv_batched(const hcsa_pool_job* jobs, int n_jobs, int B,
                             const hcsa_pages* pages, hcsa_stream stream) {
  const int rc = check_pool_jobs(jobs, n_jobs, B, pages);
  if (rc) return rc;
  const int64_t ring = raw_ring(pages);
  return hip_status(hcsa::launch_compress_batched(jobs, n_jobs, B, page_table(pages),
                                                  page_stride(pages), ring,
                                                  static_cast<hipStream_t>(stream)),
                    "hcsa_compress_kv_batched");
}

// x holds x_rows rows per sequence (x_bstride apart, checked when Bx > 1); y's sequences
// are y_bstride apart (checked when By > 1).
static int check_compress(const void* x, int x_dtype, int64_t x_bstride, int T, int64_t x_rows,
                          int Bx, int By, int D, const float* omega, int ratio, void* y,
                          int y_dtype, int64_t y_bstride, uint8_t* y_scales,
                          int64_t ys_bstride) {
  const int B = Bx > By ? Bx : By;
  if (x_dtype != HCSA_F32 && x_dtype != HCSA_BF16)
    return fail(HCSA_EDTYPE, "x_dtype must be F32 or BF16");
  if (y_dtype != HCSA_F32 && y_dtype != HCSA_BF16 && y_dtype != HCSA_MXFP4)
    return fail(HCSA_EDTYPE, "y_dtype must be F32, BF16 or MXFP4");
  if (B < 1 || B > 65535) return fail(HCSA_EINVAL, "B must be in [1, 65535]");
  if (T < 0) return fail(HCSA_EINVAL, "T must be >= 0");
  if (D < 8 || D > 2048 || D % 8 != 0) return fail(HCSA_EINVAL, "D must be a multiple of 8 in [8, 2048]");
  if (y_dtype == HCSA_MXFP4 && D % 32 != 0) return fail(HCSA_EINVAL, "MXFP4 output needs D % 32 == 0");
  if (ratio < 1 || ratio > 1024) return fail(HCSA_EINVAL, "ratio must be in [1, 1024]");
  if (!x || !y || !omega) return fail(HCSA_EINVAL, "x, omega and y must be non-null");
  if (y_dtype == HCSA_MXFP4 && !y_scales) return fail(HCSA_EINVAL, "MXFP4 output needs y_scales");
  const int n_out = T / ratio;
  if (Bx > 1 && x_bstride < x_rows * D) return fail(HCSA_EINVAL, "x_bstride < rows*D");
  if (By > 1) {
    const int64_t yrow = y_dtype == HCSA_MXFP4 ? D / 2 : D;
    if (y_bstride < static_cast<int64_t>(n_out) * yrow) return fail(HCSA_EINVAL, "y_bstride too small");
    if (y_dtype == HCSA_MXFP4 && ys_bstride < static_cast<int64_t>(n_out) * (D / 32))
      return fail(HCSA_EINVAL, "ys_bstride too small");
  }
  if (!aligned16(x) || !aligned16(y)) return fail(HCSA_EALIGN, "x and y must be 16-byte aligned");
  if ((x_bstride * elem_size(x_dtype)) % 16 != 0)
    return fail(HCSA_EALIGN, "x_bstride must keep 16-byte alignment");
  const int64_t yb = y_dtype == HCSA_MXFP4 ? y_bstride : y_bstride * elem_size(y_dtype);
  if (yb % 16 != 0) return fail(HCSA_EALIGN, "y_bstride must keep 16-byte alignment");
  return HCSA_OK;
}

int hcsa_mxfp4_quantize(const void* x, int x_dtype, int64_t rows, int D, uint8_t* packed,
                        uint8_t* scales, hcsa_stream stream) {
  if (x_dtype != HCSA_F32 && x_dtype != HCSA_BF16)
    return fail(HCSA_EDTYPE, "x_dtype must be F32 or BF16");
  if (rows < 0 || rows > 0x7fffffffLL) return fail(HCSA_EINVAL, "rows must be in [0, 2^31)");
  if (D < 32 || D > 2048 || D % 32 != 0) return fail(HCSA_EINVAL, "D must be a multiple of 32 in [32, 2048]");
  if (!x || !packed || !scales) return fail(HCSA_EINVAL, "null pointer");
  if (!aligned16(x) || !aligned16(packed)) return fail(HCSA_EALIGN, "x and packed must be 16-byte aligned");
  if (rows == 0) return ok();
  return hip_status(hcsa::launch_mxfp4_quantize(x, x_dtype, rows, D, packed, scales,
                                                static_cast<hipStream_t>(stream)),
                    "hcsa_mxfp4_quantize");
}

size_t hcsa_topk_workspace_size(int score_dtype, int B, int Nq, int N, int k) {
  if (B < 1 || Nq < 1 || N < 1 || k < 1) return 0;
  return hcsa::plan_topk(score_dtype, B * Nq, N, k).total_bytes;
}

// Per-sequence positions (ragged batches): a device array of B int64 values, each >= 0
// (not checked: device memory), or null.
static int check_seq_pos(const int64_t* seq_pos) {
  if (seq_pos && reinterpret_cast<uintptr_t>(seq_pos) % 8 != 0)
    return fail(HCSA_EALIGN, "seq_pos must be 8-byte aligned");
  return HCSA_OK;
}

static int check_topk_args(int score_dtype, int B, int Nq, int N, int ratio, int64_t pos0,
                           int k) {
  if (score_dtype != HCSA_F32 && score_dtype != HCSA_BF16)
    return fail(HCSA_EDTYPE, "score_dtype must be F32 or BF16");
  if (B < 1 || Nq < 1) return fail(HCSA_EINVAL, "B and Nq must be >= 1");
  if (static_cast<int64_t>(B) * Nq > 65535) return fail(HCSA_EINVAL, "B*Nq must be <= 65535");
  if (N < 1) return fail(HCSA_EINVAL, "N must be >= 1");
  if (!hcsa::topk_plan_ok(hcsa::plan_topk(score_dtype, B * Nq, N, 1)))
    return fail(HCSA_EINVAL, "N too large for the selector (at most 2^25 entries per row)");
  if (k < 1 || k > 4096) return fail(HCSA_EINVAL, "k must be in [1, 4096]");
  if (ratio < 1) return fail(HCSA_EINVAL, "ratio must be >= 1");
  if (pos0 < 0) return fail(HCSA_EINVAL, "pos0 must be >= 0");
  return HCSA_OK;
}

int hcsa_topk(const void* scores, int score_dtype, int64_t row_stride, int B, int Nq, int N,
              int ratio, int64_t pos0, const int64_t* seq_pos, int k, int32_t* idx,
              void* workspace, size_t ws_bytes, hcsa_stream stream) {
  int rc = check_topk_args(score_dtype, B, Nq, N, ratio, pos0, k);
  if (rc) return rc;
  rc = check_seq_pos(seq_pos);
  if (rc) return rc;
  if (row_stride < N) return fail(HCSA_EINVAL, "row_stride < N");
  if (!scores || !idx) return fail(HCSA_EINVAL, "scores and idx must be non-null");
  if (!aligned16(scores) || !aligned16(idx)) return fail(HCSA_EALIGN, "scores and idx must be 16-byte aligned");
  const hcsa::TopkPlan plan = hcsa::plan_topk(score_dtype, B * Nq, N, k);
  rc = check_ws(workspace, ws_bytes, plan.total_bytes);
  if (rc) return rc;
  return hip_status(hcsa::launch_topk(plan, scores, score_dtype, row_stride, Nq, ratio, pos0,
                                      seq_pos, idx, workspace, static_cast<hipStream_t>(stream)),
                    "hcsa_topk");
}


// Few long rows of bf16 scores over MXFP4 keys, with no score copy requested: the fused
// selection (no score array).
static bool index_topk_fused(int k_dtype, int score_dtype, int B, int Nq, int N, int k,
                             const void* scores_out) {
  return scores_out == nullptr && (k_dtype == HCSA_MXFP4 || k_dtype == HCSA_MXFP4_FP8) &&
         !hcsa::plan_topk(score_dtype, B * Nq, N, k).rows_path &&
         hcsa::mx_topk_fused_ok(B * Nq, N, score_dtype);
}

size_t hcsa_csa_index_topk_workspace_size(int B, int Nq, int N, int k, int score_dtype) {
  if (B < 1 || Nq < 1 || N < 1 || k < 1) return 0;
  const size_t scores = hcsa::align256(static_cast<size_t>(B) * Nq * N * (score_dtype == HCSA_BF16 ? 2 : 4));
  const size_t two_pass = scores + hcsa::plan_topk(score_dtype, B * Nq, N, k).total_bytes;
  // the key dtype is not an argument: cover the fused selection of MXFP4 keys too
  const size_t fused = index_topk_fused(HCSA_MXFP4, score_dtype, B, Nq, N, k, nullptr)
                           ? hcsa::mx_topk_workspace_bytes(B * Nq, N) : 0;
  return two_pass > fused ? two_pass : fused;
}

static int check_index_args(const void* q_idx, int q_dtype, const float* w_idx,
                            const void* k_idx, int k_dtype, int64_t k_bstride,
                            const uint8_t* k_scales, int64_t ks_bstride, int B, int Nq,
                            int H_I, int d_I, int N, bool paged = false) {
  if (k_dtype != HCSA_F32 && k_dtype != HCSA_BF16 && k_dtype != HCSA_MXFP4 &&
      k_dtype != HCSA_MXFP4_FP8)
    return fail(HCSA_EDTYPE, "k_dtype must be F32, BF16, MXFP4 or MXFP4_FP8");
  if (q_dtype != HCSA_F32 && q_dtype != HCSA_BF16) return fail(HCSA_EDTYPE, "q_dtype must be F32 or BF16");
  const bool mx = k_dtype == HCSA_MXFP4 || k_dtype == HCSA_MXFP4_FP8;
  if (!mx && q_dtype != k_dtype)
    return fail(HCSA_EDTYPE, "q_dtype must equal k_dtype for F32/BF16 keys");
  if (!is_pow2(H_I) || H_I > 16) return fail(HCSA_EINVAL, "H_I must be 1, 2, 4, 8 or 16");
  if (k_dtype == HCSA_F32 && d_I != 32 && d_I != 64) return fail(HCSA_EINVAL, "F32 keys need d_I in {32, 64}");
  if (k_dtype != HCSA_F32 && d_I != 32 && d_I != 64 && d_I != 128)
    return fail(HCSA_EINVAL, "d_I must be 32, 64 or 128");
  if (!q_idx || !w_idx || !k_idx) return fail(HCSA_EINVAL, "null pointer");
  if (mx && !k_scales) return fail(HCSA_EINVAL, "MXFP4 keys need k_scales");
  if (!aligned16(q_idx) || !aligned16(k_idx))
    return fail(HCSA_EALIGN, "q_idx and k_idx must be 16-byte aligned");
  if (paged) return HCSA_OK;                     // page pools: the strides are unused
  const int64_t kb = mx ? k_bstride : k_bstride * elem_size(k_dtype);
  if (kb % 16 != 0) return fail(HCSA_EALIGN, "k_bstride must keep 16-byte alignment");
  if (B > 1) {
    const int64_t row = mx ? d_I / 2 : d_I;
    if (k_bstride < static_cast<int64_t>(N) * row) return fail(HCSA_EINVAL, "k_bstride too small");
    if (mx && ks_bstride < static_cast<int64_t>(N) * (d_I / 32))
      return fail(HCSA_EINVAL, "ks_bstride too small");
  }
  return HCSA_OK;
}

int hcsa_csa_index_scores(const void* q_idx, int q_dtype, const float* w_idx,
                          const void* k_idx, int k_dtype, int64_t k_bstride,
                          const uint8_t* k_scales, int64_t ks_bstride, int B, int Nq, int H_I,
                          int d_I, int N, int ratio, int64_t pos0, const int64_t* seq_pos,
                          const hcsa_pages* pages, int score_dtype, void* scores,
                          hcsa_stream stream) {
  int rc = check_topk_args(score_dtype, B, Nq, N, ratio, pos0, 1);
  if (rc) return rc;
  rc = check_seq_pos(seq_pos);
  if (rc) return rc;
  rc = check_pages(pages, {ratio});
  if (rc) return rc;
  rc = check_index_args(q_idx, q_dtype, w_idx, k_idx, k_dtype, k_bstride, k_scales, ks_bstride,
                        B, Nq, H_I, d_I, N, is_paged(pages));
  if (rc) return rc;
  if (!scores) return fail(HCSA_EINVAL, "scores must be non-null");
  if (!aligned16(scores)) return fail(HCSA_EALIGN, "scores must be 16-byte aligned");
  return hip_status(hcsa::launch_index_scores(q_idx, q_dtype, w_idx, k_idx, k_dtype, k_bstride,
                                              k_scales, ks_bstride, B, Nq, H_I, d_I, N, ratio,
                                              pos0, seq_pos, page_table(pages),
                                              page_stride(pages), score_dtype, scores,
                                              static_cast<hipStream_t>(stream)),
                    "hcsa_csa_index_scores");
}

// Indexer + top-k, after the pooling jobs (validated) when given: in the fused selection
// the pooling runs in the floors' launch, otherwise in its own launch first.
static int index_topk_impl(const void* q_idx, int q_dtype, const float* w_idx, const void* k_idx,
                           int k_dtype, int64_t k_bstride, const uint8_t* k_scales,
                           int64_t ks_bstride, int B, int Nq, int H_I, int d_I, int N, int ratio,
                           int64_t pos0, const int64_t* seq_pos, const hcsa_pages* pages, int k,
                           int score_dtype, int32_t* topk_idx, void* scores_out, void* workspace,
                           size_t ws_bytes, hcsa_stream stream, const hcsa_pool_job* jobs,
                           int n_jobs) {
  int rc = check_topk_args(score_dtype, B, Nq, N, ratio, pos0, k);
  if (rc) return rc;
  rc = check_seq_pos(seq_pos);
  if (rc) return rc;
  rc = check_pages(pages, {ratio});
  if (rc) return rc;
  rc = check_index_args(q_idx, q_dtype, w_idx, k_idx, k_dtype, k_bstride, k_scales, ks_bstride,
                        B, Nq, H_I, d_I, N, is_paged(pages));
  if (rc) return rc;
  if (!topk_idx) return fail(HCSA_EINVAL, "topk_idx must be non-null");
  if (!aligned16(topk_idx) || (scores_out && !aligned16(scores_out)))
    return fail(HCSA_EALIGN, "topk_idx and scores_out must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool fused = index_topk_fused(k_dtype, score_dtype, B, Nq, N, k, scores_out);
  const size_t sbytes = hcsa::align256(static_cast<size_t>(B) * Nq * N * (score_dtype == HCSA_BF16 ? 2 : 4));
  const hcsa::TopkPlan plan = hcsa::plan_topk(score_dtype, B * Nq, N, k);
  rc = check_ws(workspace, ws_bytes,
                fused ? hcsa::mx_topk_workspace_bytes(B * Nq, N) : sbytes + plan.total_bytes);
  if (rc) return rc;
  if (fused)
    return hip_status(hcsa::launch_mxfp4_index_topk(
                          q_idx, q_dtype, w_idx, static_cast<const uint8_t*>(k_idx), k_bstride,
                          k_scales, ks_bstride, B, Nq, H_I, d_I, N, ratio, pos0, seq_pos,
                          page_table(pages), page_stride(pages), k, topk_idx,
                          k_dtype == HCSA_MXFP4_FP8, workspace, s, jobs, n_jobs,
                          raw_ring(pages)),
                      "hcsa_csa_index_topk (fused)");
  hipError_t e = hipSuccess;
  if (jobs && n_jobs > 0) {
    e = hcsa::launch_compress_batched(jobs, n_jobs, B, page_table(pages), page_stride(pages),
                                      raw_ring(pages), s);
    if (e != hipSuccess) return hip_status(e, "hcsa_csa_pool_index_topk (pooling)");
  }
  void* scores = scores_out ? scores_out : workspace;
  void* tws = static_cast<char*>(workspace) + sbytes;
  e = hcsa::launch_index_scores(q_idx, q_dtype, w_idx, k_idx, k_dtype, k_bstride, k_scales,
                                ks_bstride, B, Nq, H_I, d_I, N, ratio, pos0, seq_pos,
                                page_table(pages), page_stride(pages), score_dtype, scores, s);
  if (e != hipSuccess) return hip_status(e, "hcsa_csa_index_topk (scores)");
  e = hcsa::launch_topk(plan, scores, score_dtype, N, Nq, ratio, pos0, seq_pos, topk_idx, tws, s);
  return hip_status(e, "hcsa_csa_index_topk (select)");
}

int hcsa_csa_index_topk(const void* q_idx, int q_dtype, const float* w_idx, const void* k_idx,
                        int k_dtype, int64_t k_bstride, const uint8_t* k_scales,
                        int64_t ks_bstride, int B, int Nq, int H_I, int d_I, int N, int ratio,
                        int64_t pos0, const int64_t* seq_pos, const hcsa_pages* pages, int k,
                        int score_dtype, int32_t* topk_idx, void* scores_out, void* workspace,
                        size_t ws_bytes, hcsa_stream stream) {
  return index_topk_impl(q_idx, q_dtype, w_idx, k_idx, k_dtype, k_bstride, k_scales,
                         ks_bstride, B, Nq, H_I, d_I, N, ratio, pos0, seq_pos, pages, k,
                         score_dtype, topk_idx, scores_out, workspace, ws_bytes, stream,
                         nullptr, 0);
}

int hcsa_csa_pool_index_topk(const hcsa_pool_job* jobs, int n_jobs, const void* q_idx,
                             int q_dtype, const float* w_idx, const void* k_idx, int k_dtype,
                             int64_t k_bstride, const uint8_t* k_scales, int64_t ks_bstride,
                             int B, int Nq, int H_I, int d_I, int N, int ratio, int64_t pos0,
                             const int64_t* seq_pos, const hcsa_pages* pages, int k,
                             int score_dtype, int32_t* topk_idx, void* scores_out,
                             void* workspace, size_t ws_bytes, hcsa_stream stream) {
  const int rc = check_pool_jobs(jobs, n_jobs, B, pages);
  if (rc) return rc;
  return index_topk_impl(q_idx, q_dtype, w_idx, k_idx, k_dtype, k_bstride, k_scales,
                         ks_bstride, B, Nq, H_I, d_I, N, ratio, pos0, seq_pos, pages, k,
                         score_dtype, topk_idx, scores_out, workspace, ws_bytes, stream, jobs,
                         n_jobs);
}

static int attn_max_len_csa(int k, int n_win) { return k + n_win; }

size_t hcsa_csa_sparse_attn_workspace_size(int B, int Nq, int H, int d, int k, int n_win) {
  if (B < 1 || Nq < 1 || H < 1 || d < 1 || k < 0 || n_win < 0) return 0;
  // the plan depends on the dtype only through the fast-path choice; take the larger
  const size_t a = hcsa::plan_attention(true, HCSA_BF16, B, Nq, H, d, attn_max_len_csa(k, n_win)).total_bytes;
  const size_t b = hcsa::plan_attention(true, HCSA_F32, B, Nq, H, d, attn_max_len_csa(k, n_win)).total_bytes;
  return a > b ? a : b;
}

// Arguments of CSA attention (forward and backward), checked on the host.
static int check_csa(const void* q, const void* kc, const void* vc, int64_t c_bstride, int N,
                     const int32_t* topk_idx, int k, const void* k_raw, const void* v_raw,
                     int64_t raw_bstride, int64_t T_raw, int64_t raw_pos0, int n_win,
                     int ratio, int64_t pos0, const int64_t* seq_pos, const hcsa_pages* pages,
                     int kv_dtype, int B, int Nq, int H, int d, float scale, const float* out,
                     const float* lse) {
  int rc = check_attn_common(q, kv_dtype, B, Nq, H, d, scale, out, lse, ratio, pos0);
  if (rc) return rc;
  rc = check_seq_pos(seq_pos);
  if (rc) return rc;
  rc = check_pages(pages, {ratio});
  if (rc) return rc;
  const bool paged = is_paged(pages);
  const int64_t ring = raw_ring(pages);
  if ((paged || ring) && raw_pos0 != 0)
    return fail(HCSA_EINVAL, "paged or ring raw tokens need raw_pos0 == 0");
  if (k < 0 || k > 4096) return fail(HCSA_EINVAL, "k must be in [0, 4096]");
  if (n_win < 0 || n_win > 4096) return fail(HCSA_EINVAL, "n_win must be in [0, 4096]");
  if (k > 0) {
    if (N < 1) return fail(HCSA_EINVAL, "N must be >= 1 when k > 0");
    if (!kc || !vc || !topk_idx) return fail(HCSA_EINVAL, "kc, vc and topk_idx must be non-null");
    if (!aligned16(kc) || !aligned16(vc)) return fail(HCSA_EALIGN, "kc and vc must be 16-byte aligned");
    if ((c_bstride * elem_size(kv_dtype)) % 16 != 0) return fail(HCSA_EALIGN, "c_bstride alignment");
    if (!paged && B > 1 && c_bstride < static_cast<int64_t>(N) * d) return fail(HCSA_EINVAL, "c_bstride < N*d");
  }
  if (n_win > 0) {
    if (!k_raw || !v_raw) return fail(HCSA_EINVAL, "k_raw and v_raw must be non-null");
    if (!aligned16(k_raw) || !aligned16(v_raw)) return fail(HCSA_EALIGN, "k_raw and v_raw alignment");
    if ((raw_bstride * elem_size(kv_dtype)) % 16 != 0) return fail(HCSA_EALIGN, "raw_bstride alignment");
    if (T_raw < 1) return fail(HCSA_EINVAL, "T_raw must be >= 1");
    if (ring && T_raw != ring) return fail(HCSA_EINVAL, "a raw-token ring needs T_raw == raw_ring");
    // a chunk's windows span n_win + Nq - 1 positions, all of which the ring must hold
    if (ring && n_win + static_cast<int64_t>(Nq) - 1 > ring)
      return fail(HCSA_EINVAL, "n_win + Nq - 1 exceeds the raw-token ring");
    if ((ring || !paged) && B > 1 && raw_bstride < T_raw * d)
      return fail(HCSA_EINVAL, "raw_bstride < T_raw*d");
    // (with per-sequence positions, which sit in device memory, paged raw tokens or a
    // ring, the caller guarantees it)
    const int64_t first = pos0 - n_win + 1 > 0 ? pos0 - n_win + 1 : 0;
    const int64_t last = pos0 + Nq - 1;
    if (!seq_pos && !paged && !ring && (first < raw_pos0 || last >= raw_pos0 + T_raw))
      return fail(HCSA_EINVAL, "window positions [%lld, %lld] not inside the raw rows [%lld, %lld)",
                  static_cast<long long>(first), static_cast<long long>(last),
                  static_cast<long long>(raw_pos0), static_cast<long long>(raw_pos0 + T_raw));
  }
  return HCSA_OK;
}

int hcsa_csa_sparse_attn(const void* q, const void* kc, const void* vc, int64_t c_bstride,
                         int N, const int32_t* topk_idx, int k, const void* k_raw,
                         const void* v_raw, int64_t raw_bstride, int64_t T_raw,
                         int64_t raw_pos0, int n_win, int ratio, int64_t pos0,
                         const int64_t* seq_pos, const hcsa_pages* pages, int kv_dtype, int B,
                         int Nq, int H, int d, float scale, float* out, float* lse,
                         void* workspace, size_t ws_bytes, hcsa_stream stream) {
  int rc = check_csa(q, kc, vc, c_bstride, N, topk_idx, k, k_raw, v_raw, raw_bstride, T_raw,
                     raw_pos0, n_win, ratio, pos0, seq_pos, pages, kv_dtype, B, Nq, H, d, scale,
                     out, lse);
  if (rc) return rc;
  const bool paged = is_paged(pages);
  const int64_t ring = raw_ring(pages);
  (void)paged;
  const hcsa::AttnPlan plan =
      hcsa::plan_attention(true, kv_dtype, B, Nq, H, d, attn_max_len_csa(k, n_win));
  rc = check_ws(workspace, ws_bytes, plan.total_bytes);
  if (rc) return rc;
  hcsa::AttnArgs a{};
  a.q = q; a.kc = kc; a.vc = vc; a.c_bstride = c_bstride; a.N = N > 0 ? N : 0; a.ratio = ratio;
  a.idx = topk_idx; a.k = k; a.k_raw = k_raw; a.v_raw = v_raw; a.raw_bstride = raw_bstride;
  a.T_raw = T_raw; a.raw_pos0 = raw_pos0; a.n_win = n_win; a.pos0 = pos0; a.seq_pos = seq_pos;
  a.block_table = page_table(pages); a.table_stride = page_stride(pages); a.raw_ring = ring;
  a.kv_dtype = kv_dtype; a.B = B; a.Nq = Nq; a.H = H; a.d = d; a.scale = scale;
  a.out = out; a.lse = lse;
  return hip_status(hcsa::launch_attention(true, a, plan, workspace, static_cast<hipStream_t>(stream)),
                    "hcsa_csa_sparse_attn");
}

size_t hcsa_hca_dense_attn_workspace_size(int B, int Nq, int H, int d, int N) {
  if (B < 1 || Nq < 1 || H < 1 || d < 1 || N < 0) return 0;
  const size_t a = hcsa::plan_attention(false, HCSA_BF16, B, Nq, H, d, N).total_bytes;
  const size_t b = hcsa::plan_attention(false, HCSA_F32, B, Nq, H, d, N).total_bytes;
  return a > b ? a : b;
}

// Arguments of HCA attention, checked on the host.
static int check_hca(const void* q, const void* kh, const void* vh, int64_t h_bstride, int N,
                     int ratio, int64_t pos0, const int64_t* seq_pos, const hcsa_pages* pages,
                     int kv_dtype, int B, int Nq, int H, int d, float scale, const float* out,
                     const float* lse) {
  int rc = check_attn_common(q, kv_dtype, B, Nq, H, d, scale, out, lse, ratio, pos0);
  if (rc) return rc;
  rc = check_seq_pos(seq_pos);
  if (rc) return rc;
  rc = check_pages(pages, {ratio});
  if (rc) return rc;
  if (N < 0) return fail(HCSA_EINVAL, "N must be >= 0");
  if (N > 0) {
    if (!kh || !vh) return fail(HCSA_EINVAL, "kh and vh must be non-null");
    if (!aligned16(kh) || !aligned16(vh)) return fail(HCSA_EALIGN, "kh and vh must be 16-byte aligned");
    if ((h_bstride * elem_size(kv_dtype)) % 16 != 0) return fail(HCSA_EALIGN, "h_bstride alignment");
    if (!is_paged(pages) && B > 1 && h_bstride < static_cast<int64_t>(N) * d)
      return fail(HCSA_EINVAL, "h_bstride < N*d");
  }
  return HCSA_OK;
}

int hcsa_hca_dense_attn(const void* q, const void* kh, const void* vh, int64_t h_bstride,
                        int N, int ratio, int64_t pos0, const int64_t* seq_pos,
                        const hcsa_pages* pages, int kv_dtype, int B, int Nq, int H, int d,
                        float scale, float* out, float* lse, void* workspace, size_t ws_bytes,
                        hcsa_stream stream) {
  int rc = check_hca(q, kh, vh, h_bstride, N, ratio, pos0, seq_pos, pages, kv_dtype, B, Nq, H,
                     d, scale, out, lse);
  if (rc) return rc;
  const hcsa::AttnPlan plan = hcsa::plan_attention(false, kv_dtype, B, Nq, H, d, N);
  rc = check_ws(workspace, ws_bytes, plan.total_bytes);
  if (rc) return rc;
  hcsa::AttnArgs a{};
  a.q = q; a.kc = kh; a.vc = vh; a.c_bstride = h_bstride; a.N = N; a.ratio = ratio;
  a.idx = nullptr; a.k = 0; a.k_raw = nullptr; a.v_raw = nullptr; a.raw_bstride = 0;
  a.T_raw = 0; a.raw_pos0 = 0; a.n_win = 0; a.pos0 = pos0; a.seq_pos = seq_pos;
  a.block_table = page_table(pages); a.table_stride = page_stride(pages);
  a.kv_dtype = kv_dtype; a.B = B; a.Nq = Nq; a.H = H; a.d = d; a.scale = scale;
  a.out = out; a.lse = lse;
  return hip_status(hcsa::launch_attention(false, a, plan, workspace, static_cast<hipStream_t>(stream)),
                    "hcsa_hca_dense_attn");
}

// ------------------------------------------------------------------ CSA + HCA in one call

size_t hcsa_csa_hca_attn_workspace_size(int B, int Nq, int H, int d, int k, int n_win, int N_h) {
  const size_t c = hcsa_csa_sparse_attn_workspace_size(B, Nq, H, d, k, n_win);
  const size_t h = hcsa_hca_dense_attn_workspace_size(B, Nq, H, d, N_h);
  if ((B >= 1 && Nq >= 1 && H >= 1 && d >= 1) == false) return 0;
  return hcsa::align256(c) + h;
}

int hcsa_csa_hca_attn(const void* q, const void* kc, const void* vc, int64_t c_bstride, int N,
                      const int32_t* topk_idx, int k, const void* k_raw, const void* v_raw,
                      int64_t raw_bstride, int64_t T_raw, int64_t raw_pos0, int n_win,
                      int ratio, const void* kh, const void* vh, int64_t h_bstride, int N_h,
                      int ratio_h, int64_t pos0, const int64_t* seq_pos,
                      const hcsa_pages* pages, int kv_dtype, int B, int Nq, int H, int d,
                      float scale, float* out_c, float* lse_c, float* out_h, float* lse_h,
                      void* workspace, size_t ws_bytes, hcsa_stream stream) {
  int rc = check_csa(q, kc, vc, c_bstride, N, topk_idx, k, k_raw, v_raw, raw_bstride, T_raw,
                     raw_pos0, n_win, ratio, pos0, seq_pos, pages, kv_dtype, B, Nq, H, d, scale,
                     out_c, lse_c);
  if (rc) return rc;
  rc = check_hca(q, kh, vh, h_bstride, N_h, ratio_h, pos0, seq_pos, pages, kv_dtype, B, Nq, H,
                 d, scale, out_h, lse_h);
  if (rc) return rc;
  const hcsa::AttnPlan pc =
      hcsa::plan_attention(true, kv_dtype, B, Nq, H, d, attn_max_len_csa(k, n_win));
  const hcsa::AttnPlan ph = hcsa::plan_attention(false, kv_dtype, B, Nq, H, d, N_h);
  rc = check_ws(workspace, ws_bytes, hcsa::align256(pc.total_bytes) + ph.total_bytes);
  if (rc) return rc;
  hcsa::AttnArgs c{};
  c.q = q; c.kc = kc; c.vc = vc; c.c_bstride = c_bstride; c.N = N > 0 ? N : 0; c.ratio = ratio;
  c.idx = topk_idx; c.k = k; c.k_raw = k_raw; c.v_raw = v_raw; c.raw_bstride = raw_bstride;
  c.T_raw = T_raw; c.raw_pos0 = raw_pos0; c.n_win = n_win; c.pos0 = pos0; c.seq_pos = seq_pos;
  c.block_table = page_table(pages); c.table_stride = page_stride(pages);
  c.raw_ring = raw_ring(pages);
  c.kv_dtype = kv_dtype; c.B = B; c.Nq = Nq; c.H = H; c.d = d; c.scale = scale;
  c.out = out_c; c.lse = lse_c;
  hcsa::AttnArgs h{};
  h.q = q; h.kc = kh; h.vc = vh; h.c_bstride = h_bstride; h.N = N_h; h.ratio = ratio_h;
  h.pos0 = pos0; h.seq_pos = seq_pos;
  h.block_table = page_table(pages); h.table_stride = page_stride(pages);
  h.kv_dtype = kv_dtype; h.B = B; h.Nq = Nq; h.H = H; h.d = d; h.scale = scale;
  h.out = out_h; h.lse = lse_h;
  return hip_status(hcsa::launch_csa_hca(c, pc, h, ph, workspace, static_cast<hipStream_t>(stream)),
                    "hcsa_csa_hca_attn");
}

// ------------------------------------------------------------------ one decode step

size_t hcsa_decode_step_workspace_size(int B, int Nq, int N, int k, int score_dtype, int H,
                                       int d, int n_win, int N_h) {
  if (B < 1 || Nq < 1 || N < 1 || k < 1 || H < 1 || d < 1) return 0;
  // attention partials: those of the two calls, or of the four-launch form's splits,
  // whichever is larger
  const size_t two = hcsa_csa_hca_attn_workspace_size(B, Nq, H, d, k, n_win, N_h);
  const size_t four = hcsa::align256(hcsa::plan_step_csa(B, Nq, H, d, k, n_win).total_bytes) +
                      hcsa::plan_step_hca(B, Nq, H, d, N_h).total_bytes;
  return hcsa::align256(hcsa_csa_index_topk_workspace_size(B, Nq, N, k, score_dtype)) +
         hcsa::decode_step_sync_bytes(B * Nq) + std::max(two, four);
}

int hcsa_decode_step(const hcsa_pool_job* jobs, int n_jobs, const void* q_idx, int q_dtype,
                     const float* w_idx, const void* k_idx, int k_dtype, int64_t k_bstride,
                     const uint8_t* k_scales, int64_t ks_bstride, int H_I, int d_I,
                     int score_dtype, int32_t* topk_idx, const void* q, const void* kc,
                     const void* vc, int64_t c_bstride, int N, int k, const void* k_raw,
                     const void* v_raw, int64_t raw_bstride, int64_t T_raw, int64_t raw_pos0,
                     int n_win, int ratio, const void* kh, const void* vh, int64_t h_bstride,
                     int N_h, int ratio_h, int64_t pos0, const int64_t* seq_pos,
                     const hcsa_pages* pages, int kv_dtype, int B, int Nq, int H, int d,
                     float scale, float* out_c, float* lse_c, float* out_h, float* lse_h,
                     void* workspace, size_t ws_bytes, hcsa_stream stream) {
  int rc = n_jobs > 0 ? check_pool_jobs(jobs, n_jobs, B, pages) : HCSA_OK;
  if (rc) return rc;
  rc = check_topk_args(score_dtype, B, Nq, N, ratio, pos0, k);
  if (rc) return rc;
  rc = check_seq_pos(seq_pos);
  if (rc) return rc;
  rc = check_pages(pages, {ratio});
  if (rc) return rc;
  rc = check_index_args(q_idx, q_dtype, w_idx, k_idx, k_dtype, k_bstride, k_scales, ks_bstride,
                        B, Nq, H_I, d_I, N, is_paged(pages));
  if (rc) return rc;
  if (!topk_idx) return fail(HCSA_EINVAL, "topk_idx must be non-null");
  if (!aligned16(topk_idx)) return fail(HCSA_EALIGN, "topk_idx must be 16-byte aligned");
  rc = check_csa(q, kc, vc, c_bstride, N, topk_idx, k, k_raw, v_raw, raw_bstride, T_raw,
                 raw_pos0, n_win, ratio, pos0, seq_pos, pages, kv_dtype, B, Nq, H, d, scale,
                 out_c, lse_c);
  if (rc) return rc;
  rc = check_hca(q, kh, vh, h_bstride, N_h, ratio_h, pos0, seq_pos, pages, kv_dtype, B, Nq, H,
                 d, scale, out_h, lse_h);
  if (rc) return rc;
  const size_t mx_bytes = hcsa::align256(hcsa_csa_index_topk_workspace_size(B, Nq, N, k, score_dtype));
  const hcsa::AttnPlan pc =
      hcsa::plan_attention(true, kv_dtype, B, Nq, H, d, attn_max_len_csa(k, n_win));
  const hcsa::AttnPlan ph = hcsa::plan_attention(false, kv_dtype, B, Nq, H, d, N_h);
  const hcsa::AttnPlan pc_step = hcsa::plan_step_csa(B, Nq, H, d, k, n_win);
  const hcsa::AttnPlan ph_step = hcsa::plan_step_hca(B, Nq, H, d, N_h);
  const size_t attn_bytes =
      std::max(hcsa::align256(pc.total_bytes) + ph.total_bytes,
               hcsa::align256(pc_step.total_bytes) + ph_step.total_bytes);
  const size_t sync_bytes = hcsa::decode_step_sync_bytes(B * Nq);
  rc = check_ws(workspace, ws_bytes, mx_bytes + sync_bytes + attn_bytes);
  if (rc) return rc;
  hcsa::DecodeStepArgs a{};
  a.jobs = jobs; a.n_jobs = n_jobs; a.q_idx = q_idx; a.q_dtype = q_dtype; a.w_idx = w_idx;
  a.k_idx = static_cast<const uint8_t*>(k_idx); a.k_dtype = k_dtype; a.k_bstride = k_bstride;
  a.k_scales = k_scales; a.ks_bstride = ks_bstride; a.H_I = H_I; a.d_I = d_I; a.N = N;
  a.score_dtype = score_dtype; a.idx = topk_idx; a.block_table = page_table(pages);
  a.raw_ring = raw_ring(pages); a.seq_pos = seq_pos; a.B = B; a.Nq = Nq;
  hcsa::AttnArgs& c = a.c;
  c.q = q; c.kc = kc; c.vc = vc; c.c_bstride = c_bstride; c.N = N; c.ratio = ratio;
  c.idx = topk_idx; c.k = k; c.k_raw = k_raw; c.v_raw = v_raw; c.raw_bstride = raw_bstride;
  c.T_raw = T_raw; c.raw_pos0 = raw_pos0; c.n_win = n_win; c.pos0 = pos0; c.seq_pos = seq_pos;
  c.block_table = page_table(pages); c.table_stride = page_stride(pages);
  c.raw_ring = raw_ring(pages);
  c.kv_dtype = kv_dtype; c.B = B; c.Nq = Nq; c.H = H; c.d = d; c.scale = scale;
  c.out = out_c; c.lse = lse_c;
  hcsa::AttnArgs& h = a.h;
  h.q = q; h.kc = kh; h.vc = vh; h.c_bstride = h_bstride; h.N = N_h; h.ratio = ratio_h;
  h.pos0 = pos0; h.seq_pos = seq_pos;
  h.block_table = page_table(pages); h.table_stride = page_stride(pages);
  h.kv_dtype = kv_dtype; h.B = B; h.Nq = Nq; h.H = H; h.d = d; h.scale = scale;
  h.out = out_h; h.lse = lse_h;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool fused = index_topk_fused(k_dtype, score_dtype, B, Nq, N, k, nullptr);
  if (hcsa::decode_step_fast(a, pc, ph, fused))
    return hip_status(hcsa::launch_decode_step(a, pc_step, ph_step, workspace, mx_bytes,
                                               mx_bytes + sync_bytes, s),
                      "hcsa_decode_step");
  if (!fused && hcsa::decode_step_scores_ok(a, pc, ph))
    return hip_status(hcsa::launch_decode_step_scores(a, pc_step, ph_step, workspace,
                                                      mx_bytes, mx_bytes + sync_bytes, s),
                      "hcsa_decode_step");
  // other shapes: the two calls in turn, on the same parts of the workspace
  rc = index_topk_impl(q_idx, q_dtype, w_idx, k_idx, k_dtype, k_bstride, k_scales, ks_bstride,
                       B, Nq, H_I, d_I, N, ratio, pos0, seq_pos, pages, k, score_dtype,
                       topk_idx, nullptr, workspace, mx_bytes, stream,
                       n_jobs > 0 ? jobs : nullptr, n_jobs);
  if (rc) return rc;
  return hip_status(hcsa::launch_csa_hca(c, pc, h, ph,
                                         static_cast<char*>(workspace) + mx_bytes + sync_bytes,
                                         s),
                    "hcsa_decode_step (attention)");
}

// ------------------------------------------------------------------ backward (training)

static int check_bwd_grads(const float* dout, const float* dq, int B, int Nq, int H, int d) {
  if (!dout || !dq) return fail(HCSA_EINVAL, "dout and dq must be non-null");
  if (!aligned16(dout) || !aligned16(dq)) return fail(HCSA_EALIGN, "dout and dq must be 16-byte aligned");
  if (!hcsa::attn_bwd_shape_supported(H, d))
    return fail(HCSA_EINVAL, "backward needs H <= 64/c with c = 1, 2, 4 for d <= 64, 128, 256 "
                "(H rounded up to 4, 16, 32 or 64)");
  (void)B; (void)Nq;
  return HCSA_OK;
}

size_t hcsa_csa_sparse_attn_bwd_workspace_size(int B, int Nq, int H, int d, int kv_dtype, int N,
                                                int k) {
  if (B < 1 || Nq < 1 || H < 1 || d < 1) return 0;
  hcsa::AttnArgs a{};
  a.B = B; a.Nq = Nq; a.H = H; a.d = d; a.kv_dtype = kv_dtype;
  a.N = N > 0 ? N : 0; a.k = k > 0 ? k : 0;
  return hcsa::bwd_workspace_bytes(a);
}

int hcsa_csa_sparse_attn_bwd(const void* q, const void* kc, const void* vc, int64_t c_bstride,
                             int N, const int32_t* topk_idx, int k, const void* k_raw,
                             const void* v_raw, int64_t raw_bstride, int64_t T_raw,
                             int64_t raw_pos0, int n_win, int ratio, int64_t pos0,
                             const int64_t* seq_pos, int kv_dtype, int B, int Nq, int H, int d,
                             float scale, const float* out, const float* lse,
                             const float* dout, const float* dlse, float* dq, float* dkc,
                             float* dvc, int64_t dc_bstride, float* dk_raw, float* dv_raw,
                             int64_t draw_bstride, void* workspace, size_t ws_bytes,
                             hcsa_stream stream) {
  int rc = check_csa(q, kc, vc, c_bstride, N, topk_idx, k, k_raw, v_raw, raw_bstride, T_raw,
                     raw_pos0, n_win, ratio, pos0, seq_pos, nullptr, kv_dtype, B, Nq, H, d,
                     scale, out, lse);
  if (rc) return rc;
  rc = check_bwd_grads(dout, dq, B, Nq, H, d);
  if (rc) return rc;
  if (k > 0) {
    if (!dkc || !dvc) return fail(HCSA_EINVAL, "dkc and dvc must be non-null when k > 0");
    if (B > 1 && dc_bstride < static_cast<int64_t>(N) * d) return fail(HCSA_EINVAL, "dc_bstride < N*d");
  }
  if (n_win > 0) {
    if (!dk_raw || !dv_raw) return fail(HCSA_EINVAL, "dk_raw and dv_raw must be non-null when n_win > 0");
    if (B > 1 && draw_bstride < T_raw * d) return fail(HCSA_EINVAL, "draw_bstride < T_raw*d");
  }
  hcsa::AttnArgs a{};
  a.q = q; a.kc = kc; a.vc = vc; a.c_bstride = c_bstride; a.N = N > 0 ? N : 0; a.ratio = ratio;
  a.idx = topk_idx; a.k = k; a.k_raw = k_raw; a.v_raw = v_raw; a.raw_bstride = raw_bstride;
  a.T_raw = T_raw; a.raw_pos0 = raw_pos0; a.n_win = n_win; a.pos0 = pos0; a.seq_pos = seq_pos;
  a.kv_dtype = kv_dtype; a.B = B; a.Nq = Nq; a.H = H; a.d = d; a.scale = scale;
  // a null workspace is allowed: the shared keys then get their gradients query-major
  rc = workspace ? check_ws(workspace, ws_bytes, hcsa::bwd_workspace_bytes(a)) : HCSA_OK;
  if (rc) return rc;
  hcsa::AttnBwdArgs g{out, lse, dout, dlse, dq, dkc, dvc, dc_bstride, dk_raw, dv_raw,
                      draw_bstride, workspace};
  return hip_status(hcsa::launch_attention_bwd(true, a, g, static_cast<hipStream_t>(stream)),
                    "hcsa_csa_sparse_attn_bwd");
}

size_t hcsa_hca_dense_attn_bwd_workspace_size(int B, int Nq, int H, int d, int kv_dtype) {
  if (B < 1 || Nq < 1 || H < 1 || d < 1) return 0;
  hcsa::AttnArgs a{};
  a.B = B; a.Nq = Nq; a.H = H; a.d = d; a.kv_dtype = kv_dtype;
  return hcsa::bwd_workspace_bytes(a);
}

int hcsa_hca_dense_attn_bwd(const void* q, const void* kh, const void* vh, int64_t h_bstride,
                            int N, int ratio, int64_t pos0, const int64_t* seq_pos,
                            int kv_dtype, int B, int Nq, int H, int d, float scale,
                            const float* out, const float* lse, const float* dout,
                            const float* dlse, float* dq, float* dkh, float* dvh,
                            int64_t dh_bstride, void* workspace, size_t ws_bytes,
                            hcsa_stream stream) {
  int rc = check_attn_common(q, kv_dtype, B, Nq, H, d, scale, out, lse, ratio, pos0);
  if (rc) return rc;
  rc = check_seq_pos(seq_pos);
  if (rc) return rc;
  rc = check_bwd_grads(dout, dq, B, Nq, H, d);
  if (rc) return rc;
  if (N < 0) return fail(HCSA_EINVAL, "N must be >= 0");
  if (N > 0) {
    if (!kh || !vh || !dkh || !dvh) return fail(HCSA_EINVAL, "kh, vh, dkh and dvh must be non-null");
    if (!aligned16(kh) || !aligned16(vh)) return fail(HCSA_EALIGN, "kh and vh must be 16-byte aligned");
    if ((h_bstride * elem_size(kv_dtype)) % 16 != 0) return fail(HCSA_EALIGN, "h_bstride alignment");
    if (B > 1 && (h_bstride < static_cast<int64_t>(N) * d || dh_bstride < static_cast<int64_t>(N) * d))
      return fail(HCSA_EINVAL, "h_bstride and dh_bstride must be >= N*d");
  }
  hcsa::AttnArgs a{};
  a.q = q; a.kc = kh; a.vc = vh; a.c_bstride = h_bstride; a.N = N; a.ratio = ratio;
  a.pos0 = pos0; a.seq_pos = seq_pos;
  a.kv_dtype = kv_dtype; a.B = B; a.Nq = Nq; a.H = H; a.d = d; a.scale = scale;
  // a null workspace is allowed: the shared keys then get their gradients query-major
  rc = workspace ? check_ws(workspace, ws_bytes, hcsa::bwd_workspace_bytes(a)) : HCSA_OK;
  if (rc) return rc;
  hcsa::AttnBwdArgs g{out, lse, dout, dlse, dq, dkh, dvh, dh_bstride, nullptr, nullptr, 0,
                      workspace};
  return hip_status(hcsa::launch_attention_bwd(false, a, g, static_cast<hipStream_t>(stream)),
                    "hcsa_hca_dense_attn_bwd");
}

size_t hcsa_compress_kv_bwd_workspace_size(int B, int T, int ratio) {
  if (B < 1 || T < 0 || ratio < 1) return 0;
  return hcsa::compress_bwd_workspace_bytes(B, T, ratio);
}

int hcsa_compress_kv_bwd(const void* x, int x_dtype, int64_t x_bstride, int B, int T, int D,
                         const float* omega, int ratio, const float* dy, int64_t dy_bstride,
                         float* dx, int64_t dx_bstride, float* domega, void* workspace,
                         size_t ws_bytes, hcsa_stream stream) {
  if (x_dtype != HCSA_F32 && x_dtype != HCSA_BF16)
    return fail(HCSA_EDTYPE, "x_dtype must be F32 or BF16");
  if (B < 1 || B > 65535) return fail(HCSA_EINVAL, "B must be in [1, 65535]");
  if (T < 0) return fail(HCSA_EINVAL, "T must be >= 0");
  if (D < 8 || D > 2048 || D % 8 != 0) return fail(HCSA_EINVAL, "D must be a multiple of 8 in [8, 2048]");
  if (ratio < 1 || ratio > 1024) return fail(HCSA_EINVAL, "ratio must be in [1, 1024]");
  if (!x || !omega || !dy || !dx) return fail(HCSA_EINVAL, "x, omega, dy and dx must be non-null");
  if (!aligned16(x) || !aligned16(dy) || !aligned16(dx))
    return fail(HCSA_EALIGN, "x, dy and dx must be 16-byte aligned");
  if ((x_bstride * elem_size(x_dtype)) % 16 != 0 || (dy_bstride * 4) % 16 != 0 ||
      (dx_bstride * 4) % 16 != 0)
    return fail(HCSA_EALIGN, "x_bstride, dy_bstride and dx_bstride must keep 16-byte alignment");
  const int n_out = T / ratio;
  if (B > 1 && (x_bstride < static_cast<int64_t>(T) * D || dx_bstride < static_cast<int64_t>(T) * D ||
                dy_bstride < static_cast<int64_t>(n_out) * D))
    return fail(HCSA_EINVAL, "x_bstride, dx_bstride (>= T*D) or dy_bstride (>= (T/ratio)*D) too small");
  const int rc = check_ws(workspace, ws_bytes, hcsa::compress_bwd_workspace_bytes(B, T, ratio));
  if (rc) return rc;
  if (n_out == 0) return ok();
  return hip_status(hcsa::launch_compress_bwd(x, x_dtype, x_bstride, B, T, D, omega, ratio, dy,
                                              dy_bstride, dx, dx_bstride, domega, workspace,
                                              static_cast<hipStream_t>(stream)),
                    "hcsa_compress_kv_bwd");
}

}  // extern "C"
