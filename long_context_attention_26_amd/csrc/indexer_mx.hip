// Lightning-indexer scores of MXFP4 keys (the score array form): the scan kernel's score
// variants and their launchers.
//
// FP4 on the indexer's QK path with FP32 scores optionally stored as BF16 (9fzt.com digest
// item 4); the score form s_j = sum_g w_g * max(0, q_g . k_j) is the reading taken
// (Lighthouse, "deep deepseek v4 release", section 八 item 3 names the indexer without a
// formula).
#include "common.h"
#include <hip/hip_ext.h>

#include "internal.h"
#include "mx_dev.h"
#include "pool_dev.h"
#include "select_dev.h"
#include "mx_scan.h"

namespace hcsa {

namespace {

// KS: 64-channel MFMA steps the kernels hold registers for (d_I <= 64: one).  The FP8 form
// holds two: at 108 registers (4 waves per SIMD) its candidate scan took 71-74 us at batch 32
// x 1M tokens, against 80-81 us with one (72 registers, 7 waves), on the same box.
template <int HI, int KS, bool QBF16, bool F8>
hipError_t launch_mx_mfma_ks(const IdxMxDev& A, int rows, int score_dtype, hipStream_t s) {
  const int nchunks = (A.N + A.chunk - 1) / A.chunk;
  dim3 grid(nchunks, rows);
  if (score_dtype == 1)
    if (A.pm.table) launch_timed(index_scores_mx_mfma_kernel<HI, KS, QBF16, true, true, F8, false>, grid, dim3(256), s, A);
    else launch_timed(index_scores_mx_mfma_kernel<HI, KS, QBF16, true, false, F8, false>, grid, dim3(256), s, A);
  else
    if (A.pm.table) launch_timed(index_scores_mx_mfma_kernel<HI, KS, QBF16, false, true, F8, false>, grid, dim3(256), s, A);
    else launch_timed(index_scores_mx_mfma_kernel<HI, KS, QBF16, false, false, F8, false>, grid, dim3(256), s, A);
  return hipGetLastError();
}

template <int HI, bool QBF16, bool F8>
hipError_t launch_mx_mfma_hi(const IdxMxDev& A, int rows, int score_dtype, hipStream_t s) {
  if (A.d_I > 64 || F8) return launch_mx_mfma_ks<HI, 2, QBF16, F8>(A, rows, score_dtype, s);
  return launch_mx_mfma_ks<HI, 1, QBF16, F8>(A, rows, score_dtype, s);
}

template <bool QBF16, bool F8>
hipError_t launch_mx_mfma(const IdxMxDev& A, int rows, int H_I, int score_dtype, hipStream_t s) {
  switch (H_I) {
    case 1: return launch_mx_mfma_hi<1, QBF16, F8>(A, rows, score_dtype, s);
    case 2: return launch_mx_mfma_hi<2, QBF16, F8>(A, rows, score_dtype, s);
    case 4: return launch_mx_mfma_hi<4, QBF16, F8>(A, rows, score_dtype, s);
    case 8: return launch_mx_mfma_hi<8, QBF16, F8>(A, rows, score_dtype, s);
    case 16: return launch_mx_mfma_hi<16, QBF16, F8>(A, rows, score_dtype, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_mxfp4_index_scores(const void* q, int q_dtype, const float* w,
                                     const uint8_t* kx, int64_t k_bstride, const uint8_t* ks,
                                     int64_t ks_bstride, int B, int Nq, int H_I, int d_I,
                                     int N, int ratio, int64_t pos0, const int64_t* seq_pos,
                                     const int32_t* block_table, int64_t table_stride,
                                     int score_dtype, void* scores, bool fp8, hipStream_t s) {
  const IdxMxDev A = make_mx_dev(q, w, kx, k_bstride, ks, ks_bstride, B, Nq, d_I, N, ratio,
                                 pos0, seq_pos, block_table, table_stride, scores);
  if (fp8) {
    if (q_dtype == 1) return launch_mx_mfma<true, true>(A, B * Nq, H_I, score_dtype, s);
    return launch_mx_mfma<false, true>(A, B * Nq, H_I, score_dtype, s);
  }
  if (q_dtype == 1) return launch_mx_mfma<true, false>(A, B * Nq, H_I, score_dtype, s);
  return launch_mx_mfma<false, false>(A, B * Nq, H_I, score_dtype, s);
}

}  // namespace hcsa
