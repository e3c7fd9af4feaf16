// Indexer + top-k of MXFP4 keys without the score array (decode): a floor per row from
// scored samples (in the launch of the step's pooling when given), the key scan's
// per-chunk candidate lists, and the exact selection among the candidates per row, with a
// rescan of rows whose lists hold too few or too many candidates.
//
// The indexer keeps the top-k compressed entries (Lighthouse, "deep deepseek v4 release",
// section 八 item 3) from BF16 index scores of FP4 keys (9fzt.com digest item 4).
#include "common.h"
#include <hip/hip_ext.h>

#include "internal.h"
#include "mx_dev.h"
#include "pool_dev.h"
#include "select_dev.h"
#include "mx_scan.h"

namespace hcsa {

namespace {

// grid: rows * kMxFloorParts (the parts of a row adjacent); block 512.
template <int HI, int KS, bool QBF16, bool PAGED, bool F8>
__global__ __launch_bounds__(kMxFloorThreads) void mx_floor_kernel(IdxMxDev A, int k) {
  mx_floor_block<HI, KS, QBF16, PAGED, F8>(A, k, blockIdx.x / kMxFloorParts,
                                           blockIdx.x % kMxFloorParts, false);
}

// The floors and the pooling of the same tokens in one launch: blocks x < Nq * parts of
// grid row y set part x % parts of the floor of query row y*Nq + x / parts (sampling only
// entries completed before the call), the rest run the pooling jobs (sequence y).
// grid: (Nq * parts + pooling blocks, B); block 512.
template <int HI, int KS, bool QBF16, bool PAGED, bool F8>
__global__ __launch_bounds__(kMxFloorThreads) void mx_pool_floor_kernel(PoolJobs J, IdxMxDev A,
                                                                        int k) {
  __shared__ float alpha[1024];
  __shared__ float s_part[kMxFloorThreads * 8];
  const int nf = A.Nq * kMxFloorParts;
  if (static_cast<int>(blockIdx.x) < nf)
    mx_floor_block<HI, KS, QBF16, PAGED, F8>(A, k,
                                             blockIdx.y * A.Nq + blockIdx.x / kMxFloorParts,
                                             blockIdx.x % kMxFloorParts, true);
  else
    pool_jobs_block<PAGED>(J, blockIdx.x - nf, alpha, s_part, blockIdx.y);
}

// grid: rows; block 512.
template <int HI, int KS, bool QBF16, bool PAGED, bool F8>
__global__ __launch_bounds__(kMxResThreads) void mx_list_resolve_kernel(IdxMxDev A, int k,
                                                                        int32_t* idx) {
  mx_resolve_row<HI, KS, QBF16, PAGED, F8, false>(A, k, idx, blockIdx.x);
}

// pool: null, or the pooling jobs to run in the floors' launch (pool_blocks of 512 threads)
template <int HI, int KS, bool QBF16, bool F8, bool PAGED>
hipError_t launch_mx_topk_ks(const IdxMxDev& A, int rows, int k, int32_t* idx,
                             const PoolJobs* pool, int pool_blocks_n, int B, hipStream_t s) {
  if (pool && pool_blocks_n > 0)
    mx_pool_floor_kernel<HI, KS, QBF16, PAGED, F8>
        <<<dim3(A.Nq * kMxFloorParts + pool_blocks_n, B), kMxFloorThreads, 0, s>>>(*pool, A, k);
  else
    mx_floor_kernel<HI, KS, QBF16, PAGED, F8>
        <<<rows * kMxFloorParts, kMxFloorThreads, 0, s>>>(A, k);
  launch_timed(index_scores_mx_mfma_kernel<HI, KS, QBF16, true, PAGED, F8, true>,
               dim3(A.nchunks, rows), dim3(256), s, A);
  mx_list_resolve_kernel<HI, KS, QBF16, PAGED, F8><<<rows, kMxResThreads, 0, s>>>(A, k, idx);
  return hipGetLastError();
}

template <int HI, bool QBF16, bool F8, bool PAGED>
hipError_t launch_mx_topk_hi(const IdxMxDev& A, int rows, int k, int32_t* idx,
                             const PoolJobs* pool, int pool_blocks_n, int B, hipStream_t s) {
  if (A.d_I > 64 || F8)   // FP8: two register steps (see launch_mx_mfma_hi)
    return launch_mx_topk_ks<HI, 2, QBF16, F8, PAGED>(A, rows, k, idx, pool, pool_blocks_n, B, s);
  return launch_mx_topk_ks<HI, 1, QBF16, F8, PAGED>(A, rows, k, idx, pool, pool_blocks_n, B, s);
}

template <bool QBF16, bool F8, bool PAGED>
hipError_t launch_mx_topk(const IdxMxDev& A, int rows, int H_I, int k, int32_t* idx,
                          const PoolJobs* pool, int pb, int B, hipStream_t s) {
  switch (H_I) {
    case 1: return launch_mx_topk_hi<1, QBF16, F8, PAGED>(A, rows, k, idx, pool, pb, B, s);
    case 2: return launch_mx_topk_hi<2, QBF16, F8, PAGED>(A, rows, k, idx, pool, pb, B, s);
    case 4: return launch_mx_topk_hi<4, QBF16, F8, PAGED>(A, rows, k, idx, pool, pb, B, s);
    case 8: return launch_mx_topk_hi<8, QBF16, F8, PAGED>(A, rows, k, idx, pool, pb, B, s);
    case 16: return launch_mx_topk_hi<16, QBF16, F8, PAGED>(A, rows, k, idx, pool, pb, B, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_mx_candidate_scan(const IdxMxDev& A, int rows, int H_I, bool paged,
                                     hipStream_t s) {
  const dim3 grid(A.nchunks, rows);
#define HCSA_SCAN_KS(HI_, KS_, P_)                                                           \
  launch_timed(index_scores_mx_mfma_kernel<HI_, KS_, true, true, P_, false, true>, grid,    \
               dim3(256), s, A)
#define HCSA_SCAN(HI_)                                                                        \
  if (H_I == HI_) {                                                                           \
    if (A.d_I > 64) {                                                                         \
      if (paged) HCSA_SCAN_KS(HI_, 2, true);                                                  \
      else HCSA_SCAN_KS(HI_, 2, false);                                                       \
    } else {                                                                                  \
      if (paged) HCSA_SCAN_KS(HI_, 1, true);                                                  \
      else HCSA_SCAN_KS(HI_, 1, false);                                                       \
    }                                                                                         \
    return hipGetLastError();                                                                 \
  }
  HCSA_SCAN(1) HCSA_SCAN(2) HCSA_SCAN(4) HCSA_SCAN(8) HCSA_SCAN(16)
#undef HCSA_SCAN
#undef HCSA_SCAN_KS
  return hipErrorInvalidValue;
}

bool mx_topk_fused_ok(int rows, int N, int score_dtype) {
  if (score_dtype != 1 || N < 1 || rows < 1) return false;
  const int chunk = std::min(index_chunk(rows, N), 2048);
  return (N + chunk - 1) / chunk <= kMxMaxChunks;
}

size_t mx_topk_workspace_bytes(int rows, int N) { return mx_topk_layout(rows, N).total; }

hipError_t launch_mxfp4_index_topk(const void* q, int q_dtype, const float* w,
                                   const uint8_t* kx, int64_t k_bstride, const uint8_t* ks,
                                   int64_t ks_bstride, int B, int Nq, int H_I, int d_I, int N,
                                   int ratio, int64_t pos0, const int64_t* seq_pos,
                                   const int32_t* block_table, int64_t table_stride, int k,
                                   int32_t* idx, bool fp8, void* ws, hipStream_t s,
                                   const hcsa_pool_job* pool_jobs, int n_pool_jobs,
                                   int64_t raw_ring) {
  const int rows = B * Nq;
  const MxTopkLayout l = mx_topk_layout(rows, N);
  char* base = static_cast<char*>(ws);
  IdxMxDev A = make_mx_dev(q, w, kx, k_bstride, ks, ks_bstride, B, Nq, d_I, N, ratio, pos0,
                           seq_pos, block_table, table_stride, base + l.scores_off);
  A.floor = reinterpret_cast<uint32_t*>(base);
  A.counts = reinterpret_cast<uint32_t*>(base + l.counts_off);
  A.lists = reinterpret_cast<uint32_t*>(base + l.lists_off);
  PoolJobs J;
  int pb = 0;
  if (pool_jobs)
    pb = pool_jobs_fill(pool_jobs, n_pool_jobs, block_table, table_stride, raw_ring,
                        kMxFloorThreads, J);
  const PoolJobs* pj = pool_jobs ? &J : nullptr;
  const bool paged = block_table != nullptr, qb = q_dtype == 1;
  if (fp8) {
    if (qb) return paged ? launch_mx_topk<true, true, true>(A, rows, H_I, k, idx, pj, pb, B, s)
                         : launch_mx_topk<true, true, false>(A, rows, H_I, k, idx, pj, pb, B, s);
    return paged ? launch_mx_topk<false, true, true>(A, rows, H_I, k, idx, pj, pb, B, s)
                 : launch_mx_topk<false, true, false>(A, rows, H_I, k, idx, pj, pb, B, s);
  }
  if (qb) return paged ? launch_mx_topk<true, false, true>(A, rows, H_I, k, idx, pj, pb, B, s)
                       : launch_mx_topk<true, false, false>(A, rows, H_I, k, idx, pj, pb, B, s);
  return paged ? launch_mx_topk<false, false, true>(A, rows, H_I, k, idx, pj, pb, B, s)
               : launch_mx_topk<false, false, false>(A, rows, H_I, k, idx, pj, pb, B, s);
}

}  // namespace hcsa
