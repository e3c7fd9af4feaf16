// Block pooling of K / V / indexer-key streams and the MXFP4 quantizer.
//
// CSA pools every m = 4 tokens into one entry and HCA every m' = 128 tokens
// (Lighthouse, "deep deepseek v4 release", section 八 item 3; tulong.co Q&A, 技术架构创新
// item 1).  The pooling weights are a softmax over per-position logits omega, shared by
// every block and channel; the pages do not fix the weighting, this is the reading taken.
//
// HBM-streaming kernel: one thread owns 8 consecutive channels of one output entry and
// walks the r input rows of its block with 16-byte loads (a wave covers whole rows, so
// every load instruction is contiguous), accumulating in fp32 and rounding once.
#include "common.h"
#include "internal.h"
#include "pool_dev.h"

namespace hcsa {

// grid: (pool_blocks(...), B); block 256.
template <bool IN_BF16, int OUT>
__global__ __launch_bounds__(256) void compress_kernel(const void* __restrict__ x,
                                                       int64_t x_bs, int D,
                                                       const float* __restrict__ omega, int r,
                                                       void* __restrict__ y, int64_t y_bs,
                                                       uint8_t* __restrict__ ys, int64_t ys_bs,
                                                       int n_out) {
  __shared__ float alpha[1024];
  __shared__ float s_part[2048];
  if (r >= kWideRatio)
    pool_rows_wide<IN_BF16, OUT>(x, x_bs, D, omega, alpha, r, y, y_bs, ys, ys_bs, blockIdx.x,
                                 blockIdx.y, s_part);
  else
    pool_rows<IN_BF16, OUT>(x, x_bs, D, omega, alpha, r, y, y_bs, ys, ys_bs, n_out,
                            blockIdx.x, blockIdx.y);
}

template <bool PAGED>
__global__ __launch_bounds__(256) void compress_batched_kernel(PoolJobs J) {
  __shared__ float alpha[1024];
  __shared__ float s_part[2048];
  pool_jobs_block<PAGED>(J, blockIdx.x, alpha, s_part, blockIdx.y);
}

hipError_t launch_compress_batched(const hcsa_pool_job* jobs, int n, int B,
                                   const int32_t* block_table, int64_t table_stride,
                                   int64_t raw_ring, hipStream_t s) {
  PoolJobs J;
  const int blocks = pool_jobs_fill(jobs, n, block_table, table_stride, raw_ring, 256, J);
  if (blocks == 0) return hipSuccess;
  if (block_table) compress_batched_kernel<true><<<dim3(blocks, B), 256, 0, s>>>(J);
  else compress_batched_kernel<false><<<dim3(blocks, B), 256, 0, s>>>(J);
  return hipGetLastError();
}

template <bool IN_BF16>
static hipError_t launch_compress_t(const void* x, int64_t x_bs, int B, int T, int D,
                                    const float* omega, int r, void* y, int y_dtype,
                                    int64_t y_bs, uint8_t* ys, int64_t ys_bs, hipStream_t s) {
  const int n_out = T / r;
  if (n_out == 0) return hipSuccess;
  dim3 grid(static_cast<unsigned>(pool_blocks(n_out, D, r)), B);
  if (y_dtype == 0)
    compress_kernel<IN_BF16, OUT_F32><<<grid, 256, 0, s>>>(x, x_bs, D, omega, r, y, y_bs, ys,
                                                           ys_bs, n_out);
  else if (y_dtype == 1)
    compress_kernel<IN_BF16, OUT_BF16><<<grid, 256, 0, s>>>(x, x_bs, D, omega, r, y, y_bs, ys,
                                                            ys_bs, n_out);
  else
    compress_kernel<IN_BF16, OUT_MXFP4><<<grid, 256, 0, s>>>(x, x_bs, D, omega, r, y, y_bs, ys,
                                                             ys_bs, n_out);
  return hipGetLastError();
}

hipError_t launch_compress(const void* x, int x_dtype, int64_t x_bstride, int B, int T, int D,
                           const float* omega, int ratio, void* y, int y_dtype,
                           int64_t y_bstride, uint8_t* ys, int64_t ys_bstride,
                           hipStream_t s) {
  if (x_dtype == 1)
    return launch_compress_t<true>(x, x_bstride, B, T, D, omega, ratio, y, y_dtype, y_bstride,
                                   ys, ys_bstride, s);
  return launch_compress_t<false>(x, x_bstride, B, T, D, omega, ratio, y, y_dtype, y_bstride,
                                  ys, ys_bstride, s);
}

// MXFP4 quantization of [rows][D]: the pooling kernel with a single-row block and
// weight 1 (exact), so both share one quantizer.
hipError_t launch_mxfp4_quantize(const void* x, int x_dtype, int64_t rows, int D,
                                 uint8_t* packed, uint8_t* scales, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int tpr = D / 8;
  const int rpb = 256 / tpr;
  const int64_t nb = (rows + rpb - 1) / rpb;
  if (nb > 0x7fffffff) return hipErrorInvalidValue;
  dim3 grid(static_cast<unsigned>(nb), 1);
  if (x_dtype == 1)
    compress_kernel<true, OUT_MXFP4><<<grid, 256, 0, s>>>(x, 0, D, nullptr, 1, packed, 0,
                                                          scales, 0, static_cast<int>(rows));
  else
    compress_kernel<false, OUT_MXFP4><<<grid, 256, 0, s>>>(x, 0, D, nullptr, 1, packed, 0,
                                                           scales, 0, static_cast<int>(rows));
  return hipGetLastError();
}

}  // namespace hcsa
