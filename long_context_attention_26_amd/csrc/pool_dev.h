// Block pooling device code, shared by the pooling kernels and the fused pooling + indexer
// launch: one thread owns 8 consecutive channels of one output entry and walks the r input
// rows of its block with 16-byte loads, accumulating in fp32 and rounding once.
//
// CSA pools every m = 4 tokens into one entry and HCA every m' = 128 tokens (Lighthouse,
// "deep deepseek v4 release", section 八 item 3; tulong.co Q&A, 技术架构创新 item 1); the
// pooling weights are a softmax over per-position logits omega, shared by every block and
// channel (the reading taken where the pages do not fix the weighting).
#pragma once
#include "common.h"
#include "../../include/hcsa.h"

namespace hcsa {

enum { OUT_F32 = 0, OUT_BF16 = 1, OUT_MXFP4 = 2 };

// Writes 8 values of one row: F32, BF16, or MXFP4 (4 code bytes; the lane holding the
// first 8 channels of each 32-channel block also writes the block's scale byte).
template <int OUT>
__device__ __forceinline__ void store8(const float (&acc)[8], void* y, int64_t y_row_elems,
                                       uint8_t* ys, int64_t ys_row, int c8) {
  if constexpr (OUT == OUT_F32) {
    f32x4* d = reinterpret_cast<f32x4*>(static_cast<float*>(y) + y_row_elems + c8 * 8);
    d[0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
    d[1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
  } else if constexpr (OUT == OUT_BF16) {
    u32x4 w;
#pragma unroll
    for (int c = 0; c < 4; ++c) w[c] = pack_bf16x2(acc[2 * c], acc[2 * c + 1]);
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(y) + y_row_elems + c8 * 8) = w;
  } else {
    // y_row_elems is the byte offset of the packed row here.
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) amax = fmaxf(amax, __builtin_fabsf(acc[c]));
    // the 4 lanes of a 32-channel block are consecutive and quad-aligned
    amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
    amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
    const int e = mx_scale_exp(amax);
    uint32_t packed = 0;
#pragma unroll
    for (int c = 0; c < 8; ++c) packed |= e2m1_code(acc[c], e) << (4 * c);
    *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(y) + y_row_elems + c8 * 4) = packed;
    if ((c8 & 3) == 0) ys[ys_row + (c8 >> 2)] = static_cast<uint8_t>(e + 127);
  }
}


// Source row (in D-element rows) of entry j's first token and the entry's output row, for
// paged tensors: the entry's r tokens lie in one 128-token page (r divides 128 and the
// job starts on an entry boundary), so one lookup serves all of them.
__device__ __forceinline__ void paged_rows(const PageMap& pm, int b, int64_t pos0, int r,
                                           int64_t j, int64_t& xrow, int64_t& yrow) {
  xrow = row_off<true>(pm, 0, b, pos0 + j * r, 7, 1);
  yrow = row_off<true>(pm, 0, b, pos0 / r + j, __builtin_ctz(kPageTokens / r), 1);
}

// Element offset of entry j's first source token: a ring of `ring` rows per sequence
// (position t in row t mod ring; r divides 128 and the ring is a power of two >= 128, so an
// entry's r rows never wrap), a page pool (xrow from paged_rows), or rows from the job's
// first token.
template <bool PAGED>
__device__ __forceinline__ int64_t src_off(int64_t ring, int64_t x_bs, int D, int b,
                                           int64_t pos0, int r, int64_t j, int64_t xrow) {
  if (ring) return b * x_bs + ((pos0 + j * r) & (ring - 1)) * D;
  return PAGED ? xrow * D : b * x_bs + j * r * D;
}

// 8 channels of one input row as loaded (BF16: one 16-byte word, F32: two), so that a row's
// load can be issued before its pooling weight is known.
template <bool IN_BF16>
struct Row8 {
  u32x4 w[IN_BF16 ? 1 : 2];
  __device__ __forceinline__ void load(const char* p) {
    w[0] = *reinterpret_cast<const u32x4*>(p);
    if constexpr (!IN_BF16) w[1] = *reinterpret_cast<const u32x4*>(p + 16);
  }
  __device__ __forceinline__ void fma_into(float a, float (&acc)[8]) const {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if constexpr (IN_BF16) {
        acc[2 * c] = fmaf(a, bf16_lo(w[0][c]), acc[2 * c]);
        acc[2 * c + 1] = fmaf(a, bf16_hi(w[0][c]), acc[2 * c + 1]);
      } else {
        acc[c] = fmaf(a, __uint_as_float(w[0][c]), acc[c]);
        acc[4 + c] = fmaf(a, __uint_as_float(w[1][c]), acc[4 + c]);
      }
    }
  }
};

// One block of the pooling: this thread's 8 channels of entry `j` (block-local row `local`).
// The first rows are loaded before the weights softmax(omega) are formed in `alpha` (a
// block-wide step), so the two memory latencies overlap; every thread of the block calls.
template <bool IN_BF16, int OUT, bool PAGED = false>
__device__ __forceinline__ void pool_rows(const void* __restrict__ x, int64_t x_bs, int D,
                                          const float* __restrict__ omega, float* alpha, int r,
                                          void* __restrict__ y, int64_t y_bs,
                                          uint8_t* __restrict__ ys, int64_t ys_bs, int n_out,
                                          int64_t jblock, int b,
                                          const PageMap& pm = PageMap{nullptr, 0},
                                          int64_t pos0 = 0, int64_t ring = 0) {
  constexpr int PF = 4;                         // rows loaded ahead of the weights
  const int tpr = D >> 3;                       // threads per output row
  const int rows_per_block = blockDim.x / tpr;
  const int local = threadIdx.x / tpr;
  const int c8 = threadIdx.x - local * tpr;
  const int64_t j = jblock * rows_per_block + local;
  const bool active = local < rows_per_block && j < n_out;
  constexpr int ES = IN_BF16 ? 2 : 4;
  const int64_t row_bytes = static_cast<int64_t>(D) * ES;
  int64_t xrow = 0, yrow = 0;
  const char* src = nullptr;
  Row8<IN_BF16> pre[PF];
  if (active) {
    if constexpr (PAGED) paged_rows(pm, b, pos0, r, j, xrow, yrow);
    src = static_cast<const char*>(x) +
          (src_off<PAGED>(ring, x_bs, D, b, pos0, r, j, xrow) + c8 * 8) * ES;
#pragma unroll
    for (int u = 0; u < PF; ++u)
      if (u < r) pre[u].load(src + u * row_bytes);
  }
  pool_weights(omega, r, alpha);
  if (!active) return;

  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int u = 0; u < PF; ++u)
    if (u < r) pre[u].fma_into(alpha[u], acc);
#pragma unroll 4
  for (int i = PF; i < r; ++i) {
    Row8<IN_BF16> v;
    v.load(src + i * row_bytes);
    v.fma_into(alpha[i], acc);
  }

  if constexpr (OUT == OUT_MXFP4) {
    if constexpr (PAGED) store8<OUT>(acc, y, yrow * (D >> 1), ys, yrow * (D >> 5), c8);
    else store8<OUT>(acc, y, b * y_bs + j * (D >> 1), ys, b * ys_bs + j * (D >> 5), c8);
  } else {
    store8<OUT>(acc, y, PAGED ? yrow * D : b * y_bs + j * D, nullptr, 0, c8);
  }
}

// Long blocks (ratio >= kWideRatio): one block per output entry.  Thread (g, c8) sums
// rows g, g + G, g + 2G, ... of its 8 channels (G = 256 / (D/8) row groups), so all of a
// thread's loads are independent (the first PF of them issued before the weights are
// formed); the G partial sums are added in group order in LDS.
constexpr int kWideRatio = 32;

template <bool IN_BF16, int OUT, bool PAGED = false>
__device__ __forceinline__ void pool_rows_wide(const void* __restrict__ x, int64_t x_bs, int D,
                                               const float* __restrict__ omega, float* alpha,
                                               int r, void* __restrict__ y, int64_t y_bs,
                                               uint8_t* __restrict__ ys, int64_t ys_bs,
                                               int64_t j, int b, float* s_part,
                                               const PageMap& pm = PageMap{nullptr, 0},
                                               int64_t pos0 = 0, int64_t ring = 0) {
  constexpr int PF = 8;
  const int tpr = D >> 3;
  // the groups of a 256-thread block whatever the launch's block size: the partial sums,
  // and so the entry's bits, are the same in every launch that pools it
  const int G = min(static_cast<int>(blockDim.x), 256) / tpr;
  const int g = threadIdx.x / tpr;
  const int c8 = threadIdx.x - g * tpr;
  constexpr int ES = IN_BF16 ? 2 : 4;
  const int64_t row_bytes = static_cast<int64_t>(D) * ES;
  int64_t xrow = 0, yrow = 0;
  if constexpr (PAGED) paged_rows(pm, b, pos0, r, j, xrow, yrow);
  const char* src = static_cast<const char*>(x) +
                    (src_off<PAGED>(ring, x_bs, D, b, pos0, r, j, xrow) + c8 * 8) * ES;
  Row8<IN_BF16> pre[PF];
  if (g < G) {
#pragma unroll
    for (int u = 0; u < PF; ++u)
      if (g + u * G < r) pre[u].load(src + (g + u * G) * row_bytes);
  }
  pool_weights(omega, r, alpha);
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (g < G) {
#pragma unroll
    for (int u = 0; u < PF; ++u)
      if (g + u * G < r) pre[u].fma_into(alpha[g + u * G], acc);
#pragma unroll 8
    for (int i = g + PF * G; i < r; i += G) {
      Row8<IN_BF16> v;
      v.load(src + i * row_bytes);
      v.fma_into(alpha[i], acc);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) s_part[g * D + c8 * 8 + c] = acc[c];
  }
  __syncthreads();
  if (g == 0) {
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = s_part[c8 * 8 + c];
    for (int gg = 1; gg < G; ++gg)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] += s_part[gg * D + c8 * 8 + c];
    if constexpr (OUT == OUT_MXFP4) {
      if constexpr (PAGED) store8<OUT>(acc, y, yrow * (D >> 1), ys, yrow * (D >> 5), c8);
      else store8<OUT>(acc, y, b * y_bs + j * (D >> 1), ys, b * ys_bs + j * (D >> 5), c8);
    } else {
      store8<OUT>(acc, y, PAGED ? yrow * D : b * y_bs + j * D, nullptr, 0, c8);
    }
  }
}

// Blocks a pooling job needs with blocks of `threads`: one per entry for long blocks, else
// threads / (D/8) entries per block.  Long blocks need threads * 8 floats of LDS partials.
__host__ __device__ inline int64_t pool_blocks(int n_out, int D, int r, int threads = 256) {
  if (r >= kWideRatio) return n_out;
  const int rpb = threads / (D / 8);
  return (static_cast<int64_t>(n_out) + rpb - 1) / rpb;
}

// Several pooling jobs in one launch (the blocks completed by a decode token in every
// stream): grid.x is the concatenation of the jobs' block ranges.
struct PoolJobs {
  hcsa_pool_job job[HCSA_MAX_POOL_JOBS];
  int first_block[HCSA_MAX_POOL_JOBS + 1];
  int n;
  PageMap pm;        // paged caches (table null: contiguous)
  int64_t ring;      // 0, or raw tokens (every job's x) in a ring of this many rows
};

template <bool IN_BF16, int OUT, bool PAGED>
__device__ __forceinline__ void pool_job_blocks(const hcsa_pool_job& q, const PageMap& pm,
                                                int64_t ring, float* alpha, int64_t jb,
                                                int n_out, float* s_part, int b) {
  if (q.ratio >= kWideRatio)
    pool_rows_wide<IN_BF16, OUT, PAGED>(q.x, q.x_bstride, q.D, q.omega, alpha, q.ratio, q.y,
                                        q.y_bstride, q.y_scales, q.ys_bstride, jb, b,
                                        s_part, pm, q.pos0, ring);
  else
    pool_rows<IN_BF16, OUT, PAGED>(q.x, q.x_bstride, q.D, q.omega, alpha, q.ratio, q.y,
                                   q.y_bstride, q.y_scales, q.ys_bstride, n_out, jb,
                                   b, pm, q.pos0, ring);
}

// Block bx of sequence b of a batched pooling launch: finds its job and runs it.
// alpha: LDS for 1024 weights; s_part: LDS for blockDim.x * 8 floats.
template <bool PAGED>
__device__ __forceinline__ void pool_jobs_block(const PoolJobs& J, int bx, float* alpha,
                                                float* s_part, int b) {
  int t = 0;
  while (t + 1 < J.n && bx >= J.first_block[t + 1]) ++t;
  const hcsa_pool_job& q = J.job[t];
  const int64_t jb = bx - J.first_block[t];
  const int n_out = q.T / q.ratio;
  const bool ib = q.x_dtype == 1;
  const PageMap& pm = J.pm;
  const int64_t rg = J.ring;
  if (ib && q.y_dtype == 1) pool_job_blocks<true, OUT_BF16, PAGED>(q, pm, rg, alpha, jb, n_out, s_part, b);
  else if (ib && q.y_dtype == 2) pool_job_blocks<true, OUT_MXFP4, PAGED>(q, pm, rg, alpha, jb, n_out, s_part, b);
  else if (ib) pool_job_blocks<true, OUT_F32, PAGED>(q, pm, rg, alpha, jb, n_out, s_part, b);
  else if (q.y_dtype == 1) pool_job_blocks<false, OUT_BF16, PAGED>(q, pm, rg, alpha, jb, n_out, s_part, b);
  else if (q.y_dtype == 2) pool_job_blocks<false, OUT_MXFP4, PAGED>(q, pm, rg, alpha, jb, n_out, s_part, b);
  else pool_job_blocks<false, OUT_F32, PAGED>(q, pm, rg, alpha, jb, n_out, s_part, b);
}

// The jobs of a batched pooling call with their block ranges for blocks of `threads`;
// returns the total block count (jobs with no complete entry are dropped).
inline int pool_jobs_fill(const hcsa_pool_job* jobs, int n, const int32_t* block_table,
                          int64_t table_stride, int64_t raw_ring, int threads, PoolJobs& J) {
  J = PoolJobs{};
  J.n = 0;
  J.pm.table = block_table;
  J.pm.stride = table_stride;
  J.ring = raw_ring;
  int blocks = 0;
  for (int i = 0; i < n; ++i) {
    const int n_out = jobs[i].T / jobs[i].ratio;
    if (n_out == 0) continue;
    J.job[J.n] = jobs[i];
    J.first_block[J.n] = blocks;
    blocks += static_cast<int>(pool_blocks(n_out, jobs[i].D, jobs[i].ratio, threads));
    ++J.n;
  }
  J.first_block[J.n] = blocks;
  return blocks;
}

}  // namespace hcsa
