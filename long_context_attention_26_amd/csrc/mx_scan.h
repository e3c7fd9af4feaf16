// The MXFP4 key scan of the lightning indexer on the matrix cores (scores, or candidate
// lists above each row's selection floor), shared by the score and the fused-selection
// translation units; and the launch helper that lets a benchmark time the next indexer
// kernel by events recorded in its own dispatch.
//
// The indexer scores compressed entries with its own compressed keys on a low-precision QK
// path (Lighthouse, "deep deepseek v4 release", section 八 items 3 and 7; 9fzt.com digest
// item 4).
#pragma once
#include "common.h"
#include <hip/hip_ext.h>

#include "internal.h"
#include "mx_dev.h"
#include "pool_dev.h"
#include "select_dev.h"

namespace hcsa {

// The events the next indexer kernel of this thread records in its dispatch, taken (and
// cleared) by the launcher; false when none are set.
bool take_indexer_timing(hipEvent_t* start, hipEvent_t* stop);

namespace {

template <typename K, typename... Args>
void launch_timed(K kernel, dim3 grid, dim3 block, hipStream_t s, Args... args) {
  hipEvent_t e0, e1;
  if (take_indexer_timing(&e0, &e1))
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, e0, e1, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
}

// grid: (ceil(N / chunk), rows); block 256 (4 waves, 32 keys per MFMA).  Wave w takes keys
// j0 + 128u + lane%32 of the block's chunk, j0 = start + 32w + 512i, u < 4: step (i, u)
// covers 128 consecutive keys in wave order.
//  - Scores: every visible key's score, rounded to the score dtype.
//  - Candidate lists (CAND, bf16 scores): the keys whose bf16 score key is >= the row's
//    floor, as (key << 16 | index in the chunk), in index order: each wave stages a step's
//    candidates in LDS by ballot rank, and at the end the block writes the groups (step,
//    wave) in order, with its count.  Chunks are at most 2048 keys (64 groups of 32).
template <int HI, int KS, bool QBF16, bool SBF16, bool PAGED, bool F8, bool CAND>
__global__ __launch_bounds__(256) void index_scores_mx_mfma_kernel(IdxMxDev A) {
  constexpr int U = 4;
  const int row = blockIdx.y;
  const int b = row / A.Nq;
  const int64_t p = query_pos(A.seq_pos, A.pos0, b, row % A.Nq);
  const int64_t nv64 = (p + 1) / A.ratio;
  const int nv = static_cast<int>(nv64 < A.N ? nv64 : A.N);
  const int start = blockIdx.x * A.chunk;
  const int end = min(start + A.chunk, nv);
  if (start >= end) return;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int ksteps = A.d_I > 64 ? A.d_I / 64 : 1;
  __shared__ uint32_t s_qa[kMxMaxUnits][4];
  __shared__ int s_qs[kMxMaxUnits];
  __shared__ uint32_t s_stage[CAND ? 2048 : 1];
  __shared__ int s_cnt[CAND ? 64 : 1], s_off[CAND ? 64 : 1];
  uint32_t L = 0;
  if constexpr (CAND) {
    L = mx_row_floor(A, row);
    if (threadIdx.x < 64) s_cnt[threadIdx.x] = 0;   // ordered by the barrier in mx_query
  }
  const MxQuery<HI, KS> Q = mx_query<HI, KS, QBF16, F8>(A, row, s_qa, s_qs);

  const uint8_t* kbase = PAGED ? A.k : A.k + b * A.k_bstride;
  const uint8_t* sbase = PAGED ? A.ks : A.ks + b * A.ks_bstride;
  float* s32 = static_cast<float*>(A.scores) + static_cast<int64_t>(row) * A.N;
  uint16_t* s16 = static_cast<uint16_t*>(A.scores) + static_cast<int64_t>(row) * A.N;

  int it = 0;
  for (int j0 = start + wave * 32; j0 < end; j0 += 4 * 32 * U, ++it) {
    u32x4 kraw[U][KS];
    int ksc[U][KS];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * 128 + col;
      mx_load<KS, PAGED, F8>(A, kbase, sbase, b, j, j < end, kraw[u], ksc[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (j0 + u * 128 >= end) break;                 // wave-uniform
      const float s = mx_score<HI, KS, F8>(Q, kraw[u], ksc[u], ksteps);
      const int j = j0 + u * 128 + col;
      if constexpr (CAND) {
        const uint32_t kk = bf16_key(f32_to_bf16_bits(s));
        const bool c = half == 0 && j < end && kk >= L;
        const uint64_t m = __ballot(c);
        const int g = (it * U + u) * 4 + wave;
        if (c) s_stage[g * 32 + ballot_rank(m)] = (kk << 16) | static_cast<uint32_t>(j - start);
        if (lane == 0) s_cnt[g] = __popcll(m);
      } else if (half == 0 && j < end) {
        if constexpr (SBF16)
          s16[j] = static_cast<uint16_t>(f32_to_bf16_bits(s));
        else
          s32[j] = s;
      }
    }
  }
  if constexpr (CAND) {
    __syncthreads();
    if (threadIdx.x < 64) {                       // offsets of the groups in (step, wave) order
      const int c = s_cnt[threadIdx.x];
      int inc = c;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(inc, d, kWave);
        if (lane >= d) inc += y;
      }
      s_off[threadIdx.x] = inc - c;
      if (threadIdx.x == 63) A.counts[static_cast<int64_t>(row) * A.nchunks + blockIdx.x] = inc;
    }
    __syncthreads();
    uint32_t* out = A.lists + (static_cast<int64_t>(row) * A.nchunks + blockIdx.x) * A.chunk;
    const int g = threadIdx.x >> 2;
    const int c = s_cnt[g], o = s_off[g];
    for (int i = threadIdx.x & 3; i < c; i += 4) out[o + i] = s_stage[g * 32 + i];
  }
}

}  // namespace
}  // namespace hcsa
