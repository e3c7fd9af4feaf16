// One decode step of a CSA layer and an HCA layer (pooling on append, lightning indexer,
// top-k, CSA sparse attention with its window, HCA dense attention) in four launches that
// keep the HBM streams running beside the latency-bound stages.
//
// The method (Lighthouse, "deep deepseek v4 release", section 八 item 3): CSA pools every 4
// tokens into one entry, a lightning indexer keeps the top-k entries for sparse attention
// plus a window of the last 128 raw tokens; HCA pools every 128 tokens into one entry and
// attends densely.  The indexer scans MXFP4 keys (9fzt.com digest item 4: FP4 on the
// indexer's QK path, BF16 index scores).  The results are those of
// hcsa_csa_pool_index_topk followed by hcsa_csa_hca_attn, bit for bit: the same kernels'
// device code runs here in another arrangement.
//
//  1. front: the per-row selection floors (one 512-thread block per row, sampling only
//     entries completed before the step) and the pooling of the blocks the step completes,
//     side by side with the first HCA splits of every row (entries completed before the
//     step), which stream HBM on the CUs the floors leave idle.
//  2. the MXFP4 key scan writing per-chunk candidate lists (the indexer's own launch).
//  3. back: per-row resolves (the exact top-k among the candidates) beside the remaining
//     HCA splits, and the CSA splits, each of which waits for its row's selection.  The
//     blocks take their role in the order they start (a ticket counter), resolves first,
//     so a CSA block only ever waits for a block that is already running.  The selection
//     is written with agent-coherent stores and published per row by a flag.
//  4. the log-sum-exp merge of both attentions' splits.
#include "attn_dev.h"
#include "internal.h"
#include "mx_dev.h"
#include "pool_dev.h"
#include "select_dev.h"

#include <algorithm>
#include <cstdlib>

namespace hcsa {

namespace {

using namespace attn;

constexpr int kStepThreads = 512;        // two 256-thread attention units per block
constexpr int kWaitIters = 1 << 20;      // bound of a selection wait (about a second)

struct StepDev {
  IdxMxDev X;          // indexer: floors, candidate lists, rescan rows
  AttnDev C, Hd;       // CSA and HCA attention (partials in the workspace when split)
  PoolJobs J;          // pooling jobs of the step's completed blocks
  int B, rows, k;
  int pool_blocks;     // pooling blocks per sequence
  int hca_a;           // HCA splits per row run in the front launch
  int hca_b_units;     // HCA (split, row) units of the back launch
  int csa_units;       // CSA (split, row) units
  int32_t* idx;        // [rows][k] selection
  uint32_t* sync;      // [0] wait timeouts, [1] ticket, [2 + row] selection ready
  int nsync;
};

// grid: rows + B * pool_blocks + ceil(rows * hca_a / 2); block 512.
template <int HI, int KS>
__global__ __launch_bounds__(kStepThreads) void step_front_kernel(StepDev S) {
  __shared__ float alpha[1024];
  __shared__ float s_part[kStepThreads * 8];
  __shared__ float s_o[2][4][16][129];
  __shared__ float s_ml[2][4][2][16];
  const int bx = blockIdx.x;
  if (bx == 0)                                   // the back launch's counters and flags
    for (int i = threadIdx.x; i < S.nsync; i += kStepThreads) S.sync[i] = 0u;
  if (bx < S.rows) {
    mx_floor_block<HI, KS, true, false, false>(S.X, S.k, bx, true);
    return;
  }
  int b2 = bx - S.rows;
  if (b2 < S.B * S.pool_blocks) {
    pool_jobs_block<false>(S.J, b2 % S.pool_blocks, alpha, s_part, b2 / S.pool_blocks);
    return;
  }
  b2 -= S.B * S.pool_blocks;
  const int half = threadIdx.x >> 8, tid = threadIdx.x & 255;
  const int u = 2 * b2 + half;
  if (u < S.rows * S.hca_a)
    hca_decode_block<false>(S.Hd, u % S.hca_a, u / S.hca_a, s_o[half], s_ml[half], tid);
  else
    __syncthreads();                             // the unit's one barrier
}

// Thread 0 waits (bounded) until row `row`'s selection is published; counts a timeout.
__device__ __forceinline__ void wait_ready(const StepDev& S, int row) {
  uint32_t* f = S.sync + 2 + row;
  for (int it = 0; it < kWaitIters; ++it) {
    if (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) return;
    __builtin_amdgcn_s_sleep(4);
  }
  atomicAdd(S.sync, 1u);
}

// grid: rows + ceil(hca_b_units / 2) + ceil(csa_units / 2); block 512.
template <int HI, int KS>
__global__ __launch_bounds__(kStepThreads) void step_back_kernel(StepDev S) {
  __shared__ int s_role;
  __shared__ int s_code[2][kMfmaMaxChunk];
  __shared__ float s_o[2][4][16][129];
  __shared__ float s_ml[2][4][2][16];
  if (threadIdx.x == 0) s_role = static_cast<int>(atomicAdd(S.sync + 1, 1u));
  __syncthreads();
  const int t = s_role;
  if (t < S.rows) {
    mx_resolve_row<HI, KS, true, false, false, true>(S.X, S.k, S.idx, t);
    // this thread's selection stores (agent-coherent) complete before the flag: the fence
    // keeps them above the wait, the wait for every counter drains them
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0)
      __hip_atomic_store(S.sync + 2 + t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const int half = threadIdx.x >> 8, tid = threadIdx.x & 255;
  int b2 = t - S.rows;
  const int hb_blocks = (S.hca_b_units + 1) / 2;
  if (b2 < hb_blocks) {
    const int nb = S.Hd.splits - S.hca_a;
    const int u = 2 * b2 + half;
    if (u < S.hca_b_units)
      hca_decode_block<false>(S.Hd, S.hca_a + u % nb, u / nb, s_o[half], s_ml[half], tid);
    else
      __syncthreads();
    return;
  }
  b2 -= hb_blocks;
  const int u0 = 2 * b2, u = u0 + half;
  if (threadIdx.x == 0) {
    wait_ready(S, u0 / S.C.splits);
    if (u0 + 1 < S.csa_units) wait_ready(S, (u0 + 1) / S.C.splits);
  }
  __syncthreads();
  if (u < S.csa_units) {
    attn_mfma_block<true, true>(S.C, u % S.C.splits, u / S.C.splits, s_code[half], s_o[half],
                                s_ml[half], tid);
  } else {                                       // the unit's two barriers
    __syncthreads();
    __syncthreads();
  }
}

// The sync words of a step that runs as the two calls: the timeout count reads 0.
__global__ __launch_bounds__(64) void step_sync_reset_kernel(uint32_t* sync, int n) {
  for (int i = threadIdx.x; i < n; i += 64) sync[i] = 0u;
}

struct StepMerge {
  const float* part_o;
  const float* part_l;
  int splits, rows;
  float* out;
  float* lse;
};

// grid: (H, rows_c + rows_h); block d.  Rows below rows_c merge the CSA splits.
__global__ __launch_bounds__(256) void step_merge_kernel(StepMerge c, StepMerge h, int H, int d) {
  __shared__ float s_w[1024];
  __shared__ float s_red[2];
  const int y = blockIdx.y;
  const StepMerge& m = y < c.rows ? c : h;
  const int row = y < c.rows ? y : y - c.rows;
  lse_merge_row(m.part_o, m.part_l, m.splits, m.rows, H, d, m.out, m.lse, blockIdx.x, row,
                s_w, s_red);
}

template <int HI, int KS>
hipError_t launch_step_hi(const StepDev& S, int front_blocks, int back_blocks, int H_I,
                          hipStream_t s) {
  step_front_kernel<HI, KS><<<front_blocks, kStepThreads, 0, s>>>(S);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_mx_candidate_scan(S.X, S.rows, H_I, s);
  if (e != hipSuccess) return e;
  step_back_kernel<HI, KS><<<back_blocks, kStepThreads, 0, s>>>(S);
  return hipGetLastError();
}

// HCA splits per row in the front launch: about this share of each row's splits (tuning:
// HCSA_DECODE_HCA_FRONT, in per mille), limited to splits of entries completed before the
// step.
int front_hca_splits(const AttnPlan& ph, int64_t pos0, int ratio_h) {
  int permille = 500;
  if (const char* v = std::getenv("HCSA_DECODE_HCA_FRONT")) permille = std::atoi(v);
  permille = std::max(0, std::min(1000, permille));
  const int64_t prior = pos0 / ratio_h;          // entries complete before the step
  const int64_t safe = ph.chunk > 0 ? prior / ph.chunk : 0;
  const int want = (ph.splits * permille + 500) / 1000;
  return static_cast<int>(std::min<int64_t>(std::min(want, ph.splits), safe));
}

}  // namespace

// HCA splits of the four-launch step: finer than the attention call's own plan, so that
// each of the two launches holding HCA units spreads them over every CU (two 256-thread
// units per block, one block per CU): about 1024 units over the batch, at least 128
// entries each.  The split outputs are combined exactly by the merge, so the HCA result
// equals the attention call's up to the rounding of its sums.
AttnPlan plan_step_hca(int B, int Nq, int H, int d, int N_h) {
  AttnPlan p = plan_attention(false, HCSA_BF16, B, Nq, H, d, N_h);
  if (!p.hca_decode || N_h < 1) return p;
  const int64_t total = static_cast<int64_t>(p.rows) * N_h;
  int64_t c = (total + 1023) / 1024;
  c = std::max<int64_t>(128, (c + 31) / 32 * 32);
  p.chunk = static_cast<int>(std::min<int64_t>(c, kMfmaMaxChunk));
  p.splits = std::max(1, (N_h + p.chunk - 1) / p.chunk);
  p.part_bytes = 0;
  if (p.splits > 1)
    p.part_bytes = align256(static_cast<size_t>(p.splits) * p.rows * H * d * 4) +
                   align256(static_cast<size_t>(p.splits) * p.rows * H * 4);
  p.total_bytes = p.part_bytes;
  return p;
}

bool decode_step_fast(const DecodeStepArgs& a, const AttnPlan& pc, const AttnPlan& ph,
                      bool fused_selection) {
  const bool hi_ok = a.H_I == 1 || a.H_I == 2 || a.H_I == 4 || a.H_I == 8 || a.H_I == 16;
  return fused_selection && a.Nq == 1 && a.k_dtype == HCSA_MXFP4 && a.q_dtype == HCSA_BF16 &&
         a.score_dtype == HCSA_BF16 && a.block_table == nullptr && a.raw_ring == 0 &&
         a.seq_pos == nullptr && hi_ok && csa_hca_fused(pc, ph);
}

size_t decode_step_sync_bytes(int rows) { return align256((2 + static_cast<size_t>(rows)) * 4); }

hipError_t launch_decode_step_reset(void* ws, int rows, hipStream_t s) {
  step_sync_reset_kernel<<<1, 64, 0, s>>>(static_cast<uint32_t*>(ws), 2 + rows);
  return hipGetLastError();
}

hipError_t launch_decode_step(const DecodeStepArgs& a, const AttnPlan& pc, const AttnPlan& ph,
                              void* ws, size_t mx_off, size_t attn_off, hipStream_t s) {
  const int rows = a.B * a.Nq;
  char* base = static_cast<char*>(ws);
  StepDev S{};
  const MxTopkLayout l = mx_topk_layout(rows, a.N);
  char* mx = base + mx_off;
  S.X = make_mx_dev(a.q_idx, a.w_idx, a.k_idx, a.k_bstride, a.k_scales, a.ks_bstride, a.B,
                    a.Nq, a.d_I, a.N, a.c.ratio, a.c.pos0, nullptr, nullptr, 0,
                    mx + l.scores_off);
  S.X.floor = reinterpret_cast<uint32_t*>(mx);
  S.X.counts = reinterpret_cast<uint32_t*>(mx + l.counts_off);
  S.X.lists = reinterpret_cast<uint32_t*>(mx + l.lists_off);
  void* ws_c = base + attn_off;
  void* ws_h = base + attn_off + align256(pc.total_bytes);
  S.C = attn_dev_for(a.c, pc, ws_c);
  S.Hd = attn_dev_for(a.h, ph, ws_h);
  S.B = a.B;
  S.rows = rows;
  S.k = a.c.k;
  S.idx = a.idx;
  S.pool_blocks = a.n_jobs > 0 ? pool_jobs_fill(a.jobs, a.n_jobs, nullptr, 0, 0, kStepThreads, S.J)
                               : 0;
  S.hca_a = front_hca_splits(ph, a.c.pos0, a.h.ratio);
  S.hca_b_units = rows * (ph.splits - S.hca_a);
  S.csa_units = rows * pc.splits;
  S.sync = reinterpret_cast<uint32_t*>(base);
  S.nsync = 2 + rows;
  const int front = rows + a.B * S.pool_blocks + (rows * S.hca_a + 1) / 2;
  const int back = rows + (S.hca_b_units + 1) / 2 + (S.csa_units + 1) / 2;
  hipError_t e = hipErrorInvalidValue;
  const bool ks2 = a.d_I > 64;
#define HCSA_STEP(HI_)                                                              \
  if (a.H_I == HI_)                                                                 \
    e = ks2 ? launch_step_hi<HI_, 2>(S, front, back, a.H_I, s)                       \
            : launch_step_hi<HI_, 1>(S, front, back, a.H_I, s);
  HCSA_STEP(1) HCSA_STEP(2) HCSA_STEP(4) HCSA_STEP(8) HCSA_STEP(16)
#undef HCSA_STEP
  if (e != hipSuccess) return e;
  // merge of the splits: CSA rows first, then HCA rows (a call without splits needs none)
  StepMerge mc{S.C.out, S.C.lse, pc.splits, rows, a.c.out, a.c.lse};
  const StepMerge mh{S.Hd.out, S.Hd.lse, ph.splits, rows, a.h.out, a.h.lse};
  if (pc.splits == 1) mc.rows = 0;
  const int gy = mc.rows + (ph.splits > 1 ? rows : 0);
  if (gy > 0) step_merge_kernel<<<dim3(a.c.H, gy), a.c.d, 0, s>>>(mc, mh, a.c.H, a.c.d);
  return hipGetLastError();
}

}  // namespace hcsa
