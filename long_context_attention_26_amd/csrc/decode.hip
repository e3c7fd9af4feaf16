// One decode step of a CSA layer and an HCA layer (pooling on append, lightning indexer,
// top-k, CSA sparse attention with its window, HCA dense attention) in four launches that
// keep the HBM streams running beside the latency-bound stages.
//
// The method (Lighthouse, "deep deepseek v4 release", section 八 item 3): CSA pools every 4
// tokens into one entry, a lightning indexer keeps the top-k entries for sparse attention
// plus a window of the last 128 raw tokens; HCA pools every 128 tokens into one entry and
// attends densely.  The indexer scans MXFP4 keys (9fzt.com digest item 4: FP4 on the
// indexer's QK path, BF16 index scores).  The pooled caches and the selection are those of
// hcsa_csa_pool_index_topk bit for bit (the same device code runs here); the attention
// splits differ from hcsa_csa_hca_attn's, so its outputs agree up to the rounding of the
// split sums.  Paged caches, the raw-token ring and per-sequence positions take the same
// launches (the paged kernels are instantiated separately).
//
//  1. front: the per-row selection floors (kMxFloorParts 512-thread blocks per row, each
//     scoring a quarter of the samples, taken only from entries completed before the step)
//     and the pooling of the blocks the step completes.
//  2. the MXFP4 key scan writing per-chunk candidate lists (the indexer's own launch).
//  3. back: a few blocks per row each resolve the row's top-k among its candidates (the
//     same deterministic selection, so it never crosses blocks) and then run the CSA
//     attention over their split of the row's key list (selected entries and window) with
//     all 8 waves; the HCA splits run as 4-wave units, two per block, on the other CUs,
//     taken from a counter until none is left.
//  4. the log-sum-exp merge of the CSA and the HCA splits.
#include "attn_dev.h"
#include "internal.h"
#include "mx_dev.h"
#include "pool_dev.h"
#include "seg_dev.h"
#include "select_dev.h"

#include <algorithm>

namespace hcsa {

namespace {

using namespace attn;

constexpr int kStepThreads = 512;        // two 256-thread attention units per block

// Blocks per query row in the back launch.  Each runs the row's resolve and then its share of
// the row's CSA key list, so with few rows more parts spread a row's gathers over more CUs.
__host__ __device__ inline int step_row_parts(int rows) {
  return rows <= 8 ? 8 : rows <= 16 ? 4 : 2;
}

struct StepDev {
  IdxMxDev X;          // indexer: floors, candidate lists, rescan rows
  AttnDev C, Hd;       // CSA and HCA attention (partials in the workspace)
  PoolJobs J;          // pooling jobs of the step's completed blocks
  int B, rows, k;
  int pool_blocks;     // pooling blocks per sequence
  int hca_units;       // HCA (split, row) units
  int parts;           // blocks per row in the back launch
  int32_t* idx;        // [rows][k] selection
  uint32_t* hca_next;  // next HCA unit of the back launch (zeroed by the front launch)
};

// A worker block of a back launch: pairs of HCA (split, row) units, one per 4-wave half,
// taken from the counter until none is left.  Which block computes a unit does not change
// its result, so the outputs do not depend on the order the units are taken in.
template <bool PAGED>
__device__ __forceinline__ void hca_worker_loop(const AttnDev& Hd, int units, uint32_t* next,
                                                float (*s_o)[16][129], float (*s_ml)[2][16],
                                                int* s_next) {
  const int half = threadIdx.x >> 8, tid = threadIdx.x & 255;
  for (;;) {
    if (threadIdx.x == 0) *s_next = static_cast<int>(atomicAdd(next, 2u));
    __syncthreads();
    const int u0 = *s_next;
    if (u0 >= units) break;                      // block-uniform
    const int u = u0 + half;
    if (u < units)
      hca_decode_block<PAGED>(Hd, u % Hd.splits, u / Hd.splits, s_o + 4 * half,
                              s_ml + 4 * half, tid);
    else
      __syncthreads();                           // the unit's one barrier
    __syncthreads();                             // LDS and s_next free for the next pair
  }
}

// grid: rows * kMxFloorParts + B * pool_blocks; block 512.  PAGED: caches in 128-token
// pages through the block table.
template <int HI, int KS, bool PAGED>
__global__ __launch_bounds__(kStepThreads) void step_front_kernel(StepDev S) {
  __shared__ float alpha[1024];
  __shared__ float s_part[kStepThreads * 8];
  const int bx = blockIdx.x;
  if (bx == 0 && threadIdx.x == 0) *S.hca_next = 0u;   // the back launch's unit counter
  if (bx < S.rows * kMxFloorParts) {
    mx_floor_block<HI, KS, true, PAGED, false>(S.X, S.k, bx / kMxFloorParts,
                                               bx % kMxFloorParts, true);
    return;
  }
  const int b2 = bx - S.rows * kMxFloorParts;
  pool_jobs_block<PAGED>(S.J, b2 % S.pool_blocks, alpha, s_part, b2 / S.pool_blocks);
}

// grid: rows * parts + HCA workers; block 512.  Blocks below rows * parts: the
// row's resolve, then the CSA attention over split `part` of its key list by all 8 waves;
// the rest take pairs of HCA units (one per 4-wave half) from a counter until none is
// left.  Which block computes a unit does not change its result, so the outputs do not
// depend on the order the units are taken in.
template <int HI, int KS, bool PAGED>
__global__ __launch_bounds__(kStepThreads) void step_back_kernel(StepDev S) {
  __shared__ int s_code[kMfmaMaxChunk];
  __shared__ float s_o[8][16][129];
  __shared__ float s_ml[8][2][16];
  __shared__ int s_next;
  const int bx = blockIdx.x;
  if (bx < S.rows * S.parts) {
    // every part of a row runs the row's (deterministic) resolve, so each holds the same
    // selection without waiting for another block, then attends over its split of the list
    const int row = bx / S.parts, part = bx % S.parts;
    mx_resolve_row<HI, KS, true, PAGED, false, false>(S.X, S.k, S.idx, row);
    const RowKeys r = row_keys<true>(S.C, row);
    Row8State st;
    row8_init(S.C, row, st);
    // (csa_range8 begins with a barrier: the selection is then visible to the block)
    const int p0 = part * S.C.chunk, p1 = min(r.L, p0 + S.C.chunk);
    csa_range8<false>(S.C, r, row, p0, p1, s_code, st.qB, st.acc, st.m_run, st.l_run, st.sl2);
    combine_waves<8>(S.C, st.acc, st.m_run, st.l_run, s_o, s_ml, part, row, threadIdx.x);
    return;
  }
  hca_worker_loop<PAGED>(S.Hd, S.hca_units, S.hca_next, s_o, s_ml, &s_next);
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

// ---- bf16 or fp32 indexer keys: the score-array form
//
// The key scan writes the score array and the segment extract lists each segment's keys at
// or above the row's sampled floor (the selector's own launches); the back launch then
// runs the row's resolve in its row blocks, so it overlaps the HCA stream instead of
// taking a launch of its own, and the merge follows as in the MXFP4 form.  The selection
// is the selector's bit for bit (the same device code).
struct StepScoresDev {
  segsel::TopkDev P;   // the score rows (in the workspace) and the selection output
  segsel::SegWs Sg;    // floors and candidate lists of the extract launch
  int vec;             // rows readable with 16-byte loads
  AttnDev C, Hd;       // CSA and HCA attention (partials in the workspace)
  int rows, hca_units, parts;
  uint32_t* hca_next;  // next HCA unit (zeroed by the extract launch)
};

static_assert(segsel::kResThreads == kStepThreads, "the resolve runs on a step block");

// grid: rows * parts + HCA workers; block 512.  Row blocks: the row's resolve (each part
// of a row runs it, so neither waits for the other), then the CSA attention over split
// `part` of the row's key list by all 8 waves; the other blocks are HCA workers.
template <int KB, bool PAGED>
__global__ __launch_bounds__(kStepThreads) void step_back_scores_kernel(StepScoresDev S) {
  constexpr int W = kStepThreads / 64;
  __shared__ int s_code[kMfmaMaxChunk];
  // the resolve's segment prefix lives where the attention's partial outputs go later
  __shared__ union {
    float o[8][16][129];
    int pre[segsel::kResMaxSeg + 1];
  } s_u;
  __shared__ float s_ml[8][2][16];
  __shared__ int s_cnt[2][W];
  __shared__ int s_gt[W], s_eq[W], s_hb[W];
  __shared__ int s_hist[2][256];
  __shared__ int s_sel[4];
  __shared__ int s_over;
  __shared__ int s_next;
  const int bx = blockIdx.x;
  if (bx < S.rows * S.parts) {
    const int row = bx / S.parts, part = bx % S.parts;
    segsel::seg_resolve_row<KB>(S.P, S.Sg, S.vec, row, s_u.pre, s_cnt, s_gt, s_eq, s_hb, s_hist,
                                s_sel, &s_over);
    const RowKeys r = row_keys<true>(S.C, row);
    Row8State st;
    row8_init(S.C, row, st);
    // (csa_range8 begins with a barrier: the selection is then visible to the block, and
    // every thread is past its last read of the segment prefix)
    const int p0 = part * S.C.chunk, p1 = min(r.L, p0 + S.C.chunk);
    csa_range8<false>(S.C, r, row, p0, p1, s_code, st.qB, st.acc, st.m_run, st.l_run, st.sl2);
    combine_waves<8>(S.C, st.acc, st.m_run, st.l_run, s_u.o, s_ml, part, row, threadIdx.x);
    return;
  }
  hca_worker_loop<PAGED>(S.Hd, S.hca_units, S.hca_next, s_u.o, s_ml, &s_next);
}

template <int HI, int KS, bool PAGED>
hipError_t launch_step_hi(const StepDev& S, int front_blocks, int back_blocks, int H_I,
                          hipStream_t s) {
  step_front_kernel<HI, KS, PAGED><<<front_blocks, kStepThreads, 0, s>>>(S);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_mx_candidate_scan(S.X, S.rows, H_I, PAGED, s);
  if (e != hipSuccess) return e;
  step_back_kernel<HI, KS, PAGED><<<back_blocks, kStepThreads, 0, s>>>(S);
  return hipGetLastError();
}

}  // namespace

// CUs of the current device (cached per device).
static int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    const hipError_t e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess || n < 1) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Attention splits of the four-launch step.  CSA: one per row (the row block's 8 waves take
// the whole key list).  HCA: units of at least 128 entries, about four per worker
// half-block, the workers being the CUs the row blocks leave.  The HCA units' outputs are
// combined exactly by the merge, so the results equal the attention call's up to the
// rounding of the split sums.
AttnPlan plan_step_csa(int B, int Nq, int H, int d, int k, int n_win) {
  AttnPlan p = plan_attention(true, HCSA_BF16, B, Nq, H, d, k + n_win);
  // one split per block of the row
  const int parts = step_row_parts(p.rows);
  p.chunk = std::max((k + n_win + parts - 1) / parts, 1);
  p.splits = parts;
  p.part_bytes = p.total_bytes = align256(static_cast<size_t>(parts) * p.rows * H * d * 4) +
                                 align256(static_cast<size_t>(parts) * p.rows * H * 4);
  return p;
}

static int step_hca_workers(int rows) {
  return std::max(1, device_cus() - step_row_parts(rows) * rows);
}

AttnPlan plan_step_hca(int B, int Nq, int H, int d, int N_h) {
  AttnPlan p = plan_attention(false, HCSA_BF16, B, Nq, H, d, N_h);
  if (!p.hca_decode || N_h < 1) return p;
  const int64_t total = static_cast<int64_t>(p.rows) * N_h;
  const int64_t units = 2 * static_cast<int64_t>(step_hca_workers(p.rows));
  int64_t c = (total + units - 1) / units;
  // at most kMergeRegSplits splits per row, so the merge loads them all at once
  c = std::max<int64_t>(c, (N_h + kMergeRegSplits - 1) / kMergeRegSplits);
  c = std::max<int64_t>(128, (c + 31) / 32 * 32);
  p.chunk = static_cast<int>(std::min<int64_t>(c, kMfmaMaxChunk));
  p.splits = std::max(1, (N_h + p.chunk - 1) / p.chunk);
  p.part_bytes = p.splits > 1 ? align256(static_cast<size_t>(p.splits) * p.rows * H * d * 4) +
                                    align256(static_cast<size_t>(p.splits) * p.rows * H * 4)
                              : 0;
  p.total_bytes = p.part_bytes;
  return p;
}

// The log-sum-exp merge of a step's splits: CSA rows first, then HCA rows (a call without
// splits needs none).
static hipError_t launch_step_merge(const DecodeStepArgs& a, const AttnDev& C, const AttnDev& Hd,
                                    const AttnPlan& pc, const AttnPlan& ph, hipStream_t s) {
  const int rows = a.B * a.Nq;
  StepMerge mc{C.out, C.lse, pc.splits, rows, a.c.out, a.c.lse};
  const StepMerge mh{Hd.out, Hd.lse, ph.splits, rows, a.h.out, a.h.lse};
  if (pc.splits == 1) mc.rows = 0;
  const int gy = mc.rows + (ph.splits > 1 ? rows : 0);
  if (gy > 0) step_merge_kernel<<<dim3(a.c.H, gy), a.c.d, 0, s>>>(mc, mh, a.c.H, a.c.d);
  return hipGetLastError();
}

bool decode_step_fast(const DecodeStepArgs& a, const AttnPlan& pc, const AttnPlan& ph,
                      bool fused_selection) {
  const bool hi_ok = a.H_I == 1 || a.H_I == 2 || a.H_I == 4 || a.H_I == 8 || a.H_I == 16;
  return fused_selection && a.Nq == 1 && a.k_dtype == HCSA_MXFP4 && a.q_dtype == HCSA_BF16 &&
         a.score_dtype == HCSA_BF16 && hi_ok && csa_hca_fused(pc, ph) &&
         a.c.k + a.c.n_win <= kMfmaMaxChunk;
}

size_t decode_step_sync_bytes(int rows) { (void)rows; return 256; }

hipError_t launch_decode_step(const DecodeStepArgs& a, const AttnPlan& pc, const AttnPlan& ph,
                              void* ws, size_t sync_off, size_t attn_off, hipStream_t s) {
  const int rows = a.B * a.Nq;
  char* base = static_cast<char*>(ws);
  StepDev S{};
  const MxTopkLayout l = mx_topk_layout(rows, a.N);
  char* mx = base;
  S.X = make_mx_dev(a.q_idx, a.w_idx, a.k_idx, a.k_bstride, a.k_scales, a.ks_bstride, a.B,
                    a.Nq, a.d_I, a.N, a.c.ratio, a.c.pos0, a.seq_pos, a.block_table,
                    a.c.table_stride, mx + l.scores_off);
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
  S.pool_blocks = a.n_jobs > 0 ? pool_jobs_fill(a.jobs, a.n_jobs, a.block_table,
                                                a.c.table_stride, a.raw_ring, kStepThreads, S.J)
                               : 0;
  S.hca_units = rows * ph.splits;
  S.parts = pc.splits;
  S.hca_next = reinterpret_cast<uint32_t*>(base + sync_off);
  const int front = rows * kMxFloorParts + a.B * S.pool_blocks;
  const int back = S.parts * rows + std::min(step_hca_workers(rows), (S.hca_units + 1) / 2);
  hipError_t e = hipErrorInvalidValue;
  const bool ks2 = a.d_I > 64, paged = a.block_table != nullptr;
#define HCSA_STEP(HI_)                                                              \
  if (a.H_I == HI_) {                                                               \
    if (paged)                                                                      \
      e = ks2 ? launch_step_hi<HI_, 2, true>(S, front, back, a.H_I, s)               \
              : launch_step_hi<HI_, 1, true>(S, front, back, a.H_I, s);              \
    else                                                                            \
      e = ks2 ? launch_step_hi<HI_, 2, false>(S, front, back, a.H_I, s)              \
              : launch_step_hi<HI_, 1, false>(S, front, back, a.H_I, s);             \
  }
  HCSA_STEP(1) HCSA_STEP(2) HCSA_STEP(4) HCSA_STEP(8) HCSA_STEP(16)
#undef HCSA_STEP
  if (e != hipSuccess) return e;
  return launch_step_merge(a, S.C, S.Hd, pc, ph, s);
}

bool decode_step_scores_ok(const DecodeStepArgs& a, const AttnPlan& pc, const AttnPlan& ph) {
  const TopkPlan tp = plan_topk(a.score_dtype, a.B * a.Nq, a.N, a.c.k);
  return a.Nq == 1 && (a.k_dtype == HCSA_BF16 || a.k_dtype == HCSA_F32) &&
         (a.score_dtype == HCSA_BF16 || a.score_dtype == HCSA_F32) && !tp.rows_path &&
         topk_plan_ok(tp) && csa_hca_fused(pc, ph) && a.c.k + a.c.n_win <= kMfmaMaxChunk;
}

hipError_t launch_decode_step_scores(const DecodeStepArgs& a, const AttnPlan& pc,
                                     const AttnPlan& ph, void* ws, size_t sync_off,
                                     size_t attn_off, hipStream_t s) {
  const int rows = a.B * a.Nq;
  char* base = static_cast<char*>(ws);
  // the selection state as the selector's own call lays it out: scores, then its plan
  const TopkPlan tp = plan_topk(a.score_dtype, rows, a.N, a.c.k);
  const size_t sbytes =
      align256(static_cast<size_t>(rows) * a.N * (a.score_dtype == HCSA_BF16 ? 2 : 4));
  void* scores = base;
  StepScoresDev S{};
  seg_select_view(tp, scores, a.N, a.Nq, a.c.ratio, a.c.pos0, a.seq_pos, a.idx, base + sbytes,
                  &S.P, &S.Sg, &S.vec);
  S.hca_next = reinterpret_cast<uint32_t*>(base + sync_off);
  S.Sg.clear = S.hca_next;
  S.C = attn_dev_for(a.c, pc, base + attn_off);
  S.Hd = attn_dev_for(a.h, ph, base + attn_off + align256(pc.total_bytes));
  S.rows = rows;
  S.hca_units = rows * ph.splits;
  S.parts = pc.splits;
  hipError_t e = hipSuccess;
  if (a.n_jobs > 0) {
    e = launch_compress_batched(a.jobs, a.n_jobs, a.B, a.block_table, a.c.table_stride,
                                a.raw_ring, s);
    if (e != hipSuccess) return e;
  }
  e = launch_index_scores(a.q_idx, a.q_dtype, a.w_idx, a.k_idx, a.k_dtype, a.k_bstride,
                          a.k_scales, a.ks_bstride, a.B, a.Nq, a.H_I, a.d_I, a.N, a.c.ratio,
                          a.c.pos0, a.seq_pos, a.block_table, a.c.table_stride, a.score_dtype,
                          scores, s);
  if (e != hipSuccess) return e;
  e = launch_seg_extract(S.P, S.Sg, S.vec, tp.key_bits, rows, s);
  if (e != hipSuccess) return e;
  const int back = S.parts * rows + std::min(step_hca_workers(rows), (S.hca_units + 1) / 2);
  const bool paged = a.block_table != nullptr;
  if (tp.key_bits == 16) {
    if (paged) step_back_scores_kernel<16, true><<<back, kStepThreads, 0, s>>>(S);
    else step_back_scores_kernel<16, false><<<back, kStepThreads, 0, s>>>(S);
  } else {
    if (paged) step_back_scores_kernel<32, true><<<back, kStepThreads, 0, s>>>(S);
    else step_back_scores_kernel<32, false><<<back, kStepThreads, 0, s>>>(S);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_step_merge(a, S.C, S.Hd, pc, ph, s);
}


}  // namespace hcsa
