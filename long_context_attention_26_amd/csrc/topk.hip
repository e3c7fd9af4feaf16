// Top-k selector: exact and deterministic, on order-preserving integer keys of the scores.
//
// The indexer keeps the top-k compressed entries of each query (Lighthouse, "deep
// deepseek v4 release", section 八 item 3; k = 1024 Pro / 512 Flash); BF16 scores make the
// selector cheaper (9fzt.com digest, item 4).  Ties go to the lowest index and the output
// is ascending, the reading taken where the pages are silent.
//
// Keys are the score bits mapped to unsigned integers in the scores' order (-0 equal to +0).
// With T the k-th largest key of a row, the selection is every key above T and then the
// lowest-index keys equal to T, written in ascending index order (-1 padding when a row sees
// fewer than k entries).
//
// A wave64 vector instruction occupies its SIMD for four cycles, so the selectors touch
// every key only a few times.  Both paths first bound the candidates with a floor L: the
// 16-bit prefix of the m-th largest key of a sample of the row, m twice the sample rank at
// which the k-th largest key is expected plus a margin, so that typically a few percent of
// the row is >= L while at least k keys are (checked).
//  - Many short rows (prefill: >= 64 rows of <= 128K keys): one block per row streams the
//    row once (topk_rows_kernel), sampling the first chunks it loads.
//  - Otherwise (decode: a few long rows): seg_extract_kernel (a block per 2048-key segment:
//    the row's floor from 4096 keys at evenly spaced 16-byte chunks, the same in every
//    block of the row, then the segment's keys >= L into its candidate list, in index
//    order) and seg_resolve_kernel (a block per row: T among the concatenated lists by
//    8-bit LDS histogram passes, and the ordered output).
// When the candidates overflow their lists or fall short of k (massive ties, a skewed row,
// an unlucky sample), T is found bit by bit over the whole row and the output is written by
// an ordered ballot compaction.  Every step is integer-only, so results do not depend on
// scheduling.
#include "common.h"
#include "internal.h"
#include "select_dev.h"
#include "seg_dev.h"

#include <algorithm>
#include <type_traits>

namespace hcsa {

namespace {

using namespace sel;

using namespace segsel;

// ---------------------------------------------------------------- many rows: one block per row

// One 512-thread block per row streams the row from HBM once; four such blocks share a CU,
// so one block's loads overlap the others' arithmetic.  Wave w owns a contiguous run of
// chunks and walks it 64 chunks at a time (index order = wave, step, lane, element); the
// floor comes from the first key of each lane's first four chunks (up to 2048 samples,
// loaded anyway), and the stream appends the index of every key >= L to the wave's LDS
// list (the threshold search re-reads those keys from the row, which the block has just
// streamed).
constexpr int kRowsThreads = 512;
constexpr int kRowsWaves = kRowsThreads / 64;
constexpr int kRowsMaxKeys = 131072;
constexpr int kRowsWaveCap = 512;   // candidates per wave list

__host__ __device__ inline bool rows_path(int rows, int N) {
  return rows >= 64 && N <= kRowsMaxKeys;
}

// grid: rows; block 512.
template <int KB>
__global__ __launch_bounds__(kRowsThreads) void topk_rows_kernel(TopkDev P, int vec) {
  using V_t = RowView<KB>;
  constexpr int EPC = V_t::EPC;
  constexpr int STEPS = kRowsWaveCap / 64;       // list entries per lane at most
  __shared__ int32_t s_cj[kRowsWaves][kRowsWaveCap];   // candidate indices (keys re-read)
  __shared__ int s_cnt[2][kRowsWaves];
  __shared__ int s_wave[kRowsWaves], s_gt[kRowsWaves], s_eq[kRowsWaves], s_hb[kRowsWaves];
  __shared__ int s_hist[2][256];
  __shared__ int s_sel[4];
  const int row = blockIdx.x;
  const V_t V = row_view<KB>(P, row, vec);
  const int nv = V.nv;
  int32_t* out = P.idx + static_cast<int64_t>(row) * P.k;
  if (P.k >= nv) {
    take_all(nv, P.k, out, kRowsThreads);
    return;
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint64_t below = (1ull << lane) - 1;
  const int nch = V.nchunks();
  const int CW = (nch + kRowsThreads - 1) / kRowsThreads * 64;   // chunks per wave
  const int cw0 = w * CW, cw1 = min(cw0 + CW, nch);

  // first stream loads, in flight while the floor is chosen
  u32x4 cur[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int ch = cw0 + 64 * u + lane;
    cur[u] = ch < cw1 ? V.load_raw(ch) : u32x4{0u, 0u, 0u, 0u};
  }

  // ---- 1. candidate floor L (all keys are candidates when few): the m-th largest 16-bit
  // sample prefix (a 128th of a binade: a coarser floor would admit up to a whole bin of
  // extra candidates), by two LDS histograms of 8 bits (the high byte, then the low byte
  // within the chosen high byte): a few atomics per thread and four barriers in all.
  uint32_t L = 0;
  if (nv > kRowsWaves * kRowsWaveCap / 2) {
    s_hist[threadIdx.x >> 8][threadIdx.x & 255] = 0;
    uint32_t st[4];                              // 0 = no sample (never counts)
    int nmine = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool sv = cw0 + 64 * u + lane < cw1;  // first elements are visible keys
      st[u] = sv ? V_t::to_key(V_t::raw_of(cur[u], 0)) >> (KB - 16) : 0u;
      nmine += sv;
    }
    const int ns = block_total_bits<kRowsWaves, bits_for(4)>(nmine, s_cnt, 0);   // also orders the zeroing
    const int m = max(1, min(ns, static_cast<int>((2LL * P.k * ns + nv - 1) / nv) + 16));
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (st[u] != 0u) atomicAdd(&s_hist[0][st[u] >> 8], 1);
    __syncthreads();
    if (w == 0) hist_pick(s_hist[0], m, s_sel);  // s_sel = {high byte, samples above it}
    __syncthreads();
    const uint32_t hi = static_cast<uint32_t>(s_sel[0]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (st[u] != 0u && (st[u] >> 8) == hi) atomicAdd(&s_hist[1][st[u] & 255u], 1);
    __syncthreads();
    if (w == 0) hist_pick(s_hist[1], m - s_sel[1], s_sel + 2);
    __syncthreads();
    // fewer than m nonzero samples: no floor
    L = s_sel[0] < 0 || s_sel[2] < 0 ? 0u : ((hi << 8) | static_cast<uint32_t>(s_sel[2])) << (KB - 16);
  }

  // ---- 2. stream the wave's chunks 256 at a time (the next 256 loading meanwhile),
  // appending the indices of keys >= L to the wave's list.  Steps whose chunks are all
  // whole and visible (every step but a row's last, as a rule) load and test them without
  // per-chunk checks.
  const int whole = min(min(V.nfull, nv / EPC), cw1);   // chunks below: whole, visible
  int wslot = 0;
  for (int base = cw0; base < cw1; base += 256) {
    u32x4 nxt[4];
    const bool more = base + 256 < cw1;          // wave-uniform
    if (more) {
      if (base + 512 <= whole) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          nxt[u] = *reinterpret_cast<const u32x4*>(
              V.rowp + static_cast<int64_t>(base + 256 + 64 * u + lane) * EPC);
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int ch = base + 256 + 64 * u + lane;
          nxt[u] = ch < cw1 ? V.load_raw(ch) : u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
    const bool full = base + 256 <= whole;       // wave-uniform
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ch = base + 64 * u + lane;
      uint32_t msk = full ? V.ge_bits(cur[u], L) : ch < cw1 ? V.ge_mask(cur[u], ch * EPC, L) : 0u;
      int tot;
      int o = wslot + wave_prefix_bits<bits_for(EPC)>(__popc(msk), below, tot);
      while (msk) {
        const int e = __ffs(msk) - 1;
        msk &= msk - 1;
        if (o < kRowsWaveCap) s_cj[w][o] = ch * EPC + e;
        ++o;
      }
      wslot += tot;
    }
    if (more) {
#pragma unroll
      for (int u = 0; u < 4; ++u) cur[u] = nxt[u];
    }
  }
  if (lane == 0) s_wave[w] = wslot;
  __syncthreads();
  int C = 0;
  bool overflow = false;
#pragma unroll
  for (int u = 0; u < kRowsWaves; ++u) {
    C += s_wave[u];
    overflow |= s_wave[u] > kRowsWaveCap;
  }
  if (overflow || C < P.k) {
    select_exact_row<KB, kRowsThreads>(V, P.k, out, s_cnt, s_gt, s_eq);
    return;
  }

  // ---- 3. exact threshold among the candidates: lane l of wave w holds entries
  // l, l+64, ... of the wave's list; the lists are in index order, wave after wave, so the
  // output order is (wave, step, lane)
  uint32_t ck[STEPS];
  uint32_t dor = 0;
#pragma unroll
  for (int u = 0; u < STEPS; ++u) {
    const bool in = 64 * u + lane < wslot;
    ck[u] = in ? V.key(s_cj[w][64 * u + lane]) : 0u;   // the row's own key, re-read
    dor |= in ? (ck[u] ^ L) : 0u;
  }
  int hb = 0;
  for (int b = KB - 1; b >= 0; --b) {
    if (__ballot((dor >> b) & 1u)) {
      hb = b + 1;
      break;
    }
  }
  if (lane == 0) s_hb[w] = hb;
  s_hist[threadIdx.x >> 8][threadIdx.x & 255] = 0;
  __syncthreads();
  int nb = 0;
#pragma unroll
  for (int u = 0; u < kRowsWaves; ++u) nb = s_hb[u] > nb ? s_hb[u] : nb;
  // T = the k-th largest candidate, 8 bits a pass from the highest bit in which the
  // candidates differ from L: an LDS histogram of the pass's digit over the candidates that
  // match T so far (digits from the top of the differing bits spread over the bins)
  const int D = (nb + 7) / 8;
  uint32_t T = nb >= 32 ? 0u : (L >> nb) << nb;
  int rem = P.k;                                 // rank of T among the candidates still open
#pragma unroll 1
  for (int p = 0; p < D; ++p) {
    const int top = nb - 8 * p;                  // this pass: bits [sh, top)
    const int sh = top > 8 ? top - 8 : 0;
    const uint32_t dmask = (1u << (top - sh)) - 1u;
    int* hist = s_hist[p & 1];
    const uint32_t hi = top >= 32 ? 0u : T >> top;
#pragma unroll
    for (int u = 0; u < STEPS; ++u) {
      const bool in = 64 * u + lane < wslot;
      if (in && (top >= 32 || (ck[u] >> top) == hi)) atomicAdd(&hist[(ck[u] >> sh) & dmask], 1);
    }
    if (p >= 1) s_hist[(p + 1) & 1][threadIdx.x & 255] = 0;   // the previous pass's bins
    __syncthreads();
    if (w == 0) hist_pick(hist, rem, s_sel);
    __syncthreads();
    // every thread reads s_sel before it reaches the next pass's first barrier, and the
    // next pick comes after that barrier
    T |= static_cast<uint32_t>(s_sel[0]) << sh;
    rem -= s_sel[1];
  }
  // per-wave counts of entries above T and equal to T
  int gt = 0, eq = 0;
#pragma unroll
  for (int u = 0; u < STEPS; ++u) {
    const bool in = 64 * u + lane < wslot;
    gt += in && ck[u] > T;
    eq += in && ck[u] == T;
  }
  gt = wave_sum_bits<bits_for(STEPS)>(gt);
  eq = wave_sum_bits<bits_for(STEPS)>(eq);
  if (lane == 0) {
    s_gt[w] = gt;
    s_eq[w] = eq;
  }
  __syncthreads();
  int gt_before = 0, eq_rank = 0, gt_all = 0;
#pragma unroll
  for (int u = 0; u < kRowsWaves; ++u) {
    gt_before += u < w ? s_gt[u] : 0;
    eq_rank += u < w ? s_eq[u] : 0;
    gt_all += s_gt[u];
  }
  const int need = P.k - gt_all;                 // 1 <= need <= candidates equal to T
  int o = gt_before + min(need, eq_rank);
#pragma unroll
  for (int u = 0; u < STEPS; ++u) {
    if (64 * u < wslot) {                        // wave-uniform
      const bool in = 64 * u + lane < wslot;
      const bool is_eq = in && ck[u] == T;
      const uint64_t meq = __ballot(is_eq);
      const int r = eq_rank + __popcll(meq & below);
      const bool sel = in && (ck[u] > T || (is_eq && r < need));
      const uint64_t msel = __ballot(sel);
      if (sel) {
        const int oo = o + __popcll(msel & below);
        if (oo < P.k) out[oo] = s_cj[w][64 * u + lane];
      }
      o += __popcll(msel);
      eq_rank += __popcll(meq);
    }
  }
}

// ---------------------------------------------------------------- few long rows: segments


// The row's candidate floor from 4096 keys in 32 runs of 16 consecutive 16-byte chunks (two
// cache lines) at evenly spaced positions; every block of the row samples the same keys
// and so finds the same floor.  Called by all NT threads.
// Only the candidate count depends on the floor (too few or too many candidates send the
// row to the exact path), so it is an estimate of the 16-bit prefix of the m-th largest
// sample, m about twice the rank at which the k-th largest key is expected:
//  - shallow ranks (the decode case): each thread keeps the largest of its samples, and the
//    m-th largest of these group maxima stands in for the m-th largest sample (it is at or
//    below it, so it admits slightly more candidates); one ballot per tested threshold;
//  - deeper ranks: the m-th largest sample itself, every sample counted per threshold.
// Each wave finds the ceil(m/W)-th largest of its own values by radix 4 from the top
// (ballot counts, no barriers); the floor is the smallest of the W results, at or below
// the block's m-th largest.
template <int KB, int NT>
__device__ uint32_t row_floor(const RowView<KB>& V, int k, uint32_t* s_min) {
  constexpr int W = NT / 64;
  const int nv = V.nv;
  if (nv <= kSegCap) return 0u;                  // every visible key is a candidate
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  using V_t = RowView<KB>;
  constexpr int EPC = V_t::EPC;
  constexpr int NPOS = kFloorSamples / EPC;      // sampled 16-byte chunks (8 BF16 / 4 F32 keys)
  constexpr int LPT = NPOS / NT;                 // per thread
  constexpr int PT = LPT * EPC;
  constexpr int RUN = 16, NRUN = NPOS / RUN;     // runs of consecutive chunks
  const int nch = V.nchunks();                   // runs overlap when nch < NPOS
  // a missing key (past the visible count, last chunk only) reads as 0 and never counts:
  // every tested threshold is >= 1
  uint32_t top[PT];
#pragma unroll
  for (int u = 0; u < LPT; ++u) {
    const int i = threadIdx.x + u * NT, run = i / RUN;
    const int r0 = static_cast<int>(static_cast<int64_t>(run) * nch / NRUN);
    const int c = min(r0 + i % RUN, nch - 1);
    const u32x4 x = V.load_raw(c);
    const int r = nv - c * EPC;                  // visible keys of the chunk
#pragma unroll
    for (int e = 0; e < EPC; ++e)
      top[u * EPC + e] = e < r ? V_t::to_key(V_t::raw_of(x, e)) >> (KB - 16) : 0u;
  }
  const int m = min(kFloorSamples - EPC,
                    static_cast<int>((2LL * k * kFloorSamples + nv - 1) / nv) + 8);
  const int mw = (m + W - 1) / W;
  uint32_t pre = 0;
  if (mw <= 16) {
    uint32_t mx = 0;
#pragma unroll
    for (int u = 0; u < PT; ++u) mx = max(mx, top[u]);
#pragma unroll 1
    for (int sh = 14; sh >= 0; sh -= 2) {
      int cnt[3];
#pragma unroll
      for (int d = 1; d <= 3; ++d)
        cnt[d - 1] = __popcll(__ballot(mx >= (pre | (static_cast<uint32_t>(d) << sh))));
      const uint32_t d = cnt[2] >= mw ? 3u : cnt[1] >= mw ? 2u : cnt[0] >= mw ? 1u : 0u;
      pre |= d << sh;
    }
  } else {
#pragma unroll 1
    for (int sh = 14; sh >= 0; sh -= 2) {
      int cnt[3];
#pragma unroll
      for (int d = 1; d <= 3; ++d) {
        const uint32_t th = pre | (static_cast<uint32_t>(d) << sh);
        int n = 0;
#pragma unroll
        for (int u = 0; u < PT; ++u) n += top[u] >= th;
        cnt[d - 1] = wave_sum_bits<bits_for(PT)>(n);
      }
      const uint32_t d = cnt[2] >= mw ? 3u : cnt[1] >= mw ? 2u : cnt[0] >= mw ? 1u : 0u;
      pre |= d << sh;
    }
  }
  if (lane == 0) s_min[w] = pre;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < W; ++u) pre = min(pre, s_min[u]);
  return pre << (KB - 16);
}

// grid: (nseg, rows); block 256.  The row's floor (block 0 of the row stores it), then the
// segment: wave w owns 1/4 of its chunks, lane l chunks 64u + l of it (4 chunks for BF16
// keys, 8 for F32); the keys >= floor go to the segment's list in index order, and the
// segment's count (which may exceed the list) to the counters.
template <int KB>
__global__ __launch_bounds__(kSegThreads) void seg_extract_kernel(TopkDev P, SegWs S, int vec) {
  using V_t = RowView<KB>;
  constexpr int EPC = V_t::EPC;
  constexpr int W = kSegThreads / 64;
  constexpr int CPW = kSegKeys / EPC / W;        // chunks per wave
  constexpr int CPL = CPW / 64;                  // chunks per lane
  __shared__ int s_w[W];
  __shared__ uint32_t s_min[W];
  const int row = blockIdx.y, seg = blockIdx.x;
  if (S.clear != nullptr && row == 0 && seg == 0 && threadIdx.x == 0) *S.clear = 0u;
  const V_t V = row_view<KB>(P, row, vec);
  if (P.k >= V.nv || seg * kSegKeys >= V.nv) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint64_t below = (1ull << lane) - 1;
  const int nch = V.nchunks();
  const int ch0 = seg * (kSegKeys / EPC) + w * CPW + lane;
  u32x4 x[CPL];
#pragma unroll
  for (int u = 0; u < CPL; ++u) {
    const int ch = ch0 + 64 * u;
    x[u] = ch < nch ? V.load_raw(ch) : u32x4{0u, 0u, 0u, 0u};
  }
  const uint32_t L = row_floor<KB, kSegThreads>(V, P.k, s_min);
  if (seg == 0 && threadIdx.x == 0) S.floor[row] = L;
  uint32_t msk[CPL];
  int c = 0;
#pragma unroll
  for (int u = 0; u < CPL; ++u) {
    const int ch = ch0 + 64 * u;
    msk[u] = ch < nch ? V.ge_mask(x[u], ch * EPC, L) : 0u;
    c += __popc(msk[u]);
  }
  c = wave_sum_bits<bits_for(CPL * EPC)>(c);
  if (lane == 0) s_w[w] = c;
  __syncthreads();
  int slot = 0, total = 0;
#pragma unroll
  for (int u = 0; u < W; ++u) {
    slot += u < w ? s_w[u] : 0;
    total += s_w[u];
  }
  uint64_t* list = S.cand + (static_cast<int64_t>(row) * S.nseg + seg) * kSegCap;
#pragma unroll
  for (int u = 0; u < CPL; ++u) {
    const int ch = ch0 + 64 * u;
    int tot;
    int o = slot + wave_prefix_bits<bits_for(EPC)>(__popc(msk[u]), below, tot);
    uint32_t m = msk[u];
    while (m) {
      const int e = __ffs(m) - 1;
      m &= m - 1;
      if (o < kSegCap)
        list[o] = (static_cast<uint64_t>(V_t::to_key(V_t::raw_of(x[u], e))) << 32) |
                  static_cast<uint32_t>(ch * EPC + e);
      ++o;
    }
    slot += tot;
  }
  if (threadIdx.x == 0) S.cnt[static_cast<int64_t>(row) * S.nseg + seg] = static_cast<uint32_t>(total);
}

// grid: rows; block 512.
template <int KB>
__global__ __launch_bounds__(kResThreads) void seg_resolve_kernel(TopkDev P, SegWs S, int vec) {
  constexpr int W = kResThreads / 64;
  __shared__ int s_pre[kResMaxSeg + 1];
  __shared__ int s_cnt[2][W];
  __shared__ int s_gt[W], s_eq[W], s_hb[W];
  __shared__ int s_hist[2][256];
  __shared__ int s_sel[4];
  __shared__ int s_over;
  seg_resolve_row<KB>(P, S, vec, blockIdx.x, s_pre, s_cnt, s_gt, s_eq, s_hb, s_hist, s_sel,
                      &s_over);
}

}  // namespace


TopkPlan plan_topk(int score_dtype, int rows, int N, int k) {
  TopkPlan p{};
  p.rows = rows;
  p.N = N;
  p.k = k;
  p.key_bits = score_dtype == 1 ? 16 : 32;
  p.rows_path = rows_path(rows, N);
  p.nseg = N > 0 ? (N + kSegKeys - 1) / kSegKeys : 1;
  if (p.rows_path) {
    p.total_bytes = 0;                           // one block per row, all state on chip
  } else {
    p.floor_off = 0;
    p.cnt_off = align256(static_cast<size_t>(rows) * 4);
    p.cand_off = p.cnt_off + align256(static_cast<size_t>(rows) * p.nseg * 4);
    p.total_bytes = p.cand_off + static_cast<size_t>(rows) * p.nseg * kSegCap * 8;
  }
  return p;
}

bool topk_plan_ok(const TopkPlan& plan) { return plan.rows_path || plan.nseg <= kResMaxSeg; }

void seg_select_view(const TopkPlan& plan, const void* scores, int64_t row_stride, int Nq,
                     int ratio, int64_t pos0, const int64_t* seq_pos, int32_t* idx, void* ws,
                     segsel::TopkDev* P, segsel::SegWs* S, int* vec) {
  *P = segsel::TopkDev{};
  P->scores = scores;
  P->row_stride = row_stride;
  P->Nq = Nq;
  P->N = plan.N;
  P->ratio = ratio;
  P->k = plan.k;
  P->pos0 = pos0;
  P->seq_pos = seq_pos;
  P->idx = idx;
  const int esz = plan.key_bits / 8;
  *vec = (reinterpret_cast<uintptr_t>(scores) % 16 == 0) && (row_stride * esz) % 16 == 0;
  *S = segsel::SegWs{};
  if (!plan.rows_path) {
    S->floor = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + plan.floor_off);
    S->cnt = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + plan.cnt_off);
    S->cand = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + plan.cand_off);
    S->nseg = plan.nseg;
  }
}

hipError_t launch_seg_extract(const segsel::TopkDev& P, const segsel::SegWs& S, int vec,
                              int key_bits, int rows, hipStream_t s) {
  const dim3 grid(S.nseg, rows);
  if (key_bits == 16) seg_extract_kernel<16><<<grid, kSegThreads, 0, s>>>(P, S, vec);
  else seg_extract_kernel<32><<<grid, kSegThreads, 0, s>>>(P, S, vec);
  return hipGetLastError();
}

hipError_t launch_topk(const TopkPlan& plan, const void* scores, int score_dtype,
                       int64_t row_stride, int Nq, int ratio, int64_t pos0,
                       const int64_t* seq_pos, int32_t* idx, void* ws, hipStream_t s) {
  (void)score_dtype;
  TopkDev P;
  SegWs S;
  int vec = 0;
  seg_select_view(plan, scores, row_stride, Nq, ratio, pos0, seq_pos, idx, ws, &P, &S, &vec);
  if (plan.rows_path) {
    if (plan.key_bits == 16) topk_rows_kernel<16><<<plan.rows, kRowsThreads, 0, s>>>(P, vec);
    else topk_rows_kernel<32><<<plan.rows, kRowsThreads, 0, s>>>(P, vec);
    return hipGetLastError();
  }
  const hipError_t e = launch_seg_extract(P, S, vec, plan.key_bits, plan.rows, s);
  if (e != hipSuccess) return e;
  if (plan.key_bits == 16) seg_resolve_kernel<16><<<plan.rows, kResThreads, 0, s>>>(P, S, vec);
  else seg_resolve_kernel<32><<<plan.rows, kResThreads, 0, s>>>(P, S, vec);
  return hipGetLastError();
}

}  // namespace hcsa
