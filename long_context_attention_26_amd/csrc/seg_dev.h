// Top-k over a materialised row of scores for few long rows (decode), the device parts
// shared by the selector's own launches and the decode-step launch: the row view of a
// score array, the segment workspace, and the per-row resolve.
//
// The indexer keeps the top-k compressed entries of each query (Lighthouse, "deep deepseek
// v4 release", section 八 item 3); ties go to the lowest index and the output is ascending
// (the reading taken where the pages are silent).  A segment extract block per 2048 keys
// lists the keys at or above the row's sampled floor; the resolve takes the row's exact
// top-k among the concatenated lists, or falls back to the exact whole-row selection when
// a list overflowed or fewer than k keys were listed.
#pragma once
#include "common.h"
#include "select_dev.h"

namespace hcsa {
namespace segsel {

using namespace sel;

struct TopkDev {
  const void* scores;
  int64_t row_stride;   // elements
  int Nq, N, ratio, k;
  int64_t pos0;
  const int64_t* seq_pos;   // [B] or null
  int32_t* idx;         // [rows][k]
};

__device__ __forceinline__ int visible(const TopkDev& P, int row) {
  const int64_t p = query_pos(P.seq_pos, P.pos0, row / P.Nq, row % P.Nq);
  const int64_t v = (p + 1) / P.ratio;
  return static_cast<int>(v < P.N ? v : P.N);
}

// A row of scores of a call as a RowView.
template <int KB>
__device__ __forceinline__ RowView<KB> row_view(const TopkDev& P, int row, int vec) {
  using KT = typename RowView<KB>::KT;
  const char* p = static_cast<const char*>(P.scores) +
                  static_cast<int64_t>(row) * P.row_stride * sizeof(KT);
  const int nv = visible(P, row);
  return RowView<KB>(p, nv, vec ? P.N / RowView<KB>::EPC : 0);
}
constexpr int kSegKeys = 2048;            // keys per segment (one extract block)
constexpr int kSegCap = 512;              // candidate list per segment
constexpr int kSegThreads = 256;
constexpr int kFloorSamples = 4096;       // 16 per thread
constexpr int kResThreads = 512;
constexpr int kResPer = 16;               // candidates per resolve thread at most
constexpr int kResMax = kResThreads * kResPer;
constexpr int kResMaxSeg = 16384;         // segments per row (rows of up to 32M keys)

struct SegWs {
  uint32_t* floor;    // [rows]
  uint32_t* cnt;      // [rows][nseg]   keys >= floor per segment (may exceed the cap)
  uint64_t* cand;     // [rows][nseg][kSegCap]   key << 32 | index
  int nseg;
  uint32_t* clear;   // null, or a word the extract launch sets to 0 (a later launch's counter)
};

// The row's exact top-k among its segments' candidate lists, by one 512-thread block (the
// lists concatenated in segment order are the row's candidates in index order; thread t
// takes a contiguous run of them).  LDS comes from the caller: s_pre holds kResMaxSeg + 1
// ints.  Writes the row's k indices to P.idx.
template <int KB>
__device__ void seg_resolve_row(const TopkDev& P, const SegWs& S, int vec, int row, int* s_pre,
                                int (*s_cnt)[kResThreads / 64], int* s_gt, int* s_eq, int* s_hb,
                                int (*s_hist)[256], int* s_sel, int* s_over) {
  const RowView<KB> V = row_view<KB>(P, row, vec);
  const int nv = V.nv;
  int32_t* out = P.idx + static_cast<int64_t>(row) * P.k;
  if (P.k >= nv) {
    take_all(nv, P.k, out, kResThreads);
    return;
  }
  const int nseg = (nv + kSegKeys - 1) / kSegKeys;   // segments holding visible keys
  const uint32_t* cnt = S.cnt + static_cast<int64_t>(row) * S.nseg;
  if (threadIdx.x < 64) {                        // prefix of the listed counts, 64 at a time
    const int lane = threadIdx.x;
    int carry = 0;
    bool over = false;
    // the first four rounds' counts are loaded together (one memory latency for rows of up
    // to 256 segments), later rounds' as they come
    int pre4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int sg = 64 * q + lane;
      pre4[q] = sg < nseg ? static_cast<int>(cnt[sg]) : 0;
    }
    for (int base = 0; base < nseg; base += 64) {
      const int sg = base + lane;
      int c = 0;
      if (base < 256) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (base == 64 * q) c = pre4[q];
      } else {
        c = sg < nseg ? static_cast<int>(cnt[sg]) : 0;
      }
      over |= c > kSegCap;
      int inc = c < kSegCap ? c : kSegCap;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(inc, d, kWave);
        if (lane >= d) inc += y;
      }
      if (sg < nseg) s_pre[sg + 1] = carry + inc;
      carry += __shfl(inc, 63, kWave);
    }
    const bool any_over = __ballot(over) != 0;
    if (lane == 0) {
      s_pre[0] = 0;
      *s_over = any_over;
    }
  }
  __syncthreads();
  const int C = s_pre[nseg];
  if (*s_over || C < P.k || C > kResMax) {
    select_exact_row<KB, kResThreads>(V, P.k, out, s_cnt, s_gt, s_eq);
    return;
  }
  const int per = (C + kResThreads - 1) / kResThreads;
  const int g0 = min(C, static_cast<int>(threadIdx.x) * per);
  const int my = min(per, C - g0);
  // segment of the first candidate: the last s with s_pre[s] <= g0
  int lo = 0, hi = nseg - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_pre[mid] <= g0) lo = mid;
    else hi = mid - 1;
  }
  int seg = lo;
  uint32_t ck[kResPer];
  int32_t cj[kResPer];
#pragma unroll
  for (int u = 0; u < kResPer; ++u) {
    ck[u] = 0u;
    cj[u] = 0;
    if (u < my) {
      const int g = g0 + u;
      while (g >= s_pre[seg + 1]) ++seg;
      const uint64_t v = S.cand[(static_cast<int64_t>(row) * S.nseg + seg) * kSegCap + (g - s_pre[seg])];
      ck[u] = static_cast<uint32_t>(v >> 32);
      cj[u] = static_cast<int32_t>(v & 0xffffffffu);
    }
  }
  select_candidates<KB, kResThreads, kResPer>(ck, cj, my, S.floor[row], P.k, out, s_gt, s_eq,
                                              s_hb, s_hist, s_sel);
}

}  // namespace segsel
}  // namespace hcsa
