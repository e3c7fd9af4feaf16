// Top-k selector: exact and deterministic, on order-preserving integer keys of the scores.
//
// The indexer keeps the top-k compressed entries of each query (Lighthouse, "deep
// deepseek v4 release", section 八 item 3; k = 1024 Pro / 512 Flash); BF16 scores make the
// selector cheaper (9fzt.com digest, item 4).  Ties go to the lowest index and the output
// is ascending, the reading taken where the pages are silent.
//
// After a 12-bit histogram of every row's keys (built by the indexer kernel itself, or by
// topk_hist_kernel for caller-given scores; block i of a row adds into replica i % copies):
//   b0       one block per row sums the replicas and finds the bin b0 holding the row's
//            k-th largest key.
//   extract  many blocks per row: every key in bins >= b0 is appended to a replica's
//            candidate list (one atomic per block reserves its slots; list order does not
//            matter).  Typically about k + |bin b0| candidates.
//   resolve  one block per row: with the candidates in LDS, the remaining key bits give
//            the exact threshold key T and how many T-valued entries to keep; ties keep the
//            lowest indices (each tie's rank among the ties is counted); the k selected
//            indices are written in ascending order by a counting sort on their top 10 bits
//            and a rank count inside each bucket.  A row whose candidates exceed the
//            list capacity (massive ties) is resolved exactly from its full score row
//            instead, with an ordered compaction.
// Every step is integer-only, so the result does not depend on scheduling.
#include "common.h"
#include "internal.h"
#include "select_common.h"

#include <algorithm>

namespace hcsa {

namespace {

constexpr int kBins = kSelBins;    // 12-bit first digit
constexpr int kCap = kSelCap;      // candidates kept per row (over all replicas)
constexpr int kExtractChunk = 8192;

struct TopkDev {
  const void* scores;
  int64_t row_stride;
  int Nq, N, ratio, k;
  int64_t pos0;
  SelState S;
  int32_t* idx;         // [rows][k]
};

template <int KB>
__device__ __forceinline__ uint32_t key_at(const TopkDev& P, int row, int j) {
  if constexpr (KB == 16)
    return bf16_key(static_cast<const uint16_t*>(P.scores)[row * P.row_stride + j]);
  else
    return f32_key(static_cast<const uint32_t*>(P.scores)[row * P.row_stride + j]);
}

__device__ __forceinline__ int visible(const TopkDev& P, int row) {
  const int64_t p = P.pos0 + (row % P.Nq);
  const int64_t v = (p + 1) / P.ratio;
  return static_cast<int>(v < P.N ? v : P.N);
}

// Exclusive prefix of one int per thread over 256 threads (thread order).
__device__ __forceinline__ int block_scan_256(int v, int* s_w, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += t;
  }
  if (lane == kWave - 1) s_w[w] = incl;
  __syncthreads();
  int before = 0;
  for (int i = 0; i < w; ++i) before += s_w[i];
  total = s_w[0] + s_w[1] + s_w[2] + s_w[3];
  __syncthreads();
  return before + incl - v;
}

// ---------------------------------------------------------------- histogram of given scores

// grid: (ceil(N / kExtractChunk), rows); block 256; 32 keys per thread.
template <int KB>
__global__ __launch_bounds__(256) void topk_hist_kernel(TopkDev P) {
  __shared__ uint32_t h[kBins];
  const int row = blockIdx.y;
  const int nv = visible(P, row);
  if (P.k >= nv) return;
  const int start = blockIdx.x * kExtractChunk;
  const int end = min(start + kExtractChunk, nv);
  if (start >= end) return;
  for (int i = threadIdx.x; i < kBins; i += 256) h[i] = 0;
  uint32_t key[32];
#pragma unroll
  for (int u = 0; u < 32; ++u) {
    const int j = start + threadIdx.x + 256 * u;
    key[u] = j < end ? key_at<KB>(P, row, j) : 0u;
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 32; ++u)
    if (start + static_cast<int>(threadIdx.x) + 256 * u < end) atomicAdd(&h[key[u] >> (KB - 12)], 1u);
  __syncthreads();
  uint32_t* hrow = sel_hist_row(P.S, blockIdx.x % P.S.copies, row);
  for (int i = threadIdx.x; i < kBins; i += 256)
    if (h[i]) atomicAdd(&hrow[i], h[i]);
}

// ---------------------------------------------------------------- threshold bin per row

// grid: rows; block 256.  Sums the replicas and finds the 12-bit bin b0 holding the k-th
// largest key: count(bins > b0) < k <= count(bins >= b0).  Thread t owns the 16 bins
// 4095-16t .. 4080-16t (thread 0 the top ones).
__global__ __launch_bounds__(256) void topk_b0_kernel(TopkDev P) {
  __shared__ int s_w[4];
  const int row = blockIdx.x;
  const int nv = visible(P, row);
  if (P.k >= nv) return;
  const int lo = kBins - 16 * (threadIdx.x + 1);
  uint32_t v[16];
#pragma unroll
  for (int b = 0; b < 16; ++b) v[b] = 0;
  for (int c = 0; c < P.S.copies; ++c) {
    const u32x4* h4 = reinterpret_cast<const u32x4*>(sel_hist_row(P.S, c, row) + lo);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 x = h4[q];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * q + e] += x[e];
    }
  }
  int sum = 0;
#pragma unroll
  for (int b = 0; b < 16; ++b) sum += static_cast<int>(v[b]);
  int total;
  int above = block_scan_256(sum, s_w, total);
  if (above < P.k && above + sum >= P.k) {
    for (int b = 15; b >= 0; --b) {
      if (above + static_cast<int>(v[b]) >= P.k) {
        P.S.b0info[2 * row] = lo + b;
        P.S.b0info[2 * row + 1] = above;
        break;
      }
      above += static_cast<int>(v[b]);
    }
  }
}

// ---------------------------------------------------------------- extract candidates

// grid: (ceil(N / kExtractChunk), rows); block 256; 32 keys per thread.  One atomic per
// block (on its replica's counter) reserves the block's slots in the replica's list.
template <int KB>
__global__ __launch_bounds__(256) void topk_extract_kernel(TopkDev P) {
  __shared__ int s_w[4];
  __shared__ uint32_t s_base;
  const int row = blockIdx.y;
  const int nv = visible(P, row);
  if (P.k >= nv) return;
  const int start = blockIdx.x * kExtractChunk;
  const int end = min(start + kExtractChunk, nv);
  if (start >= end) return;
  uint32_t key[32];
#pragma unroll
  for (int u = 0; u < 32; ++u) {
    const int j = start + threadIdx.x + 256 * u;
    key[u] = j < end ? key_at<KB>(P, row, j) : 0u;
  }
  const uint32_t b0 = static_cast<uint32_t>(P.S.b0info[2 * row]);
  uint32_t mask = 0;
#pragma unroll
  for (int u = 0; u < 32; ++u) {
    const int j = start + threadIdx.x + 256 * u;
    if (j < end && (key[u] >> (KB - 12)) >= b0) mask |= 1u << u;
  }
  int total;
  const int before = block_scan_256(__popc(mask), s_w, total);
  const int copy = blockIdx.x % P.S.copies;
  if (threadIdx.x == 0)
    s_base = total ? atomicAdd(&P.S.cnt[copy * P.S.rows + row], static_cast<uint32_t>(total)) : 0u;
  __syncthreads();
  uint32_t slot = s_base + before;
  uint64_t* cand = P.S.cand + (static_cast<int64_t>(row) * P.S.copies + copy) * P.S.capc;
#pragma unroll
  for (int u = 0; u < 32; ++u) {
    if (mask & (1u << u)) {
      if (slot < static_cast<uint32_t>(P.S.capc)) {
        const uint32_t inv = KB == 16 ? (0xFFFFu - key[u]) : ~key[u];
        cand[slot] = (static_cast<uint64_t>(inv) << 32) |
                     static_cast<uint32_t>(start + threadIdx.x + 256 * u);
      }
      ++slot;
    }
  }
}

// ---------------------------------------------------------------- resolve one row

constexpr int kResolveThreads = 1024;

__device__ __forceinline__ int block_sum_1024(int v, int* s_red) {
  v = wave_sum_i(v);
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int i = 0; i < kResolveThreads / 64; ++i) t += s_red[i];
  __syncthreads();
  return t;
}

// Exclusive prefix of one int per thread over 1024 threads (thread order).
__device__ __forceinline__ int block_scan_1024(int v, int* s_w, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += t;
  }
  if (lane == kWave - 1) s_w[w] = incl;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < kResolveThreads / 64; ++i) {
    before += i < w ? s_w[i] : 0;
    total += s_w[i];
  }
  __syncthreads();
  return before + incl - v;
}

// Radix over the bits below the 12-bit digit: finds the exact threshold key T and the number
// `need` of T-valued keys to keep, given that `krem` keys must still be taken from bin b0.
// `get(i)` returns the key of element i of a list of n elements (keys outside bin b0 do not
// count).
template <int KB, typename Get>
__device__ void resolve_threshold(Get get, int n, uint32_t b0, int krem, uint32_t* s_h,
                                  uint32_t* s_T, int* s_need) {
  constexpr int LOW = KB - 12;                    // 4 (bf16) or 20 (fp32)
  constexpr int DIG = LOW > 10 ? 10 : LOW;        // digit width
  uint32_t prefix = b0;
  int have = LOW;
  while (have > 0) {
    const int dw = have < DIG ? have : DIG;
    const int nb = 1 << dw;
    for (int i = threadIdx.x; i < nb; i += kResolveThreads) s_h[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += kResolveThreads) {
      const uint32_t key = get(i);
      if ((key >> have) == prefix) atomicAdd(&s_h[(key >> (have - dw)) & (nb - 1)], 1u);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      int cum = 0;
      for (int d = nb - 1; d >= 0; --d) {
        const int c = static_cast<int>(s_h[d]);
        if (cum + c >= krem) {
          *s_T = (prefix << dw) | static_cast<uint32_t>(d);
          *s_need = krem - cum;
          break;
        }
        cum += c;
      }
    }
    __syncthreads();
    prefix = *s_T;
    krem = *s_need;
    have -= dw;
    __syncthreads();
  }
}

// Pads an LDS list of n indices with never-smaller sentinels up to a multiple of 4.
__device__ __forceinline__ void pad4(uint32_t* a, int n) {
  if (threadIdx.x < 4 && n + static_cast<int>(threadIdx.x) < ((n + 3) & ~3))
    a[n + threadIdx.x] = 0xFFFFFFFFu;
}

// Number of entries of the LDS list a[0..n) (padded to a multiple of 4) below j; 16-byte
// broadcast reads and independent partial counts keep the loop issue-bound.
__device__ __forceinline__ int count_below(const uint32_t* a, int n, uint32_t j) {
  const u32x4* v = reinterpret_cast<const u32x4*>(a);
  const int n4 = (n + 3) >> 2;
  int c0 = 0, c1 = 0, c2 = 0, c3 = 0;
  int m = 0;
  for (; m + 1 < n4; m += 2) {
    const u32x4 x = v[m], y = v[m + 1];
    c0 += (x[0] < j) + (y[0] < j);
    c1 += (x[1] < j) + (y[1] < j);
    c2 += (x[2] < j) + (y[2] < j);
    c3 += (x[3] < j) + (y[3] < j);
  }
  if (m < n4) {
    const u32x4 x = v[m];
    c0 += x[0] < j;
    c1 += x[1] < j;
    c2 += x[2] < j;
    c3 += x[3] < j;
  }
  return c0 + c1 + c2 + c3;
}

// grid: rows; block 1024.
template <int KB>
__global__ __launch_bounds__(kResolveThreads) void topk_resolve_kernel(TopkDev P) {
  __shared__ __align__(16) uint32_t s_key[kCap];
  __shared__ __align__(16) uint32_t s_j[kCap];
  __shared__ __align__(16) uint32_t s_tie[kCap + 4];
  __shared__ __align__(16) uint32_t s_sel[4096 + 4];
  __shared__ uint32_t s_h[1024];
  __shared__ uint32_t s_bcnt[1024];
  __shared__ uint32_t s_bstart[1024];
  __shared__ int s_red[kResolveThreads / 64];
  __shared__ int s_need, s_nsel, s_ntie;
  __shared__ uint32_t s_T;
  const int row = blockIdx.x;
  const int nv = visible(P, row);
  int32_t* out = P.idx + static_cast<int64_t>(row) * P.k;
  if (P.k >= nv) {
    for (int j = threadIdx.x; j < P.k; j += kResolveThreads) out[j] = j < nv ? j : -1;
    return;
  }
  const uint32_t b0 = static_cast<uint32_t>(P.S.b0info[2 * row]);
  const int krem = P.k - P.S.b0info[2 * row + 1];
  int C = 0;
  bool overflow = false;
  for (int c = 0; c < P.S.copies; ++c) {
    const int n = static_cast<int>(P.S.cnt[c * P.S.rows + row]);
    overflow |= n > P.S.capc;
    C += n;
  }

  if (!overflow) {
    // ---- candidates of every replica into LDS: keys and indices
    int off = 0;
    for (int c = 0; c < P.S.copies; ++c) {
      const int n = static_cast<int>(P.S.cnt[c * P.S.rows + row]);
      const uint64_t* cand = P.S.cand + (static_cast<int64_t>(row) * P.S.copies + c) * P.S.capc;
      for (int i = threadIdx.x; i < n; i += kResolveThreads) {
        const uint64_t x = cand[i];
        const uint32_t inv = static_cast<uint32_t>(x >> 32);
        s_key[off + i] = KB == 16 ? (0xFFFFu - inv) : ~inv;
        s_j[off + i] = static_cast<uint32_t>(x);
      }
      off += n;
    }
    if (threadIdx.x == 0) {
      s_nsel = 0;
      s_ntie = 0;
    }
    __syncthreads();
    auto key_of = [&](int i) -> uint32_t { return s_key[i]; };
    resolve_threshold<KB>(key_of, C, b0, krem, s_h, &s_T, &s_need);
    const uint32_t T = s_T;
    const int need = s_need;
    // keys above T are selected; T-valued ones go to the tie list
    for (int i = threadIdx.x; i < C; i += kResolveThreads) {
      const uint32_t key = s_key[i];
      if (key > T) s_sel[atomicAdd(&s_nsel, 1) & 4095] = s_j[i];
      else if (key == T) s_tie[atomicAdd(&s_ntie, 1)] = s_j[i];
    }
    __syncthreads();
    const int E = s_ntie;
    pad4(s_tie, E);
    __syncthreads();
    // the `need` lowest indices among the ties
    for (int i = threadIdx.x; i < E; i += kResolveThreads) {
      const uint32_t j = s_tie[i];
      if (E == need || count_below(s_tie, E, j) < need) s_sel[atomicAdd(&s_nsel, 1) & 4095] = j;
    }
    __syncthreads();
    const int ns = min(s_nsel, P.k);
    // ascending output: counting sort on the top (up to) 10 bits of the index, then each
    // index's rank inside its bucket
    const int bits = 32 - __clz(max(nv - 1, 1));
    const int shift = bits > 10 ? bits - 10 : 0;
    s_bcnt[threadIdx.x] = 0;
    s_h[threadIdx.x] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < ns; i += kResolveThreads) atomicAdd(&s_bcnt[s_sel[i] >> shift], 1u);
    __syncthreads();
    int tot;
    const uint32_t cnt_b = s_bcnt[threadIdx.x];
    s_bstart[threadIdx.x] = block_scan_1024(static_cast<int>(cnt_b), s_red, tot);
    __syncthreads();
    for (int i = threadIdx.x; i < ns; i += kResolveThreads) {
      const uint32_t j = s_sel[i];
      const uint32_t b = j >> shift;
      s_tie[s_bstart[b] + atomicAdd(&s_h[b], 1u)] = j;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < ns; i += kResolveThreads) {
      const uint32_t j = s_tie[i];
      const uint32_t b = j >> shift;
      const int st = static_cast<int>(s_bstart[b]);
      const int n = static_cast<int>(s_bcnt[b]);
      int rank = 0;
      for (int m = st; m < st + n; ++m) rank += s_tie[m] < j;
      out[st + rank] = static_cast<int32_t>(j);
    }
    return;
  }

  // ---- too many candidates: exact resolution from the full score row
  auto key_row = [&](int j) -> uint32_t { return key_at<KB>(P, row, j); };
  resolve_threshold<KB>(key_row, nv, b0, krem, s_h, &s_T, &s_need);
  const uint32_t T = s_T;
  const int need = s_need;
  int sel_before = 0, eq_before = 0;
  for (int base = 0; base < nv; base += kResolveThreads) {
    const int j = base + threadIdx.x;
    const uint32_t key = j < nv ? key_row(j) : 0u;
    const bool gt = j < nv && key > T;
    const bool eq = j < nv && key == T;
    int tot;
    const int er = eq_before + block_scan_1024(eq, s_red, tot);
    eq_before += tot;
    const bool sel = gt || (eq && er < need);
    const int slot = sel_before + block_scan_1024(sel, s_red, tot);
    sel_before += tot;
    if (sel && slot < P.k) out[slot] = j;
  }
}

// ---------------------------------------------------------------- many rows: one block per row

// Prefill: many rows of at most 72K BF16 (64K F32) scores.  One 1024-thread block per row
// keeps the row's keys in registers: wave w owns a contiguous span of 64*NCH 16-byte chunks
// and lane l holds chunk 64*i + l of it (coalesced loads), so key order is (wave, i, lane,
// element).  The threshold key T (the k-th largest) is found bit by bit from the top: a
// candidate bit stays set when at least k keys are >= the candidate, each step one block
// count.  Keys past the visible count are zeroed, and no candidate is 0, so they never
// count.  The selection (keys above T, then the lowest-index keys equal to T) is written in
// index order from ballots.  No shared-memory atomics: prefill scores crowd a few values
// (many are exactly 0), which would serialize a histogram.
constexpr int kRowsThreads = 1024;
constexpr int kRowsMaxBf16 = 73728, kRowsMaxF32 = 65536;   // 9 (16) chunks per thread

__host__ __device__ inline bool rows_path(int rows, int N, int key_bits) {
  return rows >= 64 && N <= (key_bits == 16 ? kRowsMaxBf16 : kRowsMaxF32);
}

template <int KB, int NCH>
__global__ __launch_bounds__(kRowsThreads) void topk_rows_kernel(TopkDev P, int vec) {
  constexpr int EPC = KB == 16 ? 8 : 4;          // keys per 16-byte chunk
  constexpr int kWaves = kRowsThreads / 64;
  __shared__ int s_cnt[2][kWaves];
  __shared__ int s_gt[kWaves], s_eq[kWaves];
  const int row = blockIdx.x;
  const int nv = visible(P, row);
  int32_t* out = P.idx + static_cast<int64_t>(row) * P.k;
  if (P.k >= nv) {
    for (int j = threadIdx.x; j < P.k; j += kRowsThreads) out[j] = j < nv ? j : -1;
    return;
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;

  // ---- keys of this lane's chunks
  const int cbase = w * 64 * NCH + lane;
  const char* rowp = static_cast<const char*>(P.scores) +
                     static_cast<int64_t>(row) * P.row_stride * (KB / 8);
  u32x4 kv[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int j0 = (cbase + 64 * i) * EPC;
    if (vec && j0 < nv && j0 + EPC <= P.N)
      kv[i] = *reinterpret_cast<const u32x4*>(rowp + static_cast<int64_t>(j0) * (KB / 8));
    else
      kv[i] = u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int i = 0; i < NCH; ++i) {                // unaligned rows, or the allocation's tail
    const int j0 = (cbase + 64 * i) * EPC;
    if (j0 < nv && !(vec && j0 + EPC <= P.N)) {
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        if (j0 + e < nv) {
          if constexpr (KB == 16) {
            const uint32_t h = reinterpret_cast<const uint16_t*>(rowp)[j0 + e];
            kv[i][e >> 1] |= h << (16 * (e & 1));
          } else {
            kv[i][e] = reinterpret_cast<const uint32_t*>(rowp)[j0 + e];
          }
        }
      }
    }
  }
  auto nvalid = [&](int i) -> int {
    const int r = nv - (cbase + 64 * i) * EPC;
    return r < 0 ? 0 : (r > EPC ? EPC : r);
  };
  // order-preserving keys; 0 past the visible count
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int nvl = nvalid(i);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t x = kv[i][c];
      if constexpr (KB == 16) {
        const uint32_t lo = 2 * c < nvl ? bf16_key(x & 0xffffu) : 0u;
        const uint32_t hi = 2 * c + 1 < nvl ? bf16_key(x >> 16) : 0u;
        kv[i][c] = lo | (hi << 16);
      } else {
        kv[i][c] = c < nvl ? f32_key(x) : 0u;
      }
    }
  }
  auto key = [&](int i, int e) -> uint32_t {
    if constexpr (KB == 16)
      return (kv[i][e >> 1] >> (16 * (e & 1))) & 0xffffu;
    else
      return kv[i][e];
  };

  // ---- T: the largest value with at least k keys >= T
  uint32_t T = 0;
#pragma unroll 1
  for (int b = KB - 1; b >= 0; --b) {
    const uint32_t cand = T | (1u << b);
    int c = 0;
#pragma unroll
    for (int i = 0; i < NCH; ++i)
#pragma unroll
      for (int e = 0; e < EPC; ++e) c += key(i, e) >= cand;
    c = wave_sum_i(c);
    if (lane == 0) s_cnt[b & 1][w] = c;
    __syncthreads();
    int tot = 0;
#pragma unroll
    for (int u = 0; u < kWaves; ++u) tot += s_cnt[b & 1][u];
    if (tot >= P.k) T = cand;
  }

  // ---- selection in index order: keys above T, and the first `need` keys equal to T
  int gt = 0, eq = 0;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int nvl = nvalid(i);
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      const uint32_t kk = key(i, e);
      gt += kk > T;
      eq += e < nvl && kk == T;
    }
  }
  gt = wave_sum_i(gt);
  eq = wave_sum_i(eq);
  if (lane == 0) {
    s_gt[w] = gt;
    s_eq[w] = eq;
  }
  __syncthreads();
  int slot = 0, eq_rank = 0, gt_all = 0;
#pragma unroll
  for (int u = 0; u < kWaves; ++u) {
    slot += u < w ? s_gt[u] : 0;
    eq_rank += u < w ? s_eq[u] : 0;
    gt_all += s_gt[u];
  }
  const int need = P.k - gt_all;                 // 1 <= need <= keys equal to T
  slot += min(need, eq_rank);
  const uint64_t below = (1ull << lane) - 1;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int nvl = nvalid(i);
    const int jc = (cbase + 64 * i) * EPC;
    // T-valued keys of the lanes before this one (and of this wave's chunk in total)
    int eq_before = 0, eq_all = 0;
    bool is_eq[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      is_eq[e] = e < nvl && key(i, e) == T;
      const uint64_t m = __ballot(is_eq[e]);
      eq_before += __popcll(m & below);
      eq_all += __popcll(m);
    }
    int r = eq_rank + eq_before;
    bool sel[EPC];
    int sel_before = 0, sel_all = 0;
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      sel[e] = key(i, e) > T || (is_eq[e] && r < need);
      r += is_eq[e];
      const uint64_t m = __ballot(sel[e]);
      sel_before += __popcll(m & below);
      sel_all += __popcll(m);
    }
    int o = slot + sel_before;
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      if (sel[e]) {
        if (o < P.k) out[o] = jc + e;
        ++o;
      }
    }
    slot += sel_all;
    eq_rank += eq_all;
  }
}

__global__ void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v) {
  for (int64_t i = blockIdx.x * 256LL + threadIdx.x; i < n; i += 256LL * gridDim.x) p[i] = v;
}

}  // namespace

static size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

TopkPlan plan_topk(int score_dtype, int rows, int N, int k) {
  TopkPlan p{};
  p.rows = rows;
  p.N = N;
  p.k = k;
  p.key_bits = score_dtype == 1 ? 16 : 32;
  p.chunk = kExtractChunk;
  p.nchunks = N > 0 ? (N + p.chunk - 1) / p.chunk : 1;
  p.copies = sel_copies(rows, N);
  if (rows_path(rows, N, p.key_bits)) {
    p.hist_bytes = p.count_bytes = 0;     // one block per row, all state in LDS
  } else {
    p.hist_bytes = align256(sel_words(rows, p.copies) * 4);               // selector words
    p.count_bytes = align256(static_cast<size_t>(rows) * kCap * 8);       // candidates
  }
  p.total_bytes = p.hist_bytes + p.count_bytes;
  return p;
}

SelState topk_sel_state(const TopkPlan& plan, void* ws) {
  return sel_state(ws, plan.rows, plan.copies, plan.hist_bytes);
}

template <int KB>
static hipError_t launch_rows_kb(const TopkPlan& plan, const TopkDev& P, int vec, hipStream_t s) {
  constexpr int EPC = KB == 16 ? 8 : 4;
  const int per = (plan.N + kRowsThreads * EPC - 1) / (kRowsThreads * EPC);   // chunks / thread
#define HCSA_ROWS(n) \
  if (per <= n) { topk_rows_kernel<KB, n><<<plan.rows, kRowsThreads, 0, s>>>(P, vec); return hipGetLastError(); }
  // BF16 keys are unpacked for comparison, so their register budget ends at 9 chunks
  HCSA_ROWS(2) HCSA_ROWS(4) HCSA_ROWS(6) HCSA_ROWS(9)
  if constexpr (KB == 32) { HCSA_ROWS(12) HCSA_ROWS(16) }
#undef HCSA_ROWS
  return hipErrorInvalidValue;
}

static hipError_t launch_topk_rows(const TopkPlan& plan, const void* scores,
                                   int64_t row_stride, int Nq, int ratio, int64_t pos0,
                                   int32_t* idx, hipStream_t s) {
  TopkDev P{};
  P.scores = scores;
  P.row_stride = row_stride;
  P.Nq = Nq;
  P.N = plan.N;
  P.ratio = ratio;
  P.k = plan.k;
  P.pos0 = pos0;
  P.idx = idx;
  const int esz = plan.key_bits / 8;
  const int vec = (reinterpret_cast<uintptr_t>(scores) % 16 == 0) && (row_stride * esz) % 16 == 0;
  return plan.key_bits == 16 ? launch_rows_kb<16>(plan, P, vec, s)
                             : launch_rows_kb<32>(plan, P, vec, s);
}

bool topk_uses_rows_path(const TopkPlan& plan) { return rows_path(plan.rows, plan.N, plan.key_bits); }

hipError_t launch_topk_clear(const TopkPlan& plan, void* ws, hipStream_t s) {
  if (rows_path(plan.rows, plan.N, plan.key_bits)) return hipSuccess;   // no shared state
  const int64_t words = static_cast<int64_t>(sel_words(plan.rows, plan.copies));
  const int blocks = static_cast<int>(std::min<int64_t>((words + 255) / 256, 4096));
  fill_u32_kernel<<<blocks, 256, 0, s>>>(static_cast<uint32_t*>(ws), words, 0u);
  return hipGetLastError();
}

hipError_t launch_topk_select(const TopkPlan& plan, const void* scores, int64_t row_stride,
                              int Nq, int ratio, int64_t pos0, int32_t* idx, void* ws,
                              bool need_hist, hipStream_t s) {
  if (rows_path(plan.rows, plan.N, plan.key_bits))
    return launch_topk_rows(plan, scores, row_stride, Nq, ratio, pos0, idx, s);
  TopkDev P;
  P.scores = scores;
  P.row_stride = row_stride;
  P.Nq = Nq;
  P.N = plan.N;
  P.ratio = ratio;
  P.k = plan.k;
  P.pos0 = pos0;
  P.S = topk_sel_state(plan, ws);
  P.idx = idx;
  const dim3 grid(plan.nchunks, plan.rows);
  if (plan.key_bits == 16) {
    if (need_hist) topk_hist_kernel<16><<<grid, 256, 0, s>>>(P);
    topk_b0_kernel<<<plan.rows, 256, 0, s>>>(P);
    topk_extract_kernel<16><<<grid, 256, 0, s>>>(P);
    topk_resolve_kernel<16><<<plan.rows, kResolveThreads, 0, s>>>(P);
  } else {
    if (need_hist) topk_hist_kernel<32><<<grid, 256, 0, s>>>(P);
    topk_b0_kernel<<<plan.rows, 256, 0, s>>>(P);
    topk_extract_kernel<32><<<grid, 256, 0, s>>>(P);
    topk_resolve_kernel<32><<<plan.rows, kResolveThreads, 0, s>>>(P);
  }
  return hipGetLastError();
}

hipError_t launch_sel_hist(const void* scores, int score_dtype, int64_t row_stride, int B,
                           int Nq, int N, int ratio, int64_t pos0, int k, void* ws,
                           hipStream_t s) {
  const TopkPlan plan = plan_topk(score_dtype, B * Nq, N, k);
  if (rows_path(plan.rows, plan.N, plan.key_bits)) return hipSuccess;   // not needed
  TopkDev P;
  P.scores = scores;
  P.row_stride = row_stride;
  P.Nq = Nq;
  P.N = N;
  P.ratio = ratio;
  P.k = k;
  P.pos0 = pos0;
  P.S = topk_sel_state(plan, ws);
  P.idx = nullptr;
  const dim3 grid(plan.nchunks, plan.rows);
  if (plan.key_bits == 16) topk_hist_kernel<16><<<grid, 256, 0, s>>>(P);
  else topk_hist_kernel<32><<<grid, 256, 0, s>>>(P);
  return hipGetLastError();
}

hipError_t launch_topk(const TopkPlan& plan, const void* scores, int score_dtype,
                       int64_t row_stride, int Nq, int ratio, int64_t pos0, int32_t* idx,
                       void* ws, hipStream_t s) {
  (void)score_dtype;
  if (rows_path(plan.rows, plan.N, plan.key_bits))
    return launch_topk_rows(plan, scores, row_stride, Nq, ratio, pos0, idx, s);
  hipError_t e = launch_topk_clear(plan, ws, s);
  if (e != hipSuccess) return e;
  return launch_topk_select(plan, scores, row_stride, Nq, ratio, pos0, idx, ws, true, s);
}

}  // namespace hcsa
