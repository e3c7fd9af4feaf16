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

// Prefill: many rows of at most 128K scores (BF16 or F32).  One 512-thread block per row
// streams the row from HBM once; four such blocks share a CU, so one block's loads overlap
// the others' arithmetic.  Wave w owns a contiguous run of 16-byte chunks and walks it 64
// chunks at a time, so index order is (wave, step, lane, element).  A wave64 vector
// instruction occupies its SIMD for four cycles, so each key gets only a few instructions:
//   1. the top 16 bits L of the m-th largest of up to 2048 sampled keys (the first key of
//      each lane's first four chunks; m twice the expected rank of the k-th largest key,
//      plus a margin) bound the candidates;
//   2. the streaming pass writes every key >= L (key and index) to its wave's LDS list, in
//      index order (a few percent of the row);
//   3. the exact threshold T and the selection are resolved among those candidates.
// When a wave's list overflows or the candidates fall short of k (many tied keys, a skewed
// row, an unlucky sample), T is found bit by bit over the whole row, re-read from the
// caches, and the selection is written from ballots.  Either way the result is the keys
// above T, then the lowest-index keys equal to T, in index order.
constexpr int kRowsThreads = 512;
constexpr int kRowsWaves = kRowsThreads / 64;
constexpr int kRowsMaxKeys = 131072;
constexpr int kRowsWaveCap = 512;   // candidates per wave list (four blocks share a CU)

__host__ __device__ inline bool rows_path(int rows, int N, int key_bits) {
  (void)key_bits;
  return rows >= 64 && N <= kRowsMaxKeys;
}

// Wave sum of a small non-negative int (< 2^BITS) from the ballots of its bits: scalar
// popcounts, no cross-lane data movement (a lane shuffle goes through the LDS crossbar).
template <int BITS>
__device__ __forceinline__ int wave_sum_bits(int v) {
  int t = 0;
#pragma unroll
  for (int b = 0; b < BITS; ++b) t += __popcll(__ballot((v >> b) & 1)) << b;
  return t;
}

// Exclusive prefix over the lanes (and wave total) of a small non-negative int.
template <int BITS>
__device__ __forceinline__ int wave_prefix_bits(int v, uint64_t below, int& total) {
  int pre = 0;
  total = 0;
#pragma unroll
  for (int b = 0; b < BITS; ++b) {
    const uint64_t m = __ballot((v >> b) & 1);
    pre += __popcll(m & below) << b;
    total += __popcll(m) << b;
  }
  return pre;
}

// Block-wide sum of a small non-negative int per thread; s[buf] is written, so consecutive
// calls without a barrier in between must alternate buf.
template <int BITS>
__device__ __forceinline__ int block_total_bits(int v, int (*s)[kRowsWaves], int buf) {
  const int t = wave_sum_bits<BITS>(v);
  if ((threadIdx.x & 63) == 0) s[buf][threadIdx.x >> 6] = t;
  __syncthreads();
  int r = 0;
#pragma unroll
  for (int u = 0; u < kRowsWaves; ++u) r += s[buf][u];
  return r;
}

// grid: rows; block 512.
template <int KB>
__global__ __launch_bounds__(kRowsThreads) void topk_rows_kernel(TopkDev P, int vec) {
  using KT = typename std::conditional<KB == 16, uint16_t, uint32_t>::type;
  constexpr int EPC = 16 / sizeof(KT);           // keys per 16-byte chunk
  constexpr int STEPS = kRowsWaveCap / 64;       // list entries per lane at most
  __shared__ uint32_t s_ck[kRowsWaves][kRowsWaveCap];
  __shared__ int32_t s_cj[kRowsWaves][kRowsWaveCap];
  __shared__ int s_cnt[2][kRowsWaves];
  __shared__ int s_wave[kRowsWaves], s_gt[kRowsWaves], s_eq[kRowsWaves], s_hb[kRowsWaves];
  __shared__ int s_rdx[2][kRowsWaves][3];
  const int row = blockIdx.x;
  const int nv = visible(P, row);
  int32_t* out = P.idx + static_cast<int64_t>(row) * P.k;
  if (P.k >= nv) {
    for (int j = threadIdx.x; j < P.k; j += kRowsThreads) out[j] = j < nv ? j : -1;
    return;
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint64_t below = (1ull << lane) - 1;
  const int nch = (nv + EPC - 1) / EPC;          // chunks holding visible keys
  const int CW = (nch + kRowsThreads - 1) / kRowsThreads * 64;   // chunks per wave
  const int cw0 = w * CW, cw1 = min(cw0 + CW, nch);
  const KT* rowp = reinterpret_cast<const KT*>(static_cast<const char*>(P.scores) +
                                               static_cast<int64_t>(row) * P.row_stride * sizeof(KT));
  const int nfull = vec ? min(nch, P.N / EPC) : 0;   // chunks read as one 16-byte load

  // raw bits of chunk ch < nch (elements past the visible count are never used)
  auto load_raw = [&](int ch) -> u32x4 {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (ch < nfull) {
      x = *reinterpret_cast<const u32x4*>(rowp + static_cast<int64_t>(ch) * EPC);
    } else {
      for (int e = 0; e < EPC && ch * EPC + e < nv; ++e) {
        const uint32_t v = rowp[ch * EPC + e];
        if constexpr (KB == 16)
          x[e >> 1] |= v << (16 * (e & 1));
        else
          x[e] = v;
      }
    }
    return x;
  };
  auto to_key = [&](uint32_t raw) -> uint32_t {
    if constexpr (KB == 16)
      return bf16_key(raw);
    else
      return f32_key(raw);
  };
  auto raw_of = [&](const u32x4& x, int e) -> uint32_t {
    if constexpr (KB == 16) {
      const int c = e >> 1;
      const uint32_t v = c == 0 ? x[0] : c == 1 ? x[1] : c == 2 ? x[2] : x[3];
      return (v >> (16 * (e & 1))) & 0xffffu;
    } else {
      return e == 0 ? x[0] : e == 1 ? x[1] : e == 2 ? x[2] : x[3];
    }
  };
  // bit e set when element e of a raw chunk (first index j0) is a visible key >= L.  For a
  // floor above +0 the keys >= L are exactly the non-negative raw values in
  // [raw(L), largest positive pattern], an unsigned range test on the raw bits.
  constexpr uint32_t kSign = KB == 16 ? 0x8000u : 0x80000000u;
  auto ge_mask = [&](const u32x4& x, int j0, uint32_t L) -> uint32_t {
    uint32_t m = 0;
    if (L > kSign) {
      const uint32_t lo_raw = L - kSign, span = kSign - 1 - lo_raw;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if constexpr (KB == 16) {
          m |= static_cast<uint32_t>((x[c] & 0xffffu) - lo_raw <= span) << (2 * c);
          m |= static_cast<uint32_t>((x[c] >> 16) - lo_raw <= span) << (2 * c + 1);
        } else {
          m |= static_cast<uint32_t>(x[c] - lo_raw <= span) << c;
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPC; ++e) m |= static_cast<uint32_t>(to_key(raw_of(x, e)) >= L) << e;
    }
    const int r = nv - j0;
    return r >= EPC ? m : m & ((1u << r) - 1u);
  };

  // first stream loads, in flight while the floor is chosen
  u32x4 cur[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int ch = cw0 + 64 * u + lane;
    cur[u] = ch < cw1 ? load_raw(ch) : u32x4{0u, 0u, 0u, 0u};
  }

  // ---- 1. candidate floor L from up to 2048 sampled keys: the first element of each of
  // the lane's four prefetched chunks (all keys are candidates when few)
  uint32_t L = 0;
  if (nv > kRowsWaves * kRowsWaveCap / 2) {
    bool sv[4];
    uint32_t st[4];
    int nmine = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      sv[u] = cw0 + 64 * u + lane < cw1;          // first elements are visible keys
      st[u] = sv[u] ? to_key(raw_of(cur[u], 0)) >> (KB - 16) : 0u;
      nmine += sv[u];
    }
    const int ns = block_total_bits<3>(nmine, s_cnt, 0);
    const int m = min(ns, static_cast<int>((2LL * P.k * ns + nv - 1) / nv) + 16);
    // radix-4 select of the m-th largest 16-bit prefix (a 128th of a binade: a coarser
    // floor would admit up to a whole bin of extra candidates): three thresholds a round
    uint32_t pre = 0;
#pragma unroll 1
    for (int sh = 14; sh >= 0; sh -= 2) {
      int cnt[3];
#pragma unroll
      for (int d = 1; d <= 3; ++d) {
        const uint32_t th = pre | (static_cast<uint32_t>(d) << sh);
        int n = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) n += sv[u] && st[u] >= th;
        cnt[d - 1] = wave_sum_bits<3>(n);
      }
      const int buf = (sh >> 1) & 1;
      if (lane == 0) {
        s_rdx[buf][w][0] = cnt[0];
        s_rdx[buf][w][1] = cnt[1];
        s_rdx[buf][w][2] = cnt[2];
      }
      __syncthreads();
      int tot[3] = {0, 0, 0};
#pragma unroll
      for (int u = 0; u < kRowsWaves; ++u) {
        tot[0] += s_rdx[buf][u][0];
        tot[1] += s_rdx[buf][u][1];
        tot[2] += s_rdx[buf][u][2];
      }
      const uint32_t d = tot[2] >= m ? 3u : tot[1] >= m ? 2u : tot[0] >= m ? 1u : 0u;
      pre |= d << sh;
    }
    L = ns > 0 ? pre << (KB - 16) : 0u;
  }

  // ---- 2. stream the wave's chunks 256 at a time (the next 256 loading meanwhile),
  // appending keys >= L to the wave's list
  int wslot = 0;
  for (int base = cw0; base < cw1; base += 256) {
    u32x4 nxt[4];
    const bool more = base + 256 < cw1;          // wave-uniform
    if (more) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int ch = base + 256 + 64 * u + lane;
        nxt[u] = ch < cw1 ? load_raw(ch) : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ch = base + 64 * u + lane;
      uint32_t msk = ch < cw1 ? ge_mask(cur[u], ch * EPC, L) : 0u;
      int tot;
      int o = wslot + wave_prefix_bits<4>(__popc(msk), below, tot);
      while (msk) {
        const int e = __ffs(msk) - 1;
        msk &= msk - 1;
        if (o < kRowsWaveCap) {
          s_ck[w][o] = to_key(raw_of(cur[u], e));
          s_cj[w][o] = ch * EPC + e;
        }
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
  int C = 0, before = 0;
  bool overflow = false;
#pragma unroll
  for (int u = 0; u < kRowsWaves; ++u) {
    before += u < w ? s_wave[u] : 0;
    C += s_wave[u];
    overflow |= s_wave[u] > kRowsWaveCap;
  }

  if (!overflow && C >= P.k) {
    // ---- 3. exact threshold among the candidates (lane l of wave w holds entries
    // l, l+64, ... of the wave's list); the bits above the highest one in which some
    // candidate differs from L are shared by every candidate and by T
    uint32_t ck[STEPS];
    uint32_t dor = 0;
#pragma unroll
    for (int u = 0; u < STEPS; ++u) {
      const bool in = 64 * u + lane < wslot;
      ck[u] = in ? s_ck[w][64 * u + lane] : 0u;
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
    __syncthreads();
    int nb = 0;
#pragma unroll
    for (int u = 0; u < kRowsWaves; ++u) nb = s_hb[u] > nb ? s_hb[u] : nb;
    uint32_t T = nb >= 32 ? 0u : (L >> nb) << nb;
#pragma unroll 1
    for (int b = nb - 1; b >= 0; --b) {
      const uint32_t cand = T | (1u << b);
      int n = 0;
#pragma unroll
      for (int u = 0; u < STEPS; ++u) n += (64 * u + lane < wslot) && ck[u] >= cand;
      if (block_total_bits<4>(n, s_cnt, b & 1) >= P.k) T = cand;
    }
    // per-wave counts of entries above T and equal to T
    int gt = 0, eq = 0;
#pragma unroll
    for (int u = 0; u < STEPS; ++u) {
      const bool in = 64 * u + lane < wslot;
      gt += in && ck[u] > T;
      eq += in && ck[u] == T;
    }
    gt = wave_sum_bits<4>(gt);
    eq = wave_sum_bits<4>(eq);
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
    const int need = P.k - gt_all;               // 1 <= need <= candidates equal to T
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
    return;
  }

  // ---- fallback: T bit by bit over the whole row, re-read from the caches (keys past the
  // visible count are 0 and every tested value is >= 1, so they never count), selection
  // from ballots
  uint32_t T = 0;
#pragma unroll 1
  for (int b = KB - 1; b >= 0; --b) {
    const uint32_t cand = T | (1u << b);
    int n = 0;
    for (int ch = cw0 + lane; ch < cw1; ch += 64) n += __popc(ge_mask(load_raw(ch), ch * EPC, cand));
    if (block_total_bits<9>(n, s_cnt, b & 1) >= P.k) T = cand;   // n <= 32 chunks * 8
  }
  // bits of a chunk: keys above T (gtm) and keys equal to T (eqm)
  auto gt_eq = [&](int ch, uint32_t& gtm, uint32_t& eqm) {
    const u32x4 x = load_raw(ch);
    const uint32_t ge = ge_mask(x, ch * EPC, T);
    gtm = T == 0xffffffffu ? 0u : ge_mask(x, ch * EPC, T + 1);
    eqm = ge & ~gtm;
  };
  int gt = 0, eq = 0;
  for (int ch = cw0 + lane; ch < cw1; ch += 64) {
    uint32_t gtm, eqm;
    gt_eq(ch, gtm, eqm);
    gt += __popc(gtm);
    eq += __popc(eqm);
  }
  gt = wave_sum_bits<9>(gt);
  eq = wave_sum_bits<9>(eq);
  if (lane == 0) {
    s_gt[w] = gt;
    s_eq[w] = eq;
  }
  __syncthreads();
  int gslot = 0, eq_rank = 0, gt_all = 0;
#pragma unroll
  for (int u = 0; u < kRowsWaves; ++u) {
    gslot += u < w ? s_gt[u] : 0;
    eq_rank += u < w ? s_eq[u] : 0;
    gt_all += s_gt[u];
  }
  const int need = P.k - gt_all;                 // 1 <= need <= keys equal to T
  gslot += min(need, eq_rank);
  for (int base = cw0; base < cw1; base += 64) {
    const int ch = base + lane;
    uint32_t gtm = 0, eqm = 0;
    if (ch < cw1) gt_eq(ch, gtm, eqm);
    int eq_tot;
    int r = eq_rank + wave_prefix_bits<4>(__popc(eqm), below, eq_tot);
    uint32_t sel = gtm;
    for (uint32_t m = eqm; m; m &= m - 1) {      // ties in index order while some are needed
      if (r < need) sel |= m & (~m + 1);
      ++r;
    }
    int tot;
    int o = gslot + wave_prefix_bits<4>(__popc(sel), below, tot);
    while (sel) {
      if (o < P.k) out[o] = ch * EPC + __ffs(sel) - 1;
      ++o;
      sel &= sel - 1;
    }
    gslot += tot;
    eq_rank += eq_tot;
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
  topk_rows_kernel<KB><<<plan.rows, kRowsThreads, 0, s>>>(P, vec);
  return hipGetLastError();
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
