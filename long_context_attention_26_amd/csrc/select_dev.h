// Exact top-k selection primitives on order-preserving integer keys of scores, shared by
// the selector kernels and the fused indexer-selector: wave and block counting by ballots,
// a view of one score row in 16-byte chunks, LDS histogram picks, exact selection over a
// whole row and over a candidate list.
//
// Keys are the score bits mapped to unsigned integers in the scores' order (-0 equal to +0).
// With T the k-th largest key of a row, the selection is every key above T and then the
// lowest-index keys equal to T, written in ascending index order.
#pragma once
#include "common.h"

#include <type_traits>

namespace hcsa {
namespace sel {

// ---------------------------------------------------------------- wave / block counting

// Bits that hold every value in [0, max_value]: the BITS argument of the ballot counts
// below for per-thread values bounded by max_value (a value needing more bits is counted
// wrongly, so callers derive BITS from their bound with this).
constexpr int bits_for(int max_value) {
  int b = 0;
  while (b < 31 && (1 << b) <= max_value) ++b;
  return b;
}
static_assert(bits_for(0) == 0 && bits_for(1) == 1 && bits_for(16) == 5 && bits_for(31) == 5 &&
                  bits_for(32) == 6,
              "bits_for");

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

// Block-wide sum (W waves) of a small non-negative int per thread; s[buf] is written, so
// consecutive calls without a barrier in between must alternate buf.
template <int W, int BITS>
__device__ __forceinline__ int block_total_bits(int v, int (*s)[W], int buf) {
  const int t = wave_sum_bits<BITS>(v);
  if ((threadIdx.x & 63) == 0) s[buf][threadIdx.x >> 6] = t;
  __syncthreads();
  int r = 0;
#pragma unroll
  for (int u = 0; u < W; ++u) r += s[buf][u];
  return r;
}

// ---------------------------------------------------------------- one score row

// A row of scores read in 16-byte chunks (8 BF16 or 4 F32 keys), as raw bits.
template <int KB>
struct RowView {
  using KT = typename std::conditional<KB == 16, uint16_t, uint32_t>::type;
  static constexpr int EPC = 16 / sizeof(KT);              // keys per chunk
  static constexpr uint32_t kSign = KB == 16 ? 0x8000u : 0x80000000u;
  const KT* rowp;
  int nv;        // visible keys
  int nfull;     // chunks read with one 16-byte load (the rest element by element)

  // keys p[0 .. nv_); chunks below full_chunks (16-byte aligned and in bounds) are read
  // with one load, the rest element by element
  __device__ RowView(const void* p, int nv_, int full_chunks) {
    nv = nv_;
    rowp = static_cast<const KT*>(p);
    nfull = min(nchunks(), full_chunks);
  }
  __device__ int nchunks() const { return (nv + EPC - 1) / EPC; }

  // raw bits of chunk ch < nchunks() (elements past the visible count are never used)
  __device__ u32x4 load_raw(int ch) const {
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
  }
  __device__ uint32_t key(int j) const { return to_key(rowp[j]); }
  __device__ static uint32_t to_key(uint32_t raw) {
    if constexpr (KB == 16)
      return bf16_key(raw);
    else
      return f32_key(raw);
  }
  // raw bits of element e (compile-time or run-time) of a chunk
  __device__ static uint32_t raw_of(const u32x4& x, int e) {
    if constexpr (KB == 16) {
      const int c = e >> 1;
      const uint32_t v = c == 0 ? x[0] : c == 1 ? x[1] : c == 2 ? x[2] : x[3];
      return (v >> (16 * (e & 1))) & 0xffffu;
    } else {
      return e == 0 ? x[0] : e == 1 ? x[1] : e == 2 ? x[2] : x[3];
    }
  }
  // bit e set when element e of a chunk (first index j0) is a visible key >= L.  For a
  // floor above +0 the keys >= L are exactly the non-negative raw values in
  // [raw(L), largest positive pattern], an unsigned range test on the raw bits.
  // bf16, both halves of a word at once: with H = 0x8000 in each half, (w | H) - raw(L)
  // per half cannot borrow across halves and keeps H exactly when the half's low 15 bits
  // are >= raw(L); and-ing with ~w keeps it only for non-negative raw values.  A byte
  // permute gathers the eight flags and a multiply packs them into the mask (about 16
  // instructions a chunk instead of 40).
  __device__ uint32_t ge_mask(const u32x4& x, int j0, uint32_t L) const {
    const uint32_t m = ge_bits(x, L);
    const int r = nv - j0;
    return r >= EPC ? m : m & ((1u << r) - 1u);
  }
  // the same for a chunk whose keys are all visible
  __device__ uint32_t ge_bits(const u32x4& x, uint32_t L) const {
    uint32_t m = 0;
    if (L > kSign) {
      const uint32_t lo_raw = L - kSign, span = kSign - 1 - lo_raw;
      if constexpr (KB == 16) {
        const uint32_t H = 0x80008000u, LL = lo_raw * 0x10001u;
        uint32_t cb[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) cb[c] = ((x[c] | H) - LL) & ~x[c] & H;
        // high bytes of the halves, keys 0..3 and 4..7: flags at bits 7, 15, 23, 31
        const uint32_t a = (__builtin_amdgcn_perm(cb[1], cb[0], 0x07050301u) >> 7) & 0x01010101u;
        const uint32_t b = (__builtin_amdgcn_perm(cb[3], cb[2], 0x07050301u) >> 7) & 0x01010101u;
        // one bit per byte -> four adjacent bits (bits 21..24 of the product)
        m = ((a * 0x204081u) >> 21 & 0xfu) | ((b * 0x204081u) >> 17 & 0xf0u);
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) m |= static_cast<uint32_t>(x[c] - lo_raw <= span) << c;
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPC; ++e) m |= static_cast<uint32_t>(to_key(raw_of(x, e)) >= L) << e;
    }
    return m;
  }
};

// A selected index written to the output: COH stores are agent-coherent (relaxed atomic
// stores), for outputs that other blocks of the same launch read.
template <bool COH>
__device__ __forceinline__ void put_idx(int32_t* p, int32_t v) {
  if constexpr (COH)
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}

// Rows that see at most k entries take all of them.
template <bool COH = false>
__device__ __forceinline__ void take_all(int nv, int k, int32_t* out, int nthreads) {
  for (int j = threadIdx.x; j < k; j += nthreads) put_idx<COH>(out + j, j < nv ? j : -1);
}

// One wave: the bin b (of 256) holding the m-th largest of the values counted in hist, and
// the number of values in the bins above it: out = {b, above}; b = -1 when the bins hold
// fewer than m values.  Lane l holds bins 255-4l .. 252-4l, so a prefix over the lanes runs
// from the largest bin down.
__device__ __forceinline__ void hist_pick(const int* hist, int m, int* out) {
  const int lane = threadIdx.x & 63;
  int c[4], sum = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    c[j] = hist[255 - 4 * lane - j];
    sum += c[j];
  }
  int inc = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(inc, d, kWave);
    if (lane >= d) inc += y;
  }
  const int exc = inc - sum;
  const bool here = exc < m && inc >= m;          // exactly one lane when the total >= m
  if (here) {
    int acc = exc, j = 3;
    bool found = false;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      if (!found && acc + c[jj] >= m) {
        j = jj;
        found = true;
      } else if (!found) {
        acc += c[jj];
      }
    }
    out[0] = 255 - 4 * lane - j;
    out[1] = acc;
  }
  if (lane == 63 && inc < m) {
    out[0] = -1;
    out[1] = 0;
  }
}

// Exact selection over a whole row by NT threads (the fallback of both paths): T bit by bit
// from the top (a bit stays set while at least k keys are >= the candidate value; keys past
// the visible count are masked), then every key above T and the first need = k - #(> T)
// keys equal to T, written in index order: wave w owns a contiguous run of chunks, so the
// order is (wave, step, lane, element) and ballots give each lane's output slots.
template <int KB, int NT, bool COH = false>
__device__ void select_exact_row(const RowView<KB>& V, int k, int32_t* out,
                                 int (*s_cnt)[NT / 64], int* s_gt, int* s_eq) {
  constexpr int W = NT / 64, EPC = RowView<KB>::EPC;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint64_t below = (1ull << lane) - 1;
  const int nch = V.nchunks();
  const int CW = (nch + NT - 1) / NT * 64;
  const int cw0 = w * CW, cw1 = min(cw0 + CW, nch);
  __syncthreads();                               // callers' shared counters are free again
  uint32_t T = 0;
#pragma unroll 1
  for (int b = KB - 1; b >= 0; --b) {
    const uint32_t cand = T | (1u << b);
    int n = 0;
    for (int ch = cw0 + lane; ch < cw1; ch += 64) n += __popc(V.ge_mask(V.load_raw(ch), ch * EPC, cand));
    if (block_total_bits<W, 24>(n, s_cnt, b & 1) >= k) T = cand;
  }
  // bits of a chunk: keys above T (gtm) and keys equal to T (eqm)
  auto gt_eq = [&](int ch, uint32_t& gtm, uint32_t& eqm) {
    const u32x4 x = V.load_raw(ch);
    const uint32_t ge = V.ge_mask(x, ch * EPC, T);
    gtm = T == 0xffffffffu ? 0u : V.ge_mask(x, ch * EPC, T + 1);
    eqm = ge & ~gtm;
  };
  int gt = 0, eq = 0;
  for (int ch = cw0 + lane; ch < cw1; ch += 64) {
    uint32_t gtm, eqm;
    gt_eq(ch, gtm, eqm);
    gt += __popc(gtm);
    eq += __popc(eqm);
  }
  gt = wave_sum_bits<24>(gt);
  eq = wave_sum_bits<24>(eq);
  if (lane == 0) {
    s_gt[w] = gt;
    s_eq[w] = eq;
  }
  __syncthreads();
  int slot = 0, eq_rank = 0, gt_all = 0;
#pragma unroll
  for (int u = 0; u < W; ++u) {
    slot += u < w ? s_gt[u] : 0;
    eq_rank += u < w ? s_eq[u] : 0;
    gt_all += s_gt[u];
  }
  const int need = k - gt_all;                   // 1 <= need <= keys equal to T
  slot += min(need, eq_rank);
  constexpr int CB = bits_for(EPC);              // a chunk's keys above / equal to T
  for (int base = cw0; base < cw1; base += 64) {
    const int ch = base + lane;
    uint32_t gtm = 0, eqm = 0;
    if (ch < cw1) gt_eq(ch, gtm, eqm);
    int eq_tot;
    int r = eq_rank + wave_prefix_bits<CB>(__popc(eqm), below, eq_tot);
    uint32_t sel = gtm;
    for (uint32_t m = eqm; m; m &= m - 1) {      // ties in index order while some are needed
      if (r < need) sel |= m & (~m + 1);
      ++r;
    }
    int tot;
    int o = slot + wave_prefix_bits<CB>(__popc(sel), below, tot);
    while (sel) {
      if (o < k) put_idx<COH>(out + o, ch * EPC + __ffs(sel) - 1);
      ++o;
      sel &= sel - 1;
    }
    slot += tot;
    eq_rank += eq_tot;
  }
}

// Exact selection among candidates (all >= L) held by NT threads in order: thread t holds
// the candidates [t*per, t*per + cnt_t) of the list (keys ck, indices cj, cnt_t <= PER).
// The bits of T above the highest one in which some candidate differs from L (bit nb - 1)
// are shared by every candidate and by T; the bits below are found 8 at a time from bit
// nb - 1 down, each pass an LDS histogram of the digit over the candidates that match T so
// far (two passes for BF16 keys, at most four for F32).  Digits taken from the top of the
// differing bits spread the candidates over the bins; digits aligned to bytes would pile
// them into the few bins of their common exponent, and LDS atomics on one address
// serialise.
template <int KB, int NT, int PER, bool COH = false>
__device__ void select_candidates(const uint32_t (&ck)[PER], const int32_t (&cj)[PER], int cnt,
                                  uint32_t L, int k, int32_t* out, int* s_gt, int* s_eq,
                                  int* s_hb, int (*s_hist)[256], int* s_sel) {
  constexpr int W = NT / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint64_t below = (1ull << lane) - 1;
  uint32_t dor = 0;
#pragma unroll
  for (int u = 0; u < PER; ++u) dor |= u < cnt ? (ck[u] ^ L) : 0u;
  int hb = 0;
  for (int b = KB - 1; b >= 0; --b) {
    if (__ballot((dor >> b) & 1u)) {
      hb = b + 1;
      break;
    }
  }
  if (lane == 0) s_hb[w] = hb;
  for (int i = threadIdx.x; i < 512; i += NT) s_hist[i >> 8][i & 255] = 0;
  __syncthreads();
  int nb = 0;
#pragma unroll
  for (int u = 0; u < W; ++u) nb = s_hb[u] > nb ? s_hb[u] : nb;
  const int D = (nb + 7) / 8;
  uint32_t T = nb >= 32 ? 0u : (L >> nb) << nb;
  int rem = k;                                   // rank of T among the candidates still open
#pragma unroll 1
  for (int p = 0; p < D; ++p) {
    const int top = nb - 8 * p;                  // this pass: bits [sh, top)
    const int sh = top > 8 ? top - 8 : 0;
    const uint32_t dmask = (1u << (top - sh)) - 1u;
    int* hist = s_hist[p & 1];
    const uint32_t hi = top >= 32 ? 0u : T >> top;
#pragma unroll
    for (int u = 0; u < PER; ++u)
      if (u < cnt && (top >= 32 || (ck[u] >> top) == hi))
        atomicAdd(&hist[(ck[u] >> sh) & dmask], 1);
    if (p >= 1)                                  // the previous pass's bins, read already
      for (int i = threadIdx.x; i < 256; i += NT) s_hist[(p + 1) & 1][i] = 0;
    __syncthreads();
    if (w == 0) hist_pick(hist, rem, s_sel);
    __syncthreads();
    // every thread reads s_sel before it reaches the next pass's first barrier, and the
    // next pick comes after that barrier
    T |= static_cast<uint32_t>(s_sel[0]) << sh;
    rem -= s_sel[1];
  }
  int gt = 0, eq = 0;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    gt += u < cnt && ck[u] > T;
    eq += u < cnt && ck[u] == T;
  }
  // a thread holds up to PER candidates, so its counts need bits_for(PER) bits (6 for 32)
  constexpr int CB = bits_for(PER);
  int gt_w, eq_w;
  const int gt_pre = wave_prefix_bits<CB>(gt, below, gt_w);
  const int eq_pre = wave_prefix_bits<CB>(eq, below, eq_w);
  if (lane == 0) {
    s_gt[w] = gt_w;
    s_eq[w] = eq_w;
  }
  __syncthreads();
  int gt_before = gt_pre, eq_rank = eq_pre, gt_all = 0;
#pragma unroll
  for (int u = 0; u < W; ++u) {
    gt_before += u < w ? s_gt[u] : 0;
    eq_rank += u < w ? s_eq[u] : 0;
    gt_all += s_gt[u];
  }
  const int need = k - gt_all;                   // 1 <= need <= candidates equal to T
  int o = gt_before + min(need, eq_rank);
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    if (u < cnt) {
      const bool sel = ck[u] > T || (ck[u] == T && eq_rank < need);
      eq_rank += ck[u] == T;
      if (sel) {
        if (o < k) put_idx<COH>(out + o, cj[u]);
        ++o;
      }
    }
  }
}

}  // namespace sel
}  // namespace hcsa
