// Device code of the lightning indexer on MXFP4 keys, shared by the indexer kernels and the
// decode-step launches: the operands of the scaled fp4 matrix-core product, the per-row
// selection floor from scored samples and the exact selection among the scan's candidate
// lists (with its rescan fallback).
//
// The indexer scores compressed entries with its own compressed keys on a low-precision QK
// path (Lighthouse, "deep deepseek v4 release", section 八 items 3 and 7; 9fzt.com digest
// item 4: FP4 on the indexer's QK path, BF16 index scores for the top-k selector).
#pragma once
#include <algorithm>

#include "common.h"
#include "internal.h"
#include "select_dev.h"

namespace hcsa {

// Keys per block of the decode kernels: enough blocks to cover every CU several times even
// for one sequence, and at least 256 keys so a block issues a few loads per lane.
// log2 of the rows a page holds of a tensor pooled at `ratio` (a divisor of 128).
inline int page_rows_log2(int ratio) {
  int l = 0;
  for (int per = kPageTokens / ratio; per > 1; per >>= 1) ++l;
  return l;
}

inline int index_chunk(int rows, int N) {
  int64_t c = static_cast<int64_t>(N) * rows / 2048;
  c = (c + 255) / 256 * 256;
  return static_cast<int>(c < 256 ? 256 : (c > 4096 ? 4096 : c));
}

// ------------------------------------------------------------------ MXFP4 keys
// Indexer keys stored as MXFP4 (e2m1 codes, one e8m0 scale per 32 channels); the query
// vectors are quantized the same way at block start.

struct IdxMxDev {
  const void* q;       // [rows][H_I][d_I] bf16 or f32
  const float* w;      // [rows][H_I]
  const uint8_t* k;    // [B][N][d_I/2] packed codes (bstride bytes)
  const uint8_t* ks;   // [B][N][d_I/32] scale bytes (bstride bytes)
  int64_t k_bstride, ks_bstride;
  int Nq, N, ratio, d_I;
  int64_t pos0;
  const int64_t* seq_pos;   // [B] or null
  PageMap pm;          // paged keys (table null: contiguous)
  int c_log2;
  void* scores;        // scores [rows][N]; the fused selection's rescan rows
  int chunk;
  // fused selection (candidate lists instead of scores)
  uint32_t* floor;     // [rows][kMxFloorParts] 16-bit key floors (the row's: their minimum)
  uint32_t* lists;     // [rows][nchunks][chunk] (key << 16 | index in the chunk)
  uint32_t* counts;    // [rows][nchunks]
  int nchunks;
};

// MXFP4 keys on the matrix cores: v_mfma_scale_f32_32x32x64_f8f6f4 with e2m1 operands and
// e8m0 scales per 32 channels computes D[head][key] for 32 keys at once (A = the quantized
// query heads as rows, B = the keys as columns), so the e2m1 codes are never unpacked.
// Operand lane layout (measured): lane l holds row/column l % 32 and the 32 channels
// 32*(l/32) .. +31 of one 64-channel step, channel e in bits 4e..4e+3 (the stored packing:
// element 2i in the low nibble of byte i); the scale operand's low byte is that block's
// e8m0 scale; D register r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l % 32.
//
// The FP8 form of the same scan (F8 = true) widens the e2m1 codes to e4m3 bytes and runs
// the instruction with e4m3 operands and the same e8m0 scales: every e2m1 value is exact in
// e4m3, so the products and the scores are the same, at twice the operand registers and
// twice the matrix-core cycles [9fzt.com digest item 4: FP4 dequantized to FP8 without
// loss; tulong.co 技术架构创新 item 2: FP4+FP8 mixed precision, equal FP4 and FP8 peaks on
// current hardware].  Its operand layout differs (measured): registers 0..3 of lane l
// hold 16 channels of the step's first 32-channel block, registers 4..7 16 channels of
// the second, lane halves l/32 = 0 and 1 taking channels 0..15 and 16..31 of each block;
// the scale operand of lane half h still scales block h.  Within a block the channel
// order is free as long as queries and keys share it, so the even and odd channels of
// every packed word are kept in separate registers, with no interleaving.
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

// Eight e2m1 codes (a packed word, channel 2i in the low nibble of byte i) to e4m3: the
// magnitude (low three bits) indexes a byte table of 0, 0.5, 1, 1.5 | 2, 3, 4, 6 in e4m3
// (a byte permute), and the sign moves from bit 3 to bit 7.  `ev` receives the even
// channels (bytes in channel order), `od` the odd ones.
__device__ __forceinline__ void e2m1x8_to_e4m3(uint32_t w, uint32_t& ev, uint32_t& od) {
  constexpr uint32_t kMagLo = 0x3C383000u, kMagHi = 0x4C484440u;
  ev = __builtin_amdgcn_perm(kMagHi, kMagLo, w & 0x07070707u) | ((w << 4) & 0x80808080u);
  od = __builtin_amdgcn_perm(kMagHi, kMagLo, (w >> 4) & 0x07070707u) | (w & 0x80808080u);
}

constexpr int kMxMaxUnits = 16 * 4;   // H_I <= 16 heads x d_I / 32 <= 4 blocks

// The MFMA operands of one query row: the heads quantized to MXFP4 (per 32-channel block,
// the same rule as the keys), this lane's A operand and scale for each 64-channel step,
// and the head weights.
template <int HI, int KS>
struct MxQuery {
  i32x8 qa[KS];
  int qs[KS];
  float w[HI];
};

// Quantizes the row's query heads into LDS (eight threads per 32-channel block, four
// channels each; the block's absolute maximum is reduced across the eight and each thread
// writes its four codes, 16 bits of the packed row) and builds this lane's operands.
// Called by every thread of the block (one barrier).
template <int HI, int KS, bool QBF16, bool F8>
__device__ __forceinline__ MxQuery<HI, KS> mx_query(const IdxMxDev& A, int row,
                                                   uint32_t (*s_qa)[4], int* s_qs) {
  const int lane = threadIdx.x & 63;
  const int col = lane & 31, half = lane >> 5;
  const int ksteps = A.d_I > 64 ? A.d_I / 64 : 1;       // 64-channel MFMA steps
  const int nblk = A.d_I / 32;                          // 32-channel scale blocks per row
  const int units = HI * nblk;
  for (int t = threadIdx.x; t < units * 8; t += blockDim.x) {   // groups of 8 stay together
    const int u = t >> 3, sub = t & 7;
    const int g = u / nblk, blk = u - g * nblk;
    const int64_t off = (static_cast<int64_t>(row) * HI + g) * A.d_I + blk * 32 + 4 * sub;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      v[e] = QBF16 ? bf16_to_f32(static_cast<const uint16_t*>(A.q)[off + e])
                   : static_cast<const float*>(A.q)[off + e];
    float amax = fmaxf(fmaxf(__builtin_fabsf(v[0]), __builtin_fabsf(v[1])),
                       fmaxf(__builtin_fabsf(v[2]), __builtin_fabsf(v[3])));
    amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
    amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
    amax = fmaxf(amax, __shfl_xor(amax, 4, kWave));
    const int se = mx_scale_exp(amax);
    uint32_t c = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) c |= e2m1_code(v[e], se) << (4 * e);
    reinterpret_cast<uint16_t*>(s_qa[u])[sub] = static_cast<uint16_t>(c);
    if (sub == 0) s_qs[u] = se + 127;
  }
  __syncthreads();
  MxQuery<HI, KS> Q;
  // A operand: this lane's head (col) and block (2*step + half)
#pragma unroll
  for (int st = 0; st < KS; ++st) {
    Q.qa[st] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
    Q.qs[st] = 127;
    const int blk = 2 * st + half;
    if (st < ksteps && col < HI && blk < nblk) {
      const int u = col * nblk + blk;
      if constexpr (!F8) {
#pragma unroll
        for (int d = 0; d < 4; ++d) Q.qa[st][d] = static_cast<int>(s_qa[u][d]);
      }
      Q.qs[st] = s_qs[u];
    }
    if constexpr (F8) {
      // registers 4q..4q+3: channels 16*half .. +15 of block 2*st + q
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int bq = 2 * st + q;
        if (st < ksteps && col < HI && bq < nblk) {
#pragma unroll
          for (int wd = 0; wd < 2; ++wd) {
            uint32_t ev, od;
            e2m1x8_to_e4m3(s_qa[col * nblk + bq][2 * half + wd], ev, od);
            Q.qa[st][4 * q + 2 * wd] = static_cast<int>(ev);
            Q.qa[st][4 * q + 2 * wd + 1] = static_cast<int>(od);
          }
        }
      }
    }
  }
#pragma unroll
  for (int g = 0; g < HI; ++g) Q.w[g] = A.w[static_cast<int64_t>(row) * HI + g];
  return Q;
}

// This lane's share of key j (sequence b) as loaded: the packed codes of its 32-channel
// blocks (fp4 operands take them as they are, 4 words per step; the FP8 form holds 8 bytes
// of each of the step's two blocks and widens them at the MFMA) and their scales.  Nothing
// is loaded when !ok (zero codes, unit scales).
template <int KS, bool PAGED, bool F8>
__device__ __forceinline__ void mx_load(const IdxMxDev& A, const uint8_t* kbase,
                                        const uint8_t* sbase, int b, int j, bool ok,
                                        u32x4 (&kraw)[KS], int (&ksc)[KS]) {
  const int half = (threadIdx.x & 63) >> 5;
  const int ksteps = A.d_I > 64 ? A.d_I / 64 : 1;
  const int nblk = A.d_I / 32;
  const int rowb = A.d_I / 2;
  const int64_t rj = PAGED && ok ? row_off<true>(A.pm, 0, b, j, A.c_log2, 1) : j;   // pool row
#pragma unroll
  for (int st = 0; st < KS; ++st) {
    kraw[st] = u32x4{0, 0, 0, 0};
    ksc[st] = 127;
    const int blk = 2 * st + half;
    if (st < ksteps && blk < nblk && ok) ksc[st] = sbase[rj * nblk + blk];
    if constexpr (!F8) {
      if (st < ksteps && blk < nblk && ok)
        kraw[st] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(kbase + rj * rowb + blk * 16));
    } else {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int bq = 2 * st + q;
        if (st < ksteps && bq < nblk && ok) {
          const u32x2 c = __builtin_nontemporal_load(
              reinterpret_cast<const u32x2*>(kbase + rj * rowb + bq * 16 + 8 * half));
          kraw[st][2 * q] = c[0];
          kraw[st][2 * q + 1] = c[1];
        }
      }
    }
  }
}

// Score of the key whose codes this lane's column holds (valid in lane half 0, and in both
// halves for H_I > 4): sum over heads of w_g * relu(q_g . k) from one or two MFMAs.
//
// The MFMA reads the operand registers of all 64 lanes whatever the EXEC mask, so every lane
// must assemble its operands before it.  With the score used only in half 0 (callers store it
// under `half == 0`), the compiler sank the FP8 form's e2m1-to-e4m3 widening and the MFMA
// into that store's branch, where half 1 never wrote its widened operand and the MFMA read
// stale registers (measured: wrong and run-dependent scores at H_I 1 and 4).  An empty
// volatile asm that takes the lane's sum in every lane keeps the MFMA, and so its operands,
// where the whole wave runs it; it emits no instruction and holds one register.
template <int HI, int KS, bool F8>
__device__ __forceinline__ float mx_score(const MxQuery<HI, KS>& Q, const u32x4 (&kraw)[KS],
                                          const int (&ksc)[KS], int ksteps) {
  const int half = (threadIdx.x & 63) >> 5;
  i32x8 kb[KS];
#pragma unroll
  for (int st = 0; st < KS; ++st) {
    kb[st] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
    if constexpr (!F8) {
#pragma unroll
      for (int d = 0; d < 4; ++d) kb[st][d] = static_cast<int>(kraw[st][d]);
    } else {
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        uint32_t ev, od;
        e2m1x8_to_e4m3(kraw[st][wd], ev, od);
        kb[st][2 * wd] = static_cast<int>(ev);
        kb[st][2 * wd + 1] = static_cast<int>(od);
      }
    }
  }
  constexpr int kFmt = F8 ? 0 : 4;                 // operand format: e4m3 or e2m1
  f32x16 d = {};
  d = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(Q.qa[0], kb[0], d, kFmt, kFmt, 0,
                                                      Q.qs[0], 0, ksc[0]);
  if constexpr (KS > 1) {
    if (ksteps > 1)
      d = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(Q.qa[KS - 1], kb[KS - 1], d, kFmt,
                                                          kFmt, 0, Q.qs[KS - 1], 0, ksc[KS - 1]);
  }
  // rows (heads) held by this lane: 8*(r/4) + 4*half + r%4
  float part = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int g = 8 * (r >> 2) + 4 * half + (r & 3);
    if (g < HI) part = fmaf(Q.w[g], relu(d[r]), part);
  }
  asm volatile("" : "+v"(part));
  if constexpr (HI > 4) part += __shfl_xor(part, 32, kWave);
  return part + 0.0f;
}

// ---------------------------------------------------------------- fused decode selection
//
// Top-k of MXFP4 scores without the score array: a floor per row from scored samples, the
// scan's candidate lists (keys >= floor), then the exact threshold among the candidates
// (sel::select_candidates).  Rows whose lists hold fewer than k or more than kMxResMax
// candidates are rescanned by their resolve block into the score rows of the workspace and
// selected over the whole row (sel::select_exact_row), so the result is always that of
// the selector on the materialized scores.

constexpr int kMxFloorThreads = 512;
constexpr int kMxFloorRuns = 32;          // sampled runs of consecutive keys
constexpr int kMxRunKeys = 128;
constexpr int kMxSamples = kMxFloorRuns * kMxRunKeys;
constexpr int kMxFloorParts = 4;          // blocks per row, each scoring a share of the runs
constexpr int kMxPartSamples = kMxSamples / kMxFloorParts;
constexpr int kMxResThreads = 512;
constexpr int kMxResPer = 32;
constexpr int kMxResMax = kMxResThreads * kMxResPer;
constexpr int kMxMaxChunks = 4096;

// One of a row's kMxFloorParts floor blocks (block 512).  The row's samples are 32 runs of
// 128 consecutive visible keys at evenly spaced positions; part p scores runs 8p .. 8p+7
// and stores the 16-bit key of about its m_p-th largest sample, m_p = ceil(m / parts) and m
// about twice the rank at which the k-th largest key is expected among the 4096 samples.
// The row's floor is the second smallest of the parts' values (mx_row_floor).  Only the
// candidate count depends on the floor (a row left with fewer than k candidates is
// rescanned).  Rank statistics of 4 parts of 1024 samples at k = 1024 of 262 144 keys put
// the floor at rank 2 747 on average (p99 4 093) against 2 557 (p99 3 595) for the m-th
// largest of all 4096 samples, and below rank k in none of 200 000 rows; the smallest part
// value would admit 3 421 on average (p99 5 385).  Within a part: for shallow ranks the
// m_p-th largest of the 512 per-thread maxima, found exactly by one wave (radix 4 from the
// top, ballot counts); deeper ranks count every sample, each wave its own ceil(m_p/W)-th,
// and take the smallest of the W.
// Rows of at most 4096 visible keys take every key (floor 0).  All sample loads are issued
// before the query is quantized.
//
// prior_only: sample only the entries completed before the sequence's first query token
// (those a pooling launch of the same tokens does not write), for the fused pooling launch.
// Called by every thread of the block.
template <int HI, int KS, bool QBF16, bool PAGED, bool F8>
__device__ __forceinline__ void mx_floor_block(const IdxMxDev& A, int k, int row, int part,
                                               bool prior_only) {
  constexpr int W = kMxFloorThreads / 64;
  constexpr int PT = kMxPartSamples / kMxFloorThreads;  // samples per thread
  __shared__ uint32_t s_qa[kMxMaxUnits][4];
  __shared__ int s_qs[kMxMaxUnits];
  __shared__ uint16_t s_samp[kMxPartSamples];
  __shared__ uint32_t s_gmax[kMxFloorThreads];
  __shared__ uint32_t s_min[W];
  const int b = row / A.Nq;
  const int64_t p = query_pos(A.seq_pos, A.pos0, b, row % A.Nq);
  const int64_t nv64 = (p + 1) / A.ratio;
  const int nv = static_cast<int>(nv64 < A.N ? nv64 : A.N);
  int ns = nv;                                         // entries the samples may read
  if (prior_only) {
    const int64_t e0 = query_pos(A.seq_pos, A.pos0, b, 0) / A.ratio;
    ns = static_cast<int>(e0 < nv ? e0 : nv);
  }
  uint32_t* floor_out = A.floor + row * kMxFloorParts + part;
  if (k >= nv || ns <= kMxSamples) {
    if (threadIdx.x == 0) *floor_out = 0u;
    return;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int ksteps = A.d_I > 64 ? A.d_I / 64 : 1;
  const uint8_t* kbase = PAGED ? A.k : A.k + b * A.k_bstride;
  const uint8_t* sbase = PAGED ? A.ks : A.ks + b * A.ks_bstride;
  // wave w scores the part's runs RPW*w .. RPW*w + RPW-1: NG groups of 32 keys, all loads
  // in flight
  constexpr int RPP = kMxFloorRuns / kMxFloorParts;    // runs per part
  constexpr int RPW = RPP / W, GPR = kMxRunKeys / 32, NG = RPW * GPR;
  static_assert(RPW >= 1 && RPW * W == RPP, "whole runs per wave");
  u32x4 kraw[NG][KS];
  int ksc[NG][KS];
#pragma unroll
  for (int u = 0; u < NG; ++u) {
    const int run = part * RPP + wave * RPW + u / GPR;
    const int r0 = static_cast<int>(static_cast<int64_t>(run) * (ns - kMxRunKeys) /
                                    (kMxFloorRuns - 1));
    mx_load<KS, PAGED, F8>(A, kbase, sbase, b, r0 + (u % GPR) * 32 + col, true, kraw[u], ksc[u]);
  }
  const MxQuery<HI, KS> Q = mx_query<HI, KS, QBF16, F8>(A, row, s_qa, s_qs);
#pragma unroll
  for (int u = 0; u < NG; ++u) {
    const int lrun = wave * RPW + u / GPR;             // run within the part
    const float s = mx_score<HI, KS, F8>(Q, kraw[u], ksc[u], ksteps);
    if (half == 0)
      s_samp[lrun * kMxRunKeys + (u % GPR) * 32 + col] =
          static_cast<uint16_t>(bf16_key(f32_to_bf16_bits(s)));
  }
  __syncthreads();
  uint32_t top[PT];
#pragma unroll
  for (int e = 0; e < PT; ++e) top[e] = s_samp[threadIdx.x * PT + e];
  const int m_all = min(kMxSamples - 8, static_cast<int>((2LL * k * kMxSamples + nv - 1) / nv) + 8);
  const int m = (m_all + kMxFloorParts - 1) / kMxFloorParts;
  if (m <= 64) {
    uint32_t mx = 0;
#pragma unroll
    for (int e = 0; e < PT; ++e) mx = max(mx, top[e]);
    s_gmax[threadIdx.x] = mx;
    __syncthreads();
    if (wave == 0) {
      constexpr int MPL = kMxFloorThreads / 64;        // maxima per lane
      uint32_t v[MPL];
#pragma unroll
      for (int e = 0; e < MPL; ++e) v[e] = s_gmax[lane * MPL + e];
      uint32_t pre = 0;
#pragma unroll 1
      for (int sh = 14; sh >= 0; sh -= 2) {
        int cnt[3];
#pragma unroll
        for (int d = 1; d <= 3; ++d) {
          const uint32_t th = pre | (static_cast<uint32_t>(d) << sh);
          int n = 0;
#pragma unroll
          for (int e = 0; e < MPL; ++e) n += v[e] >= th;
          cnt[d - 1] = sel::wave_sum_bits<sel::bits_for(MPL)>(n);
        }
        const uint32_t d = cnt[2] >= m ? 3u : cnt[1] >= m ? 2u : cnt[0] >= m ? 1u : 0u;
        pre |= d << sh;
      }
      if (lane == 0) *floor_out = pre;
    }
    return;
  }
  const int mw = (m + W - 1) / W;
  uint32_t pre = 0;
#pragma unroll 1
  for (int sh = 14; sh >= 0; sh -= 2) {
    int cnt[3];
#pragma unroll
    for (int d = 1; d <= 3; ++d) {
      const uint32_t th = pre | (static_cast<uint32_t>(d) << sh);
      int n = 0;
#pragma unroll
      for (int e = 0; e < PT; ++e) n += top[e] >= th;
      cnt[d - 1] = sel::wave_sum_bits<sel::bits_for(PT)>(n);
    }
    const uint32_t d = cnt[2] >= mw ? 3u : cnt[1] >= mw ? 2u : cnt[0] >= mw ? 1u : 0u;
    pre |= d << sh;
  }
  if (lane == 0) s_min[wave] = pre;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < W; ++u) pre = min(pre, s_min[u]);
  if (threadIdx.x == 0) *floor_out = pre;
}

// The row's floor: the second smallest of its parts' values.
__device__ __forceinline__ uint32_t mx_row_floor(const IdxMxDev& A, int row) {
  static_assert(kMxFloorParts == 4, "one 16-byte load");
  const u32x4 f = *reinterpret_cast<const u32x4*>(A.floor + row * kMxFloorParts);
  const uint32_t lo01 = min(f[0], f[1]), hi01 = max(f[0], f[1]);
  const uint32_t lo23 = min(f[2], f[3]), hi23 = max(f[2], f[3]);
  return min(max(lo01, lo23), min(hi01, hi23));
}

// The exact threshold among the row's C candidates (the concatenated chunk lists, prefix
// counts in s_pre): thread t takes a contiguous run of at most PER of them.
template <int PER, bool COH>
__device__ __forceinline__ void mx_resolve_lists(const IdxMxDev& A, int row, int nch, int C,
                                                 int k, int32_t* out, const int* s_pre,
                                                 int* s_gt, int* s_eq, int* s_hb,
                                                 int (*s_hist)[256], int* s_sel) {
  const int per = (C + kMxResThreads - 1) / kMxResThreads;
  const int g0 = min(C, static_cast<int>(threadIdx.x) * per);
  const int my = min(per, C - g0);
  int lo = 0, hi = nch - 1;                            // chunk of the first candidate
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_pre[mid] <= g0) lo = mid;
    else hi = mid - 1;
  }
  int c = lo;
  uint32_t ck[PER];
  int32_t cj[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    ck[u] = 0u;
    cj[u] = 0;
    if (u < my) {
      const int g = g0 + u;
      while (g >= s_pre[c + 1]) ++c;
      const uint32_t v =
          A.lists[(static_cast<int64_t>(row) * A.nchunks + c) * A.chunk + (g - s_pre[c])];
      ck[u] = v >> 16;
      cj[u] = c * A.chunk + static_cast<int>(v & 0xffffu);
    }
  }
  sel::select_candidates<16, kMxResThreads, PER, COH>(ck, cj, my, mx_row_floor(A, row), k, out,
                                                      s_gt, s_eq, s_hb, s_hist, s_sel);
}

// The selection of one row by a 512-thread block: the row's candidates are the
// concatenated chunk lists (index order); thread t takes a contiguous run of them.  COH:
// the selection is written with agent-coherent stores (read by other blocks of the same
// launch).  Called by every thread of the block.
template <int HI, int KS, bool QBF16, bool PAGED, bool F8, bool COH>
__device__ __forceinline__ void mx_resolve_row(const IdxMxDev& A, int k, int32_t* idx, int row) {
  constexpr int W = kMxResThreads / 64;
  __shared__ int s_pre[kMxMaxChunks + 1];
  __shared__ int s_cnt[2][W];
  __shared__ int s_gt[W], s_eq[W], s_hb[W];
  __shared__ int s_hist[2][256];
  __shared__ int s_sel[4];
  __shared__ uint32_t s_qa[kMxMaxUnits][4];
  __shared__ int s_qs[kMxMaxUnits];
  const int b = row / A.Nq;
  const int64_t p = query_pos(A.seq_pos, A.pos0, b, row % A.Nq);
  const int64_t nv64 = (p + 1) / A.ratio;
  const int nv = static_cast<int>(nv64 < A.N ? nv64 : A.N);
  int32_t* out = idx + static_cast<int64_t>(row) * k;
  if (k >= nv) {
    sel::take_all<COH>(nv, k, out, kMxResThreads);
    return;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nch = (nv + A.chunk - 1) / A.chunk;        // chunks holding visible keys
  const uint32_t* cnt = A.counts + static_cast<int64_t>(row) * A.nchunks;
  // Direct form (few chunks): tpc threads per chunk, thread (c, sub) loads the slice
  // [16 sub, 16 sub + 16) of chunk c's list together with the count, without waiting for
  // a prefix; thread order is index order.  Taken when every chunk's count fits its
  // threads' slices and the row holds at least k candidates, else the prefix form below.
  int pw = 1;
  while (pw < nch) pw <<= 1;
  const int tpc = pw <= kMxResThreads ? kMxResThreads / pw : 0;
  if (tpc > 0 && tpc * 16 <= A.chunk) {
    const int c = threadIdx.x / tpc, sub = threadIdx.x % tpc;
    int cc = 0;
    u32x4 e[4] = {};
    if (c < nch) {
      cc = static_cast<int>(cnt[c]);
      const u32x4* src = reinterpret_cast<const u32x4*>(
          A.lists + (static_cast<int64_t>(row) * A.nchunks + c) * A.chunk + 16 * sub);
#pragma unroll
      for (int v = 0; v < 4; ++v) e[v] = src[v];
    }
    const int my = min(max(cc - 16 * sub, 0), 16);
    const int over = __syncthreads_or(cc > tpc * 16);
    const int C = sel::block_total_bits<W, sel::bits_for(16)>(my, s_cnt, 0);
    if (!over && C >= k) {
      uint32_t ck[16];
      int32_t cj[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const uint32_t v = e[u >> 2][u & 3];
        ck[u] = u < my ? v >> 16 : 0u;
        cj[u] = u < my ? c * A.chunk + static_cast<int>(v & 0xffffu) : 0;
      }
      sel::select_candidates<16, kMxResThreads, 16, COH>(ck, cj, my, mx_row_floor(A, row), k,
                                                         out, s_gt, s_eq, s_hb, s_hist, s_sel);
      return;
    }
  }
  if (threadIdx.x < 64) {                              // prefix of the counts, 64 at a time
    int carry = 0;
    for (int base = 0; base < nch; base += 64) {
      const int c = base + lane < nch ? static_cast<int>(cnt[base + lane]) : 0;
      int inc = c;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(inc, d, kWave);
        if (lane >= d) inc += y;
      }
      if (base + lane < nch) s_pre[base + lane + 1] = carry + inc;
      carry += __shfl(inc, 63, kWave);
    }
    if (lane == 0) s_pre[0] = 0;
  }
  __syncthreads();
  const int C = s_pre[nch];
  if (C >= k && C <= kMxResMax) {
    if (C <= kMxResThreads * 16)
      mx_resolve_lists<16, COH>(A, row, nch, C, k, out, s_pre, s_gt, s_eq, s_hb, s_hist, s_sel);
    else
      mx_resolve_lists<kMxResPer, COH>(A, row, nch, C, k, out, s_pre, s_gt, s_eq, s_hb, s_hist,
                                  s_sel);
    return;
  }
  // too few or too many candidates: score the whole row into the workspace's score row
  // and select over it
  const MxQuery<HI, KS> Q = mx_query<HI, KS, QBF16, F8>(A, row, s_qa, s_qs);
  const int col = lane & 31, half = lane >> 5;
  const int ksteps = A.d_I > 64 ? A.d_I / 64 : 1;
  const uint8_t* kbase = PAGED ? A.k : A.k + b * A.k_bstride;
  const uint8_t* sbase = PAGED ? A.ks : A.ks + b * A.ks_bstride;
  uint16_t* srow = static_cast<uint16_t*>(A.scores) + static_cast<int64_t>(row) * A.N;
  constexpr int U = 4;
  for (int j0 = wave * 32; j0 < nv; j0 += W * 32 * U) {
    u32x4 kraw[U][KS];
    int ksc[U][KS];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * W * 32 + col;
      mx_load<KS, PAGED, F8>(A, kbase, sbase, b, j, j < nv, kraw[u], ksc[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float s = mx_score<HI, KS, F8>(Q, kraw[u], ksc[u], ksteps);
      const int j = j0 + u * W * 32 + col;
      if (half == 0 && j < nv) srow[j] = static_cast<uint16_t>(f32_to_bf16_bits(s));
    }
  }
  __syncthreads();
  const sel::RowView<16> V(srow, nv, A.N % 8 == 0 ? A.N / 8 : 0);
  sel::select_exact_row<16, kMxResThreads, COH>(V, k, out, s_cnt, s_gt, s_eq);
}

inline IdxMxDev make_mx_dev(const void* q, const float* w, const uint8_t* kx, int64_t k_bstride,
                     const uint8_t* ks, int64_t ks_bstride, int B, int Nq, int d_I, int N,
                     int ratio, int64_t pos0, const int64_t* seq_pos,
                     const int32_t* block_table, int64_t table_stride, void* scores) {
  IdxMxDev A{};
  A.q = q;
  A.w = w;
  A.k = kx;
  A.ks = ks;
  A.k_bstride = k_bstride;
  A.ks_bstride = ks_bstride;
  A.Nq = Nq;
  A.N = N;
  A.ratio = ratio;
  A.d_I = d_I;
  A.pos0 = pos0;
  A.seq_pos = seq_pos;
  A.pm.table = block_table;
  A.pm.stride = table_stride;
  A.c_log2 = page_rows_log2(ratio);
  A.scores = scores;
  // at most 2048 keys per block: more, shorter blocks shorten the grid's last round
  A.chunk = std::min(index_chunk(B * Nq, N), 2048);
  A.nchunks = (N + A.chunk - 1) / A.chunk;
  return A;
}

// Workspace of the fused selection: floors, chunk counts, chunk lists, rescan score rows.
struct MxTopkLayout {
  size_t counts_off, lists_off, scores_off, total;
};

inline MxTopkLayout mx_topk_layout(int rows, int N) {
  const int chunk = std::min(index_chunk(rows, N), 2048);
  const int64_t nchunks = (N + chunk - 1) / chunk;
  MxTopkLayout l;
  l.counts_off = align256(static_cast<size_t>(rows) * kMxFloorParts * 4);   // floors first
  l.lists_off = l.counts_off + align256(static_cast<size_t>(rows) * nchunks * 4);
  l.scores_off = l.lists_off + align256(static_cast<size_t>(rows) * nchunks * chunk * 4);
  l.total = l.scores_off + align256(static_cast<size_t>(rows) * N * 2);
  return l;
}

// The candidate scan of the fused selection (bf16 queries, MXFP4 keys on fp4 operands,
// contiguous or paged): per-chunk lists of the keys scoring at or above each row's floor.
hipError_t launch_mx_candidate_scan(const IdxMxDev& A, int rows, int H_I, bool paged,
                                     hipStream_t s);

// Scores of MXFP4 keys (fp4 operands, or widened to e4m3 with fp8) into scores [rows][N].
hipError_t launch_mxfp4_index_scores(const void* q, int q_dtype, const float* w,
                                     const uint8_t* kx, int64_t k_bstride, const uint8_t* ks,
                                     int64_t ks_bstride, int B, int Nq, int H_I, int d_I,
                                     int N, int ratio, int64_t pos0, const int64_t* seq_pos,
                                     const int32_t* block_table, int64_t table_stride,
                                     int score_dtype, void* scores, bool fp8, hipStream_t s);

}  // namespace hcsa
