// Lightning-indexer scores of the compressed indexer keys.
//
// The indexer scores compressed entries with its own compressed keys (Lighthouse, "deep
// deepseek v4 release", section 八 items 3 and 7) on a low-precision QK path whose scores
// are fp32, optionally stored as bf16 (9fzt.com digest, item 4).  The score form
// s_j = sum_g w_g * max(0, q_g . k_j) is the reading taken (the pages print no formula).
//
// Decode kernel (one or few query tokens per sequence): HBM-bound key scan.  A group of
// LPE lanes reads one key row with 16-byte loads (a wave covers 64/LPE contiguous rows per
// instruction), each lane forms H_I partial dot products with packed bf16 dot2 (or fp32
// fma), the group reduces them with cross-lane adds, and the group's first lane applies
// ReLU, the head weights (fixed order g = 0..H_I-1) and writes the score.
#include "common.h"
#include <hip/hip_ext.h>

#include "internal.h"
#include "select_common.h"

namespace hcsa {

// Optional timing of the next indexer kernel launched on this thread: the dispatch itself
// records the start and stop events (hipExtLaunchKernel), so the measured interval is the
// kernel's own execution.
static thread_local hipEvent_t t_ev_start = nullptr, t_ev_stop = nullptr;

void time_next_indexer(hipEvent_t start, hipEvent_t stop) {
  t_ev_start = start;
  t_ev_stop = stop;
}

namespace {

template <typename K, typename... Args>
void launch_timed(K kernel, dim3 grid, dim3 block, hipStream_t s, Args... args) {
  if (t_ev_start != nullptr) {
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, t_ev_start, t_ev_stop, 0, args...);
    t_ev_start = t_ev_stop = nullptr;
  } else {
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
  }
}

struct IdxDev {
  const void* q;     // [rows][H_I][d_I]
  const float* w;    // [rows][H_I]
  const void* k;     // [B][N][d_I] (bstride elements)
  int64_t k_bstride;
  int Nq, N, ratio, d_I;
  int64_t pos0;
  void* scores;      // [rows][N]
  int chunk;
  uint32_t* hist;    // optional selector workspace (see select_common.h)
  int topk;
  int rows_total;    // B*Nq*H_I (prefill GEMM)
};


__device__ __forceinline__ float dot16b_bf16(const u32x4& a, const u32x4& b, float acc) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    // copy the element out first: a bit_cast of a vector subscript is miscompiled
    // (every iteration read element 0)
    const uint32_t x = a[c], y = b[c];
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x),
                                          __builtin_bit_cast(bf16x2, y), acc, false);
  }
  return acc;
}

__device__ __forceinline__ float dot16b_f32(const u32x4& a, const u32x4& b, float acc) {
#pragma unroll
  for (int c = 0; c < 4; ++c) acc = fmaf(__uint_as_float(a[c]), __uint_as_float(b[c]), acc);
  return acc;
}

// Selector histogram fused into the score kernels: a 4096-bin LDS histogram of the 12-bit
// top digit of each stored score's order-preserving key, flushed with one global atomic per
// non-empty bin.
constexpr int kHistBins = 4096;

__device__ __forceinline__ void hist_clear(uint32_t* h, bool on) {
  if (on)
    for (int i = threadIdx.x; i < kHistBins; i += 256) h[i] = 0;
  __syncthreads();
}

template <bool SBF16>
__device__ __forceinline__ void hist_add(uint32_t* h, float s) {
  if constexpr (SBF16)
    atomicAdd(&h[bf16_key(f32_to_bf16_bits(s)) >> 4], 1u);
  else
    atomicAdd(&h[f32_key(__float_as_uint(s)) >> 20], 1u);
}

// Flushes the block histogram into replica (block % copies) of the row's histogram.
__device__ __forceinline__ void hist_flush(const uint32_t* h, uint32_t* ws, int row, int N) {
  __syncthreads();
  const SelState S = sel_state(ws, gridDim.y, sel_copies(gridDim.y, N), 0);
  uint32_t* grow = sel_hist_row(S, blockIdx.x % S.copies, row);
  for (int i = threadIdx.x; i < kHistBins; i += 256) {
    const uint32_t v = h[i];
    if (v) atomicAdd(&grow[i], v);
  }
}

// grid: (ceil(N / chunk), rows); block 256.
template <int HI, int LPE, bool KBF16, bool SBF16>
__global__ __launch_bounds__(256) void index_scores_kernel(IdxDev A) {
  constexpr int ES = KBF16 ? 2 : 4;
  constexpr int GROUPS = 256 / LPE;
  constexpr int U = 4;
  const int row = blockIdx.y;
  const int b = row / A.Nq;
  const int64_t p = A.pos0 + (row % A.Nq);
  const int64_t nv64 = (p + 1) / A.ratio;
  const int nv = static_cast<int>(nv64 < A.N ? nv64 : A.N);
  const int start = blockIdx.x * A.chunk;
  const int end = min(start + A.chunk, nv);
  if (start >= end) return;

  const int sub = threadIdx.x % LPE;
  const int grp = threadIdx.x / LPE;
  const int row_bytes = A.d_I * ES;
  __shared__ uint32_t s_hist[kHistBins];
  const bool hist = A.hist != nullptr && A.topk < nv;
  hist_clear(s_hist, hist);

  u32x4 qv[HI];
  float w[HI];
  const char* qrow = static_cast<const char*>(A.q) + static_cast<int64_t>(row) * HI * row_bytes;
#pragma unroll
  for (int g = 0; g < HI; ++g) {
    qv[g] = *reinterpret_cast<const u32x4*>(qrow + g * row_bytes + sub * 16);
    w[g] = A.w[static_cast<int64_t>(row) * HI + g];
  }
  const char* kbase = static_cast<const char*>(A.k) + b * A.k_bstride * ES + sub * 16;
  float* s32 = static_cast<float*>(A.scores) + static_cast<int64_t>(row) * A.N;
  uint16_t* s16 = static_cast<uint16_t*>(A.scores) + static_cast<int64_t>(row) * A.N;

  for (int j0 = start + grp; j0 < end; j0 += GROUPS * U) {
    u32x4 kv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * GROUPS;
      if (j < end)
        kv[u] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(kbase + static_cast<int64_t>(j) * row_bytes));
      else
        kv[u] = u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float part[HI];
#pragma unroll
      for (int g = 0; g < HI; ++g)
        part[g] = KBF16 ? dot16b_bf16(qv[g], kv[u], 0.0f) : dot16b_f32(qv[g], kv[u], 0.0f);
#pragma unroll
      for (int o = 1; o < LPE; o <<= 1)
#pragma unroll
        for (int g = 0; g < HI; ++g) part[g] += __shfl_xor(part[g], o, kWave);
      const int j = j0 + u * GROUPS;
      if (sub == 0 && j < end) {
        float s = 0.0f;
#pragma unroll
        for (int g = 0; g < HI; ++g) s = fmaf(w[g], fmaxf(part[g], 0.0f), s);
        s += 0.0f;  // -0 -> +0
        if constexpr (SBF16)
          s16[j] = static_cast<uint16_t>(f32_to_bf16_bits(s));
        else
          s32[j] = s;
        if (hist) hist_add<SBF16>(s_hist, s);
      }
    }
  }
  if (hist) hist_flush(s_hist, A.hist, row, A.N);
}

// ------------------------------------------------------------------ prefill GEMM
// Many query tokens per sequence (chunked prefill): the indexer is a GEMM
// [Nq*H_I x d_I] x [d_I x N] on v_mfma_f32_32x32x16_bf16.  A wave owns 32 rows (32/H_I query
// tokens x H_I heads, operand A kept in registers) and walks its block's key range 32 keys
// at a time (operand B loaded straight from global; the block's 4 waves read the same keys,
// so most loads hit the L1/L2).  Output lane layout: register r of lane l holds row
// 8*(r/4) + 4*(l/32) + r%4 and key l%32, so the H_I <= 4 heads of a query token sit in
// consecutive registers of one lane and the ReLU / weight / head-sum epilogue is lane-local.
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16g;

template <int HI, bool SBF16>
__global__ __launch_bounds__(256) void index_scores_gemm_kernel(IdxDev A) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 31, half = lane >> 5;
  const int64_t row0 = (static_cast<int64_t>(blockIdx.y) * 4 + wave) * 32;   // first row of the wave
  const int q_first = static_cast<int>(row0 / HI);             // first query row (b*Nq + i)
  const int rows_total = A.rows_total;                          // B*Nq*H_I
  if (row0 >= rows_total) return;
  const int b = q_first / A.Nq;                                 // whole wave in one sequence
  const int kstart = blockIdx.x * A.chunk;
  const int kend = min(kstart + A.chunk, A.N);
  // visible keys of the wave's last query token bound the keys worth computing
  const int q_last = q_first + 32 / HI - 1;
  const int64_t p_last = A.pos0 + (q_last % A.Nq);
  const int64_t nv_last64 = (p_last + 1) / A.ratio;
  const int nv_last = static_cast<int>(nv_last64 < A.N ? nv_last64 : A.N);
  const int kstop = min(kend, nv_last);
  if (kstart >= kstop) return;

  // operand A: row col of the wave (query q_first + col/HI, head col%HI), 16 channels per step
  const int ksteps = A.d_I / 16;
  const uint16_t* qrow = static_cast<const uint16_t*>(A.q) + (row0 + col) * A.d_I + 8 * half;
  u32x4 qa[8];
#pragma unroll
  for (int s = 0; s < 8; ++s)
    qa[s] = s < ksteps ? *reinterpret_cast<const u32x4*>(qrow + 16 * s) : u32x4{0, 0, 0, 0};
  // weights and visible counts of the query tokens whose scores this lane writes
  constexpr int QPL = 16 / HI;          // query tokens per lane (one per group of HI registers)
  float w[QPL][HI];
  int nvq[QPL];
  int64_t qrow_idx[QPL];
#pragma unroll
  for (int t = 0; t < QPL; ++t) {
    const int r0 = t * HI;                                      // first register of the group
    const int row_in_wave = 8 * (r0 >> 2) + 4 * half + (r0 & 3);
    const int qi = q_first + row_in_wave / HI;
    qrow_idx[t] = qi;
#pragma unroll
    for (int g = 0; g < HI; ++g) w[t][g] = A.w[static_cast<int64_t>(qi) * HI + g];
    const int64_t p = A.pos0 + (qi % A.Nq);
    const int64_t v = (p + 1) / A.ratio;
    nvq[t] = static_cast<int>(v < A.N ? v : A.N);
  }
  const uint16_t* kbase = static_cast<const uint16_t*>(A.k) + b * A.k_bstride + 8 * half;
  for (int j0 = kstart; j0 < kstop; j0 += 32) {
    const int j = j0 + col;
    u32x4 kb[8];
    const bool jv = j < kstop;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      kb[s] = (s < ksteps && jv)
                  ? *reinterpret_cast<const u32x4*>(kbase + static_cast<int64_t>(j) * A.d_I + 16 * s)
                  : u32x4{0, 0, 0, 0};
    f32x16g d = {};
#pragma unroll
    for (int s = 0; s < 8; ++s)
      if (s < ksteps)
        d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, qa[s]),
                                                    __builtin_bit_cast(bf16x8, kb[s]), d, 0, 0, 0);
#pragma unroll
    for (int t = 0; t < QPL; ++t) {
      float sc = 0.0f;
#pragma unroll
      for (int g = 0; g < HI; ++g) sc = fmaf(w[t][g], fmaxf(d[t * HI + g], 0.0f), sc);
      sc += 0.0f;
      if (jv && j < nvq[t]) {
        if constexpr (SBF16)
          static_cast<uint16_t*>(A.scores)[qrow_idx[t] * A.N + j] =
              static_cast<uint16_t>(f32_to_bf16_bits(sc));
        else
          static_cast<float*>(A.scores)[qrow_idx[t] * A.N + j] = sc;
      }
    }
  }
}

template <int HI, int LPE, bool KBF16>
hipError_t launch_hi(const IdxDev& A, int rows, int score_dtype, hipStream_t s) {
  const int nchunks = (A.N + A.chunk - 1) / A.chunk;
  dim3 grid(nchunks, rows);
  if (score_dtype == 1)
    launch_timed(index_scores_kernel<HI, LPE, KBF16, true>, grid, dim3(256), s, A);
  else
    launch_timed(index_scores_kernel<HI, LPE, KBF16, false>, grid, dim3(256), s, A);
  return hipGetLastError();
}

template <int LPE, bool KBF16>
hipError_t launch_lpe(const IdxDev& A, int rows, int H_I, int score_dtype, hipStream_t s) {
  switch (H_I) {
    case 1: return launch_hi<1, LPE, KBF16>(A, rows, score_dtype, s);
    case 2: return launch_hi<2, LPE, KBF16>(A, rows, score_dtype, s);
    case 4: return launch_hi<4, LPE, KBF16>(A, rows, score_dtype, s);
    case 8: return launch_hi<8, LPE, KBF16>(A, rows, score_dtype, s);
    case 16: return launch_hi<16, LPE, KBF16>(A, rows, score_dtype, s);
  }
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------------ MXFP4 keys
// Indexer keys stored as MXFP4 (e2m1 codes, one e8m0 scale per 32 channels); the query
// vectors are quantized the same way at block start.  One lane owns one 32-channel block
// of one key (16 code bytes + 1 scale byte), so a wave reads 64 contiguous blocks per
// instruction.  Codes become exact small integers (twice the e2m1 value, in [-12, 12])
// through a byte-permute table, and sdot4 accumulates exact integer block sums; each
// block sum times 2^(e_q + e_k - 2) is exact in fp32.

// 4 codes (one per byte, sign in bit 3) -> 4 int8 holding twice the e2m1 value.
__device__ __forceinline__ uint32_t e2m1x4_to_i8x4(uint32_t c) {
  const uint32_t m = c & 0x07070707u;
  const uint32_t pos = __builtin_amdgcn_perm(0x0C080604u, 0x03020100u, m);  // 0,1,2,3,4,6,8,12
  const uint32_t neg = __builtin_amdgcn_perm(0xF4F8FAFCu, 0xFDFEFF00u, m);  // negated
  const uint32_t mask = ((c >> 3) & 0x01010101u) * 0xFFu;
  return (neg & mask) | (pos & ~mask);
}

struct IdxMxDev {
  const void* q;       // [rows][H_I][d_I] bf16 or f32
  const float* w;      // [rows][H_I]
  const uint8_t* k;    // [B][N][d_I/2] packed codes (bstride bytes)
  const uint8_t* ks;   // [B][N][d_I/32] scale bytes (bstride bytes)
  int64_t k_bstride, ks_bstride;
  int Nq, N, ratio, d_I;
  int64_t pos0;
  void* scores;
  int chunk;
  uint32_t* hist;
  int topk;
};

// grid: (ceil(N / kChunk), rows); block 256.  LPE = d_I / 32 lanes per key.
template <int HI, int LPE, bool QBF16, bool SBF16>
__global__ __launch_bounds__(256) void index_scores_mx_kernel(IdxMxDev A) {
  constexpr int GROUPS = 256 / LPE;
  constexpr int U = 4;
  const int row = blockIdx.y;
  const int b = row / A.Nq;
  const int64_t p = A.pos0 + (row % A.Nq);
  const int64_t nv64 = (p + 1) / A.ratio;
  const int nv = static_cast<int>(nv64 < A.N ? nv64 : A.N);
  const int start = blockIdx.x * A.chunk;
  const int end = min(start + A.chunk, nv);
  if (start >= end) return;
  const int sub = threadIdx.x % LPE;
  const int grp = threadIdx.x / LPE;

  // Quantize every 32-channel block of every query head once per block (LDS), then each
  // lane keeps the blocks it needs: words 0..3 hold elements 8c, 8c+2, 8c+4, 8c+6 and
  // words 4..7 elements 8c+1, 8c+3, 8c+5, 8c+7 (c = word index mod 4), as int8 = 2*value.
  __shared__ uint32_t s_q[16][4][8];
  __shared__ int s_qe[16][4];
  __shared__ uint32_t s_hist[kHistBins];
  const bool hist = A.hist != nullptr && A.topk < nv;
  if (hist)
    for (int i = threadIdx.x; i < kHistBins; i += 256) s_hist[i] = 0;
  if (threadIdx.x < HI * LPE) {
    const int g = threadIdx.x / LPE, blk = threadIdx.x % LPE;
    const int64_t off = (static_cast<int64_t>(row) * HI + g) * A.d_I + blk * 32;
    float amax = 0.0f;
    for (int e = 0; e < 32; ++e) {
      const float v = QBF16 ? bf16_to_f32(static_cast<const uint16_t*>(A.q)[off + e])
                            : static_cast<const float*>(A.q)[off + e];
      amax = fmaxf(amax, __builtin_fabsf(v));
    }
    const int se = mx_scale_exp(amax);
    s_qe[g][blk] = se;
    for (int c = 0; c < 4; ++c) {
      uint32_t lo = 0, hi = 0;
      for (int t = 0; t < 4; ++t) {
        const int64_t i0 = off + 8 * c + 2 * t;
        const float v0 = QBF16 ? bf16_to_f32(static_cast<const uint16_t*>(A.q)[i0])
                               : static_cast<const float*>(A.q)[i0];
        const float v1 = QBF16 ? bf16_to_f32(static_cast<const uint16_t*>(A.q)[i0 + 1])
                               : static_cast<const float*>(A.q)[i0 + 1];
        lo |= (static_cast<uint32_t>(e2m1_twice(e2m1_code(v0, se))) & 0xFFu) << (8 * t);
        hi |= (static_cast<uint32_t>(e2m1_twice(e2m1_code(v1, se))) & 0xFFu) << (8 * t);
      }
      s_q[g][blk][c] = lo;
      s_q[g][blk][4 + c] = hi;
    }
  }
  __syncthreads();
  uint32_t qlo[HI][4], qhi[HI][4];
  int qe[HI];
  float w[HI];
#pragma unroll
  for (int g = 0; g < HI; ++g) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      qlo[g][c] = s_q[g][sub][c];
      qhi[g][c] = s_q[g][sub][4 + c];
    }
    qe[g] = s_qe[g][sub];
    w[g] = A.w[static_cast<int64_t>(row) * HI + g];
  }

  const uint8_t* kbase = A.k + b * A.k_bstride + sub * 16;
  const uint8_t* sbase = A.ks + b * A.ks_bstride + sub;
  const int rowb = A.d_I / 2;
  const int rows_s = A.d_I / 32;
  float* s32 = static_cast<float*>(A.scores) + static_cast<int64_t>(row) * A.N;
  uint16_t* s16 = static_cast<uint16_t*>(A.scores) + static_cast<int64_t>(row) * A.N;

  for (int j0 = start + grp; j0 < end; j0 += GROUPS * U) {
    u32x4 kv[U];
    int ke[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * GROUPS;
      if (j < end) {
        kv[u] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(kbase + static_cast<int64_t>(j) * rowb));
        ke[u] = static_cast<int>(sbase[static_cast<int64_t>(j) * rows_s]) - 127;
      } else {
        kv[u] = u32x4{0, 0, 0, 0};
        ke[u] = 0;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      uint32_t klo[4], khi[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        klo[c] = e2m1x4_to_i8x4(kv[u][c] & 0x0F0F0F0Fu);
        khi[c] = e2m1x4_to_i8x4((kv[u][c] >> 4) & 0x0F0F0F0Fu);
      }
      float part[HI];
#pragma unroll
      for (int g = 0; g < HI; ++g) {
        int acc = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          acc = __builtin_amdgcn_sdot4(static_cast<int>(qlo[g][c]), static_cast<int>(klo[c]), acc, false);
          acc = __builtin_amdgcn_sdot4(static_cast<int>(qhi[g][c]), static_cast<int>(khi[c]), acc, false);
        }
        part[g] = __builtin_ldexpf(static_cast<float>(acc), qe[g] + ke[u] - 2);
      }
#pragma unroll
      for (int o = 1; o < LPE; o <<= 1)
#pragma unroll
        for (int g = 0; g < HI; ++g) part[g] += __shfl_xor(part[g], o, kWave);
      const int j = j0 + u * GROUPS;
      if (sub == 0 && j < end) {
        float s = 0.0f;
#pragma unroll
        for (int g = 0; g < HI; ++g) s = fmaf(w[g], fmaxf(part[g], 0.0f), s);
        s += 0.0f;
        if constexpr (SBF16)
          s16[j] = static_cast<uint16_t>(f32_to_bf16_bits(s));
        else
          s32[j] = s;
        if (hist) hist_add<SBF16>(s_hist, s);
      }
    }
  }
  if (hist) hist_flush(s_hist, A.hist, row, A.N);
}

// MXFP4 keys on the matrix cores: v_mfma_scale_f32_32x32x64_f8f6f4 with e2m1 operands and
// e8m0 scales per 32 channels computes D[head][key] for 32 keys at once (A = the quantized
// query heads as rows, B = the keys as columns), so the e2m1 codes are never unpacked.
// Operand lane layout (measured): lane l holds row/column l % 32 and the 32 channels
// 32*(l/32) .. +31 of one 64-channel step, channel e in bits 4e..4e+3 (the stored packing:
// element 2i in the low nibble of byte i); the scale operand's low byte is that block's
// e8m0 scale; D register r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l % 32.
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

// grid: (ceil(N / chunk), rows); block 256 (4 waves, 32 keys per MFMA).
template <int HI, bool QBF16, bool SBF16>
__global__ __launch_bounds__(256) void index_scores_mx_mfma_kernel(IdxMxDev A) {
  constexpr int U = 4;
  const int row = blockIdx.y;
  const int b = row / A.Nq;
  const int64_t p = A.pos0 + (row % A.Nq);
  const int64_t nv64 = (p + 1) / A.ratio;
  const int nv = static_cast<int>(nv64 < A.N ? nv64 : A.N);
  const int start = blockIdx.x * A.chunk;
  const int end = min(start + A.chunk, nv);
  if (start >= end) return;
  __shared__ uint32_t s_hist[kHistBins];
  const bool hist = A.hist != nullptr && A.topk < nv;
  hist_clear(s_hist, hist);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int ksteps = A.d_I > 64 ? A.d_I / 64 : 1;       // 64-channel MFMA steps
  const int nblk = A.d_I / 32;                          // 32-channel scale blocks per row

  // A operand: this lane's head (col) and block (2*step + half), quantized here.
  i32x8 qa[2];
  int qs[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    qa[st] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
    qs[st] = 127;
    const int blk = 2 * st + half;
    if (st < ksteps && col < HI && blk < nblk) {
      const int64_t off = (static_cast<int64_t>(row) * HI + col) * A.d_I + blk * 32;
      float v[32];
      float amax = 0.0f;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        v[e] = QBF16 ? bf16_to_f32(static_cast<const uint16_t*>(A.q)[off + e])
                     : static_cast<const float*>(A.q)[off + e];
        amax = fmaxf(amax, __builtin_fabsf(v[e]));
      }
      const int se = mx_scale_exp(amax);
      qs[st] = se + 127;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) w |= e2m1_code(v[8 * d + e], se) << (4 * e);
        qa[st][d] = static_cast<int>(w);
      }
    }
  }
  float w[HI];
#pragma unroll
  for (int g = 0; g < HI; ++g) w[g] = A.w[static_cast<int64_t>(row) * HI + g];

  const int rowb = A.d_I / 2;
  const uint8_t* kbase = A.k + b * A.k_bstride;
  const uint8_t* sbase = A.ks + b * A.ks_bstride;
  float* s32 = static_cast<float*>(A.scores) + static_cast<int64_t>(row) * A.N;
  uint16_t* s16 = static_cast<uint16_t*>(A.scores) + static_cast<int64_t>(row) * A.N;

  for (int j0 = start + wave * 32; j0 < end; j0 += 4 * 32 * U) {
    i32x8 kb[U][2];
    int ksc[U][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * 128 + col;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        kb[u][st] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
        ksc[u][st] = 127;
        const int blk = 2 * st + half;
        if (st < ksteps && blk < nblk && j < end) {
          const u32x4 c = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4*>(kbase + static_cast<int64_t>(j) * rowb + blk * 16));
          kb[u][st][0] = static_cast<int>(c[0]);
          kb[u][st][1] = static_cast<int>(c[1]);
          kb[u][st][2] = static_cast<int>(c[2]);
          kb[u][st][3] = static_cast<int>(c[3]);
          ksc[u][st] = sbase[static_cast<int64_t>(j) * nblk + blk];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (j0 + u * 128 >= end) break;                 // wave-uniform
      f32x16 d = {};
      d = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa[0], kb[u][0], d, 4, 4, 0, qs[0],
                                                          0, ksc[u][0]);
      if (ksteps > 1)
        d = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa[1], kb[u][1], d, 4, 4, 0,
                                                            qs[1], 0, ksc[u][1]);
      // rows (heads) held by this lane: 8*(r/4) + 4*half + r%4
      float part = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int g = 8 * (r >> 2) + 4 * half + (r & 3);
        if (g < HI) part = fmaf(w[g], fmaxf(d[r], 0.0f), part);
      }
      if constexpr (HI > 4) part += __shfl_xor(part, 32, kWave);
      const int j = j0 + u * 128 + col;
      if (half == 0 && j < end) {
        const float s = part + 0.0f;
        if constexpr (SBF16)
          s16[j] = static_cast<uint16_t>(f32_to_bf16_bits(s));
        else
          s32[j] = s;
        if (hist) hist_add<SBF16>(s_hist, s);
      }
    }
  }
  if (hist) hist_flush(s_hist, A.hist, row, A.N);
}

template <int HI, bool QBF16>
hipError_t launch_mx_mfma_hi(const IdxMxDev& A, int rows, int score_dtype, hipStream_t s) {
  const int nchunks = (A.N + A.chunk - 1) / A.chunk;
  dim3 grid(nchunks, rows);
  if (score_dtype == 1)
    launch_timed(index_scores_mx_mfma_kernel<HI, QBF16, true>, grid, dim3(256), s, A);
  else
    launch_timed(index_scores_mx_mfma_kernel<HI, QBF16, false>, grid, dim3(256), s, A);
  return hipGetLastError();
}

template <bool QBF16>
hipError_t launch_mx_mfma(const IdxMxDev& A, int rows, int H_I, int score_dtype, hipStream_t s) {
  switch (H_I) {
    case 1: return launch_mx_mfma_hi<1, QBF16>(A, rows, score_dtype, s);
    case 2: return launch_mx_mfma_hi<2, QBF16>(A, rows, score_dtype, s);
    case 4: return launch_mx_mfma_hi<4, QBF16>(A, rows, score_dtype, s);
    case 8: return launch_mx_mfma_hi<8, QBF16>(A, rows, score_dtype, s);
    case 16: return launch_mx_mfma_hi<16, QBF16>(A, rows, score_dtype, s);
  }
  return hipErrorInvalidValue;
}

template <int HI, int LPE, bool QBF16>
hipError_t launch_mx_hi(const IdxMxDev& A, int rows, int score_dtype, hipStream_t s) {
  const int nchunks = (A.N + A.chunk - 1) / A.chunk;
  dim3 grid(nchunks, rows);
  if (score_dtype == 1)
    index_scores_mx_kernel<HI, LPE, QBF16, true><<<grid, 256, 0, s>>>(A);
  else
    index_scores_mx_kernel<HI, LPE, QBF16, false><<<grid, 256, 0, s>>>(A);
  return hipGetLastError();
}

template <int LPE, bool QBF16>
hipError_t launch_mx_lpe(const IdxMxDev& A, int rows, int H_I, int score_dtype, hipStream_t s) {
  switch (H_I) {
    case 1: return launch_mx_hi<1, LPE, QBF16>(A, rows, score_dtype, s);
    case 2: return launch_mx_hi<2, LPE, QBF16>(A, rows, score_dtype, s);
    case 4: return launch_mx_hi<4, LPE, QBF16>(A, rows, score_dtype, s);
    case 8: return launch_mx_hi<8, LPE, QBF16>(A, rows, score_dtype, s);
    case 16: return launch_mx_hi<16, LPE, QBF16>(A, rows, score_dtype, s);
  }
  return hipErrorInvalidValue;
}

template <bool QBF16>
hipError_t launch_mx_q(const IdxMxDev& A, int rows, int H_I, int score_dtype, hipStream_t s) {
  switch (A.d_I / 32) {
    case 1: return launch_mx_lpe<1, QBF16>(A, rows, H_I, score_dtype, s);
    case 2: return launch_mx_lpe<2, QBF16>(A, rows, H_I, score_dtype, s);
    case 4: return launch_mx_lpe<4, QBF16>(A, rows, H_I, score_dtype, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_mxfp4_index_scores(const void* q, int q_dtype, const float* w,
                                     const uint8_t* kx, int64_t k_bstride, const uint8_t* ks,
                                     int64_t ks_bstride, int B, int Nq, int H_I, int d_I,
                                     int N, int ratio, int64_t pos0, int score_dtype,
                                     void* scores, uint32_t* hist, int k, hipStream_t s) {
  IdxMxDev A;
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
  A.scores = scores;
  A.chunk = index_chunk(B * Nq, N);
  if (hist != nullptr && topk_uses_rows_path(plan_topk(score_dtype, B * Nq, N, k))) hist = nullptr;
  A.hist = hist;
  A.topk = k;
  if (q_dtype == 1) return launch_mx_mfma<true>(A, B * Nq, H_I, score_dtype, s);
  return launch_mx_mfma<false>(A, B * Nq, H_I, score_dtype, s);
}


hipError_t launch_index_scores(const void* q, int q_dtype, const float* w, const void* kx,
                               int k_dtype, int64_t k_bstride, const uint8_t* ks,
                               int64_t ks_bstride, int B, int Nq, int H_I, int d_I, int N,
                               int ratio, int64_t pos0, int score_dtype, void* scores,
                               uint32_t* hist, int k, hipStream_t s) {
  if (k_dtype == 2)
    return launch_mxfp4_index_scores(q, q_dtype, w, static_cast<const uint8_t*>(kx), k_bstride,
                                     ks, ks_bstride, B, Nq, H_I, d_I, N, ratio, pos0,
                                     score_dtype, scores, hist, k, s);
  IdxDev A;
  A.q = q;
  A.w = w;
  A.k = kx;
  A.k_bstride = k_bstride;
  A.Nq = Nq;
  A.N = N;
  A.ratio = ratio;
  A.d_I = d_I;
  A.pos0 = pos0;
  A.scores = scores;
  A.chunk = index_chunk(B * Nq, N);
  // rows resolved one block per row need no shared histogram
  if (hist != nullptr && topk_uses_rows_path(plan_topk(score_dtype, B * Nq, N, k))) hist = nullptr;
  A.hist = hist;
  A.topk = k;
  const int rows = B * Nq;
  // many query tokens per sequence: the GEMM form on the matrix cores
  if (k_dtype == 1 && (H_I == 1 || H_I == 2 || H_I == 4) && Nq * H_I >= 128 &&
      (Nq * H_I) % 32 == 0 && d_I % 16 == 0 && d_I <= 128) {
    A.rows_total = rows * H_I;
    A.chunk = 4096;
    dim3 grid((N + A.chunk - 1) / A.chunk, (A.rows_total + 127) / 128);
    hipError_t e;
    if (H_I == 1) {
      if (score_dtype == 1) launch_timed(index_scores_gemm_kernel<1, true>, grid, dim3(256), s, A);
      else launch_timed(index_scores_gemm_kernel<1, false>, grid, dim3(256), s, A);
    } else if (H_I == 2) {
      if (score_dtype == 1) launch_timed(index_scores_gemm_kernel<2, true>, grid, dim3(256), s, A);
      else launch_timed(index_scores_gemm_kernel<2, false>, grid, dim3(256), s, A);
    } else {
      if (score_dtype == 1) launch_timed(index_scores_gemm_kernel<4, true>, grid, dim3(256), s, A);
      else launch_timed(index_scores_gemm_kernel<4, false>, grid, dim3(256), s, A);
    }
    e = hipGetLastError();
    if (e != hipSuccess || hist == nullptr) return e;
    return launch_sel_hist(scores, score_dtype, N, B, Nq, N, ratio, pos0, k, hist, s);
  }
  const int lpe = d_I * (k_dtype == 1 ? 2 : 4) / 16;
  if (k_dtype == 1) {
    if (lpe == 4) return launch_lpe<4, true>(A, rows, H_I, score_dtype, s);
    if (lpe == 8) return launch_lpe<8, true>(A, rows, H_I, score_dtype, s);
    if (lpe == 16) return launch_lpe<16, true>(A, rows, H_I, score_dtype, s);
  } else {
    if (lpe == 8) return launch_lpe<8, false>(A, rows, H_I, score_dtype, s);
    if (lpe == 16) return launch_lpe<16, false>(A, rows, H_I, score_dtype, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace hcsa
