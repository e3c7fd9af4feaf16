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
#include "select_dev.h"
#include "pool_dev.h"
#include "mx_dev.h"
#include "mx_scan.h"

namespace hcsa {

// Optional timing of the next indexer kernel launched on this thread: the dispatch itself
// records the start and stop events (hipExtLaunchKernel), so the measured interval is the
// kernel's own execution.
static thread_local hipEvent_t t_ev_start = nullptr, t_ev_stop = nullptr;

void time_next_indexer(hipEvent_t start, hipEvent_t stop) {
  t_ev_start = start;
  t_ev_stop = stop;
}

bool take_indexer_timing(hipEvent_t* start, hipEvent_t* stop) {
  if (t_ev_start == nullptr) return false;
  *start = t_ev_start;
  *stop = t_ev_stop;
  t_ev_start = t_ev_stop = nullptr;
  return true;
}

namespace {

struct IdxDev {
  const void* q;     // [rows][H_I][d_I]
  const float* w;    // [rows][H_I]
  const void* k;     // [B][N][d_I] (bstride elements)
  int64_t k_bstride;
  int Nq, N, ratio, d_I;
  int64_t pos0;
  const int64_t* seq_pos;   // [B] or null
  PageMap pm;        // paged keys (table null: contiguous)
  int c_log2;        // log2 of the keys' rows per page
  void* scores;      // [rows][N]
  int chunk;
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

// grid: (ceil(N / chunk), rows); block 256.
template <int HI, int LPE, bool KBF16, bool SBF16, bool PAGED>
__global__ __launch_bounds__(256) void index_scores_kernel(IdxDev A) {
  constexpr int ES = KBF16 ? 2 : 4;
  constexpr int GROUPS = 256 / LPE;
  constexpr int U = 4;
  const int row = blockIdx.y;
  const int b = row / A.Nq;
  const int64_t p = query_pos(A.seq_pos, A.pos0, b, row % A.Nq);
  const int64_t nv64 = (p + 1) / A.ratio;
  const int nv = static_cast<int>(nv64 < A.N ? nv64 : A.N);
  const int start = blockIdx.x * A.chunk;
  const int end = min(start + A.chunk, nv);
  if (start >= end) return;

  const int sub = threadIdx.x % LPE;
  const int grp = threadIdx.x / LPE;
  const int row_bytes = A.d_I * ES;

  u32x4 qv[HI];
  float w[HI];
  const char* qrow = static_cast<const char*>(A.q) + static_cast<int64_t>(row) * HI * row_bytes;
#pragma unroll
  for (int g = 0; g < HI; ++g) {
    qv[g] = *reinterpret_cast<const u32x4*>(qrow + g * row_bytes + sub * 16);
    w[g] = A.w[static_cast<int64_t>(row) * HI + g];
  }
  const char* kbase = static_cast<const char*>(A.k) + sub * 16;
  float* s32 = static_cast<float*>(A.scores) + static_cast<int64_t>(row) * A.N;
  uint16_t* s16 = static_cast<uint16_t*>(A.scores) + static_cast<int64_t>(row) * A.N;

  for (int j0 = start + grp; j0 < end; j0 += GROUPS * U) {
    u32x4 kv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * GROUPS;
      if (j < end)
        kv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
            kbase + row_off<PAGED>(A.pm, A.k_bstride * ES, b, j, A.c_log2, row_bytes)));
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
        for (int g = 0; g < HI; ++g) s = fmaf(w[g], relu(part[g]), s);
        s += 0.0f;  // -0 -> +0
        if constexpr (SBF16)
          s16[j] = static_cast<uint16_t>(f32_to_bf16_bits(s));
        else
          s32[j] = s;
      }
    }
  }
}

// ------------------------------------------------------------------ prefill GEMM
// Many query tokens per sequence (chunked prefill): the indexer is a GEMM
// [Nq*H_I x d_I] x [d_I x N] on v_mfma_f32_32x32x16_bf16.  A block of W waves owns 32*W
// consecutive rows (row = query token * H_I + head, all in one sequence); each wave keeps
// its 32-row tile of operand A in registers.  The block walks its key range 128 keys at a
// time: the 128 x d_I key tile is loaded once per block into LDS (double buffered, the next
// tile's global loads in flight during the current tile's MFMAs) and every wave reads its
// operand B from there.  Within a tile the four 32-key sub-tiles ping-pong between two
// accumulator sets, so one sub-tile's epilogue overlaps the next one's MFMAs.  Output lane
// layout: register r of lane l holds row 8*(r/4) + 4*(l/32) + r%4 of the tile and key l%32,
// so the H_I <= 4 heads of a query token sit in consecutive registers of one lane and the
// ReLU / weight / head-sum epilogue is lane-local.  A wave stages its tokens' scores in LDS
// and writes them with 16-byte stores: a whole 128-key tile per token (one 256-byte run at
// bf16) when every token of the block sees the tile and the staging fits in 4 KB per wave,
// else each 32-key sub-tile; sub-tiles that straddle the causal edge of the block's tokens are
// written score by score, masked.  The kernel is held to four waves per SIMD.
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16g;

// fp32 -> bf16 bits, round to nearest even (the gfx950 conversion instruction): a pair
// (a in the low half) and one value
__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  typedef float f32x2v __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{a, b}, bf16x2v));
}
__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return static_cast<uint16_t>(bf16_pair(x, x) & 0xffffu);
}

constexpr int kGemmKeys = 32;           // keys per MFMA tile
constexpr int kGemmTile = 128;          // keys per LDS tile (four MFMA tiles)

template <int HI, bool SBF16, int KSTEPS, int NT>
__global__ __launch_bounds__(NT, 4) void index_scores_gemm_kernel(IdxDev A) {
  constexpr int DI = KSTEPS * 16;                 // channels
  constexpr int STRIDE = DI + 8;                  // LDS row pitch (elements): no bank conflicts
  constexpr int CHUNKS = kGemmTile * DI / 8;      // 16-byte pieces of one key tile
  constexpr int QPL = 16 / HI;                    // query tokens per lane
  constexpr int TOK = 32 / HI;                    // query tokens of a wave
  constexpr int ES = SBF16 ? 2 : 4;               // score bytes
  __shared__ __align__(16) uint16_t s_k[2][kGemmTile * STRIDE];
  // a whole tile's scores of the wave's tokens are staged when they fit in 4 KB per wave,
  // so each token's 128 scores leave as one contiguous run
  constexpr bool STAGE = TOK * kGemmTile * ES <= 4096;
  constexpr int SO = (STAGE ? kGemmTile : kGemmKeys) * TOK * ES / 4;
  __shared__ __align__(16) uint32_t s_o[NT / 64][SO];   // per wave
  // 16-byte score stores need 16-byte aligned rows
  const bool vec_out = (A.N * ES) % 16 == 0 && reinterpret_cast<uintptr_t>(A.scores) % 16 == 0;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 31, half = lane >> 5;
  constexpr int64_t rows_block = NT / 64 * 32;
  const int64_t row0_block = blockIdx.y * rows_block;
  const int64_t row0 = row0_block + static_cast<int64_t>(wave) * 32;   // wave's first row
  const int64_t tok0 = row0 / HI;                 // the wave's first query token
  const int b = static_cast<int>(row0_block / HI) / A.Nq;   // the block's sequence
  const int kstart = blockIdx.x * A.chunk;
  const int kend = min(kstart + A.chunk, A.N);
  auto visible_tok = [&](int64_t tok) -> int {
    const int64_t p = query_pos(A.seq_pos, A.pos0, b, static_cast<int>(tok % A.Nq));
    const int64_t v = (p + 1) / A.ratio;
    return static_cast<int>(v < A.N ? v : A.N);
  };
  // tokens ascend with rows: the block's first token sees the fewest keys, its last the most
  const int nv_lo = visible_tok(row0_block / HI);
  const int kstop = min(kend, visible_tok((row0_block + rows_block - 1) / HI));
  if (kstart >= kstop) return;                    // whole block: no barrier reached

  u32x4 qa[KSTEPS];                               // operand A: row col, 16 channels per step
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(A.q) + (row0 + col) * DI + 8 * half;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qa[s] = *reinterpret_cast<const u32x4*>(qrow + 16 * s);
  }
  // this lane's score groups t: rows 8*(t*HI/4) + 4*half + t*HI%4 .. +HI-1 of the tile
  float w[QPL][HI];
  int qloc[QPL];                    // token within the wave
  int nvt[QPL];                     // its visible count (sub-tiles at the causal edge)
#pragma unroll
  for (int t = 0; t < QPL; ++t) {
    const int r0 = t * HI;
    qloc[t] = (8 * (r0 >> 2) + 4 * half + (r0 & 3)) / HI;
#pragma unroll
    for (int g = 0; g < HI; ++g) w[t][g] = A.w[(tok0 + qloc[t]) * HI + g];
    nvt[t] = visible_tok(tok0 + qloc[t]);
  }
  const uint16_t* kpool = static_cast<const uint16_t*>(A.k);
  auto krow = [&](int j) -> int64_t {
    return A.pm.table ? row_off<true>(A.pm, 0, b, j, A.c_log2, DI)
                      : static_cast<int64_t>(b) * A.k_bstride + static_cast<int64_t>(j) * DI;
  };
  constexpr int PPT = (CHUNKS + NT - 1) / NT;     // key-tile pieces per thread
  u32x4 pf[PPT];
  auto fetch = [&](int j0) {
    if (!A.pm.table && j0 + kGemmTile <= A.N) {
      // contiguous keys, the whole tile in the row: one run of kGemmTile * DI elements,
      // piece c at element 8c
      const uint16_t* tile = kpool + static_cast<int64_t>(b) * A.k_bstride +
                             static_cast<int64_t>(j0) * DI;
#pragma unroll
      for (int u = 0; u < PPT; ++u) {
        const int c = threadIdx.x + u * NT;
        pf[u] = c < CHUNKS ? *reinterpret_cast<const u32x4*>(tile + 8 * c) : u32x4{0u, 0u, 0u, 0u};
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int c = threadIdx.x + u * NT;
      const int key = c / (DI / 8), part = c % (DI / 8);
      pf[u] = (c < CHUNKS && j0 + key < A.N)
                  ? *reinterpret_cast<const u32x4*>(kpool + krow(j0 + key) + 8 * part)
                  : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int c = threadIdx.x + u * NT;
      if (c < CHUNKS) {
        const int key = c / (DI / 8), part = c % (DI / 8);
        *reinterpret_cast<u32x4*>(&s_k[buf][key * STRIDE + 8 * part]) = pf[u];
      }
    }
  };
  auto mma = [&](f32x16g& d, int buf, int sub) {
    u32x4 kb[KSTEPS];                             // operand B: key col, channels 16s + 8*half
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
      kb[s] = *reinterpret_cast<const u32x4*>(
          &s_k[buf][(sub * kGemmKeys + col) * STRIDE + 16 * s + 8 * half]);
    d = f32x16g{};
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
      d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, qa[s]),
                                                  __builtin_bit_cast(bf16x8, kb[s]), d, 0, 0, 0);
  };
  // scores sum_g w_g max(d_g, 0) of the sub-tile starting at key js (a +0-started chain
  // never ends at -0)
  auto emit = [&](const f32x16g& d, int js, bool stage, int u) {
    const int j = js + col;
    float sc[QPL];
#pragma unroll
    for (int t = 0; t < QPL; ++t) {
      float v = 0.0f;
#pragma unroll
      for (int g = 0; g < HI; ++g) v = fmaf(w[t][g], relu(d[t * HI + g]), v);
      sc[t] = v;
    }
    if (STAGE && stage) {
      // into the wave's staging rows (one per token, kGemmTile scores), sub-tile u
#pragma unroll
      for (int t = 0; t < QPL; t += 2) {
        if constexpr (SBF16) {
          uint16_t* o16 = reinterpret_cast<uint16_t*>(&s_o[wave][0]);
          const uint32_t pk = bf16_pair(sc[t], sc[t + 1]);
          o16[qloc[t] * kGemmTile + u * kGemmKeys + col] = static_cast<uint16_t>(pk & 0xffffu);
          o16[qloc[t + 1] * kGemmTile + u * kGemmKeys + col] = static_cast<uint16_t>(pk >> 16);
        } else {
          float* o32 = reinterpret_cast<float*>(&s_o[wave][0]);
          o32[qloc[t] * kGemmTile + u * kGemmKeys + col] = sc[t];
          o32[qloc[t + 1] * kGemmTile + u * kGemmKeys + col] = sc[t + 1];
        }
      }
      return;
    }
    if (vec_out && js + kGemmKeys <= nv_lo) {
      // every token of the block sees the whole sub-tile
#pragma unroll
      for (int t = 0; t < QPL; t += 2) {
        if constexpr (SBF16) {
          uint16_t* o16 = reinterpret_cast<uint16_t*>(&s_o[wave][0]);
          const uint32_t pk = bf16_pair(sc[t], sc[t + 1]);
          o16[qloc[t] * kGemmKeys + col] = static_cast<uint16_t>(pk & 0xffffu);
          o16[qloc[t + 1] * kGemmKeys + col] = static_cast<uint16_t>(pk >> 16);
        } else {
          float* o32 = reinterpret_cast<float*>(&s_o[wave][0]);
          o32[qloc[t] * kGemmKeys + col] = sc[t];
          o32[qloc[t + 1] * kGemmKeys + col] = sc[t + 1];
        }
      }
      constexpr int EPP = 16 / ES;                 // scores per 16-byte piece
      constexpr int PPQ = kGemmKeys / EPP;         // pieces per token
      constexpr int NPIECE = TOK * PPQ;
#pragma unroll
      for (int p0 = 0; p0 < NPIECE; p0 += 64) {
        const int p = p0 + lane;
        if (NPIECE % 64 == 0 || p < NPIECE) {
          const int ql = p / PPQ, kp = p % PPQ;
          const u32x4 v = *reinterpret_cast<const u32x4*>(
              reinterpret_cast<const char*>(&s_o[wave][0]) + (ql * kGemmKeys + kp * EPP) * ES);
          *reinterpret_cast<u32x4*>(static_cast<char*>(A.scores) +
                                    ((tok0 + ql) * A.N + js + kp * EPP) * ES) = v;
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < QPL; ++t) {
        if (j < nvt[t] && j < kstop) {
          const int64_t o = (tok0 + qloc[t]) * A.N + j;
          if constexpr (SBF16)
            static_cast<uint16_t*>(A.scores)[o] = bf16_bits(sc[t]);
          else
            static_cast<float*>(A.scores)[o] = sc[t];
        }
      }
    }
  };

  // a staged tile's scores: token ql's kGemmTile scores from key j0 as 16-byte pieces
  auto store_tile = [&](int j0) {
    constexpr int EPP = 16 / ES;                 // scores per 16-byte piece
    constexpr int PPQ = kGemmTile / EPP;         // pieces per token
    constexpr int NPIECE = TOK * PPQ;
#pragma unroll
    for (int p0 = 0; p0 < NPIECE; p0 += 64) {
      const int p = p0 + lane;
      if (NPIECE % 64 == 0 || p < NPIECE) {
        const int ql = p / PPQ, kp = p % PPQ;
        const u32x4 v = *reinterpret_cast<const u32x4*>(
            reinterpret_cast<const char*>(&s_o[wave][0]) + (ql * kGemmTile + kp * EPP) * ES);
        *reinterpret_cast<u32x4*>(static_cast<char*>(A.scores) +
                                  ((tok0 + ql) * A.N + j0 + kp * EPP) * ES) = v;
      }
    }
  };

  fetch(kstart);
  stash(0);
  __syncthreads();
  int buf = 0;
  for (int j0 = kstart; j0 < kstop; j0 += kGemmTile) {
    const bool more = j0 + kGemmTile < kstop;
    if (more) fetch(j0 + kGemmTile);              // in flight during this tile
    const int nsub = min(kGemmTile, kstop - j0 + kGemmKeys - 1) / kGemmKeys;   // block-uniform
    // every token of the block sees the whole tile: stage it and store whole runs
    const bool stage = STAGE && vec_out && j0 + kGemmTile <= nv_lo;   // block-uniform
    f32x16g da, db;
    mma(da, buf, 0);
#pragma unroll
    for (int u = 0; u < kGemmTile / kGemmKeys; u += 2) {
      if (u + 1 < nsub) mma(db, buf, u + 1);
      if (u < nsub) emit(da, j0 + u * kGemmKeys, stage, u);
      if (u + 2 < nsub) mma(da, buf, u + 2);
      if (u + 1 < nsub) emit(db, j0 + (u + 1) * kGemmKeys, stage, u + 1);
    }
    if (stage) store_tile(j0);
    if (more) stash(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
}

template <int HI, int LPE, bool KBF16>
hipError_t launch_hi(const IdxDev& A, int rows, int score_dtype, hipStream_t s) {
  const int nchunks = (A.N + A.chunk - 1) / A.chunk;
  dim3 grid(nchunks, rows);
  if (score_dtype == 1)
    if (A.pm.table) launch_timed(index_scores_kernel<HI, LPE, KBF16, true, true>, grid, dim3(256), s, A);
    else launch_timed(index_scores_kernel<HI, LPE, KBF16, true, false>, grid, dim3(256), s, A);
  else
    if (A.pm.table) launch_timed(index_scores_kernel<HI, LPE, KBF16, false, true>, grid, dim3(256), s, A);
    else launch_timed(index_scores_kernel<HI, LPE, KBF16, false, false>, grid, dim3(256), s, A);
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

}  // namespace

hipError_t launch_index_scores(const void* q, int q_dtype, const float* w, const void* kx,
                               int k_dtype, int64_t k_bstride, const uint8_t* ks,
                               int64_t ks_bstride, int B, int Nq, int H_I, int d_I, int N,
                               int ratio, int64_t pos0, const int64_t* seq_pos,
                               const int32_t* block_table, int64_t table_stride,
                               int score_dtype, void* scores, hipStream_t s) {
  if (k_dtype == 2 || k_dtype == 3)   // MXFP4 keys: e2m1 operands, or widened to e4m3
    return launch_mxfp4_index_scores(q, q_dtype, w, static_cast<const uint8_t*>(kx), k_bstride,
                                     ks, ks_bstride, B, Nq, H_I, d_I, N, ratio, pos0, seq_pos,
                                     block_table, table_stride, score_dtype, scores,
                                     k_dtype == 3, s);
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
  A.seq_pos = seq_pos;
  A.pm.table = block_table;
  A.pm.stride = table_stride;
  A.c_log2 = page_rows_log2(ratio);
  A.scores = scores;
  A.chunk = index_chunk(B * Nq, N);
  const int rows = B * Nq;
  // many query tokens per sequence: the GEMM form on the matrix cores, for sequences whose
  // rows split into whole blocks of 256 rows (8 waves) or 128 rows (4 waves)
  const int seq_rows = Nq * H_I;
  if (k_dtype == 1 && (H_I == 1 || H_I == 2 || H_I == 4) && seq_rows % 128 == 0 &&
      (d_I == 32 || d_I == 64 || d_I == 128)) {
    A.rows_total = rows * H_I;
    const int nt = seq_rows % 256 == 0 ? 512 : 256;
    A.chunk = 2048;
    dim3 grid((N + A.chunk - 1) / A.chunk, A.rows_total / (nt / 2));
    dim3 block(nt);
    const bool sb = score_dtype == 1;
#define HCSA_GEMM(HI_, KS_, NT_)                                                        \
  if (H_I == HI_ && d_I == 16 * KS_ && nt == NT_) {                                    \
    if (sb) launch_timed(index_scores_gemm_kernel<HI_, true, KS_, NT_>, grid, block, s, A); \
    else launch_timed(index_scores_gemm_kernel<HI_, false, KS_, NT_>, grid, block, s, A);   \
  }
#define HCSA_GEMM_HI(HI_) \
  HCSA_GEMM(HI_, 2, 256) HCSA_GEMM(HI_, 2, 512) HCSA_GEMM(HI_, 4, 256) \
  HCSA_GEMM(HI_, 4, 512) HCSA_GEMM(HI_, 8, 256) HCSA_GEMM(HI_, 8, 512)
    HCSA_GEMM_HI(1) HCSA_GEMM_HI(2) HCSA_GEMM_HI(4)
#undef HCSA_GEMM_HI
#undef HCSA_GEMM
    return hipGetLastError();
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
