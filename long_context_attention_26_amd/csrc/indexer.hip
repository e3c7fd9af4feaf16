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
  const int64_t* seq_pos;   // [B] or null
  PageMap pm;        // paged keys (table null: contiguous)
  int c_log2;        // log2 of the keys' rows per page
  void* scores;      // [rows][N]
  int chunk;
  int rows_total;    // B*Nq*H_I (prefill GEMM)
};

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
// ReLU / weight / head-sum epilogue is lane-local.  A wave stages a sub-tile's scores in LDS
// as [token][32 keys] and writes each token's 32 scores with 16-byte stores; sub-tiles that
// straddle the causal edge of the block's tokens are written score by score, masked.
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
__global__ __launch_bounds__(NT) void index_scores_gemm_kernel(IdxDev A) {
  constexpr int DI = KSTEPS * 16;                 // channels
  constexpr int STRIDE = DI + 8;                  // LDS row pitch (elements): no bank conflicts
  constexpr int CHUNKS = kGemmTile * DI / 8;      // 16-byte pieces of one key tile
  constexpr int QPL = 16 / HI;                    // query tokens per lane
  constexpr int TOK = 32 / HI;                    // query tokens of a wave
  constexpr int ES = SBF16 ? 2 : 4;               // score bytes
  __shared__ __align__(16) uint16_t s_k[2][kGemmTile * STRIDE];
  __shared__ __align__(16) uint32_t s_o[NT / 64][TOK * kGemmKeys * ES / 4];   // per wave
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
  auto emit = [&](const f32x16g& d, int js) {
    const int j = js + col;
    float sc[QPL];
#pragma unroll
    for (int t = 0; t < QPL; ++t) {
      float v = 0.0f;
#pragma unroll
      for (int g = 0; g < HI; ++g) v = fmaf(w[t][g], relu(d[t * HI + g]), v);
      sc[t] = v;
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

  fetch(kstart);
  stash(0);
  __syncthreads();
  int buf = 0;
  for (int j0 = kstart; j0 < kstop; j0 += kGemmTile) {
    const bool more = j0 + kGemmTile < kstop;
    if (more) fetch(j0 + kGemmTile);              // in flight during this tile
    const int nsub = min(kGemmTile, kstop - j0 + kGemmKeys - 1) / kGemmKeys;   // block-uniform
    f32x16g da, db;
    mma(da, buf, 0);
#pragma unroll
    for (int u = 0; u < kGemmTile / kGemmKeys; u += 2) {
      if (u + 1 < nsub) mma(db, buf, u + 1);
      if (u < nsub) emit(da, j0 + u * kGemmKeys);
      if (u + 2 < nsub) mma(da, buf, u + 2);
      if (u + 1 < nsub) emit(db, j0 + (u + 1) * kGemmKeys);
    }
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
  uint32_t* floor;     // [rows] 16-bit key floor of each row
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
  if constexpr (HI > 4) part += __shfl_xor(part, 32, kWave);
  return part + 0.0f;
}

// grid: (ceil(N / chunk), rows); block 256 (4 waves, 32 keys per MFMA).  Wave w takes keys
// j0 + 128u + lane%32 of the block's chunk, j0 = start + 32w + 512i, u < 4: step (i, u)
// covers 128 consecutive keys in wave order.
//  - Scores: every visible key's score, rounded to the score dtype.
//  - Candidate lists (CAND, bf16 scores): the keys whose bf16 score key is >= the row's
//    floor, as (key << 16 | index in the chunk), in index order: each wave stages a step's
//    candidates in LDS by ballot rank, and at the end the block writes the groups (step,
//    wave) in order, with its count.  Chunks are at most 2048 keys (64 groups of 32).
template <int HI, int KS, bool QBF16, bool SBF16, bool PAGED, bool F8, bool CAND>
__global__ __launch_bounds__(256) void index_scores_mx_mfma_kernel(IdxMxDev A) {
  constexpr int U = 4;
  const int row = blockIdx.y;
  const int b = row / A.Nq;
  const int64_t p = query_pos(A.seq_pos, A.pos0, b, row % A.Nq);
  const int64_t nv64 = (p + 1) / A.ratio;
  const int nv = static_cast<int>(nv64 < A.N ? nv64 : A.N);
  const int start = blockIdx.x * A.chunk;
  const int end = min(start + A.chunk, nv);
  if (start >= end) return;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int ksteps = A.d_I > 64 ? A.d_I / 64 : 1;
  __shared__ uint32_t s_qa[kMxMaxUnits][4];
  __shared__ int s_qs[kMxMaxUnits];
  __shared__ uint32_t s_stage[CAND ? 2048 : 1];
  __shared__ int s_cnt[CAND ? 64 : 1], s_off[CAND ? 64 : 1];
  uint32_t L = 0;
  if constexpr (CAND) {
    L = A.floor[row];
    if (threadIdx.x < 64) s_cnt[threadIdx.x] = 0;   // ordered by the barrier in mx_query
  }
  const MxQuery<HI, KS> Q = mx_query<HI, KS, QBF16, F8>(A, row, s_qa, s_qs);

  const uint8_t* kbase = PAGED ? A.k : A.k + b * A.k_bstride;
  const uint8_t* sbase = PAGED ? A.ks : A.ks + b * A.ks_bstride;
  float* s32 = static_cast<float*>(A.scores) + static_cast<int64_t>(row) * A.N;
  uint16_t* s16 = static_cast<uint16_t*>(A.scores) + static_cast<int64_t>(row) * A.N;

  int it = 0;
  for (int j0 = start + wave * 32; j0 < end; j0 += 4 * 32 * U, ++it) {
    u32x4 kraw[U][KS];
    int ksc[U][KS];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * 128 + col;
      mx_load<KS, PAGED, F8>(A, kbase, sbase, b, j, j < end, kraw[u], ksc[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (j0 + u * 128 >= end) break;                 // wave-uniform
      const float s = mx_score<HI, KS, F8>(Q, kraw[u], ksc[u], ksteps);
      const int j = j0 + u * 128 + col;
      if constexpr (CAND) {
        const uint32_t kk = bf16_key(f32_to_bf16_bits(s));
        const bool c = half == 0 && j < end && kk >= L;
        const uint64_t m = __ballot(c);
        const int g = (it * U + u) * 4 + wave;
        if (c) s_stage[g * 32 + ballot_rank(m)] = (kk << 16) | static_cast<uint32_t>(j - start);
        if (lane == 0) s_cnt[g] = __popcll(m);
      } else if (half == 0 && j < end) {
        if constexpr (SBF16)
          s16[j] = static_cast<uint16_t>(f32_to_bf16_bits(s));
        else
          s32[j] = s;
      }
    }
  }
  if constexpr (CAND) {
    __syncthreads();
    if (threadIdx.x < 64) {                       // offsets of the groups in (step, wave) order
      const int c = s_cnt[threadIdx.x];
      int inc = c;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(inc, d, kWave);
        if (lane >= d) inc += y;
      }
      s_off[threadIdx.x] = inc - c;
      if (threadIdx.x == 63) A.counts[static_cast<int64_t>(row) * A.nchunks + blockIdx.x] = inc;
    }
    __syncthreads();
    uint32_t* out = A.lists + (static_cast<int64_t>(row) * A.nchunks + blockIdx.x) * A.chunk;
    const int g = threadIdx.x >> 2;
    const int c = s_cnt[g], o = s_off[g];
    for (int i = threadIdx.x & 3; i < c; i += 4) out[o + i] = s_stage[g * 32 + i];
  }
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
constexpr int kMxResThreads = 512;
constexpr int kMxResPer = 32;
constexpr int kMxResMax = kMxResThreads * kMxResPer;
constexpr int kMxMaxChunks = 4096;

// grid: rows; block 512.  Scores 32 runs of 128 consecutive visible keys at evenly spaced
// positions and sets the row's floor: the 16-bit key of about the m-th largest sample, m
// about twice the rank at which the k-th largest key is expected (only the candidate count
// depends on it).  For shallow ranks it is the m-th largest of the 512 per-thread maxima
// (8 consecutive samples each), which is at or below the m-th largest sample, found exactly
// by one wave (radix 4 from the top, ballot counts); deeper ranks count every sample, each
// wave its own ceil(m/W)-th, and take the smallest of the W.  Rows of at most 4096 visible
// keys take every key (floor 0).  All sample loads are issued before the query is
// quantized.
//
// prior_only: sample only the entries completed before the sequence's first query token
// (those a pooling launch of the same tokens does not write), for the fused pooling launch.
// One 512-thread block; called by every thread.
template <int HI, int KS, bool QBF16, bool PAGED, bool F8>
__device__ __forceinline__ void mx_floor_block(const IdxMxDev& A, int k, int row,
                                               bool prior_only) {
  constexpr int W = kMxFloorThreads / 64;
  constexpr int PT = kMxSamples / kMxFloorThreads;      // samples per thread
  __shared__ uint32_t s_qa[kMxMaxUnits][4];
  __shared__ int s_qs[kMxMaxUnits];
  __shared__ uint16_t s_samp[kMxSamples];
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
  if (k >= nv || ns <= kMxSamples) {
    if (threadIdx.x == 0) A.floor[row] = 0u;
    return;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int ksteps = A.d_I > 64 ? A.d_I / 64 : 1;
  const uint8_t* kbase = PAGED ? A.k : A.k + b * A.k_bstride;
  const uint8_t* sbase = PAGED ? A.ks : A.ks + b * A.ks_bstride;
  // wave w scores runs RPW*w .. RPW*w + RPW-1: NG groups of 32 keys, all loads in flight
  constexpr int RPW = kMxFloorRuns / W, GPR = kMxRunKeys / 32, NG = RPW * GPR;
  u32x4 kraw[NG][KS];
  int ksc[NG][KS];
#pragma unroll
  for (int u = 0; u < NG; ++u) {
    const int run = wave * RPW + u / GPR;
    const int r0 = static_cast<int>(static_cast<int64_t>(run) * (ns - kMxRunKeys) /
                                    (kMxFloorRuns - 1));
    mx_load<KS, PAGED, F8>(A, kbase, sbase, b, r0 + (u % GPR) * 32 + col, true, kraw[u], ksc[u]);
  }
  const MxQuery<HI, KS> Q = mx_query<HI, KS, QBF16, F8>(A, row, s_qa, s_qs);
#pragma unroll
  for (int u = 0; u < NG; ++u) {
    const int run = wave * RPW + u / GPR;
    const float s = mx_score<HI, KS, F8>(Q, kraw[u], ksc[u], ksteps);
    if (half == 0)
      s_samp[run * kMxRunKeys + (u % GPR) * 32 + col] =
          static_cast<uint16_t>(bf16_key(f32_to_bf16_bits(s)));
  }
  __syncthreads();
  uint32_t top[PT];
#pragma unroll
  for (int e = 0; e < PT; ++e) top[e] = s_samp[threadIdx.x * PT + e];
  const int m = min(kMxSamples - 8, static_cast<int>((2LL * k * kMxSamples + nv - 1) / nv) + 8);
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
      if (lane == 0) A.floor[row] = pre;
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
  if (threadIdx.x == 0) A.floor[row] = pre;
}

// grid: rows; block 512.
template <int HI, int KS, bool QBF16, bool PAGED, bool F8>
__global__ __launch_bounds__(kMxFloorThreads) void mx_floor_kernel(IdxMxDev A, int k) {
  mx_floor_block<HI, KS, QBF16, PAGED, F8>(A, k, blockIdx.x, false);
}

// The floors and the pooling of the same tokens in one launch: blocks x < Nq of grid row y
// set the floor of query row y*Nq + x (sampling only entries completed before the call),
// the rest run the pooling jobs (sequence y).  grid: (Nq + pooling blocks, B); block 512.
template <int HI, int KS, bool QBF16, bool PAGED, bool F8>
__global__ __launch_bounds__(kMxFloorThreads) void mx_pool_floor_kernel(PoolJobs J, IdxMxDev A,
                                                                        int k) {
  __shared__ float alpha[1024];
  __shared__ float s_part[kMxFloorThreads * 8];
  if (static_cast<int>(blockIdx.x) < A.Nq)
    mx_floor_block<HI, KS, QBF16, PAGED, F8>(A, k, blockIdx.y * A.Nq + blockIdx.x, true);
  else
    pool_jobs_block<PAGED>(J, blockIdx.x - A.Nq, alpha, s_part);
}

// The exact threshold among the row's C candidates (the concatenated chunk lists, prefix
// counts in s_pre): thread t takes a contiguous run of at most PER of them.
template <int PER>
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
  sel::select_candidates<16, kMxResThreads, PER>(ck, cj, my, A.floor[row], k, out, s_gt, s_eq,
                                                 s_hb, s_hist, s_sel);
}

// grid: rows; block 512.  The row's candidates are the concatenated chunk lists (index
// order); thread t takes a contiguous run of them.
template <int HI, int KS, bool QBF16, bool PAGED, bool F8>
__global__ __launch_bounds__(kMxResThreads) void mx_list_resolve_kernel(IdxMxDev A, int k,
                                                                        int32_t* idx) {
  constexpr int W = kMxResThreads / 64;
  __shared__ int s_pre[kMxMaxChunks + 1];
  __shared__ int s_cnt[2][W];
  __shared__ int s_gt[W], s_eq[W], s_hb[W];
  __shared__ int s_hist[2][256];
  __shared__ int s_sel[4];
  __shared__ uint32_t s_qa[kMxMaxUnits][4];
  __shared__ int s_qs[kMxMaxUnits];
  const int row = blockIdx.x;
  const int b = row / A.Nq;
  const int64_t p = query_pos(A.seq_pos, A.pos0, b, row % A.Nq);
  const int64_t nv64 = (p + 1) / A.ratio;
  const int nv = static_cast<int>(nv64 < A.N ? nv64 : A.N);
  int32_t* out = idx + static_cast<int64_t>(row) * k;
  if (k >= nv) {
    sel::take_all(nv, k, out, kMxResThreads);
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
      sel::select_candidates<16, kMxResThreads, 16>(ck, cj, my, A.floor[row], k, out, s_gt,
                                                    s_eq, s_hb, s_hist, s_sel);
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
      mx_resolve_lists<16>(A, row, nch, C, k, out, s_pre, s_gt, s_eq, s_hb, s_hist, s_sel);
    else
      mx_resolve_lists<kMxResPer>(A, row, nch, C, k, out, s_pre, s_gt, s_eq, s_hb, s_hist,
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
  sel::select_exact_row<16, kMxResThreads>(V, k, out, s_cnt, s_gt, s_eq);
}

// KS: 64-channel MFMA steps the kernels hold registers for (d_I <= 64: one).  The FP8
// form keeps two: built with one, its scores differed from the FP4 form's (measured; the
// cause was not found), with two they are identical, as the tests require.
template <int HI, int KS, bool QBF16, bool F8>
hipError_t launch_mx_mfma_ks(const IdxMxDev& A, int rows, int score_dtype, hipStream_t s) {
  const int nchunks = (A.N + A.chunk - 1) / A.chunk;
  dim3 grid(nchunks, rows);
  if (score_dtype == 1)
    if (A.pm.table) launch_timed(index_scores_mx_mfma_kernel<HI, KS, QBF16, true, true, F8, false>, grid, dim3(256), s, A);
    else launch_timed(index_scores_mx_mfma_kernel<HI, KS, QBF16, true, false, F8, false>, grid, dim3(256), s, A);
  else
    if (A.pm.table) launch_timed(index_scores_mx_mfma_kernel<HI, KS, QBF16, false, true, F8, false>, grid, dim3(256), s, A);
    else launch_timed(index_scores_mx_mfma_kernel<HI, KS, QBF16, false, false, F8, false>, grid, dim3(256), s, A);
  return hipGetLastError();
}

template <int HI, bool QBF16, bool F8>
hipError_t launch_mx_mfma_hi(const IdxMxDev& A, int rows, int score_dtype, hipStream_t s) {
  if (A.d_I > 64 || F8) return launch_mx_mfma_ks<HI, 2, QBF16, F8>(A, rows, score_dtype, s);
  return launch_mx_mfma_ks<HI, 1, QBF16, F8>(A, rows, score_dtype, s);
}

// pool: null, or the pooling jobs to run in the floors' launch (pool_blocks of 512 threads)
template <int HI, int KS, bool QBF16, bool F8, bool PAGED>
hipError_t launch_mx_topk_ks(const IdxMxDev& A, int rows, int k, int32_t* idx,
                             const PoolJobs* pool, int pool_blocks_n, int B, hipStream_t s) {
  if (pool && pool_blocks_n > 0)
    mx_pool_floor_kernel<HI, KS, QBF16, PAGED, F8>
        <<<dim3(A.Nq + pool_blocks_n, B), kMxFloorThreads, 0, s>>>(*pool, A, k);
  else
    mx_floor_kernel<HI, KS, QBF16, PAGED, F8><<<rows, kMxFloorThreads, 0, s>>>(A, k);
  launch_timed(index_scores_mx_mfma_kernel<HI, KS, QBF16, true, PAGED, F8, true>,
               dim3(A.nchunks, rows), dim3(256), s, A);
  mx_list_resolve_kernel<HI, KS, QBF16, PAGED, F8><<<rows, kMxResThreads, 0, s>>>(A, k, idx);
  return hipGetLastError();
}

template <int HI, bool QBF16, bool F8, bool PAGED>
hipError_t launch_mx_topk_hi(const IdxMxDev& A, int rows, int k, int32_t* idx,
                             const PoolJobs* pool, int pool_blocks_n, int B, hipStream_t s) {
  if (A.d_I > 64 || F8)
    return launch_mx_topk_ks<HI, 2, QBF16, F8, PAGED>(A, rows, k, idx, pool, pool_blocks_n, B, s);
  return launch_mx_topk_ks<HI, 1, QBF16, F8, PAGED>(A, rows, k, idx, pool, pool_blocks_n, B, s);
}

template <bool QBF16, bool F8>
hipError_t launch_mx_mfma(const IdxMxDev& A, int rows, int H_I, int score_dtype, hipStream_t s) {
  switch (H_I) {
    case 1: return launch_mx_mfma_hi<1, QBF16, F8>(A, rows, score_dtype, s);
    case 2: return launch_mx_mfma_hi<2, QBF16, F8>(A, rows, score_dtype, s);
    case 4: return launch_mx_mfma_hi<4, QBF16, F8>(A, rows, score_dtype, s);
    case 8: return launch_mx_mfma_hi<8, QBF16, F8>(A, rows, score_dtype, s);
    case 16: return launch_mx_mfma_hi<16, QBF16, F8>(A, rows, score_dtype, s);
  }
  return hipErrorInvalidValue;
}

template <bool QBF16, bool F8, bool PAGED>
hipError_t launch_mx_topk(const IdxMxDev& A, int rows, int H_I, int k, int32_t* idx,
                          const PoolJobs* pool, int pb, int B, hipStream_t s) {
  switch (H_I) {
    case 1: return launch_mx_topk_hi<1, QBF16, F8, PAGED>(A, rows, k, idx, pool, pb, B, s);
    case 2: return launch_mx_topk_hi<2, QBF16, F8, PAGED>(A, rows, k, idx, pool, pb, B, s);
    case 4: return launch_mx_topk_hi<4, QBF16, F8, PAGED>(A, rows, k, idx, pool, pb, B, s);
    case 8: return launch_mx_topk_hi<8, QBF16, F8, PAGED>(A, rows, k, idx, pool, pb, B, s);
    case 16: return launch_mx_topk_hi<16, QBF16, F8, PAGED>(A, rows, k, idx, pool, pb, B, s);
  }
  return hipErrorInvalidValue;
}

IdxMxDev make_mx_dev(const void* q, const float* w, const uint8_t* kx, int64_t k_bstride,
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

MxTopkLayout mx_topk_layout(int rows, int N) {
  const int chunk = std::min(index_chunk(rows, N), 2048);
  const int64_t nchunks = (N + chunk - 1) / chunk;
  MxTopkLayout l;
  l.counts_off = align256(static_cast<size_t>(rows) * 4);
  l.lists_off = l.counts_off + align256(static_cast<size_t>(rows) * nchunks * 4);
  l.scores_off = l.lists_off + align256(static_cast<size_t>(rows) * nchunks * chunk * 4);
  l.total = l.scores_off + align256(static_cast<size_t>(rows) * N * 2);
  return l;
}

}  // namespace

hipError_t launch_mxfp4_index_scores(const void* q, int q_dtype, const float* w,
                                     const uint8_t* kx, int64_t k_bstride, const uint8_t* ks,
                                     int64_t ks_bstride, int B, int Nq, int H_I, int d_I,
                                     int N, int ratio, int64_t pos0, const int64_t* seq_pos,
                                     const int32_t* block_table, int64_t table_stride,
                                     int score_dtype, void* scores, bool fp8, hipStream_t s) {
  const IdxMxDev A = make_mx_dev(q, w, kx, k_bstride, ks, ks_bstride, B, Nq, d_I, N, ratio,
                                 pos0, seq_pos, block_table, table_stride, scores);
  if (fp8) {
    if (q_dtype == 1) return launch_mx_mfma<true, true>(A, B * Nq, H_I, score_dtype, s);
    return launch_mx_mfma<false, true>(A, B * Nq, H_I, score_dtype, s);
  }
  if (q_dtype == 1) return launch_mx_mfma<true, false>(A, B * Nq, H_I, score_dtype, s);
  return launch_mx_mfma<false, false>(A, B * Nq, H_I, score_dtype, s);
}

bool mx_topk_fused_ok(int rows, int N, int score_dtype) {
  if (score_dtype != 1 || N < 1 || rows < 1) return false;
  const int chunk = std::min(index_chunk(rows, N), 2048);
  return (N + chunk - 1) / chunk <= kMxMaxChunks;
}

size_t mx_topk_workspace_bytes(int rows, int N) { return mx_topk_layout(rows, N).total; }

hipError_t launch_mxfp4_index_topk(const void* q, int q_dtype, const float* w,
                                   const uint8_t* kx, int64_t k_bstride, const uint8_t* ks,
                                   int64_t ks_bstride, int B, int Nq, int H_I, int d_I, int N,
                                   int ratio, int64_t pos0, const int64_t* seq_pos,
                                   const int32_t* block_table, int64_t table_stride, int k,
                                   int32_t* idx, bool fp8, void* ws, hipStream_t s,
                                   const hcsa_pool_job* pool_jobs, int n_pool_jobs,
                                   int64_t raw_ring) {
  const int rows = B * Nq;
  const MxTopkLayout l = mx_topk_layout(rows, N);
  char* base = static_cast<char*>(ws);
  IdxMxDev A = make_mx_dev(q, w, kx, k_bstride, ks, ks_bstride, B, Nq, d_I, N, ratio, pos0,
                           seq_pos, block_table, table_stride, base + l.scores_off);
  A.floor = reinterpret_cast<uint32_t*>(base);
  A.counts = reinterpret_cast<uint32_t*>(base + l.counts_off);
  A.lists = reinterpret_cast<uint32_t*>(base + l.lists_off);
  PoolJobs J;
  int pb = 0;
  if (pool_jobs)
    pb = pool_jobs_fill(pool_jobs, n_pool_jobs, block_table, table_stride, raw_ring,
                        kMxFloorThreads, J);
  const PoolJobs* pj = pool_jobs ? &J : nullptr;
  const bool paged = block_table != nullptr, qb = q_dtype == 1;
  if (fp8) {
    if (qb) return paged ? launch_mx_topk<true, true, true>(A, rows, H_I, k, idx, pj, pb, B, s)
                         : launch_mx_topk<true, true, false>(A, rows, H_I, k, idx, pj, pb, B, s);
    return paged ? launch_mx_topk<false, true, true>(A, rows, H_I, k, idx, pj, pb, B, s)
                 : launch_mx_topk<false, true, false>(A, rows, H_I, k, idx, pj, pb, B, s);
  }
  if (qb) return paged ? launch_mx_topk<true, false, true>(A, rows, H_I, k, idx, pj, pb, B, s)
                       : launch_mx_topk<true, false, false>(A, rows, H_I, k, idx, pj, pb, B, s);
  return paged ? launch_mx_topk<false, false, true>(A, rows, H_I, k, idx, pj, pb, B, s)
               : launch_mx_topk<false, false, false>(A, rows, H_I, k, idx, pj, pb, B, s);
}


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
