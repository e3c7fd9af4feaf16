// MFMA attention units (bf16, 16 heads x 128) and the log-sum-exp merge of splits, shared by
// the attention kernels and the decode-step launches.
//
// CSA attends over the top-k compressed entries plus a sliding window of n_win = 128 raw
// tokens; HCA attends densely over every compressed entry (Lighthouse, "deep deepseek v4
// release", section 八 item 3).  One softmax runs over each query's key list; a unit owns
// one contiguous range (split) of it and writes the split's normalized output and
// log-sum-exp, which the merge combines exactly.
#pragma once
#include "attn_keys.h"
#include "common.h"

namespace hcsa {
namespace attn {

// ------------------------------------------------------------------ MFMA path (H=16, d=128)

constexpr int kMfmaMaxChunk = 4096;

__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4& a, const u32x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// One 32-key step of the MFMA attention (16 heads, d = 128), for lane (head col, k-group g):
// S^T tiles t = 0, 1 from the K rows ka[t] (keys 16t + col of the step), online softmax of
// the logits of keys 16*(j/4) + 4g + j%4 (valid where ok[j]), O^T += V^T P^T with the V rows
// vv[j] of the same keys.
__device__ __forceinline__ void attend_step(const u32x4 (&ka)[2][4], const u32x4 (&vv)[8],
                                            const bool (&ok)[8], const u32x4 (&qB)[4],
                                            f32x4 (&acc)[8], float& m_run, float& l_run,
                                            float sl2) {
  // ---- S^T tiles: lane holds logits of keys (tile t, 4g + i) for head col
  f32x4 st[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    st[t] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < 4; ++s) st[t] = mfma16x16x32(ka[t][s], qB[s], st[t]);
  }
  float lg[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) lg[j] = ok[j] ? st[j >> 2][j & 3] * sl2 : -INFINITY;
  float mt = lg[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) mt = fmaxf(mt, lg[j]);
  mt = fmaxf(mt, __shfl_xor(mt, 16, kWave));
  mt = fmaxf(mt, __shfl_xor(mt, 32, kWave));
  const float m_new = fmaxf(m_run, mt);
  if (m_new == -INFINITY) return;        // nothing visible yet for this head
  const float alpha = exp2_unit(m_run - m_new);
  m_run = m_new;
  float pj[8];
  float psum = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    pj[j] = exp2_unit(lg[j] - m_new);
    psum += pj[j];
  }
  l_run = l_run * alpha + psum;
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] *= alpha;
  u32x4 pB;
#pragma unroll
  for (int m = 0; m < 4; ++m) pB[m] = pack_bf16x2(pj[2 * m], pj[2 * m + 1]);
  // ---- O^T tiles: channel 8*i + t for tile t, row i
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
    u32x4 va;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      va[m] = __builtin_amdgcn_perm(vv[2 * m + 1][t >> 1], vv[2 * m][t >> 1], sel);
    acc[t] = mfma16x16x32(va, pB, acc[t]);
  }
}

// The W waves' partial results of one (split, row) unit merged in LDS and written as the
// split's normalized output and log-sum-exp (or the final ones with a single split).
//
// tid: the thread's index in its 64*W-thread unit (a block may hold two 4-wave units, each
// with its own LDS; both reach the same barriers).
template <int W = 4>
__device__ __forceinline__ void combine_waves(const AttnDev& A, const f32x4 (&acc)[8],
                                              float m_run, float l_run, float (*s_o)[16][129],
                                              float (*s_ml)[2][16], int split, int row,
                                              int tid) {
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 15, g = lane >> 4;
  // per-head totals across the 4 k-groups
  l_run += __shfl_xor(l_run, 16, kWave);
  l_run += __shfl_xor(l_run, 32, kWave);
  // lane holds O^T[channel 32g + 8i + t][head col] = acc[t][i]
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int t = 0; t < 8; ++t) s_o[wave][col][32 * g + 8 * i + t] = acc[t][i];
  if (g == 0) {
    s_ml[wave][0][col] = m_run;
    s_ml[wave][1][col] = l_run;
  }
  __syncthreads();

  float* o = A.out + (static_cast<int64_t>(split) * A.rows + row) * 2048;
  float* ls = A.lse + static_cast<int64_t>(split) * A.rows * 16 + static_cast<int64_t>(row) * 16;
  for (int t = tid; t < 2048; t += 64 * W) {
    const int h = t >> 7, c = t & 127;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, s_ml[w][0][h]);
    float num = 0.0f, den = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float mw = s_ml[w][0][h];
        if (mw != -INFINITY) {
          const float f = exp2f(mw - M);
          num = fmaf(f, s_o[w][h][c], num);
          den = fmaf(f, s_ml[w][1][h], den);
        }
      }
    }
    o[t] = den > 0.0f ? num / den : 0.0f;
    if (c == 0) ls[h] = den > 0.0f ? (M + log2f(den)) * 0.6931471805599453f : -INFINITY;
  }
}

// One (split, row) unit of the MFMA attention (256 threads, tid its thread index); LDS
// passed in by the kernel.  COH: the selection (CSA) is read with agent-coherent loads, for
// a selection written by another block of the same launch.
template <bool CSA, bool COH = false>
__device__ __forceinline__ void attn_mfma_block(const AttnDev& A, int split, int row,
                                                int* s_code, float (*s_o)[16][129],
                                                float (*s_ml)[2][16], int tid) {
  const RowKeys r = row_keys<CSA>(A, row);
  const int k0 = split * A.chunk;
  const int cnt = max(0, min(A.chunk, r.L - k0));
  // Contiguous caches (raw rows contiguous or in a ring) whose element offsets within a
  // sequence fit in 31 bits: the list holds each key's element offset instead of its code
  // (>= 0: compressed row, < 0: -1 - offset of a raw row, kNoKey: none), so a load is one
  // add to the sequence's base.  Paged caches keep the codes.
  constexpr int kNoKey = INT32_MIN;
  const int64_t raw_rows = A.raw_ring ? A.raw_ring : A.T_raw;
  const bool flat = A.pm.table == nullptr && static_cast<int64_t>(A.N) * A.d < (int64_t{1} << 31) &&
                    raw_rows * A.d < (int64_t{1} << 31);          // block-uniform
  for (int i = tid; i < cnt; i += 256) {
    const int c = key_code<CSA, COH>(A, r, row, k0 + i);
    int v = c;
    if (flat) {
      if (c == -1) {
        v = kNoKey;
      } else if (c >= 0) {
        v = c * A.d;
      } else {
        const int64_t t = -static_cast<int64_t>(c) - 2;
        v = -1 - static_cast<int>((A.raw_ring ? (t & (A.raw_ring - 1)) : t) * A.d);
      }
    }
    s_code[i] = v;
  }
  __syncthreads();

  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 15;   // head owned by this lane
  const int g = lane >> 4;     // k-group
  const uint16_t* kc_b = static_cast<const uint16_t*>(A.kc) + r.b * A.c_bstride;
  const uint16_t* vc_b = static_cast<const uint16_t*>(A.vc) + r.b * A.c_bstride;
  const uint16_t* kr_b = static_cast<const uint16_t*>(A.k_raw) + r.b * A.raw_bstride;
  const uint16_t* vr_b = static_cast<const uint16_t*>(A.v_raw) + r.b * A.raw_bstride;

  // B operand of S^T = K Q^T: Q[head col][32s + 8g .. +8] for s = 0..3.
  u32x4 qB[4];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(A.q) + (static_cast<int64_t>(row) * 16 + col) * 128;
#pragma unroll
    for (int s = 0; s < 4; ++s) qB[s] = *reinterpret_cast<const u32x4*>(qrow + 32 * s + 8 * g);
  }

  f32x4 acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = f32x4{0, 0, 0, 0};
  float m_run = -INFINITY;
  float l_run = 0.0f;
  const float sl2 = A.scale * 1.4426950408889634f;  // logits in base 2

  // K rows for the A operand (keys base + col and base + 16 + col) and V slices (keys
  // base + 4g + j for j < 4 and base + 16 + 4g + (j - 4), channels 8col..8col+7)
  auto load = [&](int base, u32x4 (&ka)[2][4], u32x4 (&vv)[8], bool (&ok)[8]) {
    if (flat) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int pos = base + 16 * t + col;
        const int v = pos < cnt ? s_code[pos] : kNoKey;
        if (v != kNoKey) {
          const uint16_t* kr = v >= 0 ? kc_b + v : kr_b + (-1 - v);
#pragma unroll
          for (int s = 0; s < 4; ++s) ka[t][s] = *reinterpret_cast<const u32x4*>(kr + 32 * s + 8 * g);
        } else {
#pragma unroll
          for (int s = 0; s < 4; ++s) ka[t][s] = u32x4{0, 0, 0, 0};
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int pos = base + (j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4));
        const int v = pos < cnt ? s_code[pos] : kNoKey;
        ok[j] = v != kNoKey;
        vv[j] = ok[j] ? *reinterpret_cast<const u32x4*>((v >= 0 ? vc_b + v : vr_b + (-1 - v)) + 8 * col)
                      : u32x4{0, 0, 0, 0};
      }
      return;
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int pos = base + 16 * t + col;
      const int c = pos < cnt ? s_code[pos] : -1;
      if (c != -1) {
        const uint16_t* kr = key_row<uint16_t>(A, r.b, c, false);
#pragma unroll
        for (int s = 0; s < 4; ++s) ka[t][s] = *reinterpret_cast<const u32x4*>(kr + 32 * s + 8 * g);
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) ka[t][s] = u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int pos = base + (j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4));
      const int c = pos < cnt ? s_code[pos] : -1;
      ok[j] = c != -1;
      vv[j] = ok[j] ? *reinterpret_cast<const u32x4*>(key_row<uint16_t>(A, r.b, c, true) + 8 * col)
                    : u32x4{0, 0, 0, 0};
    }
  };
  // wave w takes the 32-key steps at w*32, w*32 + 128, ...; the next step's rows load while
  // the current one is computed (the same steps in the same order as one at a time)
  u32x4 kaA[2][4], vvA[8], kaB[2][4], vvB[8];
  bool okA[8], okB[8];
  const int w0 = wave * 32;
  if (w0 < cnt) load(w0, kaA, vvA, okA);
  for (int base = w0; base < cnt; base += 256) {
    if (base + 128 < cnt) load(base + 128, kaB, vvB, okB);
    attend_step(kaA, vvA, okA, qB, acc, m_run, l_run, sl2);
    if (base + 128 >= cnt) break;
    if (base + 256 < cnt) load(base + 256, kaA, vvA, okA);
    attend_step(kaB, vvB, okB, qB, acc, m_run, l_run, sl2);
  }

  combine_waves(A, acc, m_run, l_run, s_o, s_ml, split, row, tid);
}

// CSA attention of one query row by an 8-wave (512-thread) block over ranges of its key
// list, accumulated into one online softmax (acc, m_run, l_run held by the caller): wave w
// takes steps of 32 positions at p0 + w*32, p0 + w*32 + 256, ..., with the next step's K rows
// and V slices in flight while the current step is computed.  A range holds at most
// kMfmaMaxChunk positions.  COH: the selection is read with agent-coherent loads (written
// by another block of the same launch).  The step math is that of the split kernels; only
// the partition of the key list differs.
template <bool COH>
__device__ __forceinline__ void csa_range8(const AttnDev& A, const RowKeys& r, int row, int p0,
                                           int p1, int* s_code, const u32x4 (&qB)[4],
                                           f32x4 (&acc)[8], float& m_run, float& l_run,
                                           float sl2) {
  const int cnt = max(0, min(p1 - p0, kMfmaMaxChunk));
  __syncthreads();                                 // s_code free again
  for (int i = threadIdx.x; i < cnt; i += 512) s_code[i] = key_code<true, COH>(A, r, row, p0 + i);
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, g = lane >> 4;
  // K rows of keys base + 16t + col; V slices (channels 8col..) of keys base + 16*(j/4) +
  // 4g + j%4 (the layouts of attend_step)
  auto load = [&](int base, u32x4 (&ka)[2][4], u32x4 (&vv)[8], bool (&ok)[8]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int pos = base + 16 * t + col;
      const int c = pos < cnt ? s_code[pos] : -1;
      if (c != -1) {
        const uint16_t* kr = key_row<uint16_t>(A, r.b, c, false);
#pragma unroll
        for (int s = 0; s < 4; ++s) ka[t][s] = *reinterpret_cast<const u32x4*>(kr + 32 * s + 8 * g);
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) ka[t][s] = u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int pos = base + 16 * (j >> 2) + 4 * g + (j & 3);
      const int c = pos < cnt ? s_code[pos] : -1;
      ok[j] = c != -1;
      vv[j] = ok[j] ? *reinterpret_cast<const u32x4*>(key_row<uint16_t>(A, r.b, c, true) + 8 * col)
                    : u32x4{0, 0, 0, 0};
    }
  };
  u32x4 kaA[2][4], vvA[8], kaB[2][4], vvB[8];
  bool okA[8], okB[8];
  const int w0 = wave * 32;
  if (w0 < cnt) load(w0, kaA, vvA, okA);
  for (int base = w0; base < cnt; base += 512) {
    if (base + 256 < cnt) load(base + 256, kaB, vvB, okB);
    attend_step(kaA, vvA, okA, qB, acc, m_run, l_run, sl2);
    if (base + 256 >= cnt) break;
    if (base + 512 < cnt) load(base + 512, kaA, vvA, okA);
    attend_step(kaB, vvB, okB, qB, acc, m_run, l_run, sl2);
  }
}

// The query operand and empty accumulators of an 8-wave CSA row unit.
struct Row8State {
  u32x4 qB[4];                                     // B of S^T: Q[head col][32s + 8g .. +8]
  f32x4 acc[8];
  float m_run, l_run, sl2;
};

__device__ __forceinline__ void row8_init(const AttnDev& A, int row, Row8State& st) {
  const int lane = threadIdx.x & 63, col = lane & 15, g = lane >> 4;
  const uint16_t* qrow = static_cast<const uint16_t*>(A.q) + (static_cast<int64_t>(row) * 16 + col) * 128;
#pragma unroll
  for (int s = 0; s < 4; ++s) st.qB[s] = *reinterpret_cast<const u32x4*>(qrow + 32 * s + 8 * g);
#pragma unroll
  for (int t = 0; t < 8; ++t) st.acc[t] = f32x4{0, 0, 0, 0};
  st.m_run = -INFINITY;
  st.l_run = 0.0f;
  st.sl2 = A.scale * 1.4426950408889634f;          // logits in base 2
}

// Decode HCA: the visible entries 0..nv-1 are contiguous, so no key list is built; each of
// a block's 4 waves streams its own contiguous run of the block's chunk, 32 entries a step,
// the next step's K and V rows loaded while the current step is computed.
template <bool PAGED>
__device__ __forceinline__ void hca_decode_block(const AttnDev& A, int split, int row,
                                                 float (*s_o)[16][129], float (*s_ml)[2][16],
                                                 int tid) {
  const RowKeys r = row_keys<false>(A, row);       // r.L = visible entries
  const int k0 = split * A.chunk;
  const int cnt = max(0, min(A.chunk, r.L - k0));
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, g = lane >> 4;
  const int per = (cnt + 127) / 128 * 32;          // a quarter of the chunk, whole steps
  const int w0 = k0 + wave * per;
  const int w1 = min(w0 + per, k0 + cnt);

  u32x4 qB[4];                                     // B of S^T: Q[head col][32s + 8g .. +8]
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(A.q) + (static_cast<int64_t>(row) * 16 + col) * 128;
#pragma unroll
    for (int s = 0; s < 4; ++s) qB[s] = *reinterpret_cast<const u32x4*>(qrow + 32 * s + 8 * g);
  }
  f32x4 acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = f32x4{0, 0, 0, 0};
  float m_run = -INFINITY, l_run = 0.0f;
  const float sl2 = A.scale * 1.4426950408889634f;   // logits in base 2

  const uint16_t* kb = static_cast<const uint16_t*>(A.kc);
  const uint16_t* vb = static_cast<const uint16_t*>(A.vc);
  auto erow = [&](int e) { return row_off<PAGED>(A.pm, A.c_bstride, r.b, e, A.c_log2, 128); };
  // K rows of keys base + 16t + col; V slices (channels 8col..) of keys base + 16*(j/4) + 4g + j%4
  auto load = [&](int base, u32x4 (&ka)[2][4], u32x4 (&vv)[8], bool (&ok)[8]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int e = base + 16 * t + col;
      const int64_t o = e < w1 ? erow(e) : 0;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        ka[t][s] = e < w1 ? *reinterpret_cast<const u32x4*>(kb + o + 32 * s + 8 * g)
                          : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = base + 16 * (j >> 2) + 4 * g + (j & 3);
      ok[j] = e < w1;
      vv[j] = ok[j] ? *reinterpret_cast<const u32x4*>(vb + erow(e) + 8 * col)
                    : u32x4{0, 0, 0, 0};
    }
  };
  // a step wholly inside the run (the wave-uniform common case) loads without per-entry
  // checks; only the run's last step may be partial
  auto load_step = [&](int base, u32x4 (&ka)[2][4], u32x4 (&vv)[8], bool (&ok)[8]) {
    if (base + 32 > w1) {
      load(base, ka, vv, ok);
      return;
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int64_t o = erow(base + 16 * t + col);
#pragma unroll
      for (int s = 0; s < 4; ++s) ka[t][s] = *reinterpret_cast<const u32x4*>(kb + o + 32 * s + 8 * g);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      ok[j] = true;
      vv[j] = *reinterpret_cast<const u32x4*>(vb + erow(base + 16 * (j >> 2) + 4 * g + (j & 3)) + 8 * col);
    }
  };
  u32x4 kaA[2][4], vvA[8], kaB[2][4], vvB[8];
  bool okA[8], okB[8];
  if (w0 < w1) load_step(w0, kaA, vvA, okA);
  for (int base = w0; base < w1; base += 64) {
    if (base + 32 < w1) load_step(base + 32, kaB, vvB, okB);
    attend_step(kaA, vvA, okA, qB, acc, m_run, l_run, sl2);
    if (base + 32 >= w1) break;
    if (base + 64 < w1) load_step(base + 64, kaA, vvA, okA);
    attend_step(kaB, vvB, okB, qB, acc, m_run, l_run, sl2);
  }
  combine_waves(A, acc, m_run, l_run, s_o, s_ml, split, row, tid);
}

constexpr int kMergeRegSplits = 16;

// grid: (H, rows); block = d threads (<= 256).  Up to kMergeRegSplits splits every thread
// issues all of its loads -- the splits' log-sum-exps and its channel's partial outputs --
// before using any, so the merge costs one memory latency; beyond that the split weights
// are formed once in LDS and each thread sums its channel over the splits.
__device__ __forceinline__ void lse_merge_row(const float* __restrict__ part_o,
                                              const float* __restrict__ part_l, int splits,
                                              int rows, int H, int d, float* __restrict__ out,
                                              float* __restrict__ lse, int h, int row,
                                              float* s_w, float* s_red) {
  const int64_t lstride = static_cast<int64_t>(rows) * H;
  const int64_t ostride = static_cast<int64_t>(rows) * H * d;
  const float* pl = part_l + static_cast<int64_t>(row) * H + h;
  const int c = threadIdx.x;
  const float* po = part_o + (static_cast<int64_t>(row) * H + h) * d + min(c, d - 1);
  float* orow = out + (static_cast<int64_t>(row) * H + h) * d;
  if (splits <= kMergeRegSplits) {
    float l[kMergeRegSplits], v[kMergeRegSplits];
#pragma unroll
    for (int u = 0; u < kMergeRegSplits; ++u) {
      l[u] = u < splits ? pl[u * lstride] : -INFINITY;
      v[u] = u < splits ? po[u * ostride] : 0.0f;
    }
    float M = -INFINITY;
#pragma unroll
    for (int u = 0; u < kMergeRegSplits; ++u) M = fmaxf(M, l[u]);
    float num = 0.0f, den = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int u = 0; u < kMergeRegSplits; ++u) {
        // an empty split has lse -inf and a zero partial: weight 0
        const float w = l[u] == -INFINITY ? 0.0f : expf(l[u] - M);
        den += w;
        num = fmaf(w, v[u], num);
      }
    }
    if (c < d) orow[c] = den > 0.0f ? num / den : 0.0f;
    if (c == 0) lse[static_cast<int64_t>(row) * H + h] = den > 0.0f ? M + logf(den) : -INFINITY;
    return;
  }
  if (threadIdx.x < kWave) {
    float M = -INFINITY;
    for (int s = threadIdx.x; s < splits; s += kWave) M = fmaxf(M, pl[s * lstride]);
    M = wave_max(M);
    float den = 0.0f;
    for (int s = threadIdx.x; s < splits; s += kWave) {
      const float l = pl[s * lstride];
      const float w = (M == -INFINITY || l == -INFINITY) ? 0.0f : expf(l - M);
      if (s < 1024) s_w[s] = w;
      den += w;
    }
    den = wave_sum(den);
    if (threadIdx.x == 0) {
      s_red[0] = M;
      s_red[1] = den;
    }
  }
  __syncthreads();
  const float M = s_red[0], den = s_red[1];
  if (c < d) {
    float num = 0.0f;
    int s = 0;
    if (splits <= 1024) {
      // eight independent loads in flight; a zero weight multiplies a finite partial (empty
      // splits store zeros), so no branch is needed
      float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (; s + 8 <= splits; s += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = po[(s + u) * ostride];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc[u] = fmaf(s_w[s + u], v[u], acc[u]);
      }
      for (; s < splits; ++s) acc[0] = fmaf(s_w[s], po[s * ostride], acc[0]);
#pragma unroll
      for (int u = 0; u < 8; ++u) num += acc[u];
    } else {
      for (; s < splits; ++s) {
        const float l = pl[s * lstride];
        const float w = (M == -INFINITY || l == -INFINITY) ? 0.0f : expf(l - M);
        if (w != 0.0f) num = fmaf(w, po[s * ostride], num);
      }
    }
    orow[c] = den > 0.0f ? num / den : 0.0f;
    if (c == 0) lse[static_cast<int64_t>(row) * H + h] = den > 0.0f ? M + logf(den) : -INFINITY;
  }
}

}  // namespace attn
}  // namespace hcsa
