// CSA sparse attention and HCA dense attention, split over the key list, with an
// online-softmax log-sum-exp merge of the splits.
//
// CSA attends over the top-k compressed entries plus a sliding window of n_win = 128 raw
// tokens; HCA attends densely over every compressed entry (Lighthouse, "deep deepseek v4
// release", section 八 item 3).  One softmax runs over the concatenated key list (the
// reading taken for how the window branch joins the sparse branch).  All query heads
// share one KV head (MQA).
//
// Key list of a query token at position p:
//   CSA: positions 0..k-1 are the selected entries (entries outside [0, n_c(p)) are
//        skipped), positions k.. are the raw tokens max(0, p-n_win+1) .. p.
//   HCA: positions 0..n_h(p)-1 are the entries themselves.
// A block owns one contiguous range (split) of one query's key list and writes either
// the final output (one split) or a normalized partial plus its log-sum-exp.
//
// Kernels:
//   attn_mfma_kernel     bf16, 16 heads, head dim 128 (the MI355X fast path).  Each wave
//                        takes 32 keys per step; S^T = K Q^T and O^T += V^T P^T run on
//                        v_mfma_f32_16x16x32_bf16 with every lane owning one head, so the
//                        softmax statistics never cross lanes except across the 4 k-groups.
//                        K rows feed the A operand straight from 16-byte global loads; each
//                        lane reads a 16-byte slice of 8 V rows and byte-permutes them into
//                        the A operand of 8 channel tiles (channel 8*i + tile), so no LDS
//                        transpose is needed.  The 4 waves of a block merge in LDS.
//   hca_tiled_kernel     HCA with many query tokens per sequence (chunked prefill): 16
//                        tokens share each streamed tile of entries (see its comment).
//   attn_generic_kernel  any head count / head dim, fp32 or bf16, plain VALU (small and
//                        fp32 shapes).
//   lse_merge_kernel     o = sum_s e^{lse_s - L} o_s, L = log sum_s e^{lse_s}.
#include "attn_dev.h"
#include "attn_keys.h"
#include "common.h"
#include "internal.h"

#include <algorithm>

namespace hcsa {

namespace {

using namespace attn;

// ------------------------------------------------------------------ generic VALU path

constexpr int kGenChunk = 64;


// grid: (splits, rows); block 256; dynamic LDS: H*d + H*kGenChunk floats + kGenChunk ints.
template <bool CSA, bool BF16>
__global__ __launch_bounds__(256) void attn_generic_kernel(AttnDev A) {
  extern __shared__ float smem[];
  float* qf = smem;                              // [H][d]
  float* pr = qf + A.H * A.d;                    // [H][kGenChunk] logits, then weights
  int* code = reinterpret_cast<int*>(pr + A.H * kGenChunk);
  __shared__ float s_m[64], s_sum[64];
  typedef typename std::conditional<BF16, uint16_t, float>::type TE;

  const int row = blockIdx.y;
  const int split = blockIdx.x;
  const RowKeys r = row_keys<CSA>(A, row);
  const int k0 = split * A.chunk;
  const int cnt = max(0, min(A.chunk, r.L - k0));
  const int H = A.H, d = A.d;

  for (int i = threadIdx.x; i < H * d; i += 256)
    qf[i] = ld<BF16>(A.q, static_cast<int64_t>(row) * H * d + i);
  for (int i = threadIdx.x; i < cnt; i += 256) code[i] = key_code<CSA>(A, r, row, k0 + i);
  __syncthreads();

  for (int t = threadIdx.x; t < H * cnt; t += 256) {
    const int h = t / cnt, i = t - h * cnt;
    float lg = -INFINITY;
    if (code[i] != -1) {
      const TE* kr = key_row<TE>(A, r.b, code[i], false);
      float acc = 0.0f;
      for (int c = 0; c < d; ++c) acc = fmaf(qf[h * d + c], ld<BF16>(kr, c), acc);
      lg = acc * A.scale;
    }
    pr[h * kGenChunk + i] = lg;
  }
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int h = wave; h < H; h += 4) {
    const float lg = lane < cnt ? pr[h * kGenChunk + lane] : -INFINITY;
    const float m = wave_max(lg);
    const float e = (m == -INFINITY || lg == -INFINITY) ? 0.0f : expf(lg - m);
    const float s = wave_sum(e);
    if (lane < cnt) pr[h * kGenChunk + lane] = e;
    if (lane == 0) {
      s_m[h] = m;
      s_sum[h] = s;
    }
  }
  __syncthreads();

  float* o = A.out + (static_cast<int64_t>(split) * A.rows + row) * H * d;
  float* ls = A.lse + static_cast<int64_t>(split) * A.rows * H + static_cast<int64_t>(row) * H;
  for (int t = threadIdx.x; t < H * d; t += 256) {
    const int h = t / d, c = t - h * d;
    const float s = s_sum[h];
    float acc = 0.0f;
    if (s > 0.0f) {
      for (int i = 0; i < cnt; ++i) {
        const float pw = pr[h * kGenChunk + i];
        if (pw != 0.0f) acc = fmaf(pw, ld<BF16>(key_row<TE>(A, r.b, code[i], true), c), acc);
      }
      acc = acc / s;
    }
    o[t] = acc;
    if (c == 0) ls[h] = s > 0.0f ? s_m[h] + logf(s) : -INFINITY;
  }
}

// grid: (splits, rows); block 256 (4 waves).
template <bool CSA>
__global__ __launch_bounds__(256, 2) void attn_mfma_kernel(AttnDev A) {
  __shared__ int s_code[kMfmaMaxChunk];
  __shared__ float s_o[4][16][129];
  __shared__ float s_ml[4][2][16];
  attn_mfma_block<CSA>(A, blockIdx.x, blockIdx.y, s_code, s_o, s_ml, threadIdx.x);
}

// ------------------------------------------------------------------ HCA, one token per sequence

// grid: (splits, rows); block 256.
template <bool PAGED>
__global__ __launch_bounds__(256, 2) void hca_decode_kernel(AttnDev A) {
  __shared__ float s_o[4][16][129];
  __shared__ float s_ml[4][2][16];
  hca_decode_block<PAGED>(A, blockIdx.x, blockIdx.y, s_o, s_ml, threadIdx.x);
}

// CSA and HCA attention of the same decode tokens in one launch: blocks 0 .. nH-1 are the
// HCA (split, row) blocks (the long streaming ones, started first), the rest the CSA blocks,
// so the CSA gathers run beside the HCA stream instead of after it.  grid: nH + nC; block 256.
template <bool PAGED>
__global__ __launch_bounds__(256, 2) void csa_hca_decode_kernel(AttnDev C, AttnDev Hd) {
  __shared__ int s_code[kMfmaMaxChunk];
  __shared__ float s_o[4][16][129];
  __shared__ float s_ml[4][2][16];
  const int nH = Hd.splits * Hd.rows;
  const int b = blockIdx.x;
  if (b < nH) hca_decode_block<PAGED>(Hd, b % Hd.splits, b / Hd.splits, s_o, s_ml, threadIdx.x);
  else attn_mfma_block<true>(C, (b - nH) % C.splits, (b - nH) / C.splits, s_code, s_o, s_ml,
                             threadIdx.x);
}

// ------------------------------------------------------------------ HCA, many query tokens

// Chunked prefill (many query tokens per sequence): consecutive tokens see almost the same
// HCA entries, so a block takes 16 tokens x 16 heads (8 waves, each 2 tokens x 16 heads =
// 32 query rows) and streams the entries once for all of them in 64-entry tiles through
// LDS (K rows and V transposed, double buffered, the next tile's loads in flight).  Per
// 32-entry half tile a wave computes S^T = K Q^T on v_mfma_f32_32x32x16_bf16: lane
// (column) = query row, register r = entry 8*(r/4) + 4*(lane/32) + r%4, so the online
// softmax is lane-local (two lanes share a row) and the probabilities, packed to bf16, are
// already the B operand of O^T += V^T P^T: step s takes registers 8s..8s+7, which hold
// entries 16s + 8*(e/4) + 4*(lane/32) + e%4 -- the A operand (V^T) reads the same
// entries, two runs of four, from the transposed tile.  Both halves' S^T products are
// issued before the softmax so the matrix cores stay busy, there is one running-max update
// per tile, and the accumulator rescale is skipped when no row's maximum moved.
constexpr int kTokTile = 16;              // query tokens per block
constexpr int kHKeys = 64;                // entries per tile (two MFMA tiles)
constexpr int kKPitch = 128 + 8;          // K tile row pitch (elements): no bank conflicts
constexpr int kVPitch = kHKeys + 8;       // V^T tile row pitch (elements)

// Entry e of V^T row (channel) ch sits at e ^ vt_swizzle(ch) within the row.  The XOR moves
// whole 8-entry groups, so the P.V reads (two aligned runs of four entries) stay contiguous;
// it spreads the transposing writes, whose 16 channel groups would otherwise all fall on
// one bank (8 x 36 dwords is a multiple of the bank count), over all banks, and keeps the
// reads free of conflicts, with 32 banks of 4 bytes and with 64.
__device__ __forceinline__ int vt_swizzle(int ch) {
  return 8 * (((ch >> 3) & 1) ^ ((ch >> 4) & 7));
}

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16a;

__device__ __forceinline__ f32x16a mfma32x32x16(const u32x4& a, const u32x4& b, f32x16a c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// grid: (ceil(Nq / 16), B); block 512.
__global__ __launch_bounds__(512) void hca_tiled_kernel(AttnDev A) {
  __shared__ __align__(16) uint16_t s_k[2][kHKeys * kKPitch];
  __shared__ __align__(16) uint16_t s_vt[2][128 * kVPitch];
  const int b = blockIdx.y;
  const int t0 = blockIdx.x * kTokTile;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 31, hh = lane >> 5;
  const int tok = t0 + 2 * wave + (col >> 4);     // this lane's query row: token, head
  const int head = col & 15;
  const bool tok_ok = tok < A.Nq;
  auto visible = [&](int t) -> int {
    const int64_t p = query_pos(A.seq_pos, A.pos0, b, t);
    const int64_t v = (p + 1) / A.ratio;
    return static_cast<int>(v < A.N ? v : A.N);
  };
  const int nv = tok_ok ? visible(tok) : 0;
  const int nv_max = visible(min(t0 + kTokTile, A.Nq) - 1);   // tokens ascend
  const int nv_min = visible(t0);                 // every token of the block sees these
  const int ntiles = (nv_max + kHKeys - 1) / kHKeys;
  const int64_t row = static_cast<int64_t>(b) * A.Nq + tok;

  u32x4 qb[8];                                    // B of S^T: Q[row][16s + 8hh .. +7]
  {
    const uint16_t* qr = static_cast<const uint16_t*>(A.q) + (row * 16 + head) * 128 + 8 * hh;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      qb[s] = tok_ok ? *reinterpret_cast<const u32x4*>(qr + 16 * s) : u32x4{0u, 0u, 0u, 0u};
  }
  const uint16_t* kpool = static_cast<const uint16_t*>(A.kc);
  const uint16_t* vpool = static_cast<const uint16_t*>(A.vc);
  auto erow = [&](int e) -> int64_t {
    return A.pm.table ? row_off<true>(A.pm, 0, b, e, A.c_log2, 128)
                      : b * A.c_bstride + static_cast<int64_t>(e) * 128;
  };
  // tile loads: thread i moves K channels 8*(i%16) .. +7 of entries i/16 and i/16 + 32, and
  // V channels 8*(i%16) .. +7 of entries 2*(i/16) and 2*(i/16)+1 (packed in pairs for the
  // transposed tile)
  const int lkey = threadIdx.x >> 4, lpart = threadIdx.x & 15;
  u32x4 kf[2], vf[2];
  auto fetch = [&](int tile) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int ek = tile * kHKeys + lkey + 32 * u;
      kf[u] = ek < A.N ? *reinterpret_cast<const u32x4*>(kpool + erow(ek) + 8 * lpart)
                       : u32x4{0u, 0u, 0u, 0u};
      const int ev = tile * kHKeys + 2 * lkey + u;
      vf[u] = ev < A.N ? *reinterpret_cast<const u32x4*>(vpool + erow(ev) + 8 * lpart)
                       : u32x4{0u, 0u, 0u, 0u};
    }
  };
  const int e_st = (2 * lkey) ^ vt_swizzle(8 * lpart);   // the same for all 8 channels
  auto stash = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
      *reinterpret_cast<u32x4*>(&s_k[buf][(lkey + 32 * u) * kKPitch + 8 * lpart]) = kf[u];
#pragma unroll
    for (int c = 0; c < 4; ++c) {                 // channel 8*lpart + 2c (+1): entries 2*lkey, +1
      const uint32_t lo = (vf[0][c] & 0xffffu) | (vf[1][c] << 16);
      const uint32_t hi = (vf[0][c] >> 16) | (vf[1][c] & 0xffff0000u);
      *reinterpret_cast<uint32_t*>(&s_vt[buf][(8 * lpart + 2 * c) * kVPitch + e_st]) = lo;
      *reinterpret_cast<uint32_t*>(&s_vt[buf][(8 * lpart + 2 * c + 1) * kVPitch + e_st]) = hi;
    }
  };

  f32x16a acc[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) acc[ct] = f32x16a{};
  float m_run = -INFINITY, l_run = 0.0f;
  const float sl2 = A.scale * 1.4426950408889634f;   // logits in base 2

  if (ntiles > 0) {
    fetch(0);
    stash(0);
  }
  __syncthreads();
  for (int tile = 0; tile < ntiles; ++tile) {
    const int buf = tile & 1;
    const bool more = tile + 1 < ntiles;
    if (more) fetch(tile + 1);
    // S^T of both halves: A = K rows (entry 32h + col), k-slots 16s + 8hh
    f32x16a st[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      st[h2] = f32x16a{};
#pragma unroll
      for (int s = 0; s < 8; ++s)
        st[h2] = mfma32x32x16(
            *reinterpret_cast<const u32x4*>(&s_k[buf][(32 * h2 + col) * kKPitch + 16 * s + 8 * hh]),
            qb[s], st[h2]);
    }
    const int kb = tile * kHKeys;
    float mx = -INFINITY;
    // the logits stay unscaled (scale > 0 keeps their order); the scale enters the
    // exponent's fma below
    if (kb + kHKeys <= nv_min) {                  // block-uniform: no entry of the tile masked
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[h2][r]);
    } else {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int e = kb + 32 * h2 + 8 * (r >> 2) + 4 * hh + (r & 3);
          st[h2][r] = e < nv ? st[h2][r] : -INFINITY;
          mx = fmaxf(mx, st[h2][r]);
        }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave)) * sl2;
    const float m_new = fmaxf(m_run, mx);
    if (__ballot(m_new > m_run)) {                // some row's maximum moved: rescale
      const float alpha = m_new > m_run ? exp2_unit(m_run - m_new) : 1.0f;   // exp2(-inf) = 0
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) acc[ct] *= alpha;
      l_run *= alpha;
      m_run = m_new;
    }
    const float mneg = m_run == -INFINITY ? 0.0f : -m_run;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      u32x4 pb[2];
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const float p0 = exp2_unit(fmaf(st[h2][8 * s + 2 * m], sl2, mneg));
          const float p1 = exp2_unit(fmaf(st[h2][8 * s + 2 * m + 1], sl2, mneg));
          l_run += p0 + p1;
          pb[s][m] = pack_bf16x2(p0, p1);
        }
      // O^T tiles: A = V^T rows (channel 32ct + col), entries 32h + 16s + 4hh + 0..3 and +8
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int ch = 32 * ct + col, sw = vt_swizzle(ch);
        const uint16_t* vrow = &s_vt[buf][ch * kVPitch];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int e = 32 * h2 + 16 * s + 4 * hh;
          const uint2 lo = *reinterpret_cast<const uint2*>(vrow + (e ^ sw));
          const uint2 hi = *reinterpret_cast<const uint2*>(vrow + ((e + 8) ^ sw));
          acc[ct] = mfma32x32x16(u32x4{lo.x, lo.y, hi.x, hi.y}, pb[s], acc[ct]);
        }
      }
    }
    if (more) stash(buf ^ 1);
    __syncthreads();
  }

  if (!tok_ok) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  float* o = A.out + (row * 16 + head) * 128;
  // acc[ct] register r: channel 32ct + 8*(r/4) + 4*hh + r%4
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<f32x4*>(o + 32 * ct + 8 * q + 4 * hh) =
          f32x4{acc[ct][4 * q] * inv, acc[ct][4 * q + 1] * inv, acc[ct][4 * q + 2] * inv,
                acc[ct][4 * q + 3] * inv};
  if (hh == 0)
    A.lse[row * 16 + head] = l_tot > 0.0f ? (m_run + log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
}

// ------------------------------------------------------------------ merge

__global__ __launch_bounds__(256) void lse_merge_kernel(const float* __restrict__ part_o,
                                                        const float* __restrict__ part_l,
                                                        int splits, int rows, int H, int d,
                                                        float* __restrict__ out,
                                                        float* __restrict__ lse) {
  __shared__ float s_w[1024];
  __shared__ float s_red[2];
  lse_merge_row(part_o, part_l, splits, rows, H, d, out, lse, blockIdx.x, blockIdx.y, s_w, s_red);
}

// The merges of two attention calls in one launch: rows 0 .. a.rows-1 of grid.y merge the
// first call's splits, the rest the second's.  grid: (H, rows_a + rows_b); block d threads.
struct MergeJob {
  const float* part_o;
  const float* part_l;
  int splits, rows;
  float* out;
  float* lse;
};
__global__ __launch_bounds__(256) void lse_merge2_kernel(MergeJob a, MergeJob b, int H, int d) {
  __shared__ float s_w[1024];
  __shared__ float s_red[2];
  const int y = blockIdx.y;
  const MergeJob& m = y < a.rows ? a : b;
  const int row = y < a.rows ? y : y - a.rows;
  lse_merge_row(m.part_o, m.part_l, m.splits, m.rows, H, d, m.out, m.lse, blockIdx.x, row,
                s_w, s_red);
}

}  // namespace


// Split count asked for by hcsa_set_attn_splits (0: the plan's own choice), this thread.
static thread_local int t_attn_splits = 0;
void set_attn_splits(int splits) { t_attn_splits = splits; }

AttnPlan plan_attention(bool csa, int kv_dtype, int B, int Nq, int H, int d, int max_len) {
  AttnPlan p{};
  p.rows = B * Nq;
  p.max_len = max_len;
  p.mfma = kv_dtype == 1 && H == 16 && d == 128;
  p.tiled = !csa && p.mfma && Nq >= kTokTile;
  if (p.tiled) {                                  // one pass per 16-token tile, no splits
    p.chunk = std::max(max_len, 1);
    p.splits = 1;
    p.part_bytes = p.total_bytes = 0;
    return p;
  }
  p.hca_decode = !csa && p.mfma;
  if (p.hca_decode) {
    // about one block per CU over the whole call, 128-entry granules
    const int64_t total = static_cast<int64_t>(p.rows) * std::max(max_len, 1);
    int64_t c = (total + 255) / 256;
    c = (c + 127) / 128 * 128;
    p.chunk = static_cast<int>(std::min<int64_t>(std::max<int64_t>(c, 128), kMfmaMaxChunk));
  } else if (p.mfma) {
    // about two blocks per CU over the whole call, 128-key granules, at most kMfmaMaxChunk
    const int64_t total = static_cast<int64_t>(p.rows) * std::max(max_len, 1);
    int64_t c = (total + 511) / 512;
    c = (c + 127) / 128 * 128;
    c = std::max<int64_t>(c, 128);
    c = std::min<int64_t>(c, kMfmaMaxChunk);
    p.chunk = static_cast<int>(c);
  } else {
    p.chunk = kGenChunk;
  }
  if (t_attn_splits > 0 && p.mfma) {
    // the split kernels take any key range per block up to their LDS key list
    const int L = std::max(max_len, 1);
    p.chunk = std::min((L + t_attn_splits - 1) / t_attn_splits, kMfmaMaxChunk);
  }
  p.splits = std::max(1, (max_len + p.chunk - 1) / p.chunk);
  if (p.splits > 1) {
    const size_t o = align256(static_cast<size_t>(p.splits) * p.rows * H * d * 4);
    const size_t l = align256(static_cast<size_t>(p.splits) * p.rows * H * 4);
    p.part_bytes = o + l;
  }
  p.total_bytes = p.part_bytes;
  return p;
}

hipError_t launch_attention(bool csa, const AttnArgs& a, const AttnPlan& plan, void* ws,
                            hipStream_t s) {
  AttnDev A = attn_dev_for(a, plan, ws);
  float* part_o = plan.splits > 1 ? A.out : nullptr;
  float* part_l = plan.splits > 1 ? A.lse : nullptr;
  if (plan.tiled) {
    hca_tiled_kernel<<<dim3((a.Nq + kTokTile - 1) / kTokTile, a.B), 512, 0, s>>>(A);
    return hipGetLastError();
  }
  dim3 grid(plan.splits, plan.rows);
  if (plan.hca_decode) {
    if (a.block_table) hca_decode_kernel<true><<<grid, 256, 0, s>>>(A);
    else hca_decode_kernel<false><<<grid, 256, 0, s>>>(A);
  } else if (plan.mfma) {
    if (csa) attn_mfma_kernel<true><<<grid, 256, 0, s>>>(A);
    else attn_mfma_kernel<false><<<grid, 256, 0, s>>>(A);
  } else {
    const size_t lds = (static_cast<size_t>(a.H) * a.d + static_cast<size_t>(a.H) * kGenChunk +
                        kGenChunk) * 4;
    const bool bf = a.kv_dtype == 1;
    if (csa && bf) attn_generic_kernel<true, true><<<grid, 256, lds, s>>>(A);
    else if (csa) attn_generic_kernel<true, false><<<grid, 256, lds, s>>>(A);
    else if (bf) attn_generic_kernel<false, true><<<grid, 256, lds, s>>>(A);
    else attn_generic_kernel<false, false><<<grid, 256, lds, s>>>(A);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.splits == 1) return e;
  lse_merge_kernel<<<dim3(a.H, plan.rows), a.d, 0, s>>>(part_o, part_l, plan.splits,
                                                          plan.rows, a.H, a.d, a.out, a.lse);
  return hipGetLastError();
}

bool csa_hca_fused(const AttnPlan& pc, const AttnPlan& ph) {
  return pc.mfma && !pc.tiled && ph.hca_decode;
}

hipError_t launch_csa_hca(const AttnArgs& c, const AttnPlan& pc, const AttnArgs& h,
                          const AttnPlan& ph, void* ws, hipStream_t s) {
  void* ws_h = static_cast<char*>(ws) + align256(pc.total_bytes);
  if (!csa_hca_fused(pc, ph)) {
    hipError_t e = launch_attention(true, c, pc, ws, s);
    if (e != hipSuccess) return e;
    return launch_attention(false, h, ph, ws_h, s);
  }
  const AttnDev C = attn_dev_for(c, pc, ws);
  const AttnDev Hd = attn_dev_for(h, ph, ws_h);
  const int blocks = pc.splits * pc.rows + ph.splits * ph.rows;
  if (blocks > 0) {
    if (h.block_table) csa_hca_decode_kernel<true><<<blocks, 256, 0, s>>>(C, Hd);
    else csa_hca_decode_kernel<false><<<blocks, 256, 0, s>>>(C, Hd);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const MergeJob mc{C.out, C.lse, pc.splits, pc.rows, c.out, c.lse};
  const MergeJob mh{Hd.out, Hd.lse, ph.splits, ph.rows, h.out, h.lse};
  if (pc.splits > 1 && ph.splits > 1)
    lse_merge2_kernel<<<dim3(c.H, pc.rows + ph.rows), c.d, 0, s>>>(mc, mh, c.H, c.d);
  else if (pc.splits > 1)
    lse_merge_kernel<<<dim3(c.H, pc.rows), c.d, 0, s>>>(C.out, C.lse, pc.splits, pc.rows, c.H,
                                                          c.d, c.out, c.lse);
  else if (ph.splits > 1)
    lse_merge_kernel<<<dim3(h.H, ph.rows), h.d, 0, s>>>(Hd.out, Hd.lse, ph.splits, ph.rows,
                                                          h.H, h.d, h.out, h.lse);
  return hipGetLastError();
}

}  // namespace hcsa
