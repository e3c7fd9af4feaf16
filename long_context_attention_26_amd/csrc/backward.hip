// Backward of the CSA / HCA attention and of the block pooling, for training (the sparse
// attention is trained from the 64K stage of the length curriculum: Lighthouse, "deep
// deepseek v4 release", section 八 item 2).  The selection (top-k indices) is an input and
// is not differentiated.
//
// Attention: with the forward's output o and log-sum-exp per head, every key j of a
// query's list gets the probability P_hj = exp(scale q_h.k_j - lse_h) back exactly, and
//   dS_hj = P_hj (dout_h.v_j - dout_h.o_h + dlse_h)
//   dq_h  = scale sum_j dS_hj k_j          (written)
//   dk_j += scale sum_h dS_hj q_h          (accumulated: keys are shared by queries)
//   dv_j += sum_h P_hj dout_h              (accumulated)
// attn_bwd_kernel takes one query token per block; its 4 waves split the key list.  Lanes
// own channels (c = lane + 64 t), so a key's K and V rows are read, and its dk/dv rows
// added, as whole coalesced rows.  The 2H dot products of a key (q_h.k and dout_h.v) are
// summed over the 64 lanes together: two half-swapping lane permutes leave each 16-lane group
// a quarter of the values, summed over 4 lanes, and DPP row rotations finish the sums.
//
// Pooling: y_j = sum_i alpha_i x_{jr+i} with alpha = softmax(omega) gives
//   dx_{jr+i} += alpha_i dy_j,   domega_k += alpha_k (g_k - sum_i alpha_i g_i),
//   g_i = sum_{b,j} dy_j . x_{jr+i}.
// pool_bwd_dx_kernel updates dx and writes each token's dot dy_j . x_t; pool_bwd_g_kernel
// sums the dots of one position i over all entries in a fixed order (deterministic);
// pool_bwd_omega_kernel forms domega.
#include "attn_keys.h"
#include "common.h"
#include "internal.h"

#include <type_traits>

namespace hcsa {

namespace {

using namespace attn;

struct AttnBwdDev {
  AttnDev A;
  const float* out;      // [rows][H][d]
  const float* lse;      // [rows][H]
  const float* dout;     // [rows][H][d]
  const float* dlse;     // [rows][H] or null
  float* dq;             // [rows][H][d]
  float* dkc;            // compressed-entry gradients [B][N][d] (dc_bstride)
  float* dvc;
  int64_t dc_bstride;
  float* dkr;            // raw-row gradients [B][T_raw][d] (dr_bstride)
  float* dvr;
  int64_t dr_bstride;
  float* dt_out;         // [rows][16] or null: dout.o - dlse per head, for the key-major pass
  const uint16_t* dout16;  // [rows][16][128] bf16 copy of dout for the key-major pass, or null
  // CSA selected entries key-major (else null): the dq pass stores each valid (row, position)
  // pair's P and dS per head, bf16, at rec[row][slot[row][position]] (16 words: P pairs of
  // heads 2m, 2m + 1 in words m, dS pairs in words 8 + m)
  const uint16_t* slot;  // [rows][k]
  uint32_t* rec;         // [rows][k][16]
  // with the records: rows listing an entry twice (dup[row] = 1) are left out of the dq
  // pass and taken whole by the query-major kernel with dK / dV (which skips the others)
  const uint8_t* dup;    // [rows] or null
};

// Sums each of the N values v[0..N) over the 64 lanes of the wave with no lane-dependent
// selection: v_permlane32_swap exchanges lanes 32..63 of one register with lanes 0..31 of
// another, so adding the two results sums value i over lanes l, l^32 in the lower half-wave
// and value i + N/2 in the upper one; v_permlane16_swap does the same for 16-lane rows; the
// rest is summed within each 16-lane row by DPP rotations of 8, 4, 2 and 1.  Afterwards
// lane group g = lane / 16 holds the full sums of values g*N/4 .. g*N/4 + N/4 - 1 in u.
template <int N>
__device__ __forceinline__ void wave_sum_quarters(const float (&v)[N], float (&u)[N / 4]) {
  float w[N / 2];
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]),
                                                    __float_as_uint(v[i + N / 2]), false, false);
    w[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
#pragma unroll
  for (int i = 0; i < N / 4; ++i) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(w[i]),
                                                    __float_as_uint(w[i + N / 4]), false, false);
    float x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    // DPP row_ror:8, 4, 2, 1 (controls 0x128, 0x124, 0x122, 0x121)
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xF, 0xF, false));
    u[i] = x;
  }
}

__device__ __forceinline__ float bcast(float v, int src_lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src_lane));
}

// grid: rows (B * Nq); block 256 (4 waves).  HH >= H heads, CPL * 64 >= d channels.
template <bool CSA, bool BF16, int HH, int CPL>
__global__ __launch_bounds__(256) void attn_bwd_kernel(AttnBwdDev G) {
  constexpr int NV = 2 * HH;                     // q.k and dout.v per head
  constexpr int HQ = HH / 4;                     // heads per 16-lane group after the sums
  __shared__ float s_dq[4096];
  __shared__ float s_dt[HH];
  const AttnDev& A = G.A;
  const int row = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int H = A.H, d = A.d;
  const RowKeys r = row_keys<CSA>(A, row);

  // this lane's channels of q and dout for every head; D_h = dout_h . o_h per head
  float qv[HH][CPL], dov[HH][CPL], dqv[HH][CPL];
  const int64_t hb = static_cast<int64_t>(row) * H * d;
#pragma unroll
  for (int h = 0; h < HH; ++h) {
    float part = 0.0f;
#pragma unroll
    for (int t = 0; t < CPL; ++t) {
      const int c = lane + 64 * t;
      const bool ok = h < H && c < d;
      qv[h][t] = ok ? ld<BF16>(A.q, hb + h * d + c) : 0.0f;
      dov[h][t] = ok ? G.dout[hb + h * d + c] : 0.0f;
      dqv[h][t] = 0.0f;
      if (ok) part = fmaf(dov[h][t], G.out[hb + h * d + c], part);
    }
    part = wave_sum(part);
    if (threadIdx.x == 0) s_dt[h] = part;
  }
  __syncthreads();
  // the heads whose sums this lane's group holds: g*HQ + m
  const int g = lane >> 4;
  float my_lse[HQ], my_dt[HQ];
#pragma unroll
  for (int m = 0; m < HQ; ++m) {
    const int h = g * HQ + m;
    const int64_t li = static_cast<int64_t>(row) * H + h;
    my_lse[m] = h < H ? G.lse[li] : -INFINITY;
    my_dt[m] = h < H ? s_dt[h] - (G.dlse ? G.dlse[li] : 0.0f) : 0.0f;
  }

  for (int pos = wave; pos < r.L; pos += 4) {
    const int code = key_code<CSA>(A, r, row, pos);
    if (code == -1) continue;                      // wave-uniform
    using TE = typename std::conditional<BF16, uint16_t, float>::type;
    const TE* kp = key_row<TE>(A, r.b, code, false);
    const TE* vp = key_row<TE>(A, r.b, code, true);
    float kv[CPL], vv[CPL];
#pragma unroll
    for (int t = 0; t < CPL; ++t) {
      const int c = lane + 64 * t;
      kv[t] = c < d ? ld<BF16>(kp, c) : 0.0f;
      vv[t] = c < d ? ld<BF16>(vp, c) : 0.0f;
    }
    float v[NV];
#pragma unroll
    for (int h = 0; h < HH; ++h) {
      float sk = 0.0f, dp = 0.0f;
#pragma unroll
      for (int t = 0; t < CPL; ++t) {
        sk = fmaf(qv[h][t], kv[t], sk);
        dp = fmaf(dov[h][t], vv[t], dp);
      }
      v[2 * h] = sk;
      v[2 * h + 1] = dp;
    }
    float u[NV / 4];
    wave_sum_quarters<NV>(v, u);
    float p[HQ], ds[HQ];
#pragma unroll
    for (int m = 0; m < HQ; ++m) {
      p[m] = my_lse[m] == -INFINITY ? 0.0f : __expf(A.scale * u[2 * m] - my_lse[m]);
      ds[m] = p[m] * (u[2 * m + 1] - my_dt[m]);
    }
    // every head's P and dS, read from the first lane of the group that holds it
    float dk[CPL], dv[CPL];
#pragma unroll
    for (int t = 0; t < CPL; ++t) dk[t] = dv[t] = 0.0f;
#pragma unroll
    for (int h = 0; h < HH; ++h) {
      if (h >= H) break;
      const float ph = bcast(p[h % HQ], 16 * (h / HQ));
      const float dsh = bcast(ds[h % HQ], 16 * (h / HQ));
#pragma unroll
      for (int t = 0; t < CPL; ++t) {
        dk[t] = fmaf(dsh, qv[h][t], dk[t]);
        dv[t] = fmaf(ph, dov[h][t], dv[t]);
        dqv[h][t] = fmaf(dsh, kv[t], dqv[h][t]);
      }
    }
    float* dkrow;
    float* dvrow;
    if (code >= 0) {
      const int64_t o = r.b * G.dc_bstride + static_cast<int64_t>(code) * d;
      dkrow = G.dkc + o;
      dvrow = G.dvc + o;
    } else {
      const int64_t o = r.b * G.dr_bstride + static_cast<int64_t>(-code - 2) * d;
      dkrow = G.dkr + o;
      dvrow = G.dvr + o;
    }
#pragma unroll
    for (int t = 0; t < CPL; ++t) {
      const int c = lane + 64 * t;
      if (c < d) {
        unsafeAtomicAdd(dkrow + c, A.scale * dk[t]);
        unsafeAtomicAdd(dvrow + c, dv[t]);
      }
    }
  }

  // dq: the 4 waves' sums added in wave order, then written scaled
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int h = 0; h < HH; ++h)
#pragma unroll
        for (int t = 0; t < CPL; ++t) {
          const int c = lane + 64 * t;
          if (h < H && c < d) {
            if (w == 0) s_dq[h * d + c] = dqv[h][t];
            else s_dq[h * d + c] += dqv[h][t];
          }
        }
    }
    __syncthreads();
  }
  for (int i = threadIdx.x; i < H * d; i += 256) G.dq[hb + i] = A.scale * s_dq[i];
}


// ------------------------------------------------------------------ matrix-core path (bf16, 16 x 128)

typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;
typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mma32(const u32x4& a, const u32x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(const u32x2& a, const u32x2& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                   __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// Backward of one query token's 16 heads over its key list, 32 keys per wave step, on the
// matrix cores (bf16 operands, fp32 accumulation).  Lane (col = lane % 16, g = lane / 16).
// The logits and dout.v products are formed twice, as S^T = K Q^T (lane = head col, keys
// 4g + i of each 16-key tile) and as S = Q K^T (lane = key col, heads 4g + i), so that every
// later product finds its operand in the accumulator layout it already has:
//   dQ^T += K^T dS^T  (16x16x32, the forward's V^T P^T form with K slices for V),
//   dK    = dS^T Q,  dV = P^T dout  (16x16x16 over the 16 heads, one per 16-channel tile),
// and the dK / dV tiles go to memory with atomics, 4 rows x 16 channels per instruction.
// With DKV false only dq is formed (the key-major kernel below takes dK and dV), and the
// per-head terms dout.o - dlse are stored for it.
template <bool CSA, bool DKV>
__global__ __launch_bounds__(256) void attn_bwd_mfma_kernel(AttnBwdDev G) {
  __shared__ float s_dq[4][16][129];
  __shared__ float s_lse2[16];
  __shared__ float s_dt[16];
  constexpr float kLog2e = 1.4426950408889634f;
  const AttnDev& A = G.A;
  const int row = blockIdx.x;
  if (G.dup && (G.dup[row] != 0) != DKV) return;   // block-uniform
  const RowKeys r = row_keys<CSA>(A, row);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, g = lane >> 4;
  const int64_t hb = static_cast<int64_t>(row) * 2048;
  const uint16_t* q16 = static_cast<const uint16_t*>(A.q) + hb;
  const float* dout = G.dout + hb;

  // per-head terms: D_h = dout_h . o_h - dlse_h, and lse_h in base 2 (16 threads per head)
  {
    const int h = threadIdx.x >> 4, c0 = (threadIdx.x & 15) * 8;
    float part = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) part = fmaf(dout[h * 128 + c0 + e], G.out[hb + h * 128 + c0 + e], part);
    part += __shfl_xor(part, 8, kWave);
    part += __shfl_xor(part, 4, kWave);
    part += __shfl_xor(part, 2, kWave);
    part += __shfl_xor(part, 1, kWave);
    if ((threadIdx.x & 15) == 0) {
      const int64_t li = static_cast<int64_t>(row) * 16 + h;
      s_dt[h] = part - (G.dlse ? G.dlse[li] : 0.0f);
      s_lse2[h] = G.lse[li] * kLog2e;
      if (G.dt_out) G.dt_out[li] = s_dt[h];
    }
  }
  __syncthreads();

  // q and dout (rounded to bf16) as operands: rows of head col at channels 32s + 8g (16x16x32)
  // and heads 4g..4g+3 at channel 16c + col (16x16x16 B operand)
  u32x4 qB[4], doB[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    qB[s] = *reinterpret_cast<const u32x4*>(q16 + col * 128 + 32 * s + 8 * g);
    const float* dr = dout + col * 128 + 32 * s + 8 * g;
#pragma unroll
    for (int m = 0; m < 4; ++m) doB[s][m] = pack_bf16x2(dr[2 * m], dr[2 * m + 1]);
  }
  u32x2 qT[8], doT[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int h0 = 4 * g + 2 * m, ch = 16 * c + col;
      qT[c][m] = static_cast<uint32_t>(q16[h0 * 128 + ch]) |
                 (static_cast<uint32_t>(q16[(h0 + 1) * 128 + ch]) << 16);
      doT[c][m] = pack_bf16x2(dout[h0 * 128 + ch], dout[(h0 + 1) * 128 + ch]);
    }
  }
  const float lse2_col = s_lse2[col], dt_col = s_dt[col];
  float lse2_g[4], dt_g[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lse2_g[i] = s_lse2[4 * g + i];
    dt_g[i] = s_dt[4 * g + i];
  }
  const float sl2 = A.scale * kLog2e;

  f32x4 acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = f32x4{0, 0, 0, 0};

  for (int base = wave * 32; base < r.L; base += 128) {
    // key codes: operand rows base + 16t + col, and keys base + 16(j/4) + 4g + j%4
    int ca[2], cs[8];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int pos = base + 16 * t + col;
      ca[t] = pos < r.L ? key_code<CSA>(A, r, row, pos) : -1;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int pos = base + 16 * (j >> 2) + 4 * g + (j & 3);
      cs[j] = pos < r.L ? key_code<CSA>(A, r, row, pos) : -1;
    }
    u32x4 ka[2][4], va[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (ca[t] != -1) {
        const uint16_t* kr = key_row<uint16_t>(A, r.b, ca[t], false);
        const uint16_t* vr = key_row<uint16_t>(A, r.b, ca[t], true);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          ka[t][s] = *reinterpret_cast<const u32x4*>(kr + 32 * s + 8 * g);
          va[t][s] = *reinterpret_cast<const u32x4*>(vr + 32 * s + 8 * g);
        }
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) ka[t][s] = va[t][s] = u32x4{0, 0, 0, 0};
      }
    }
    u32x4 ks[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      ks[j] = cs[j] != -1 ? *reinterpret_cast<const u32x4*>(key_row<uint16_t>(A, r.b, cs[j], false) + 8 * col)
                          : u32x4{0, 0, 0, 0};

    // ---- lane = head: S^T and dP^T, dS^T for keys 16(j/4) + 4g + j%4
    f32x4 st[2], dpt[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      st[t] = dpt[t] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        st[t] = mma32(ka[t][s], qB[s], st[t]);
        dpt[t] = mma32(va[t][s], doB[s], dpt[t]);
      }
    }
    float dsT[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float pj = cs[j] != -1 ? exp2_unit(st[j >> 2][j & 3] * sl2 - lse2_col) : 0.0f;
      dsT[j] = pj * (dpt[j >> 2][j & 3] - dt_col);
      if (CSA && !DKV && G.rec) {
        // the selected entry's record: even lanes store P of heads col, col + 1, odd lanes
        // dS of heads col - 1, col (the partner lane holds the same key)
        const float mine = (col & 1) ? dsT[j] : pj;
        const float other = __shfl_xor((col & 1) ? pj : dsT[j], 1, kWave);
        if (cs[j] >= 0) {
          const int pos = base + 16 * (j >> 2) + 4 * g + (j & 3);
          const int64_t rb = static_cast<int64_t>(row) * A.k;
          uint32_t* rp = G.rec + (rb + G.slot[rb + pos]) * 16;
          if (col & 1) rp[8 + (col >> 1)] = pack_bf16x2(other, mine);
          else rp[col >> 1] = pack_bf16x2(mine, other);
        }
      }
    }
    u32x4 dsB;
#pragma unroll
    for (int m = 0; m < 4; ++m) dsB[m] = pack_bf16x2(dsT[2 * m], dsT[2 * m + 1]);
    // dQ^T tiles: channel 8 col + ct of the K slices, as the forward's V^T
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      const uint32_t sel = (ct & 1) ? 0x07060302u : 0x05040100u;
      u32x4 kA;
#pragma unroll
      for (int m = 0; m < 4; ++m)
        kA[m] = __builtin_amdgcn_perm(ks[2 * m + 1][ct >> 1], ks[2 * m][ct >> 1], sel);
      acc[ct] = mma32(kA, dsB, acc[ct]);
    }

    // ---- lane = key: S and dP of key base + 16t + col for heads 4g + i; dK, dV tiles
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if constexpr (!DKV) break;
      f32x4 sk = f32x4{0, 0, 0, 0}, dp = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        sk = mma32(qB[s], ka[t][s], sk);
        dp = mma32(doB[s], va[t][s], dp);
      }
      float pk[4], dsk[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pk[i] = ca[t] != -1 ? exp2_unit(sk[i] * sl2 - lse2_g[i]) : 0.0f;
        dsk[i] = pk[i] * (dp[i] - dt_g[i]);
      }
      const u32x2 pA = {pack_bf16x2(pk[0], pk[1]), pack_bf16x2(pk[2], pk[3])};
      const u32x2 dsA = {pack_bf16x2(dsk[0], dsk[1]), pack_bf16x2(dsk[2], dsk[3])};
      float* dkr[4];
      float* dvr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int code = cs[4 * t + i];
        dkr[i] = dvr[i] = nullptr;
        if (code >= 0) {
          const int64_t o = r.b * G.dc_bstride + static_cast<int64_t>(code) * 128;
          dkr[i] = G.dkc + o;
          dvr[i] = G.dvc + o;
        } else if (code != -1 && G.dkr) {           // window rows (unless taken key-major)
          const int64_t o = r.b * G.dr_bstride + static_cast<int64_t>(-code - 2) * 128;
          dkr[i] = G.dkr + o;
          dvr[i] = G.dvr + o;
        }
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const f32x4 dkt = mma16(dsA, qT[c], f32x4{0, 0, 0, 0});
        const f32x4 dvt = mma16(pA, doT[c], f32x4{0, 0, 0, 0});
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (dkr[i]) {
            unsafeAtomicAdd(dkr[i] + 16 * c + col, A.scale * dkt[i]);
            unsafeAtomicAdd(dvr[i] + 16 * c + col, dvt[i]);
          }
        }
      }
    }
  }

  // dQ: lane holds dQ^T[channel 32g + 8i + t][head col] = acc[t][i]; the 4 waves add up
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int t = 0; t < 8; ++t) s_dq[wave][col][32 * g + 8 * i + t] = acc[t][i];
  __syncthreads();
  for (int e = threadIdx.x; e < 2048; e += 256) {
    const int h = e >> 7, c = e & 127;
    G.dq[hb + e] = A.scale * (((s_dq[0][h][c] + s_dq[1][h][c]) + s_dq[2][h][c]) + s_dq[3][h][c]);
  }
}

// Key-major dK / dV for keys shared by many query tokens (bf16, 16 heads x 128): the HCA
// entries (every later token sees them) and the CSA window rows (the next n_win tokens see
// each).  A block owns 16 keys for a chunk of 128 query tokens; each wave takes two tokens
// (32 query rows) per step.  S = Q K^T and dP = dout V^T run with lane = key (16x16x32, K as
// the B operand), so P and dS are already the B operand of
//   dK^T += Q^T dS,  dV^T += dout^T P   (16x16x32 over the step's 32 rows; Q^T and dout^T
// built from 16-byte row slices by byte permutes, as the forward builds V^T),
// accumulated over the chunk in registers, summed over the 4 waves in LDS and added to
// memory once per element.  dout.o - dlse per (token, head) comes from the dq pass, dout as
// a bf16 copy (the MFMA operand precision) made once before this pass.
// HCA: grid (ceil(N / 16), chunks, B), keys e0 = 16 * blockIdx.x.  Window: grid
// (ceil((128 + n_win - 1) / 16), chunks, B), the tiles covering the band of raw rows that the
// chunk's windows reach, from its first query's window start on.
constexpr int kDkvEntries = 16;
constexpr int kDkvTokens = 128;

// block 256.
template <bool WIN>
__global__ __launch_bounds__(256) void key_bwd_kernel(AttnBwdDev G) {
  __shared__ float s_acc[2][kDkvEntries][129];
  constexpr float kLog2e = 1.4426950408889634f;
  const AttnDev& A = G.A;
  const int t0 = blockIdx.y * kDkvTokens, b = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, g = lane >> 4;
  const int64_t pfirst = query_pos(A.seq_pos, A.pos0, b, t0);
  const int64_t plast = query_pos(A.seq_pos, A.pos0, b, min(t0 + kDkvTokens, A.Nq) - 1);
  int64_t e0;                         // first key of the tile: entry, or raw row
  if constexpr (WIN) {
    e0 = pfirst - A.n_win + 1 - A.raw_pos0 + static_cast<int64_t>(blockIdx.x) * kDkvEntries;
    // rows of the tile inside the raw rows and reached by some window of the chunk
    if (e0 + kDkvEntries <= 0 || e0 >= A.T_raw || A.raw_pos0 + e0 > plast) return;
  } else {
    e0 = static_cast<int64_t>(blockIdx.x) * kDkvEntries;
    // the chunk's last token must see the tile's first entry, else nothing to do
    if ((e0 + 1) * A.ratio > plast + 1) return;                          // block-uniform
  }

  const int64_t e = e0 + col;
  const bool e_ok = WIN ? (e >= 0 && e < A.T_raw) : (e < A.N);
  const int64_t kpos = A.raw_pos0 + e;      // window: the key's position
  u32x4 ka[4], va[4];                 // B operand: K[e][32s + 8g ..], V likewise
  {
    const uint16_t* kr = WIN ? static_cast<const uint16_t*>(A.k_raw) + b * A.raw_bstride + e * 128
                             : static_cast<const uint16_t*>(A.kc) + b * A.c_bstride + e * 128;
    const uint16_t* vr = WIN ? static_cast<const uint16_t*>(A.v_raw) + b * A.raw_bstride + e * 128
                             : static_cast<const uint16_t*>(A.vc) + b * A.c_bstride + e * 128;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      ka[s] = e_ok ? *reinterpret_cast<const u32x4*>(kr + 32 * s + 8 * g) : u32x4{0, 0, 0, 0};
      va[s] = e_ok ? *reinterpret_cast<const u32x4*>(vr + 32 * s + 8 * g) : u32x4{0, 0, 0, 0};
    }
  }
  f32x4 accK[8], accV[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) accK[t] = accV[t] = f32x4{0, 0, 0, 0};
  const float sl2 = A.scale * kLog2e;
  const uint16_t* q16 = static_cast<const uint16_t*>(A.q);

  for (int it = 0; it < kDkvTokens / 8; ++it) {
    const int ta = t0 + 2 * wave + 8 * it;          // tokens ta (rows 0..15), ta + 1 (16..31)
    float pv[2][4], dsv[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int tok = ta + tt;
      const bool t_ok = tok < A.Nq;
      const int64_t row = static_cast<int64_t>(b) * A.Nq + (t_ok ? tok : 0);
      const int64_t p = query_pos(A.seq_pos, A.pos0, b, t_ok ? tok : 0);
      const bool vis = t_ok && e_ok &&
                       (WIN ? (kpos <= p && kpos > p - A.n_win) : (e + 1) * A.ratio <= p + 1);
      // A operands: q and dout rows of head col at channels 32s + 8g
      u32x4 qa[4], da[4];
      const uint16_t* qrow = q16 + (row * 16 + col) * 128;
      const uint16_t* drow = G.dout16 + (row * 16 + col) * 128;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        qa[s] = *reinterpret_cast<const u32x4*>(qrow + 32 * s + 8 * g);
        da[s] = *reinterpret_cast<const u32x4*>(drow + 32 * s + 8 * g);
      }
      f32x4 sv = f32x4{0, 0, 0, 0}, dp = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        sv = mma32(qa[s], ka[s], sv);               // S[head 4g + i][entry col]
        dp = mma32(da[s], va[s], dp);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t li = row * 16 + 4 * g + i;
        const float pe = vis ? exp2_unit(sv[i] * sl2 - G.lse[li] * kLog2e) : 0.0f;
        pv[tt][i] = pe;
        dsv[tt][i] = pe * (dp[i] - G.dt_out[li]);
      }
    }
    // B operands: rows k = 8g + j <-> (token ta + j / 4, head 4g + j % 4)
    const u32x4 pB = {pack_bf16x2(pv[0][0], pv[0][1]), pack_bf16x2(pv[0][2], pv[0][3]),
                      pack_bf16x2(pv[1][0], pv[1][1]), pack_bf16x2(pv[1][2], pv[1][3])};
    const u32x4 dsB = {pack_bf16x2(dsv[0][0], dsv[0][1]), pack_bf16x2(dsv[0][2], dsv[0][3]),
                       pack_bf16x2(dsv[1][0], dsv[1][1]), pack_bf16x2(dsv[1][2], dsv[1][3])};
    // row slices (channels 8col .. 8col + 7) of the same 8 rows, q and dout
    u32x4 qs[8], ds8[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int tok = ta + (j >> 2);
      const int64_t row = static_cast<int64_t>(b) * A.Nq + (tok < A.Nq ? tok : 0);
      const int64_t hrow = row * 16 + 4 * g + (j & 3);
      qs[j] = *reinterpret_cast<const u32x4*>(q16 + hrow * 128 + 8 * col);
      ds8[j] = *reinterpret_cast<const u32x4*>(G.dout16 + hrow * 128 + 8 * col);
    }
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      const uint32_t sel = (ct & 1) ? 0x07060302u : 0x05040100u;
      u32x4 qA, dA;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        qA[m] = __builtin_amdgcn_perm(qs[2 * m + 1][ct >> 1], qs[2 * m][ct >> 1], sel);
        dA[m] = __builtin_amdgcn_perm(ds8[2 * m + 1][ct >> 1], ds8[2 * m][ct >> 1], sel);
      }
      accK[ct] = mma32(qA, dsB, accK[ct]);          // dK^T[channel 32g + 8i + ct][entry col]
      accV[ct] = mma32(dA, pB, accV[ct]);
    }
  }
  // the 4 waves' tiles summed in wave order, then one atomic add per element
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int c = 32 * g + 8 * i + t;
          if (w == 0) {
            s_acc[0][col][c] = accK[t][i];
            s_acc[1][col][c] = accV[t][i];
          } else {
            s_acc[0][col][c] += accK[t][i];
            s_acc[1][col][c] += accV[t][i];
          }
        }
    }
    __syncthreads();
  }
  for (int x = threadIdx.x; x < 2 * kDkvEntries * 128; x += 256) {
    const int m = x >> 11, r = (x >> 7) & 15, c = x & 127;
    const int64_t er = e0 + r;
    if (WIN ? (er >= 0 && er < A.T_raw) : (er < A.N)) {
      float* dst = WIN ? (m ? G.dvr : G.dkr) + b * G.dr_bstride + er * 128 + c
                       : (m ? G.dvc : G.dkc) + b * G.dc_bstride + er * 128 + c;
      unsafeAtomicAdd(dst, m ? s_acc[1][r][c] : A.scale * s_acc[0][r][c]);
    }
  }
}

// bf16 copy (round to nearest even) of n8 groups of 8 floats; grid-stride, block 256.
__global__ __launch_bounds__(256) void bf16_copy_kernel(const float* __restrict__ x,
                                                        uint16_t* __restrict__ y, int64_t n8) {
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n8; i += static_cast<int64_t>(gridDim.x) * 256) {
    const f32x4 a = reinterpret_cast<const f32x4*>(x)[2 * i];
    const f32x4 b = reinterpret_cast<const f32x4*>(x)[2 * i + 1];
    reinterpret_cast<u32x4*>(y)[i] = u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]),
                                            pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])};
  }
}

// ------------------------------------------------------------------ CSA selected entries, key-major
//
// A query token's selected entries differ from its neighbours', so no block of consecutive
// tokens shares them; the pairs are instead grouped by entry.  The entries are cut into
// tiles of kSelE; each row's valid selections are bucket-sorted by tile (sel_sort_kernel),
// the dq pass stores every pair's P and dS (bf16) in the row's sorted order, and
// sel_bwd_kernel takes one tile for a chunk of query tokens.  For a batch of tokens it
// scatters their pairs' P and dS into a dense [token][entry] table in LDS (zero where a
// token did not select the entry), and then per token
//   dK[tile entries] += dS^T Q,   dV[tile entries] += P^T dout
// run as 32x32x8 products over the 16 heads with the tile's entries as rows, summed in
// registers over the whole chunk: no atomics until one add per element per block at the
// end, where the query-major pass needs one per element per pair.  A row that lists an
// entry twice is left to the query-major kernel (its pairs are not sorted), which keeps
// each listed position its own key.
constexpr int kSelE = 128;              // entries per tile
constexpr int kSelTokens = 4096;        // query tokens per block
constexpr int kSelBatch = 8;            // tokens staged at once
constexpr int kSelThreads = 64 * kSelBatch;
constexpr int kSelMaxN = 262144;        // entries a row's sort can mark in an LDS bitmap

struct SelDev {
  const uint32_t* qT;    // [rows][128][16] bf16: q, channel-major (heads adjacent)
  const uint32_t* doT;   // [rows][128][16] bf16: dout rounded, channel-major
  uint16_t* slot;        // [rows][k] sorted position of a valid (row, position) pair
  uint8_t* el;           // [rows][k] entry within the tile of each sorted pair
  uint16_t* off;         // [tiles + 1][rows] first sorted position of each tile's pairs
  uint8_t* dup;          // [rows] 1: the row lists an entry twice (query-major instead)
  const uint32_t* rec;   // [rows][k][16] the dq pass's P / dS records, sorted order
  int tiles, rows;
};

// grid: rows; block 256.  A pair (row, position p) is valid when its entry e lies in the
// row's visible entries [0, nv); it goes to tile e / kSelE.  off[t][row] is the row's
// exclusive count of pairs in tiles before t (off[tiles][row]: all valid pairs); within a
// tile the order is that of the LDS counter (not deterministic).  A row with a repeated
// valid entry gets no pairs (all offsets 0) and dup[row] = 1.
__global__ __launch_bounds__(256) void sel_sort_kernel(AttnBwdDev G, SelDev S) {
  __shared__ uint32_t s_bits[kSelMaxN / 32];
  __shared__ uint32_t s_cnt[kSelMaxN / kSelE + 1];
  __shared__ uint32_t s_part[256];
  __shared__ int s_dup;
  const AttnDev& A = G.A;
  const int row = blockIdx.x;
  const RowKeys r = row_keys<true>(A, row);
  const int64_t rb = static_cast<int64_t>(row) * A.k;
  const int32_t* ip = A.idx + rb;
  const int nt = S.tiles;
  for (int t = threadIdx.x; t <= nt; t += 256) s_cnt[t] = 0;
  for (int w = threadIdx.x; w < (r.nv + 31) / 32; w += 256) s_bits[w] = 0;
  if (threadIdx.x == 0) s_dup = 0;
  __syncthreads();
  for (int p = threadIdx.x; p < A.k; p += 256) {
    const int e = ip[p];
    if (e >= 0 && e < r.nv) {
      const uint32_t bit = 1u << (e & 31);
      if (atomicOr(&s_bits[e >> 5], bit) & bit) s_dup = 1;
      atomicAdd(&s_cnt[e / kSelE], 1u);
    }
  }
  __syncthreads();
  if (s_dup) {                                   // block-uniform
    for (int t = threadIdx.x; t <= nt; t += 256) S.off[static_cast<int64_t>(t) * S.rows + row] = 0;
    if (threadIdx.x == 0) S.dup[row] = 1;
    return;
  }
  // exclusive scan of s_cnt[0..nt]: thread u takes the segment [u seg, (u + 1) seg)
  const int seg = (nt + 1 + 255) / 256;
  const int s0 = threadIdx.x * seg;
  uint32_t sum = 0;
  for (int i = 0; i < seg; ++i)
    if (s0 + i <= nt) sum += s_cnt[s0 + i];
  s_part[threadIdx.x] = sum;
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {       // inclusive scan of the 256 segment sums
    const uint32_t v = threadIdx.x >= d ? s_part[threadIdx.x - d] : 0u;
    __syncthreads();
    s_part[threadIdx.x] += v;
    __syncthreads();
  }
  uint32_t run = s_part[threadIdx.x] - sum;
  for (int i = 0; i < seg; ++i) {
    if (s0 + i <= nt) {
      const uint32_t c = s_cnt[s0 + i];
      s_cnt[s0 + i] = run;
      S.off[static_cast<int64_t>(s0 + i) * S.rows + row] = static_cast<uint16_t>(run);
      run += c;
    }
  }
  if (threadIdx.x == 0) S.dup[row] = 0;
  __syncthreads();
  for (int p = threadIdx.x; p < A.k; p += 256) {
    const int e = ip[p];
    if (e >= 0 && e < r.nv) {
      const int t = e / kSelE;
      const uint32_t sl = atomicAdd(&s_cnt[t], 1u);
      S.slot[rb + p] = static_cast<uint16_t>(sl);
      S.el[rb + sl] = static_cast<uint8_t>(e - t * kSelE);
    }
  }
}

// grid: rows; block 256.  q [row][16][128] bf16 and dout [row][16][128] f32 to channel-major
// bf16 copies [row][128][16] (dout rounded to nearest even, the products' operand precision).
__global__ __launch_bounds__(256) void sel_transpose_kernel(const uint16_t* __restrict__ q,
                                                            const float* __restrict__ dout,
                                                            uint32_t* __restrict__ qT,
                                                            uint32_t* __restrict__ doT) {
  __shared__ uint16_t s_q[16][130];
  __shared__ uint16_t s_d[16][130];
  const int64_t row = blockIdx.x;
  for (int x = threadIdx.x; x < 2048; x += 256) {
    const int h = x >> 7, c = x & 127;
    s_q[h][c] = q[row * 2048 + x];
    s_d[h][c] = static_cast<uint16_t>(f32_to_bf16_bits(dout[row * 2048 + x]));
  }
  __syncthreads();
  // thread u: channel u / 2, heads 8 (u % 2) .. + 7 -> four words of each copy
  const int c = threadIdx.x >> 1, h0 = 8 * (threadIdx.x & 1);
  u32x4 wq, wd;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    wq[m] = static_cast<uint32_t>(s_q[h0 + 2 * m][c]) | (static_cast<uint32_t>(s_q[h0 + 2 * m + 1][c]) << 16);
    wd[m] = static_cast<uint32_t>(s_d[h0 + 2 * m][c]) | (static_cast<uint32_t>(s_d[h0 + 2 * m + 1][c]) << 16);
  }
  reinterpret_cast<u32x4*>(qT + row * 1024)[threadIdx.x] = wq;
  reinterpret_cast<u32x4*>(doT + row * 1024)[threadIdx.x] = wd;
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mma32x16(const u32x4& a, const u32x4& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// grid: (tiles, ceil(Nq / kSelTokens), B); block kSelThreads (8 waves).  Wave w forms dK
// (w < 4) or dV (w >= 4) of channels 32 (w % 4) .. + 31 for all kSelE entries of the tile:
// four 32-entry row blocks, each a 32x32 accumulator (lane l: column l % 32, rows
// 8 (r / 4) + 4 (l / 32) + r % 4 of register r), one 32x32x16 product per block and token
// over its 16 heads.  A operand: the staged dS or P of entries 32m + l % 32, heads
// 8 (l / 32) .. + 7; B operand: q or dout of the same heads at channel 32 (w % 4) + l % 32,
// from the channel-major copies.
// Table rows hold a record's eight 8-byte slots (P heads 4j .. 4j + 3 in slot j, dS in
// slot 4 + j) in the permuted order of sel_slot.
// Staging: wave u stages token u of a batch, lane l its pairs l / 4 + 16 n (16-byte quarter
// l % 4).  The table is double-buffered: the next batch's records and B operands are read
// into registers while the current batch's products run, one barrier per batch.
constexpr int kSelRegPairs = 4;          // pairs per staging thread held in registers

// Word offset of 8-byte slot s of table row e: the slots are XOR-permuted by (e / 4) % 8,
// so that the 32 rows one operand read takes (32m .. 32m + 31, one slot each) fall in 32
// different bank pairs (a row is 16 words: unpermuted, rows 4 apart share banks).
__device__ __forceinline__ int sel_slot(int e, int s) { return 2 * (s ^ ((e >> 2) & 7)); }

struct SelStage {
  u32x4 v[kSelRegPairs];
  int e[kSelRegPairs];
};

__global__ __launch_bounds__(kSelThreads) void sel_bwd_kernel(AttnBwdDev G, SelDev S) {
  __shared__ uint32_t s_A[2][kSelBatch][kSelE][16];  // P pairs (words 0..7), dS (8..15)
  __shared__ uint16_t s_lo[kSelTokens + kSelBatch], s_hi[kSelTokens + kSelBatch];
  const AttnDev& A = G.A;
  const int tile = blockIdx.x, b = blockIdx.z;
  const int t0 = blockIdx.y * kSelTokens, t1 = min(t0 + kSelTokens, A.Nq);
  // the chunk's last token must see the tile's first entry, else nothing to do
  const int64_t plast = query_pos(A.seq_pos, A.pos0, b, t1 - 1);
  if (static_cast<int64_t>(tile * kSelE + 1) * A.ratio > plast + 1) return;   // block-uniform
  const int64_t row0 = static_cast<int64_t>(b) * A.Nq + t0;
  const int nb = (t1 - t0 + kSelBatch - 1) / kSelBatch;
  for (int x = threadIdx.x; x < nb * kSelBatch; x += kSelThreads) {
    const bool in = t0 + x < t1;
    s_lo[x] = in ? S.off[static_cast<int64_t>(tile) * S.rows + row0 + x] : 0;
    s_hi[x] = in ? S.off[static_cast<int64_t>(tile + 1) * S.rows + row0 + x] : 0;
  }
  for (int x = threadIdx.x; x < 2 * kSelBatch * kSelE * 16 / 4; x += kSelThreads)
    reinterpret_cast<u32x4*>(&s_A[0][0][0][0])[x] = u32x4{0u, 0u, 0u, 0u};
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lc = lane & 31, kg = lane >> 5;
  const bool isV = wave >= 4;
  const int ch = 32 * (wave & 3) + lc;
  const uint32_t* bsrc = (isV ? S.doT : S.qT) + ch * 8 + 4 * kg;
  const int as = (isV ? 0 : 4) + 2 * kg;           // A operand slots of heads 8kg .. 8kg + 7
  const int q4 = lane >> 2, qr = lane & 3;
  f32x16 acc[4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[m][r] = 0.0f;
  __syncthreads();

  // reads of batch i's staging (this thread's pairs of token `wave`) and B operands
  auto fetch = [&](int i, SelStage& st, u32x4 (&bop)[kSelBatch]) {
    const int x = i * kSelBatch + wave;
    const int lo = s_lo[x], hi = s_hi[x];
    const int64_t rb = (row0 + x) * A.k;
#pragma unroll
    for (int n = 0; n < kSelRegPairs; ++n) {
      const int j = lo + q4 + 16 * n;
      st.e[n] = -1;
      if (j < hi) {
        st.e[n] = S.el[rb + j];
        st.v[n] = reinterpret_cast<const u32x4*>(S.rec + (rb + j) * 16)[qr];
      }
    }
#pragma unroll
    for (int u = 0; u < kSelBatch; ++u) {
      const int t = t0 + i * kSelBatch + u < t1 ? i * kSelBatch + u : 0;
      bop[u] = *reinterpret_cast<const u32x4*>(bsrc + (row0 + t) * 1024);
    }
  };
  // write (or, with clear, zero) batch i's staged pairs in buffer i & 1: quarter qr of a
  // record is its 8-byte slots 2qr and 2qr + 1
  auto put = [&](uint32_t (*tab)[16], int e, const u32x4& v) {
    *reinterpret_cast<u32x2*>(&tab[e][sel_slot(e, 2 * qr)]) = u32x2{v[0], v[1]};
    *reinterpret_cast<u32x2*>(&tab[e][sel_slot(e, 2 * qr + 1)]) = u32x2{v[2], v[3]};
  };
  auto stage = [&](int i, const SelStage& st, bool clear) {
    const int x = i * kSelBatch + wave;
    const int lo = s_lo[x], hi = s_hi[x];
    uint32_t(*tab)[16] = s_A[i & 1][wave];
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int n = 0; n < kSelRegPairs; ++n)
      if (st.e[n] >= 0) put(tab, st.e[n], clear ? z : st.v[n]);
    // pairs beyond the registers' (a row holding most of the tile), read in place
    const int64_t rb = (row0 + x) * A.k;
    for (int j = lo + q4 + 16 * kSelRegPairs; j < hi; j += 16) {
      const int e = S.el[rb + j];
      put(tab, e, clear ? z : reinterpret_cast<const u32x4*>(S.rec + (rb + j) * 16)[qr]);
    }
  };

  SelStage cur, nxt;
  u32x4 bcur[kSelBatch], bnxt[kSelBatch];
  fetch(0, cur, bcur);
  // the first batch's reads complete here: the loop then carries no read in flight into
  // its products, whose operands would otherwise wait on the prefetch (the counter of
  // vector reads is in order)
  __builtin_amdgcn_s_waitcnt(0);
  for (int i = 0; i < nb; ++i) {
    stage(i, cur, false);
    if (i + 1 < nb) fetch(i + 1, nxt, bnxt);
    __syncthreads();              // batch i staged; batch i - 1's buffer cleared
#pragma unroll
    for (int u = 0; u < kSelBatch; ++u) {
      const int x = i * kSelBatch + u;
      if (s_hi[x] == s_lo[x]) continue;           // block-uniform: no pair in the tile
      u32x4 a[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int r = 32 * m + lc;
        const uint32_t* ar = s_A[i & 1][u][r];
        const u32x2 a0 = *reinterpret_cast<const u32x2*>(ar + sel_slot(r, as));
        const u32x2 a1 = *reinterpret_cast<const u32x2*>(ar + sel_slot(r, as + 1));
        a[m] = u32x4{a0[0], a0[1], a1[0], a1[1]};
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) acc[m] = mma32x16(a[m], bcur[u], acc[m]);
    }
    __syncthreads();              // every wave done with batch i's buffer
    stage(i, cur, true);
    cur = nxt;
#pragma unroll
    for (int u = 0; u < kSelBatch; ++u) bcur[u] = bnxt[u];
  }
  float* dst = (isV ? G.dvc : G.dkc) + b * G.dc_bstride + ch;
  const float f = isV ? 1.0f : A.scale;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t er = static_cast<int64_t>(tile) * kSelE + 32 * m + 8 * (r >> 2) + 4 * kg + (r & 3);
      if (er < A.N && acc[m][r] != 0.0f) unsafeAtomicAdd(dst + er * 128, f * acc[m][r]);
    }
}

// ------------------------------------------------------------------ pooling backward

// grid: (ceil(n_out * r / rows_per_block), B); block 256.  Thread (local row, c8) handles 8
// channels of one pooled token t = j*r + i: dx_t += alpha_i dy_j, and the row's dot
// dy_j . x_t (summed over its D/8 threads in channel order) goes to dots[b][t].
template <bool IN_BF16>
__global__ __launch_bounds__(256) void pool_bwd_dx_kernel(const void* __restrict__ x, int64_t x_bs,
                                                          int D, const float* __restrict__ omega,
                                                          int r, int n_out,
                                                          const float* __restrict__ dy,
                                                          int64_t dy_bs, float* __restrict__ dx,
                                                          int64_t dx_bs, float* __restrict__ dots,
                                                          int64_t T) {
  __shared__ float alpha[1024];
  __shared__ float s_dot[256];
  pool_weights(omega, r, alpha);
  const int tpr = D >> 3;
  const int rpb = 256 / tpr;
  const int local = threadIdx.x / tpr, c8 = threadIdx.x - local * tpr;
  const int b = blockIdx.y;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * rpb + local;
  const bool live = local < rpb && t < static_cast<int64_t>(n_out) * r;
  float dot = 0.0f;
  if (live) {
    const int64_t j = t / r;
    const int i = static_cast<int>(t - j * r);
    const float* dyp = dy + b * dy_bs + j * D + c8 * 8;
    float* dxp = dx + b * dx_bs + t * D + c8 * 8;
    float xv[8];
    if constexpr (IN_BF16) {
      load8<true>(static_cast<const char*>(x) + (b * x_bs + t * D + c8 * 8) * 2, xv);
    } else {
      load8<false>(static_cast<const char*>(x) + (b * x_bs + t * D + c8 * 8) * 4, xv);
    }
    const float a = alpha[i];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float g = dyp[c];
      dxp[c] = fmaf(a, g, dxp[c]);
      dot = fmaf(g, xv[c], dot);
    }
  }
  s_dot[threadIdx.x] = dot;
  __syncthreads();
  if (live && c8 == 0) {
    float sum = 0.0f;
    for (int c = 0; c < tpr; ++c) sum += s_dot[threadIdx.x + c];
    dots[b * T + t] = sum;
  }
}

// grid: r; block 256.  g_i = sum over sequences b and entries j of dots[b][j*r + i]: thread
// u sums every 256th term from u on, then the 256 partial sums are added in a fixed tree.
__global__ __launch_bounds__(256) void pool_bwd_g_kernel(const float* __restrict__ dots, int64_t T,
                                                         int B, int r, int n_out,
                                                         float* __restrict__ g) {
  __shared__ float s_part[256];
  const int i = blockIdx.x;
  const int64_t terms = static_cast<int64_t>(B) * n_out;
  float acc = 0.0f;
  for (int64_t u = threadIdx.x; u < terms; u += 256) {
    const int64_t b = u / n_out, j = u - b * n_out;
    acc += dots[b * T + j * r + i];
  }
  s_part[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (static_cast<int>(threadIdx.x) < w) s_part[threadIdx.x] += s_part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) g[i] = s_part[0];
}

// one block of 256: domega_k += alpha_k (g_k - sum_i alpha_i g_i).
__global__ __launch_bounds__(256) void pool_bwd_omega_kernel(const float* __restrict__ omega,
                                                             int r, const float* __restrict__ g,
                                                             float* __restrict__ domega) {
  __shared__ float alpha[1024];
  __shared__ float s_part[256];
  pool_weights(omega, r, alpha);
  float acc = 0.0f;
  for (int i = threadIdx.x; i < r; i += 256) acc = fmaf(alpha[i], g[i], acc);
  s_part[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (static_cast<int>(threadIdx.x) < w) s_part[threadIdx.x] += s_part[threadIdx.x + w];
    __syncthreads();
  }
  const float mean = s_part[0];
  for (int k = threadIdx.x; k < r; k += 256) domega[k] += alpha[k] * (g[k] - mean);
}

template <bool CSA, bool BF16>
hipError_t launch_bwd_typed(const AttnBwdDev& G, int rows, int hh, int cpl, hipStream_t s) {
#define HCSA_BWD(HH_, CPL_)                                                              \
  if (hh == HH_ && cpl == CPL_) {                                                        \
    attn_bwd_kernel<CSA, BF16, HH_, CPL_><<<rows, 256, 0, s>>>(G);                      \
    return hipGetLastError();                                                            \
  }
  HCSA_BWD(4, 1) HCSA_BWD(4, 2) HCSA_BWD(4, 4)
  HCSA_BWD(16, 1) HCSA_BWD(16, 2) HCSA_BWD(16, 4)
  HCSA_BWD(32, 1) HCSA_BWD(32, 2) HCSA_BWD(64, 1)
#undef HCSA_BWD
  return hipErrorInvalidValue;
}

}  // namespace

bool bwd_key_major(const AttnArgs& a) {
  return a.kv_dtype == 1 && a.H == 16 && a.d == 128 && a.Nq >= 16;
}

// CSA selected entries key-major: needs the sort's offsets to fit 16 bits and its entry
// bitmap to fit LDS
static int sel_tiles(int N) { return (N + kSelE - 1) / kSelE; }
static bool bwd_sel_key_major(const AttnArgs& a) {
  return bwd_key_major(a) && a.k > 0 && a.k <= 65535 && a.N > 0 && a.N <= kSelMaxN;
}

// Workspace of the key-major passes: dout.o - dlse [rows][16] f32, dout as bf16
// [rows][16][128]; for the CSA selected entries also the channel-major q and dout copies,
// the records [rows][k][16] words, the sorted slots [rows][k] u16, the tile entries
// [rows][k] u8 and the tile offsets [tiles + 1][rows] u16.
struct BwdWs {
  size_t dt, d16, qT, doT, rec, slot, el, off, dup, total;
};
static BwdWs bwd_ws_layout(const AttnArgs& a) {
  BwdWs w{};
  if (!bwd_key_major(a)) return w;
  const size_t rows = static_cast<size_t>(a.B) * a.Nq;
  size_t o = 0;
  w.dt = o;  o += align256(rows * 16 * 4);
  w.d16 = o; o += align256(rows * 2048 * 2);
  if (bwd_sel_key_major(a)) {
    const size_t k = static_cast<size_t>(a.k);
    w.qT = o;   o += align256(rows * 2048 * 2);
    w.doT = o;  o += align256(rows * 2048 * 2);
    w.rec = o;  o += align256(rows * k * 64);
    w.slot = o; o += align256(rows * k * 2);
    w.el = o;   o += align256(rows * k);
    w.off = o;  o += align256((static_cast<size_t>(sel_tiles(a.N)) + 1) * rows * 2);
    w.dup = o;  o += align256(rows);
  }
  w.total = o;
  return w;
}

size_t bwd_workspace_bytes(const AttnArgs& a) { return bwd_ws_layout(a).total; }

bool attn_bwd_shape_supported(int H, int d) {
  const int hh = bwd_heads(H), cpl = bwd_cpl(d);
  return hh > 0 && cpl > 0 && hh * cpl <= 64;
}

hipError_t launch_attention_bwd(bool csa, const AttnArgs& a, const AttnBwdArgs& g,
                                hipStream_t s) {
  AttnBwdDev G;
  G.A = make_attn_dev(a);
  G.A.rows = a.B * a.Nq;
  G.out = g.out;
  G.lse = g.lse;
  G.dout = g.dout;
  G.dlse = g.dlse;
  G.dq = g.dq;
  G.dkc = g.dkc;
  G.dvc = g.dvc;
  G.dc_bstride = g.dc_bstride;
  G.dkr = g.dkr;
  G.dvr = g.dvr;
  G.dr_bstride = g.dr_bstride;
  G.dt_out = nullptr;
  G.dout16 = nullptr;
  const int rows = a.B * a.Nq;
  G.slot = nullptr;
  G.rec = nullptr;
  G.dup = nullptr;
  const BwdWs wl = bwd_ws_layout(a);
  char* wsb = static_cast<char*>(g.ws);
  // the key-major pass's inputs in the workspace: dt_out, and dout converted to bf16 once
  auto key_major_inputs = [&]() {
    G.dt_out = reinterpret_cast<float*>(wsb + wl.dt);
    uint16_t* d16 = reinterpret_cast<uint16_t*>(wsb + wl.d16);
    G.dout16 = d16;
    const int64_t n8 = static_cast<int64_t>(rows) * 16 * 128 / 8;
    const int blocks = static_cast<int>(std::min<int64_t>((n8 + 255) / 256, 4096));
    bf16_copy_kernel<<<blocks, 256, 0, s>>>(g.dout, d16, n8);
  };
  if (rows == 0) return hipSuccess;
  const int hh = bwd_heads(a.H), cpl = bwd_cpl(a.d);
  const bool bf = a.kv_dtype == 1;
  if (bf && a.H == 16 && a.d == 128) {          // the matrix-core path
    const int chunks = (a.Nq + kDkvTokens - 1) / kDkvTokens;
    if (csa && g.ws && bwd_sel_key_major(a)) {
      // selected entries key-major by tile (sort, dq pass storing the pairs' P and dS,
      // tile pass), window rows key-major by token chunk
      key_major_inputs();
      SelDev S{};
      S.qT = reinterpret_cast<const uint32_t*>(wsb + wl.qT);
      S.doT = reinterpret_cast<const uint32_t*>(wsb + wl.doT);
      S.slot = reinterpret_cast<uint16_t*>(wsb + wl.slot);
      S.el = reinterpret_cast<uint8_t*>(wsb + wl.el);
      S.off = reinterpret_cast<uint16_t*>(wsb + wl.off);
      S.rec = reinterpret_cast<const uint32_t*>(wsb + wl.rec);
      S.dup = reinterpret_cast<uint8_t*>(wsb + wl.dup);
      S.tiles = sel_tiles(a.N);
      S.rows = rows;
      sel_sort_kernel<<<rows, 256, 0, s>>>(G, S);
      sel_transpose_kernel<<<rows, 256, 0, s>>>(static_cast<const uint16_t*>(a.q), g.dout,
                                                const_cast<uint32_t*>(S.qT),
                                                const_cast<uint32_t*>(S.doT));
      AttnBwdDev Gq = G;
      Gq.slot = S.slot;
      Gq.rec = reinterpret_cast<uint32_t*>(wsb + wl.rec);
      Gq.dup = S.dup;
      attn_bwd_mfma_kernel<true, false><<<rows, 256, 0, s>>>(Gq);
      // rows that list an entry twice: dq and the selected entries' dK / dV query-major
      Gq.dkr = Gq.dvr = nullptr;
      attn_bwd_mfma_kernel<true, true><<<rows, 256, 0, s>>>(Gq);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      dim3 sgrid(S.tiles, (a.Nq + kSelTokens - 1) / kSelTokens, a.B);
      sel_bwd_kernel<<<sgrid, kSelThreads, 0, s>>>(G, S);
      e = hipGetLastError();
      if (e != hipSuccess || a.n_win == 0) return e;
      dim3 grid((kDkvTokens + a.n_win - 1 + kDkvEntries - 1) / kDkvEntries, chunks, a.B);
      key_bwd_kernel<true><<<grid, 256, 0, s>>>(G);
    } else if (csa && bwd_key_major(a) && g.ws && a.n_win > 0) {
      // the window rows, shared by consecutive query tokens, key-major; the rest per query
      key_major_inputs();
      AttnBwdDev Gq = G;
      Gq.dkr = Gq.dvr = nullptr;
      attn_bwd_mfma_kernel<true, true><<<rows, 256, 0, s>>>(Gq);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      dim3 grid((kDkvTokens + a.n_win - 1 + kDkvEntries - 1) / kDkvEntries, chunks, a.B);
      key_bwd_kernel<true><<<grid, 256, 0, s>>>(G);
    } else if (csa) {
      attn_bwd_mfma_kernel<true, true><<<rows, 256, 0, s>>>(G);
    } else if (bwd_key_major(a) && g.ws) {
      // many query tokens share the entries: dq query-major, dK / dV key-major
      key_major_inputs();
      attn_bwd_mfma_kernel<false, false><<<rows, 256, 0, s>>>(G);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      if (a.N > 0) {
        dim3 grid((a.N + kDkvEntries - 1) / kDkvEntries, chunks, a.B);
        key_bwd_kernel<false><<<grid, 256, 0, s>>>(G);
      }
    } else {
      attn_bwd_mfma_kernel<false, true><<<rows, 256, 0, s>>>(G);
    }
    return hipGetLastError();
  }
  if (csa) return bf ? launch_bwd_typed<true, true>(G, rows, hh, cpl, s)
                     : launch_bwd_typed<true, false>(G, rows, hh, cpl, s);
  return bf ? launch_bwd_typed<false, true>(G, rows, hh, cpl, s)
            : launch_bwd_typed<false, false>(G, rows, hh, cpl, s);
}

size_t compress_bwd_workspace_bytes(int B, int T, int ratio) {
  return align256(static_cast<size_t>(B) * T * 4) + align256(static_cast<size_t>(ratio) * 4);
}

hipError_t launch_compress_bwd(const void* x, int x_dtype, int64_t x_bstride, int B, int T,
                               int D, const float* omega, int ratio, const float* dy,
                               int64_t dy_bstride, float* dx, int64_t dx_bstride,
                               float* domega, void* ws, hipStream_t s) {
  const int n_out = T / ratio;
  if (n_out == 0) return hipSuccess;
  float* dots = static_cast<float*>(ws);
  float* g = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                      align256(static_cast<size_t>(B) * T * 4));
  const int rpb = 256 / (D / 8);
  const int64_t rows = static_cast<int64_t>(n_out) * ratio;
  dim3 grid(static_cast<unsigned>((rows + rpb - 1) / rpb), B);
  if (x_dtype == 1)
    pool_bwd_dx_kernel<true><<<grid, 256, 0, s>>>(x, x_bstride, D, omega, ratio, n_out, dy,
                                                  dy_bstride, dx, dx_bstride, dots, T);
  else
    pool_bwd_dx_kernel<false><<<grid, 256, 0, s>>>(x, x_bstride, D, omega, ratio, n_out, dy,
                                                   dy_bstride, dx, dx_bstride, dots, T);
  if (domega) {
    pool_bwd_g_kernel<<<ratio, 256, 0, s>>>(dots, T, B, ratio, n_out, g);
    pool_bwd_omega_kernel<<<1, 256, 0, s>>>(omega, ratio, g, domega);
  }
  return hipGetLastError();
}

}  // namespace hcsa
