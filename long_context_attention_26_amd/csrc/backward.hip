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
// summed over the 64 lanes in one batched butterfly: every exchange step halves the
// values a lane keeps, so 2H values cost about 2H shuffles instead of 12 H.
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
};

// Sums each of the N values v[0..N) over the 64 lanes of the wave.  Each step pairs value i
// with value i + n/2: the lane with the step's lane bit set keeps the upper one, its partner
// the lower one, and each adds what the other sends.  With N <= 64 the lane ends holding
// value j = lane >> (6 - log2 N) in v[0]; with N = 128, values 2 lane and 2 lane + 1 in
// v[0], v[1].
template <int N>
__device__ __forceinline__ void wave_reduce_scatter(float (&v)[N], int lane) {
  constexpr int R = N >= 64 ? 6 : (N >= 32 ? 5 : (N >= 16 ? 4 : (N >= 8 ? 3 : (N >= 4 ? 2 : 1))));
#pragma unroll
  for (int st = 0; st < R; ++st) {
    const int delta = 32 >> st;
    const bool up = (lane & delta) != 0;
    const int half = (N >> (st + 1));
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const float keep = up ? v[i + half] : v[i];
      const float send = up ? v[i] : v[i + half];
      v[i] = keep + __shfl_xor(send, delta, kWave);
    }
  }
  if constexpr (N <= 64) {
#pragma unroll
    for (int delta = 32 >> R; delta >= 1; delta >>= 1) v[0] += __shfl_xor(v[0], delta, kWave);
  }
}

__device__ __forceinline__ float bcast(float v, int src_lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src_lane));
}

// grid: rows (B * Nq); block 256 (4 waves).  HH >= H heads, CPL * 64 >= d channels.
template <bool CSA, bool BF16, int HH, int CPL>
__global__ __launch_bounds__(256) void attn_bwd_kernel(AttnBwdDev G) {
  constexpr int NV = 2 * HH;                     // q.k and dout.v per head
  constexpr int R = NV >= 64 ? 6 : (NV >= 32 ? 5 : (NV >= 16 ? 4 : 3));
  __shared__ float s_dq[4096];
  const AttnDev& A = G.A;
  const int row = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int H = A.H, d = A.d;
  const RowKeys r = row_keys<CSA>(A, row);

  // this lane's channels of q, dout and o for every head; per-head D_h = dout_h . o_h
  float qv[HH][CPL], dov[HH][CPL], dqv[HH][CPL];
  float dterm[HH];
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
    dterm[h] = wave_sum(part);
  }
  // the head whose (q.k, dout.v) pair this lane holds after the reduction, and its terms
  const int my_h = NV <= 64 ? (lane >> (7 - R)) : lane;
  float my_lse = -INFINITY, my_dt = 0.0f;
#pragma unroll
  for (int h = 0; h < HH; ++h) {
    if (h == my_h && h < H) {
      my_lse = G.lse[static_cast<int64_t>(row) * H + h];
      my_dt = dterm[h] - (G.dlse ? G.dlse[static_cast<int64_t>(row) * H + h] : 0.0f);
    }
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
      float s = 0.0f, dp = 0.0f;
#pragma unroll
      for (int t = 0; t < CPL; ++t) {
        s = fmaf(qv[h][t], kv[t], s);
        dp = fmaf(dov[h][t], vv[t], dp);
      }
      v[2 * h] = s;
      v[2 * h + 1] = dp;
    }
    wave_reduce_scatter<NV>(v, lane);
    float s_my, dp_my;
    if constexpr (NV <= 64) {
      // lanes of value 2h hold q.k, lanes of value 2h + 1 dout.v: swap to have both
      const float other = __shfl_xor(v[0], 1 << (6 - R), kWave);
      const bool odd = ((lane >> (6 - R)) & 1) != 0;
      s_my = odd ? other : v[0];
      dp_my = odd ? v[0] : other;
    } else {
      s_my = v[0];
      dp_my = v[1];
    }
    const float p = my_lse == -INFINITY ? 0.0f : __expf(A.scale * s_my - my_lse);
    const float ds = p * (dp_my - my_dt);
    // every head's P and dS, broadcast from the lane that holds it
    float dk[CPL], dv[CPL];
#pragma unroll
    for (int t = 0; t < CPL; ++t) dk[t] = dv[t] = 0.0f;
#pragma unroll
    for (int h = 0; h < HH; ++h) {
      if (h >= H) break;
      const int src = NV <= 64 ? (h << (7 - R)) : h;
      const float ph = bcast(p, src), dsh = bcast(ds, src);
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
  const int rows = a.B * a.Nq;
  if (rows == 0) return hipSuccess;
  const int hh = bwd_heads(a.H), cpl = bwd_cpl(a.d);
  const bool bf = a.kv_dtype == 1;
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
