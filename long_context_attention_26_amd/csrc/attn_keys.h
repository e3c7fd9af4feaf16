// Key lists of the CSA and HCA attention, shared by the forward and backward kernels.
//
// Key list of a query token at position p:
//   CSA: positions 0..k-1 are the selected entries (entries outside [0, n_c(p)) are
//        skipped), positions k.. are the raw tokens max(0, p-n_win+1) .. p.
//   HCA: positions 0..n_h(p)-1 are the entries themselves.
#pragma once
#include "common.h"
#include "internal.h"

namespace hcsa {
namespace attn {

struct AttnDev {
  const void* q;
  const void* kc;
  const void* vc;
  int64_t c_bstride;
  int N, ratio;
  const int32_t* idx;
  int k;
  const void* k_raw;
  const void* v_raw;
  int64_t raw_bstride, T_raw, raw_pos0;
  int n_win;
  int64_t pos0;
  const int64_t* seq_pos;   // [B] or null
  PageMap pm;               // paged caches (table null: contiguous)
  int c_log2;               // log2 of the compressed cache's rows per page
  int64_t raw_ring;         // 0, or raw tokens in a ring of raw_ring (a power of two) rows
  int Nq, H, d;
  float scale;
  int chunk, splits, rows;
  float* out;      // final [rows][H][d] (splits == 1) or partial [splits][rows][H][d]
  float* lse;      // final [rows][H] or partial [splits][rows][H]
};

// 2^x on the transcendental unit.  The library's exp2f only adds a rescaling for results
// below the smallest normal float (x < -126); a softmax weight that small changes no sum,
// and 2^-inf is still 0.
__device__ __forceinline__ float exp2_unit(float x) { return __builtin_amdgcn_exp2f(x); }

// Key-list geometry of one query row.
struct RowKeys {
  int b;
  int nv;          // visible compressed entries
  int L;           // key list length
  int64_t wstart;  // first window position (CSA)
};

template <bool CSA>
__device__ __forceinline__ RowKeys row_keys(const AttnDev& A, int row) {
  RowKeys r;
  r.b = row / A.Nq;
  const int64_t p = query_pos(A.seq_pos, A.pos0, r.b, row % A.Nq);
  const int64_t v = (p + 1) / A.ratio;
  r.nv = static_cast<int>(v < A.N ? v : A.N);
  if constexpr (CSA) {
    r.wstart = p - A.n_win + 1 > 0 ? p - A.n_win + 1 : 0;
    const int winlen = A.n_win > 0 ? static_cast<int>(p - r.wstart + 1) : 0;
    r.L = A.k + winlen;
  } else {
    r.wstart = 0;
    r.L = r.nv;
  }
  return r;
}

// Source of key-list position `pos`: >= 0 compressed row, -1 none, <= -2 raw row -(code+2).
// COH: the selection is read with agent-coherent loads (written by another block of the same
// launch).
template <bool CSA, bool COH = false>
__device__ __forceinline__ int key_code(const AttnDev& A, const RowKeys& r, int row, int pos) {
  if (pos >= r.L) return -1;
  if constexpr (CSA) {
    if (pos < A.k) {
      const int32_t* ip = A.idx + static_cast<int64_t>(row) * A.k + pos;
      const int e = COH ? __hip_atomic_load(const_cast<int32_t*>(ip), __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT)
                        : *ip;
      return (e >= 0 && e < r.nv) ? e : -1;
    }
    const int64_t t = r.wstart + (pos - A.k) - A.raw_pos0;
    return -static_cast<int>(t) - 2;
  } else {
    return pos;
  }
}

template <typename TE>
__device__ __forceinline__ const TE* key_row(const AttnDev& A, int b, int code, bool value) {
  if (code >= 0) {
    const TE* base = static_cast<const TE*>(value ? A.vc : A.kc);
    if (A.pm.table) return base + row_off<true>(A.pm, 0, b, code, A.c_log2, A.d);
    return base + b * A.c_bstride + static_cast<int64_t>(code) * A.d;
  }
  const TE* base = static_cast<const TE*>(value ? A.v_raw : A.k_raw);
  // raw rows: one per token at position raw_pos0 + row; in a ring, position t sits in row
  // t mod raw_ring; paged, 128 per page
  if (A.raw_ring)
    return base + b * A.raw_bstride + ((-code - 2) & (A.raw_ring - 1)) * A.d;
  if (A.pm.table) return base + row_off<true>(A.pm, 0, b, A.raw_pos0 + (-code - 2), 7, A.d);
  return base + b * A.raw_bstride + static_cast<int64_t>(-code - 2) * A.d;
}

template <bool BF16>
__device__ __forceinline__ float ld(const void* p, int64_t i) {
  if constexpr (BF16) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  else return static_cast<const float*>(p)[i];
}

// Kernel-side geometry of an attention call (outputs and splits are set by the caller).
inline AttnDev make_attn_dev(const AttnArgs& a) {
  AttnDev A{};
  A.q = a.q;
  A.kc = a.kc;
  A.vc = a.vc;
  A.c_bstride = a.c_bstride;
  A.N = a.N;
  A.ratio = a.ratio;
  A.idx = a.idx;
  A.k = a.k;
  A.k_raw = a.k_raw;
  A.v_raw = a.v_raw;
  A.raw_bstride = a.raw_bstride;
  A.T_raw = a.T_raw;
  A.raw_pos0 = a.raw_pos0;
  A.n_win = a.n_win;
  A.pos0 = a.pos0;
  A.seq_pos = a.seq_pos;
  A.pm.table = a.block_table;
  A.pm.stride = a.table_stride;
  A.raw_ring = a.raw_ring;
  A.c_log2 = 0;
  for (int per = kPageTokens / a.ratio; per > 1; per >>= 1) ++A.c_log2;
  A.Nq = a.Nq;
  A.H = a.H;
  A.d = a.d;
  A.scale = a.scale;
  return A;
}

// Kernel arguments of one attention call: with splits, the partials go to the workspace
// (outputs [splits][rows][H][d], then log-sum-exps [splits][rows][H]).
inline AttnDev attn_dev_for(const AttnArgs& a, const AttnPlan& plan, void* ws) {
  AttnDev A = make_attn_dev(a);
  A.chunk = plan.chunk;
  A.splits = plan.splits;
  A.rows = plan.rows;
  if (plan.splits > 1) {
    A.out = static_cast<float*>(ws);
    A.lse = reinterpret_cast<float*>(
        static_cast<char*>(ws) +
        align256(static_cast<size_t>(plan.splits) * plan.rows * a.H * a.d * 4));
  } else {
    A.out = a.out;
    A.lse = a.lse;
  }
  return A;
}

}  // namespace attn
}  // namespace hcsa
