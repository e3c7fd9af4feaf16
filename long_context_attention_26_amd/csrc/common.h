// Device helpers shared by the libhcsa kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hcsa {

constexpr int kWave = 64;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

// ---------------------------------------------------------------- bf16 <-> fp32

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest, ties to even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7fffffffu) > 0x7f800000u) return (b >> 16) | 0x40u;
  b += 0x7fffu + ((b >> 16) & 1u);
  return b >> 16;
}

// Two values to bf16 (lo in the low half) by the conversion instruction: round to nearest
// even, the same bits as f32_to_bf16_bits for every non-NaN value (a NaN stays a NaN).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  typedef float f32x2v __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{lo, hi}, bf16x2v));
}

// ---------------------------------------------------------------- order-preserving keys
// Larger score <=> larger unsigned key; -0 and +0 map to the same key.

__device__ __forceinline__ uint32_t f32_key(uint32_t b) {
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint32_t bf16_key(uint32_t h) {
  if (h == 0x8000u) h = 0u;
  return (h & 0x8000u) ? (~h & 0xffffu) : (h | 0x8000u);
}

// max(x, 0) in one instruction (median of x, 0, +inf); fmaxf costs a canonicalizing max
// first.  The sign of a zero result is not defined; callers add it to a +0-started sum.
// Paged caches: positions [128 * blk, 128 * blk + 128) of sequence b live in page
// table[b * stride + blk] of every cache tensor; a tensor pooled at ratio r (r divides 128)
// holds 128 / r rows per page, so its pointer is a pool [pages][128 / r][row].  A null
// table means contiguous tensors [B][...] with a per-sequence stride.
constexpr int kPageTokens = 128;

struct PageMap {
  const int32_t* table;
  int64_t stride;
};

// Offset (in row units of `row` elements or bytes) of row j of sequence b in a tensor with
// 2^per_log2 rows per page, or b * bstride + j * row when contiguous.
template <bool PAGED>
__device__ __forceinline__ int64_t row_off(const PageMap& pm, int64_t bstride, int b, int64_t j,
                                           int per_log2, int row) {
  if constexpr (PAGED) {
    const int64_t pg = pm.table[b * pm.stride + (j >> per_log2)];
    return ((pg << per_log2) + (j & ((1 << per_log2) - 1))) * row;
  } else {
    return b * bstride + j * row;
  }
}

// Position of query token i of sequence b: seq_pos[b] + i when a per-sequence array is
// given (ragged batches), else pos0 + i.
__device__ __forceinline__ int64_t query_pos(const int64_t* seq_pos, int64_t pos0, int b, int i) {
  return (seq_pos ? seq_pos[b] : pos0) + i;
}

// max(x, 0) for every finite x in one median-of-three instruction (with +inf as the third
// operand the compiler turns the median into a maximum that first canonicalizes x: two
// instructions).  A sum of weighted ReLUs starting from +0 never ends at -0 whichever zero
// this gives for -0.
__device__ __forceinline__ float relu(float x) {
  return __builtin_amdgcn_fmed3f(x, 0.0f, 3.40282347e+38f);
}

// ---------------------------------------------------------------- wave reductions

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Eight consecutive values (F32, or BF16 widened) from a 16-byte aligned address.
template <bool IN_BF16>
__device__ __forceinline__ void load8(const void* p, float (&v)[8]) {
  if constexpr (IN_BF16) {
    u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      v[2 * c] = bf16_lo(w[c]);
      v[2 * c + 1] = bf16_hi(w[c]);
    }
  } else {
    f32x4 a = reinterpret_cast<const f32x4*>(p)[0];
    f32x4 b = reinterpret_cast<const f32x4*>(p)[1];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      v[c] = a[c];
      v[4 + c] = b[c];
    }
  }
}

// Softmax of the pooling logits into LDS (weight 1 when omega is null and r == 1).
__device__ __forceinline__ void pool_weights(const float* __restrict__ omega, int r,
                                             float* alpha) {
  if (threadIdx.x < kWave) {
    if (omega == nullptr) {
      if (threadIdx.x == 0) alpha[0] = 1.0f;
    } else {
      float m = -INFINITY;
      for (int i = threadIdx.x; i < r; i += kWave) m = fmaxf(m, omega[i]);
      m = wave_max(m);
      float s = 0.0f;
      for (int i = threadIdx.x; i < r; i += kWave) {
        const float e = expf(omega[i] - m);
        alpha[i] = e;
        s += e;
      }
      s = wave_sum(s);
      for (int i = threadIdx.x; i < r; i += kWave) alpha[i] = alpha[i] / s;
    }
  }
  __syncthreads();
}

__device__ __forceinline__ unsigned lane_id() { return __lane_id(); }

// Number of set bits of a 64-bit wave ballot below this lane.
__device__ __forceinline__ int ballot_rank(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}

// ---------------------------------------------------------------- MXFP4 (OCP MX e2m1/e8m0)

// floor(log2 |a|) for a finite non-zero float (subnormals included).
__device__ __forceinline__ int ilog2_floor(float a) {
  return __builtin_amdgcn_frexp_expf(a) - 1;
}

// Shared scale exponent of a block whose largest magnitude is amax.
__device__ __forceinline__ int mx_scale_exp(float amax) {
  if (!(amax > 0.0f)) return -127;
  int e = ilog2_floor(amax) - 2;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// e2m1 code (sign in bit 3) of v / 2^e, nearest-even on {0,.5,1,1.5,2,3,4,6}, saturating.
// Each comparison is a decision boundary of the grid; ">=" where the tie goes up (to an
// even code), ">" where it stays down.
__device__ __forceinline__ uint32_t e2m1_code(float v, int e) {
  float t = __builtin_fabsf(__builtin_ldexpf(v, -e));
  uint32_t m = (t > 0.25f) + (t >= 0.75f) + (t > 1.25f) + (t >= 1.75f) + (t > 2.5f) +
               (t >= 3.5f) + (t > 5.0f);
  return m | ((__float_as_uint(v) >> 28) & 8u);
}

// Value of an e2m1 code times 2 (an integer in [-12, 12]).
__device__ __forceinline__ int e2m1_twice(uint32_t c) {
  int m = c & 7u;
  int v = m < 4 ? m : (m == 4 ? 4 : (m == 5 ? 6 : (m == 6 ? 8 : 12)));
  return (c & 8u) ? -v : v;
}

__device__ __forceinline__ float exp2_int(int e) { return __builtin_ldexpf(1.0f, e); }

}  // namespace hcsa
