// Selector state shared by the indexer kernels (which build it) and the top-k kernels.
//
// Workspace layout for `rows` score rows (all 32-bit words, zeroed by the clear step):
//   hist   [rows][4096]   counts of the 12-bit top digit of each row's score keys
//   cnt    [rows]         candidates appended so far
//   ticket [rows]         blocks of the row that finished their histogram
//   b0info [rows][2]      threshold bin b0 and count of keys in bins above it
//   cand   [rows][kCap]   candidate list (64-bit), after the words above
#pragma once

#include "common.h"

namespace hcsa {

constexpr int kSelBins = 4096;
constexpr int kSelCap = 8192;

struct SelState {
  uint32_t* hist;
  uint32_t* cnt;
  uint32_t* ticket;
  int32_t* b0info;
  uint64_t* cand;
};

__host__ __device__ inline size_t sel_words(int rows) {
  return static_cast<size_t>(rows) * (kSelBins + 4);
}

__host__ __device__ inline SelState sel_state(void* ws, int rows, size_t cand_offset) {
  SelState s;
  s.hist = static_cast<uint32_t*>(ws);
  s.cnt = s.hist + static_cast<size_t>(rows) * kSelBins;
  s.ticket = s.cnt + rows;
  s.b0info = reinterpret_cast<int32_t*>(s.ticket + rows);
  s.cand = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + cand_offset);
  return s;
}

// Wave 0 finds the 12-bit bin b0 holding the k-th largest key: count(bins > b0) < k <=
// count(bins >= b0).  Lane l owns bins 4095-64l .. 4032-64l.  Results go to *s_b0, *s_above.
__device__ inline void find_b0(const uint32_t* hrow, int k, int* s_b0, int* s_above) {
  if (threadIdx.x >= kWave) return;
  const int lane = threadIdx.x;
  const int top = kSelBins - 1 - 64 * lane;
  uint32_t sum = 0;
  const u32x4* h4 = reinterpret_cast<const u32x4*>(hrow + top - 63);
  u32x4 v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = __builtin_nontemporal_load(h4 + i);
#pragma unroll
  for (int i = 0; i < 16; ++i) sum += v[i][0] + v[i][1] + v[i][2] + v[i][3];
  uint32_t incl = sum;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t t = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += t;
  }
  uint32_t above = incl - sum;
  int found = -1, found_above = 0;
  if (above < static_cast<uint32_t>(k) && incl >= static_cast<uint32_t>(k)) {
    for (int b = 63; b >= 0; --b) {       // bins top .. top-63, descending
      const uint32_t c = v[b >> 2][b & 3];
      if (above + c >= static_cast<uint32_t>(k)) {
        found = top - 63 + b;
        found_above = static_cast<int>(above);
        break;
      }
      above += c;
    }
  }
  const uint64_t who = __ballot(found >= 0);
  const int src = who ? __builtin_ctzll(who) : 0;
  found = __shfl(found, src, kWave);
  found_above = __shfl(found_above, src, kWave);
  if (lane == 0) {
    *s_b0 = found;
    *s_above = found_above;
  }
}

// Called by every block of a row after its histogram atomics: the last block of the row
// (blocks_in_row of them take part) finds b0 for the row and stores it in b0info.
__device__ inline void sel_finish_row(const SelState& S, int row, int blocks_in_row, int k) {
  __shared__ int s_last, s_b0, s_above;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = atomicAdd(&S.ticket[row], 1u) == static_cast<uint32_t>(blocks_in_row - 1);
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  find_b0(S.hist + static_cast<size_t>(row) * kSelBins, k, &s_b0, &s_above);
  __syncthreads();
  if (threadIdx.x == 0) {
    S.b0info[2 * row] = s_b0;
    S.b0info[2 * row + 1] = s_above;
  }
}

}  // namespace hcsa
