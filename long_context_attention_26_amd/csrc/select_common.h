// Selector state shared by the indexer kernels (which build the histogram) and the top-k
// kernels.
//
// Workspace layout for `rows` score rows and `copies` replicas (32-bit words first, all
// zeroed by the clear step; block i of a row adds into replica i % copies, so the atomics
// of one row spread over several addresses):
//   hist   [copies][rows][4096]  counts of the 12-bit top digit of each row's score keys
//   cnt    [copies][rows]        candidates appended to each replica's list
//   b0info [rows][2]             threshold bin b0 and the count of keys in bins above it
//   cand   [rows][copies][capc]  64-bit candidates, after the words above (256-aligned)
#pragma once

#include "common.h"

namespace hcsa {

constexpr int kSelBins = 4096;
constexpr int kSelCap = 8192;   // candidates per row over all replicas

struct SelState {
  uint32_t* hist;
  uint32_t* cnt;
  int32_t* b0info;
  uint64_t* cand;
  int rows, copies, capc;
};

// Keys per block of the decode indexer kernels: enough blocks to cover every CU several
// times even for one sequence, and at least 256 keys so a block issues a few loads per lane.
__host__ __device__ inline int index_chunk(int rows, int N) {
  int64_t c = static_cast<int64_t>(N) * rows / 2048;
  c = (c + 255) / 256 * 256;
  return static_cast<int>(c < 256 ? 256 : (c > 4096 ? 4096 : c));
}

// Replicas: one per 16 indexer blocks of a row, at most 8.
__host__ __device__ inline int sel_copies(int rows, int N) {
  const int ch = index_chunk(rows, N);
  const int blocks = (N + ch - 1) / ch;
  const int c = blocks / 16;
  return c < 1 ? 1 : (c > 8 ? 8 : c);
}

__host__ __device__ inline size_t sel_words(int rows, int copies) {
  return static_cast<size_t>(rows) * copies * (kSelBins + 1) + static_cast<size_t>(rows) * 2;
}

__host__ __device__ inline SelState sel_state(void* ws, int rows, int copies,
                                              size_t cand_offset) {
  SelState s;
  s.rows = rows;
  s.copies = copies;
  s.capc = kSelCap / copies;
  s.hist = static_cast<uint32_t*>(ws);
  s.cnt = s.hist + static_cast<size_t>(copies) * rows * kSelBins;
  s.b0info = reinterpret_cast<int32_t*>(s.cnt + static_cast<size_t>(copies) * rows);
  s.cand = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + cand_offset);
  return s;
}

__device__ inline uint32_t* sel_hist_row(const SelState& S, int copy, int row) {
  return S.hist + (static_cast<size_t>(copy) * S.rows + row) * kSelBins;
}

}  // namespace hcsa
