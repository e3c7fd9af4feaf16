// Host emulation of the wave64 device primitives used by the selection helpers, for
// compiling that device code with a host C++ compiler in CPU tests.  Every thread of a
// block is an OS thread; a wave's 64 threads meet at a barrier for each ballot or shuffle
// (values exchanged through a per-wave array), and the block's threads at another for
// __syncthreads.  Only the primitives the selection code calls are provided.
#pragma once
#include <algorithm>
#include <atomic>
#include <barrier>
#include <cstdint>
#include <memory>
#include <vector>

#define __device__
#define __host__
#define __forceinline__ inline
#define __global__

struct EmuDim3 {
  unsigned x = 0, y = 0, z = 0;
};
inline thread_local EmuDim3 threadIdx;
inline thread_local EmuDim3 blockIdx;

namespace emu {
struct Block {
  int nt;
  std::unique_ptr<std::barrier<>> block_bar;
  std::vector<std::unique_ptr<std::barrier<>>> wave_bar;
  std::vector<int64_t> xchg;       // one slot per thread
  explicit Block(int nthreads) : nt(nthreads), xchg(nthreads) {
    block_bar = std::make_unique<std::barrier<>>(nthreads);
    for (int w = 0; w < nthreads / 64; ++w) wave_bar.push_back(std::make_unique<std::barrier<>>(64));
  }
};
inline Block* g_block = nullptr;

// every lane of the calling wave publishes v; returns the 64 values of the wave
inline void exchange(int64_t v, int64_t (&all)[64]) {
  const int w = threadIdx.x / 64, base = w * 64;
  g_block->xchg[threadIdx.x] = v;
  g_block->wave_bar[w]->arrive_and_wait();
  for (int l = 0; l < 64; ++l) all[l] = g_block->xchg[base + l];
  g_block->wave_bar[w]->arrive_and_wait();
}
}  // namespace emu

inline uint64_t __ballot(int pred) {
  int64_t all[64];
  emu::exchange(pred != 0, all);
  uint64_t m = 0;
  for (int l = 0; l < 64; ++l) m |= static_cast<uint64_t>(all[l] != 0) << l;
  return m;
}
inline int __shfl_up(int v, unsigned d, int width = 64) {
  (void)width;
  int64_t all[64];
  emu::exchange(v, all);
  const int l = threadIdx.x % 64;
  return l >= static_cast<int>(d) ? static_cast<int>(all[l - d]) : v;
}
inline int __shfl(int v, int src, int width = 64) {
  (void)width;
  int64_t all[64];
  emu::exchange(v, all);
  return static_cast<int>(all[src & 63]);
}
inline int __shfl_xor(int v, int mask, int width = 64) {
  (void)width;
  int64_t all[64];
  emu::exchange(v, all);
  return static_cast<int>(all[(threadIdx.x % 64) ^ mask]);
}
inline void __syncthreads() { emu::g_block->block_bar->arrive_and_wait(); }
inline int atomicAdd(int* p, int v) { return std::atomic_ref<int>(*p).fetch_add(v); }
#define __HIP_MEMORY_SCOPE_AGENT 3
template <typename T>
inline void __hip_atomic_store(T* p, T v, int order, int scope) {
  (void)scope;
  __atomic_store_n(p, v, order);
}
// v_perm_b32: byte i of the result is chosen by byte i of sel from the eight bytes of
// (hi:lo), lo's bytes 0..3 first; selector 12 gives 0x00, 13 and above 0xff, and 8..11
// replicate the sign bit of bytes 1, 3, 5, 7 (the ISA manual's table).
inline uint32_t __builtin_amdgcn_perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  const uint64_t v = (static_cast<uint64_t>(hi) << 32) | lo;
  uint32_t r = 0;
  for (int i = 0; i < 4; ++i) {
    const uint32_t s = (sel >> (8 * i)) & 0xffu;
    uint32_t b;
    if (s < 8)
      b = static_cast<uint32_t>(v >> (8 * s)) & 0xffu;
    else if (s < 12)
      b = (v >> (16 * (s - 8) + 15)) & 1u ? 0xffu : 0u;
    else
      b = s == 12 ? 0u : 0xffu;
    r |= b << (8 * i);
  }
  return r;
}
inline int __popcll(uint64_t m) { return __builtin_popcountll(m); }
inline int __popc(uint32_t m) { return __builtin_popcount(m); }
inline int __ffs(uint32_t m) { return __builtin_ffs(static_cast<int>(m)); }
inline int min(int a, int b) { return std::min(a, b); }
inline int max(int a, int b) { return std::max(a, b); }

namespace hcsa {
constexpr int kWave = 64;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
inline uint32_t f32_key(uint32_t b) {
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
inline uint32_t bf16_key(uint32_t h) {
  if (h == 0x8000u) h = 0u;
  return (h & 0x8000u) ? (~h & 0xffffu) : (h | 0x8000u);
}
}  // namespace hcsa
