// Runs sel::select_candidates (the selection code of the library, compiled for the host on
// the SIMT emulation) over a candidate list read from stdin and prints the selection.
// Input: PER NT C k L, then C lines "key index" (keys >= L, indices ascending).
// The list is split over the threads as the resolve kernels split it: thread t holds
// candidates [t*per, t*per + my), per = ceil(C / NT).  Output: k indices, one per line.
#include <cstdio>
#include <thread>
#include <vector>

#include "select_dev_under_test.h"

template <int PER, int NT>
static int run(int C, int k, uint32_t L, const std::vector<uint32_t>& key,
               const std::vector<int32_t>& idx) {
  if ((C + NT - 1) / NT > PER) return 2;
  constexpr int W = NT / 64;
  std::vector<int32_t> out(k, -7);
  int s_gt[W], s_eq[W], s_hb[W], s_hist[2][256], s_sel[4];
  emu::Block blk(NT);
  emu::g_block = &blk;
  std::vector<std::thread> th;
  for (int t = 0; t < NT; ++t) {
    th.emplace_back([&, t] {
      threadIdx.x = t;
      const int per = (C + NT - 1) / NT;
      const int g0 = std::min(C, t * per);
      const int my = std::min(per, C - g0);
      uint32_t ck[PER];
      int32_t cj[PER];
      for (int u = 0; u < PER; ++u) {
        ck[u] = u < my ? key[g0 + u] : 0u;
        cj[u] = u < my ? idx[g0 + u] : 0;
      }
      hcsa::sel::select_candidates<16, NT, PER>(ck, cj, my, L, k, out.data(), s_gt, s_eq, s_hb,
                                                s_hist, s_sel);
    });
  }
  for (auto& x : th) x.join();
  for (int i = 0; i < k; ++i) std::printf("%d\n", out[i]);
  return 0;
}

int main() {
  int per, nt, C, k;
  unsigned L;
  if (std::scanf("%d %d %d %d %u", &per, &nt, &C, &k, &L) != 5) return 3;
  std::vector<uint32_t> key(C);
  std::vector<int32_t> idx(C);
  for (int i = 0; i < C; ++i)
    if (std::scanf("%u %d", &key[i], &idx[i]) != 2) return 3;
  if (nt != 512) return 4;
  if (per == 16) return run<16, 512>(C, k, L, key, idx);
  if (per == 32) return run<32, 512>(C, k, L, key, idx);
  return 4;
}
