// Runs sel::select_candidates (the selection code of the library, compiled for the host on
// the SIMT emulation) over a candidate list read from stdin and prints the selection.
// Input: PER NT C k L, then C lines "key index" (keys >= L, indices ascending).
// The list is split over the threads as the resolve kernels split it: thread t holds
// candidates [t*per, t*per + my), per = ceil(C / NT).  Output: k indices, one per line.
#include <cstdio>
#include <cstring>
#include <random>
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

// RowView<16>::ge_mask (the word-parallel test of two bf16 keys at once) against the
// element-by-element comparison of the keys, over random chunks whose raw values sit near
// the floor (equal, one step either side), at +-0 and at the extremes, for floors on both
// sides of the sign split and every tail length.  Prints the number of mismatches.
static int check_ge_mask() {
  std::mt19937 g(20260424);
  const uint16_t specials[] = {0x0000, 0x8000, 0x7f80, 0xff80, 0x7f7f, 0xff7f, 0x0001, 0x8001,
                               0x7fff, 0x3f80, 0xbf80, 0x4000};
  long bad = 0, runs = 0;
  uint16_t buf[8];
  for (int it = 0; it < 400000; ++it) {
    const uint32_t L = it % 4 == 0 ? (g() & 0xffffu) : (0x8000u + (g() % 0x7f81u));
    const uint16_t rawL = static_cast<uint16_t>(L >= 0x8000u ? L - 0x8000u : ~L & 0xffffu);
    for (int e = 0; e < 8; ++e) {
      const uint32_t c = g() % 6;
      uint16_t v;
      if (c == 0) v = specials[g() % 12];
      else if (c <= 2) v = static_cast<uint16_t>(rawL + static_cast<int>(g() % 3) - 1);
      else if (c == 3) v = static_cast<uint16_t>(rawL ^ 0x8000u);
      else v = static_cast<uint16_t>(g());
      buf[e] = v;
    }
    const int nv = 1 + static_cast<int>(g() % 8);
    hcsa::sel::RowView<16> rv(buf, nv, 1);
    const hcsa::u32x4 x = rv.load_raw(0);
    const uint32_t m = rv.ge_mask(x, 0, L);
    uint32_t want = 0;
    for (int e = 0; e < nv; ++e) want |= static_cast<uint32_t>(hcsa::bf16_key(buf[e]) >= L) << e;
    bad += m != want;
    ++runs;
  }
  std::printf("%ld %ld\n", bad, runs);
  return 0;
}

int main(int argc, char** argv) {
  if (argc > 1 && std::strcmp(argv[1], "gemask") == 0) return check_ge_mask();
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
