// Host-side unit check of the fast N:M superblock decode: on random valid 2:4
// and 6:8 superblocks it must equal the bit-by-bit reference decode.
// Built and run by tests/test_nm_decode_host.py (CPU only, no GPU calls).
#include "common.hpp"
#include <cstdio>
#include <random>
#include <algorithm>
#include <vector>
using namespace bl;
template <Pattern P> int run(std::mt19937 &rng, const uint8_t *tab) {
  constexpr int M = P == Pattern::NM24 ? 4 : 8, N = P == Pattern::NM24 ? 2 : 6, VW = P == Pattern::NM24 ? 2 : 3;
  int bad = 0;
  for (int it = 0; it < 200000; ++it) {
    uint32_t vals[3] = {0, 0, 0}, masks[2] = {0, 0};
    int c = 0;
    for (int g = 0; g < 64 / M; ++g) {
      uint32_t mk = 0; int cnt = 0;
      std::vector<int> idx(M); for (int i = 0; i < M; ++i) idx[i] = i;
      std::shuffle(idx.begin(), idx.end(), rng);
      for (int i = 0; i < N; ++i) mk |= 1u << idx[i];
      (void)cnt;
      if (M == 4) masks[g >> 3] |= mk << (4 * (g & 7)); else masks[g >> 2] |= mk << (8 * (g & 3));
      for (int r = 0; r < N; ++r, ++c) vals[c >> 4] |= (uint32_t)(rng() % 3) << code_bit(c & 15);
    }
    uint32_t a[4], b[4];
    decode_superblock<P>(vals, masks, a);
    decode_superblock_fast<P>(vals, masks, b, tab);
    for (int d = 0; d < 4; ++d) bad += a[d] != b[d];
    (void)VW;
  }
  return bad;
}
int main() {
  std::mt19937 rng(1);
  uint8_t tab[256];
  for (int i = 0; i < 256; ++i) tab[i] = nm24_table_entry(i);
  int b24 = run<Pattern::NM24>(rng, tab), b68 = run<Pattern::NM68>(rng, tab);
  printf("mismatches 2:4 %d 6:8 %d\n", b24, b68);
  return b24 || b68;
}
