// Host-side unit check of the fast N:M superblock decode: on random valid 2:4
// and 6:8 superblocks it must equal the bit-by-bit reference decode.  Also
// checks the one-token N:M dot product (byte permutes of 64 * t bytes) against
// sum (c - 1) * x over the reference decode, with v_perm_b32 and v_dot4
// emulated as their ISA descriptions define them.
// Built and run by tests/test_nm_decode_host.py (CPU only, no GPU calls).
#include "common.hpp"
#include <cstdio>
#include <random>
#include <algorithm>
#include <vector>
using namespace bl;
struct HostOps {
  static int bad_selector;
  // v_perm_b32: selector byte 0-3 picks a byte of s1, 4-7 of s0, 12 gives 0
  static uint32_t perm(uint32_t s0, uint32_t s1, uint32_t sel) {
    const uint64_t d = ((uint64_t)s0 << 32) | s1;
    uint32_t r = 0;
    for (int i = 0; i < 4; ++i) {
      const uint32_t v = (sel >> (8 * i)) & 0xFF;
      uint32_t b = 0;
      if (v < 8) b = (uint32_t)(d >> (8 * v)) & 0xFF;
      else if (v != 12) ++bad_selector;
      r |= b << (8 * i);
    }
    return r;
  }
  // v_dot4_i32_i8: four signed byte products added to c
  static int dot4(int a, int b, int c) {
    for (int i = 0; i < 4; ++i) c += (int8_t)(a >> (8 * i)) * (int8_t)(b >> (8 * i));
    return c;
  }
};
int HostOps::bad_selector = 0;
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
    // one-token dot: 64 * sum (c - 1) * x over the dense decode
    static uint32_t sel[2 * 512];
    static bool init = false;
    if (!init) { for (int i = 0; i < nm_sel_entries(P); ++i) nm_sel_entry<P>(i, &sel[2 * i], &sel[2 * i + 1]); init = true; }
    int32_t xw[16];
    int64_t ref = 0;
    for (int w = 0; w < 16; ++w) {
      uint32_t word = 0;
      for (int i = 0; i < 4; ++i) {
        const int x = (int)(rng() % 256) - 128;
        word |= (uint32_t)(x & 0xFF) << (8 * i);
        const int j = 4 * w + i;                         // position in the superblock
        const int code = (a[j >> 4] >> code_bit(j & 15)) & 3;
        ref += (int64_t)(code - 1) * x;
      }
      xw[w] = (int32_t)word;
    }
    int acc[4] = {0, 0, 0, 0};
    nm_dot_superblock<P, HostOps>(vals, masks, sel, xw, acc);
    const int64_t got = (int64_t)acc[0] + acc[1] + acc[2] + acc[3];
    bad += got != 64 * ref;
  }
  return bad + HostOps::bad_selector;
}
int main() {
  std::mt19937 rng(1);
  uint8_t tab[256];
  for (int i = 0; i < 256; ++i) tab[i] = nm24_table_entry(i);
  int b24 = run<Pattern::NM24>(rng, tab), b68 = run<Pattern::NM68>(rng, tab);
  printf("mismatches 2:4 %d 6:8 %d\n", b24, b68);
  return b24 || b68;
}
