// Independent Philox4x32-10 reference for the oracle's pin: PyTorch's
// header-only at::philox_engine (ATen/core/PhiloxRNGEngine.h).  Its key is the
// 64-bit seed (low word first) and its counter is (offset_lo, offset_hi,
// subsequence_lo, subsequence_hi); the first draw is word 0 of the block.
// Reads lines "c0 c1 c2 c3 k0 k1" (decimal) on stdin, prints the four words.
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdio>
#include <cstdint>

int main() {
  unsigned long long c0, c1, c2, c3, k0, k1;
  while (std::scanf("%llu %llu %llu %llu %llu %llu", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    const uint64_t seed = (uint64_t)k0 | ((uint64_t)k1 << 32);
    const uint64_t subseq = (uint64_t)c2 | ((uint64_t)c3 << 32);
    const uint64_t offset = (uint64_t)c0 | ((uint64_t)c1 << 32);
    at::philox_engine eng(seed, subseq, offset);
    uint32_t w[4];
    for (int i = 0; i < 4; ++i) w[i] = eng();
    std::printf("%u %u %u %u\n", w[0], w[1], w[2], w[3]);
  }
  return 0;
}
