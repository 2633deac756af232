// Independent reference for the oracle's Philox4x32-10: rocRAND's header-only
// host/device engine, built for the host only (no GPU needed).
//
// Usage: rocrand_philox <seed> <row> <stage> <nblocks>
// Prints, one block per line, the four 32-bit words of Philox4x32-10 at
// counter (i, row, stage, 0), key (seed mod 2^32, seed >> 32), i = 0..nblocks-1.
// rocRAND keeps the low 64 counter bits as "offset / 4" and the high 64 bits
// as "subsequence", so that counter is offset 4*(i + row*2^32), subsequence
// = stage.  The offset is 64-bit, so row must stay below 2^30 here.
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>
#include <cstdlib>

int main(int argc, char** argv) {
  if (argc != 5) {
    std::fprintf(stderr, "usage: %s seed row stage nblocks\n", argv[0]);
    return 2;
  }
  const unsigned long long seed = std::strtoull(argv[1], nullptr, 0);
  const unsigned long long row = std::strtoull(argv[2], nullptr, 0);
  const unsigned long long stage = std::strtoull(argv[3], nullptr, 0);
  const unsigned long long nblocks = std::strtoull(argv[4], nullptr, 0);
  for (unsigned long long i = 0; i < nblocks; ++i) {
    rocrand_state_philox4x32_10 st;
    rocrand_init(seed, stage, 4ull * (i + (row << 32)), &st);
    unsigned int w[4];
    for (int j = 0; j < 4; ++j) w[j] = rocrand(&st);
    std::printf("%u %u %u %u\n", w[0], w[1], w[2], w[3]);
  }
  return 0;
}
