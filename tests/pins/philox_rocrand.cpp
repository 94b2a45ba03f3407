// Test helper (not product code): prints rocRAND's Philox4x32-10 output block
// for (key, counter) tuples read from stdin, one "seed c0 c1 c2 c3" per line.
// rocRAND's engine is an independent implementation of the published
// generator (Random123); the CPU tests use it to pin the oracle's Philox.
#include <cstdio>
#include <rocrand/rocrand_philox4x32_10.h>

int main() {
  unsigned long long seed;
  unsigned c0, c1, c2, c3;
  while (std::scanf("%llu %u %u %u %u", &seed, &c0, &c1, &c2, &c3) == 5) {
    unsigned long long offset = 4ull * ((unsigned long long)c1 << 32 | c0);
    unsigned long long subseq = (unsigned long long)c3 << 32 | c2;
    rocrand_device::philox4x32_10_engine eng(seed, subseq, offset);
    uint4 r = eng.next4();
    std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
