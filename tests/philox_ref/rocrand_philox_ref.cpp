// Philox4x32-10 blocks from rocRAND's engine (rocrand/rocrand_philox4x32_10.h, host side),
// an implementation of the Salmon et al. (SC'11) generator written apart from this
// repository.  Reads lines "c0 c1 c2 c3 k0 k1" (decimal words of the counter and key),
// prints the four output words of each block.  Built and run by
// tests/test_oracle_philox_rocrand.py to pin the oracle's Philox4x32-10.
#include <cstdio>

#include <rocrand/rocrand_philox4x32_10.h>

int main() {
  unsigned long long c0, c1, c2, c3, k0, k1;
  while (std::scanf("%llu %llu %llu %llu %llu %llu", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    // the engine keys on the seed's two words and starts at counter (0, 0, sub_lo, sub_hi);
    // an offset of 4 n outputs advances words 0-1 by n with carries
    if (c1 >= (1ull << 30)) return 2;
    rocrand_device::philox4x32_10_engine eng(k0 | (k1 << 32), c2 | (c3 << 32), 4ull * (c0 | (c1 << 32)));
    const unsigned a = eng.next(), b = eng.next(), c = eng.next(), d = eng.next();
    std::printf("%u %u %u %u\n", a, b, c, d);
  }
  return 0;
}
