// Reference Philox4x32-10 words from rocRAND's engine (a separate implementation of the
// generator published by Salmon et al., SC'11), used to pin the oracle's Philox.
// Host-only: the engine's methods are __host__ __device__.  Build with hipcc.
//
// stdin : lines "seed x0 x1 x2 x3" (counter words), decimal
// stdout: the four output words of that block, decimal
//
// rocRAND maps a (seed, subsequence, offset) to the counter (offset / 4 as a 64-bit value
// in words 0-1, subsequence in words 2-3), so counter (x0, x1, x2, x3) is reached with
// subsequence = x2 + 2^32 x3 and offset = 4 (x0 + 2^32 x1).
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>

int main() {
  unsigned long long seed, x0, x1, x2, x3;
  while (std::scanf("%llu %llu %llu %llu %llu", &seed, &x0, &x1, &x2, &x3) == 5) {
    const unsigned long long subseq = x2 | (x3 << 32);
    const unsigned long long offset = 4ull * (x0 | (x1 << 32));
    rocrand_device::philox4x32_10_engine eng(seed, subseq, offset);
    unsigned int w[4];
    for (int i = 0; i < 4; ++i) w[i] = eng.next();
    std::printf("%u %u %u %u\n", w[0], w[1], w[2], w[3]);
  }
  return 0;
}
