// Host-side reference for the oracle's Philox4x32-10: prints the block that rocRAND's
// philox4x32_10 engine produces for key = seed and counter = (c0, c1, c2, c3).
// rocRAND's engine starts at counter 0, adds `subsequence` to counter words 2-3 and offset/4 to
// counter words 0-1, so (c0, c1) -> offset 4*(c0 | c1 << 32) (needs c1 < 2^30) and
// (c2, c3) -> subsequence c2 | c3 << 32.
// Input on stdin: lines "seed c0 c1 c2 c3"; output: lines "x0 x1 x2 x3".
#include <hip/hip_runtime.h>
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>

int main() {
  unsigned long long seed;
  unsigned c0, c1, c2, c3;
  while (std::scanf("%llu %u %u %u %u", &seed, &c0, &c1, &c2, &c3) == 5) {
    unsigned long long sub = (unsigned long long)c2 | ((unsigned long long)c3 << 32);
    unsigned long long off = 4ull * ((unsigned long long)c0 | ((unsigned long long)c1 << 32));
    rocrand_device::philox4x32_10_engine e(seed, sub, off);
    unsigned a = e(), b = e(), c = e(), d = e();
    std::printf("%u %u %u %u\n", a, b, c, d);
  }
  return 0;
}
