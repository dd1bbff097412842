// Prints the first four 32-bit outputs of PyTorch's header-only Philox4x32-10
// engine for each "seed subsequence offset" line on stdin.  PyTorch's engine
// keys with the 64-bit seed and starts at the counter
// (offset lo, offset hi, subsequence lo, subsequence hi); it is an independent
// implementation used only to pin the oracle's Philox.
#include <ATen/core/PhiloxRNGEngine.h>

#include <cstdio>

int main() {
  unsigned long long seed, sub, off;
  while (std::scanf("%llu %llu %llu", &seed, &sub, &off) == 3) {
    at::philox_engine e(seed, sub, off);
    unsigned w0 = e(), w1 = e(), w2 = e(), w3 = e();
    std::printf("%u %u %u %u\n", w0, w1, w2, w3);
  }
  return 0;
}
