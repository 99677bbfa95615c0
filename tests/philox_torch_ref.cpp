// Prints Philox4x32-10 output blocks computed by PyTorch's own header-only
// engine (at::philox_engine), an implementation independent of the oracle's.
// stdin: lines "seed stream block"; stdout: the four 32-bit words of the
// block whose counter is (block lo, block hi, stream lo, stream hi) under
// key (seed lo, seed hi).
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdio>

int main() {
  unsigned long long seed, stream, block;
  while (std::scanf("%llu %llu %llu", &seed, &stream, &block) == 3) {
    // philox_engine(seed, subsequence, offset): subsequence fills counter
    // words 2..3, offset (in 128-bit blocks) fills counter words 0..1.
    at::philox_engine eng(seed, stream, block);
    unsigned w[4];
    for (int i = 0; i < 4; ++i) w[i] = eng();
    std::printf("%u %u %u %u\n", w[0], w[1], w[2], w[3]);
  }
  return 0;
}
