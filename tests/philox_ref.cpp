// Reference Philox4x32-10 blocks from rocRAND's header engine (an independent
// implementation of the generator), for the sampler oracle's pins. Reads lines
// "seed subsequence c" and prints the block at counter (c mod 2^32, c / 2^32,
// subsequence mod 2^32, subsequence / 2^32) under key (seed mod 2^32, seed /
// 2^32): the engine places a subsequence in the counter's upper 64 bits and
// skips 4 c numbers (c blocks) in its lower 64 bits. Host code only.
#include <cstdio>

#include <rocrand/rocrand_philox4x32_10.h>

int main() {
  unsigned long long seed, sub, c;
  while (std::scanf("%llu %llu %llu", &seed, &sub, &c) == 3) {
    rocrand_device::philox4x32_10_engine e(seed, sub, 4ull * c);
    const uint4 r = e.next4();
    std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
