// Test-side reference for the oracle's Philox4x32-10: reads
// "key64 c0 c1 c2 c3" lines (hex) on stdin and prints the four output words of
// rocRAND's host-side philox4x32_10 engine for that key and counter.
// rocRAND seeds the key with the 64-bit seed, puts the subsequence in counter
// words 2..3 and advances words 0..1 by offset/4, so any counter is reachable.
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
#include <cstdint>

int main() {
  unsigned long long key, c0, c1, c2, c3;
  while (std::scanf("%llx %llx %llx %llx %llx", &key, &c0, &c1, &c2, &c3) == 5) {
    rocrand_state_philox4x32_10 st;
    const unsigned long long sub = (c3 << 32) | c2;
    rocrand_init(key, sub, 0ULL, &st);
    unsigned long long left = (c1 << 32) | c0;   // counter words 0..1 as one 64-bit offset
    const unsigned long long chunk = 1ULL << 60;
    while (left) {
      const unsigned long long step = left < chunk ? left : chunk;
      st.discard(4ULL * step);
      left -= step;
    }
    const uint4 r = rocrand4(&st);
    std::printf("%08x %08x %08x %08x\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
