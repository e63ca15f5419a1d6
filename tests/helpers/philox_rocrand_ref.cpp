// Independent Philox4x32-10 reference for the oracle's tests: evaluates the
// ten-round block function of rocRAND's header-only engine on the host.
// Reads lines "c0 c1 c2 c3 k0 k1" (decimal uint32) from stdin and prints the
// four output words per line.
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

// The block function is a protected member; a derived class exposes it.
struct BlockFn : rocrand_device::philox4x32_10_engine {
  uint4 run(uint4 ctr, uint2 key) { return ten_rounds(ctr, key); }
};

int main() {
  unsigned c0, c1, c2, c3, k0, k1;
  BlockFn eng;
  while (std::scanf("%u %u %u %u %u %u", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    uint4 ctr = {c0, c1, c2, c3};
    uint2 key = {k0, k1};
    uint4 out = eng.run(ctr, key);
    std::printf("%u %u %u %u\n", out.x, out.y, out.z, out.w);
  }
  return 0;
}
