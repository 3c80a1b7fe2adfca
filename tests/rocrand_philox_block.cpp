// Prints the Philox4x32-10 block of each input line "c0 c1 c2 c3 k0 k1" (hex
// words), computed by rocRAND's own engine: an implementation of the generator
// independent of the oracle's, used only to check it.
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>

struct Block : rocrand_device::philox4x32_10_engine {
  static uint4 of(uint4 c, uint2 k) { return Block().ten_rounds(c, k); }
};

int main() {
  unsigned c[4], k[2];
  while (std::scanf("%x %x %x %x %x %x", &c[0], &c[1], &c[2], &c[3], &k[0], &k[1]) == 6) {
    uint4 cc;
    cc.x = c[0], cc.y = c[1], cc.z = c[2], cc.w = c[3];
    uint2 kk;
    kk.x = k[0], kk.y = k[1];
    const uint4 o = Block::of(cc, kk);
    std::printf("%08x %08x %08x %08x\n", o.x, o.y, o.z, o.w);
  }
  return 0;
}
