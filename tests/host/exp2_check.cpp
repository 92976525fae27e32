// Host-side check of the forward's software exponential: prints, for each
// float bit pattern read from stdin (hex), the bit pattern of poly_exp2.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../exact_attention_80_amd/csrc/fa_exp2.h"

int main() {
  unsigned int bits;
  while (std::scanf("%x", &bits) == 1) {
    float x;
    std::memcpy(&x, &bits, 4);
    const float y = fa::poly_exp2(x);
    unsigned int out;
    std::memcpy(&out, &y, 4);
    std::printf("%08x\n", out);
  }
  return 0;
}
