// Host-side check of the fixed-point dQ exponent: prints, for each float bit
// pattern read from stdin (hex), the exponent e that the preprocess assigns
// to a row whose bound is that value.
#include <cstdio>
#include <cstring>

#include "../../exact_attention_80_amd/csrc/fa_launch.h"

int main() {
  unsigned int bits;
  while (std::scanf("%x", &bits) == 1) {
    float beta;
    std::memcpy(&beta, &bits, 4);
    std::printf("%d\n", fa::dq_fixed_exponent(beta));
  }
  return 0;
}
