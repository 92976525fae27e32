// Host-side check of the per-tile buffer range used by the direct copies:
// prints, for each (row0, len, row_bytes, data_bytes, tile_rows) read from
// stdin, the 32-bit range the kernels give the buffer descriptor.
#include <cstdio>

#include "../../exact_attention_80_amd/csrc/fa_common.h"

int main() {
  long row0, len, row_bytes, data_bytes, tile_rows;
  while (std::scanf("%ld %ld %ld %ld %ld", &row0, &len, &row_bytes, &data_bytes, &tile_rows) == 5)
    std::printf("%u\n", fa::tile_range((int)row0, (int)len, row_bytes, (int)data_bytes,
                                       (int)tile_rows));
  return 0;
}
