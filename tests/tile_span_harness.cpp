// Host build of the tile geometry the attention kernels use (csrc/tile_span.h):
// reads "s_kv kt row_bytes last_bytes" per line, prints "row0 rows span".
#include <cstdio>

#include "tile_span.h"

int main() {
  long long s_kv;
  int kt;
  unsigned row_bytes, last_bytes;
  while (std::scanf("%lld %d %u %u", &s_kv, &kt, &row_bytes, &last_bytes) == 4) {
    const long long row0 = (long long)h3a::tile_index_clamped(kt) * h3a::kSpanTileRows;
    std::printf("%lld %d %u\n", row0, h3a::rows_to_end(s_kv, kt), h3a::tile_span(s_kv, kt, row_bytes, last_bytes));
  }
  return 0;
}
