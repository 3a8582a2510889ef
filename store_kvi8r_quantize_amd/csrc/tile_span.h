// Geometry of a K/V store read in 64-row tiles through buffer resources: which
// row a tile starts at and how many bytes its buffer resource spans.  Plain
// integer arithmetic, compiled into the attention kernels and, for tests, into
// a host program.
//
// A tile's resource runs from the tile's first row to the end of the store, so
// rows past the end read as zero through the range check.  A negative tile
// index reads as tile 0: no buffer base can precede the store.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define H3A_HD __host__ __device__
#else
#define H3A_HD
#endif

namespace h3a {

constexpr int kSpanTileRows = 64;

// Tile index used for addressing: kt, or 0 when kt is negative.
H3A_HD inline int32_t tile_index_clamped(int32_t kt) { return kt > 0 ? kt : 0; }

// Rows from tile kt's first row to the end of a store of s_kv rows (s_kv < 2^31);
// zero or negative when the tile starts at or past the end.
H3A_HD inline int32_t rows_to_end(int64_t s_kv, int32_t kt) {
  return (int32_t)s_kv - tile_index_clamped(kt) * kSpanTileRows;
}

// Bytes from the tile's first row to the end of the store when rows > 0: rows - 1
// rows of row_bytes, then the last_bytes the last row is read with.  Not saturated.
H3A_HD inline uint64_t span_bytes(int32_t rows, uint32_t row_bytes, uint32_t last_bytes) {
  return (uint64_t)(uint32_t)(rows - 1) * row_bytes + last_bytes;
}

// The resource size of tile kt: span_bytes saturated at 2^32 - 1, 0 for a tile at
// or past the end of the store (the kernels compute the same in scalar registers).
H3A_HD inline uint32_t tile_span(int64_t s_kv, int32_t kt, uint32_t row_bytes, uint32_t last_bytes) {
  const int32_t rows = rows_to_end(s_kv, kt);
  if (rows <= 0) return 0u;
  const uint64_t b = span_bytes(rows, row_bytes, last_bytes);
  return (b >> 32) ? 0xFFFFFFFFu : (uint32_t)b;
}

}  // namespace h3a
