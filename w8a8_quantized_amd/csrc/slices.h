// Launch slices for 32-bit buffer offsets (host code, no HIP dependency).
//
// The GEMM kernels address each operand through a buffer resource whose size
// and per-lane offsets are 32-bit: a launch over R rows of K bytes computes
// offsets up to (R + tile) * K (rows past the edge, up to one tile, read as
// zeros through the range check), and the out-of-range offset 0x7FFFFFF0 must
// lie beyond R * K.  The host therefore splits R into slices of at most
// rows_per_slice(K, tile) rows, a multiple of the tile, with
// (rows_per_slice + tile) * K <= 2^31.  K <= 133144 (the int32 accumulator
// bound) keeps the slice at 15872 rows or more for tiles up to 256.
#pragma once
#include <stdint.h>

namespace sq {

inline int64_t rows_per_slice(int64_t K, int64_t tile) {
  const int64_t lim = (int64_t)1 << 31;
  return ((lim / K - tile) / tile) * tile;
}

}  // namespace sq
