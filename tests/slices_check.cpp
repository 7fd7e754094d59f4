// Host check of the GEMM launch slicing (w8a8_quantized_amd/csrc/slices.h), the
// arithmetic every 32-bit buffer offset of the GEMM kernels relies on.  For each
// K and tile it walks the slices exactly as the launchers do and checks: each
// slice has at least one row and is a multiple of the tile (but the last);
// every offset a tile can form, overhang included, fits int32; the buffer size
// R * K fits int32 and stays below the out-of-range offset 0x7FFFFFF0; the
// slices cover the rows exactly once.  Prints "ok" and exits 0 when all hold.
#include <cstdint>
#include <cstdio>
#include "../w8a8_quantized_amd/csrc/slices.h"

int main() {
  const int64_t Ks[] = {16, 32, 48, 80, 1000, 1040, 4096, 8192, 8208, 12288, 16384, 16400, 28672,
                        65536, 100000, 131072, 133136, 133144};
  const int64_t tiles[] = {16, 32, 64, 128, 256};
  const int64_t lim = (int64_t)1 << 31;
  long checks = 0;
  for (int64_t K : Ks)
    for (int64_t tile : tiles) {
      const int64_t step = sq::rows_per_slice(K, tile);
      if (step < tile || step % tile != 0) { std::printf("bad slice %lld for K %lld tile %lld\n", (long long)step, (long long)K, (long long)tile); return 1; }
      const int64_t Rs[] = {1, tile - 1, tile, step - 1, step, step + 1, 2 * step + tile / 2, 5 * step + 3,
                            lim / K + 7, 3 * (lim / K)};
      for (int64_t R : Rs) {
        if (R < 1) continue;
        int64_t covered = 0;
        for (int64_t r0 = 0; r0 < R; r0 += step) {
          const int64_t rows = R - r0 < step ? R - r0 : step;
          const int64_t tiles_here = (rows + tile - 1) / tile;
          const int64_t max_off = (tiles_here * tile) * K - 1;   // last byte a tile may address
          if (rows < 1 || max_off > INT32_MAX || rows * K > INT32_MAX || rows * K > 0x7FFFFFF0 ||
              (rows + tile) * K > lim) {
            std::printf("slice violates the bounds: K %lld tile %lld R %lld r0 %lld rows %lld\n", (long long)K,
                        (long long)tile, (long long)R, (long long)r0, (long long)rows);
            return 1;
          }
          covered += rows;
          ++checks;
        }
        if (covered != R) { std::printf("slices cover %lld of %lld rows\n", (long long)covered, (long long)R); return 1; }
      }
    }
  std::printf("ok %ld slices\n", checks);
  return 0;
}
