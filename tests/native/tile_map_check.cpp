// Host-side check of the workgroup -> work-unit maps the kernels use
// (remap_xcd, tile_coords, work_coords in gfx950_prims.hpp): over many grid
// shapes, every launch index maps to a distinct (tile row, tile column, K
// range) and together they cover the whole grid exactly once, so any
// dispatch order computes every tile of C once.  Built and run by
// tests/test_tile_map.py (hipcc, host code only); prints "ok <cases>" or the
// first failing case and exits non-zero.
#include <cstdio>
#include <vector>

#include "../../dense_gemm_12_amd/csrc/gfx950_prims.hpp"

int main() {
  long cases = 0;
  // remap_xcd alone: a permutation of [0, tiles) for every grid size
  for (int tiles = 1; tiles <= 5000; ++tiles) {
    std::vector<char> seen(tiles, 0);
    for (int b = 0; b < tiles; ++b) {
      const int l = mg::remap_xcd(b, tiles);
      if (l < 0 || l >= tiles || seen[l]) {
        std::printf("remap_xcd not a bijection: tiles=%d b=%d -> %d\n", tiles, b, l);
        return 1;
      }
      seen[l] = 1;
    }
    ++cases;
  }
  // work_coords: tiles_m x tiles_n tiles, `splits` K ranges, raster group heights
  const int group_ms[] = {1, 2, 3, 8, 16, 64};
  const int K = 4096;
  for (int tm_n = 1; tm_n <= 70; tm_n += (tm_n < 12 ? 1 : 7)) {
    for (int tn_n = 1; tn_n <= 70; tn_n += (tn_n < 12 ? 1 : 9)) {
      for (int splits : {1, 2, 3, 5, 8, 17, 64}) {
        const int chunk = (K + splits - 1) / splits;
        for (int gm : group_ms) {
          const int tiles = tm_n * tn_n;
          std::vector<char> seen((size_t)tiles * splits, 0);
          for (int b = 0; b < tiles * splits; ++b) {
            int tm, tn, k0, kl;
            mg::work_coords(b, tm_n, tn_n, gm, splits, K, chunk, tm, tn, k0, kl);
            const int s = k0 / chunk;
            const bool ok = tm >= 0 && tm < tm_n && tn >= 0 && tn < tn_n && k0 % chunk == 0 && s < splits &&
                            kl == (splits > 1 ? (K - k0 < chunk ? K - k0 : chunk) : K);
            const size_t id = ((size_t)s * tm_n + tm) * tn_n + tn;
            if (!ok || seen[id]) {
              std::printf("work_coords: tiles %dx%d splits=%d group_m=%d b=%d -> (%d,%d,k0=%d,kl=%d)%s\n", tm_n,
                          tn_n, splits, gm, b, tm, tn, k0, kl, ok ? " twice" : " out of range");
              return 1;
            }
            seen[id] = 1;
          }
          ++cases;
        }
      }
    }
  }
  std::printf("ok %ld\n", cases);
  return 0;
}
