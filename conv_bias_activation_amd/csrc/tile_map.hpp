// tile_map.hpp — workgroup id -> output tile mapping shared by the GEMM and
// conv kernels of the biasact library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace biasact {

// Workgroup id -> work-item index such that every XCD gets one contiguous
// range of indices.  The dispatcher hands workgroup b to XCD b % 8, so
// consecutive work items (neighbouring tiles or patches, which read the same
// operand panels or input rows) would otherwise land on eight different L2s.
__device__ __forceinline__ uint32_t xcd_contiguous(uint32_t bid, uint32_t nblk) {
  const uint32_t xcd = bid & 7u, idx = bid >> 3;
  const uint32_t q = nblk >> 3, r = nblk & 7u;
  return xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

// Workgroup id -> output tile.  Every XCD takes one contiguous range of tile
// ids (xcd_contiguous), and the
// grouped raster (8 tile rows at a time, row index fastest) makes the tiles of
// one range share A row panels and B column panels in that XCD's L2.
__device__ __forceinline__ void map_tile(uint32_t bid, uint32_t nblk, uint32_t tiles_m,
                                         uint32_t tiles_n, uint32_t& tm, uint32_t& tn) {
  const uint32_t t = xcd_contiguous(bid, nblk);
  constexpr uint32_t GM = 8;
  const uint32_t per_group = GM * tiles_n;
  const uint32_t first_m = (t / per_group) * GM;
  const uint32_t gm = min(tiles_m - first_m, GM);
  const uint32_t in = t - (t / per_group) * per_group;
  tm = first_m + in % gm;
  tn = in / gm;
}

}  // namespace biasact
