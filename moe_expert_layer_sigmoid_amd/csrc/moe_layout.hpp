// Packed ("MFMA-operand order") layout of the MXFP4 expert weights.
//
// A weight matrix W [R rows, K] of one slot (R = 2F, K = H for W1; R = H,
// K = F for W2) is cut into 16-row tiles and 256-wide K steps.  Step st of a
// tile feeds two block-scaled 16x16x128 MFMAs (i = 0, 1); lane L = 16 g + r of
// MFMA i holds row r, 32-block st*8 + 4i + g (32 e2m1 values, 16 bytes, low
// nibble first), i.e. the natural K order of the instruction.
//
//   data:   [tile][step][i][lane][16 B]        2 KB per (tile, step)
//   scales: [tile][step / 4][lane][8 B]         512 B per (tile, 4 steps);
//           byte 2 * (step % 4) + i of lane L = e8m0 scale of row r,
//           32-block st*8 + 4i + g
//
// The step count is padded to a multiple of 4 (K up to the next multiple of
// 1024); padded weight bytes and scales are zero, so padded steps add exact
// zeros.  Every wave load of weights is then one contiguous 1 KB, and one
// 8-byte scale load per lane covers four steps of a tile.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

struct PackGeom {
  uint32_t rows;       // R
  uint32_t K;          // reduction length
  uint32_t steps;      // padded step count (multiple of 4)
  uint32_t tiles;      // R / 16
  size_t data_tile;    // bytes of one tile's data
  size_t scale_tile;   // bytes of one tile's scales
  size_t data_slot;    // bytes of one slot's data
  size_t scale_slot;   // bytes of one slot's scales
};

__host__ __device__ inline PackGeom pack_geom(uint32_t rows, uint32_t K) {
  PackGeom g;
  g.rows = rows;
  g.K = K;
  g.steps = (K + 1023) / 1024 * 4;
  g.tiles = rows / 16;
  g.data_tile = (size_t)g.steps * 2048;
  g.scale_tile = (size_t)(g.steps / 4) * 512;
  g.data_slot = g.data_tile * g.tiles;
  g.scale_slot = g.scale_tile * g.tiles;
  return g;
}

}  // namespace moe
