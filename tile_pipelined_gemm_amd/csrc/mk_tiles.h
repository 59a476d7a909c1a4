// Tile configurations shared by the entry points and the per-shape defaults.
#pragma once

#include <stdint.h>

enum MkTile {
  TILE_AUTO = 0,
  TILE_256x256 = 1,  // 4 waves, 128x128 per wave: highest MFMA density, 1 workgroup per CU
  TILE_128x128 = 2,  // 4 waves, 64x64 per wave: small or ragged problems
  TILE_256x128 = 3,  // 4 waves, 128x64 per wave
  TILE_128x256 = 4,  // 4 waves, 64x128 per wave
  TILE_256x256_DMA = 5,  // 256x256, direct-to-LDS operand loads, 4-stage ring (K % 128 == 0)
  TILE_128x128_DMA = 6,  // the same engine at 128x128 (64 KiB LDS, 2 workgroups per CU)
  TILE_256x128_DMA = 7,
  TILE_128x256_DMA = 8,
  TILE_128x128_DMA8 = 9,  // 128x128 direct-to-LDS with an 8-slice ring (128 KiB LDS, 1 workgroup per CU,
                          // K % 256 == 0): twice the operand bytes in flight, for GEMMs that stream B
  TILE_256x256_DMA_W8 = 10,  // 256x256 direct-to-LDS with 8 waves (2x4, two per SIMD; K % 128 == 0)
  TILE_128x128_PC = 11,  // 128x128 producer/consumer: 4 compute waves load A into registers, 4 producer
                         // waves stream B into a 16-slice LDS ring (K % 128 == 0; skinny, bandwidth-bound)
  TILE_COUNT
};

// The direct-to-LDS version of a register-staged tile shape (K % 128 == 0).
inline int mk_dma_tile(int t) {
  switch (t) {
    case TILE_256x256: return TILE_256x256_DMA;
    case TILE_128x128: return TILE_128x128_DMA;
    case TILE_256x128: return TILE_256x128_DMA;
    case TILE_128x256: return TILE_128x256_DMA;
    default: return t;
  }
}
inline bool mk_is_dma_tile(int t) { return t >= TILE_256x256_DMA && t <= TILE_128x256_DMA; }

// Per-shape default: the largest tile that still gives every CU work.
inline int mk_default_tile(int64_t M, int64_t N, int64_t K) {
  (void)K;
  const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
  if (M >= 256 && N >= 256 && t256 >= 256) return TILE_256x256;
  const int64_t t128x256 = ((M + 127) / 128) * ((N + 255) / 256);
  if (N >= 256 && t128x256 >= 256) return TILE_128x256;
  return TILE_128x128;
}
