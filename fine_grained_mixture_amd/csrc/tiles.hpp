// Tile shapes of the bf16 grouped GEMMs (fp32 problems use fixed small
// tiles in the launchers).  TileCfg<T, BM, BN, waves along M, waves along N,
// pipeline stages, slab bytes KB, paired gate|up columns>.
//
//   UpWide/Mid/Narrow   up-projection: 128 slot rows x (gate half | up half),
//                       half = 256 / 128 / 64 gate columns
//   RowsWide/Mid/Narrow down-projection and dX-tilde: 128 slot rows x 512 /
//                       256 / 128 output columns
//   DhWide              dH for n = 256: 128 slot rows x all 256 columns
//   GradSquare/Tall/Small  dW1 / dW2 (varlen-K): 256x256 / 128x256 / 128x128
#pragma once

#include "gemm.hpp"

namespace moe {

#ifndef MOE_TILE_VARIANT
#define MOE_TILE_VARIANT 0
#endif

#if MOE_TILE_VARIANT == 1
// 64-byte slabs: three stages for the 128 x 512 tiles, four for 256 x 256
using UpWide = TileCfg<bf16_t, 128, 512, 2, 4, 3, 64, true>;
using RowsWide = TileCfg<bf16_t, 128, 512, 2, 4, 3, 64>;
using GradSquare = TileCfg<bf16_t, 256, 256, 2, 4, 4, 64>;
using DhWide = TileCfg<bf16_t, 128, 256, 2, 4, 3, 128>;
#elif MOE_TILE_VARIANT == 2
// as the default, with four stages of 64-byte slabs for the weight gradients
using UpWide = TileCfg<bf16_t, 128, 512, 2, 4, 2, 128, true>;
using RowsWide = TileCfg<bf16_t, 128, 512, 2, 4, 2, 128>;
using GradSquare = TileCfg<bf16_t, 256, 256, 2, 4, 4, 64>;
using DhWide = TileCfg<bf16_t, 128, 256, 2, 4, 3, 128>;
#elif MOE_TILE_VARIANT == 3
// as the default, with four stages of 64-byte slabs for dH
using UpWide = TileCfg<bf16_t, 128, 512, 2, 4, 2, 128, true>;
using RowsWide = TileCfg<bf16_t, 128, 512, 2, 4, 2, 128>;
using GradSquare = TileCfg<bf16_t, 256, 256, 2, 4, 2, 128>;
using DhWide = TileCfg<bf16_t, 128, 256, 2, 4, 4, 64>;
#else
// 128-byte slabs (one full cache line per row), two stages for the wide
// tiles, three for dH (whose H reloads in the epilogue favour a deeper ring)
using UpWide = TileCfg<bf16_t, 128, 512, 2, 4, 2, 128, true>;
using RowsWide = TileCfg<bf16_t, 128, 512, 2, 4, 2, 128>;
using GradSquare = TileCfg<bf16_t, 256, 256, 2, 4, 2, 128>;
using DhWide = TileCfg<bf16_t, 128, 256, 2, 4, 3, 128>;
#endif

using DhWide512 = TileCfg<bf16_t, 64, 512, 1, 4, 2, 128>;  // dH for n = 512 (one wave per SIMD)
using UpMid = TileCfg<bf16_t, 128, 256, 2, 4, 3, 128, true>;
using UpNarrow = TileCfg<bf16_t, 128, 128, 2, 2, 3, 128, true>;
using RowsMid = TileCfg<bf16_t, 128, 256, 2, 4, 3, 128>;
using RowsNarrow = TileCfg<bf16_t, 128, 128, 2, 2, 3, 128>;
using GradTall = TileCfg<bf16_t, 128, 256, 2, 4, 3, 128>;
using GradSmall = TileCfg<bf16_t, 128, 128, 2, 2, 3, 128>;

}  // namespace moe
