// Tile shapes of the bf16 grouped GEMMs (fp32 problems use fixed small
// tiles in the launchers).  TileCfg<T, BM, BN, waves along M, waves along N,
// pipeline stages, slab bytes KB, paired gate|up columns, loader waves>.
//
//   UpWide/Mid/Narrow   up-projection: 128 slot rows x (gate half | up half),
//                       half = 256 / 128 / 64 gate columns
//   RowsWide/Mid/Narrow down-projection and dX-tilde: 128 slot rows x 512 /
//                       256 / 128 output columns
//   RowsSplit           the same, 128 x 256, four compute and four loader
//                       waves, in persistent launches (one workgroup per CU)
//   DhWide              dH for n = 256: 128 slot rows x all 256 columns
//   GradSplit256/Split  dW1 / dW2 (varlen-K), 256 x 256 / 128 x 256 with
//                       loader waves, in persistent launches
//   GradSquare/Tall/Small  dW1 / dW2 (varlen-K): 256x256 / 128x256 / 128x128
#pragma once

#include "gemm.hpp"

namespace moe {

// 128-byte slabs (one full cache line per row), two stages for the wide
// tiles, three for dH (whose H reloads in the epilogue favour a deeper ring)
using UpWide = TileCfg<bf16_t, 128, 512, 2, 4, 2, 128, true>;
using RowsWide = TileCfg<bf16_t, 128, 512, 2, 4, 2, 128>;
// three 48 KB stages; loader waves 4-7 beside compute waves 0-3
using RowsSplit = TileCfg<bf16_t, 128, 256, 2, 2, 3, 128, false, 4>;
// dX-tilde with the dH rows in registers: 32 x 128 per compute wave, W1
// slabs of 16 KB, two per stage, in a three-stage ring
using RowsReg = TileCfg<bf16_t, 128, 128, 4, 1, 3, 128, false, 4>;
using GradSquare = TileCfg<bf16_t, 256, 256, 2, 4, 2, 128>;
// dW1 / dW2 in persistent launches: 256 x 256 with eight compute and four
// loader waves (three per SIMD, so 168 registers each) in two 64 KB stages;
// else 128 x 256 with four of each in three 48 KB stages
using GradSplit256 = TileCfg<bf16_t, 256, 256, 2, 4, 2, 128, false, 4>;
using GradSplit = TileCfg<bf16_t, 128, 256, 2, 2, 3, 128, false, 4>;
using DhWide = TileCfg<bf16_t, 128, 256, 2, 4, 3, 128>;

using DhWide512 = TileCfg<bf16_t, 64, 512, 1, 4, 2, 128>;  // dH for n = 512 (one wave per SIMD)
using UpMid = TileCfg<bf16_t, 128, 256, 2, 4, 3, 128, true>;
using UpNarrow = TileCfg<bf16_t, 128, 128, 2, 2, 3, 128, true>;
using RowsMid = TileCfg<bf16_t, 128, 256, 2, 4, 3, 128>;
using RowsNarrow = TileCfg<bf16_t, 128, 128, 2, 2, 3, 128>;
using GradTall = TileCfg<bf16_t, 128, 256, 2, 4, 3, 128>;
using GradSmall = TileCfg<bf16_t, 128, 128, 2, 2, 3, 128>;

}  // namespace moe
