// Building blocks of the grouped GEMMs on gfx950: LDS tiles, operand loaders
// with the token gather fused into the global->LDS copy, and a
// double-buffered bf16/fp32 MFMA main loop.
//
// Operand convention.  Every GEMM computes C[i][j] = sum_k A[i][k] B[k][j]
// for one BM x BN output tile.  Both operands are staged in LDS "k-major per
// row": the A tile as BM rows of BK k-values, the B tile as BN rows (one per
// output column j) of BK k-values, each row padded by 16 bytes so that the
// 16-byte fragment reads of 16 consecutive rows hit distinct LDS banks.
//
// Loaders:
//   DirectLoader  source rows already hold k contiguously (X, dO, A, dH,
//                 and the weights when the contraction runs along their
//                 rows); each thread copies fixed 8-element octets, with a
//                 per-row element offset that carries the gather.
//   TransLoader   source rows are indexed by k (the weights along their
//                 columns, and both operands of the varlen-K weight-gradient
//                 GEMMs); each thread reads an 8x8 block (8 k rows x 8
//                 columns), transposes it in registers and writes 8 LDS rows.
//
// The MFMA is issued with the B fragment as its first operand, so each
// accumulator block holds C^T: lane l owns output row (l % 32) of the block
// and, for accumulator element r, column (r/4)*8 + (l/32)*4 + r%4.  Four
// consecutive r therefore address four consecutive columns of one row, which
// the epilogues store as one vector.
#pragma once

#include "common.hpp"

namespace moe {

template <class T_, int BM_, int BN_, int WGM_, int WGN_, bool PAIRED_ = false>
struct TileCfg {
  using T = T_;
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_;
  static constexpr bool PAIRED = PAIRED_;  // B tile = [gate cols | up cols]
  static constexpr int kThreads = 256;
  static_assert(WGM * WGN == 4, "four waves per workgroup");
  static constexpr int BK = 128 / int(sizeof(T));     // 128 bytes of k per row
  static constexpr int LD = BK + 16 / int(sizeof(T));  // padded LDS row (144 B)
  static constexpr int WTM = BM / WGM, WTN = BN / WGN;
  static constexpr int MB = WTM / 32, NB = WTN / 32;
  static_assert(MB >= 1 && NB >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
  static_assert(!PAIRED || NB % 2 == 0, "paired tiles split each wave's columns");
  static constexpr int OCTS = BK / 8;  // octets per LDS row
  static constexpr int KCH = BK / 16;  // 16-wide k chunks per slab
  static constexpr int A_ELEMS = BM * LD, B_ELEMS = BN * LD;
  static constexpr int LDS_ELEMS = 2 * (A_ELEMS + B_ELEMS);

  // LDS column (B-tile row) of the first column of wave column-block nb.
  __device__ static constexpr int colblock(int wn, int nb) {
    if constexpr (PAIRED) {
      constexpr int half = BN / 2, per = half / WGN, hb = NB / 2;
      return nb < hb ? wn * per + nb * 32 : half + wn * per + (nb - hb) * 32;
    } else {
      return wn * WTN + nb * 32;
    }
  }
};

// Rows whose k-values are contiguous in memory.  row_off(r) gives the element
// offset of row r's first k-value from `base`, or -1 for a row that is zero
// (past the end of the expert).
template <class Cfg, int ROWS>
struct DirectLoader {
  using T = typename Cfg::T;
  static constexpr int N_OCT = ROWS * Cfg::OCTS;
  static constexpr int PER = (N_OCT + Cfg::kThreads - 1) / Cfg::kThreads;
  const T* base;
  int off[PER];
  Oct<T> reg[PER];

  template <class RowOff>
  __device__ __forceinline__ void init(const T* b, RowOff row_off) {
    base = b;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = threadIdx.x + i * Cfg::kThreads;
      const int r = q / Cfg::OCTS, o = q % Cfg::OCTS;
      int v = -1;
      if (q < N_OCT) {
        const int ro = row_off(r);
        v = ro < 0 ? -1 : ro + o * 8;
      }
      off[i] = v;
    }
  }
  __device__ __forceinline__ void load(int k0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (off[i] >= 0) oct_load(reg[i], base + off[i] + k0);
      else oct_zero(reg[i]);
    }
  }
  __device__ __forceinline__ void store(T* stage) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = threadIdx.x + i * Cfg::kThreads;
      if (q < N_OCT) oct_store(stage + (q / Cfg::OCTS) * Cfg::LD + (q % Cfg::OCTS) * 8, reg[i]);
    }
  }
  __device__ __forceinline__ void fetch(int s) { load(s * Cfg::BK); }
  __device__ __forceinline__ void put(T* stage) const { store(stage); }
};

// Rows indexed by k.  For slab s, k_off(s, k) gives the element offset of
// source row k (0 <= k < BK) of that slab from `base`, or -1 for a zero row;
// col_off(cg) gives the column offset of LDS column group cg (8 columns).
template <class Cfg, int COLS, class KOff, class ColOff>
struct TransLoader {
  using T = typename Cfg::T;
  static constexpr int KG = Cfg::BK / 8;
  static constexpr int N_UNITS = (COLS / 8) * KG;
  static constexpr int PER = (N_UNITS + Cfg::kThreads - 1) / Cfg::kThreads;
  const T* base;
  KOff k_off;
  ColOff col_off;
  Oct<T> reg[PER][8];

  __device__ __forceinline__ TransLoader(const T* b, KOff ko, ColOff co)
      : base(b), k_off(ko), col_off(co) {}

  __device__ __forceinline__ void fetch(int s) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int u = threadIdx.x + i * Cfg::kThreads;
      const int kg = u % KG, cg = u / KG;
      const int co = (u < N_UNITS) ? col_off(cg) : 0;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int ro = (u < N_UNITS) ? k_off(s, kg * 8 + m) : -1;
        if (ro >= 0) oct_load(reg[i][m], base + ro + co);
        else oct_zero(reg[i][m]);
      }
    }
  }
  __device__ __forceinline__ void put(T* stage) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int u = threadIdx.x + i * Cfg::kThreads;
      if (u >= N_UNITS) continue;
      const int kg = u % KG, cg = u / KG;
      Oct<T> out[8];
      oct_transpose(out, reg[i]);
#pragma unroll
      for (int c = 0; c < 8; ++c) oct_store(stage + (cg * 8 + c) * Cfg::LD + kg * 8, out[c]);
    }
  }
};

template <class Cfg, int COLS, class KOff, class ColOff>
__device__ __forceinline__ TransLoader<Cfg, COLS, KOff, ColOff> make_trans(
    const typename Cfg::T* base, KOff ko, ColOff co) {
  return TransLoader<Cfg, COLS, KOff, ColOff>(base, ko, co);
}

template <class Cfg>
struct Accum {
  using T = typename Cfg::T;
  f32x16_t acc[Cfg::MB][Cfg::NB];
  int wm, wn, lane;

  __device__ __forceinline__ void init() {
    const int wave = threadIdx.x >> 6;
    lane = threadIdx.x & 63;
    wm = wave / Cfg::WGN;
    wn = wave % Cfg::WGN;
#pragma unroll
    for (int a = 0; a < Cfg::MB; ++a)
#pragma unroll
      for (int b = 0; b < Cfg::NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;
  }

  // One BK slab from LDS.
  __device__ __forceinline__ void slab(const T* As, const T* Bs) {
    const int r32 = lane & 31, h = lane >> 5;
#pragma unroll
    for (int kc = 0; kc < Cfg::KCH; ++kc) {
      Oct<T> fa[Cfg::MB], fb[Cfg::NB];
      const int ko = kc * 16 + h * 8;
#pragma unroll
      for (int a = 0; a < Cfg::MB; ++a)
        oct_load(fa[a], As + (wm * Cfg::WTM + a * 32 + r32) * Cfg::LD + ko);
#pragma unroll
      for (int b = 0; b < Cfg::NB; ++b)
        oct_load(fb[b], Bs + (Cfg::colblock(wn, b) + r32) * Cfg::LD + ko);
#pragma unroll
      for (int a = 0; a < Cfg::MB; ++a)
#pragma unroll
        for (int b = 0; b < Cfg::NB; ++b) mma16(acc[a][b], fb[b], fa[a]);
    }
  }

  // Tile-local row of block a for this lane, and tile-local first column of
  // the 4-column group q (0..3) of block b.
  __device__ __forceinline__ int row(int a) const { return wm * Cfg::WTM + a * 32 + (lane & 31); }
  __device__ __forceinline__ int col(int b, int q) const {
    return Cfg::colblock(wn, b) + q * 8 + (lane >> 5) * 4;
  }
};

// Double-buffered main loop over `nslabs` BK-slabs: global loads of slab s+1
// are in flight while slab s is multiplied from LDS.  One barrier per slab.
template <class Cfg, class LA, class LB>
__device__ __forceinline__ void mainloop(Accum<Cfg>& acc, typename Cfg::T* lds, int nslabs,
                                         LA&& load_a, LB&& load_b) {
  using T = typename Cfg::T;
  T* As0 = lds;
  T* As1 = lds + Cfg::A_ELEMS;
  T* Bs0 = lds + 2 * Cfg::A_ELEMS;
  T* Bs1 = Bs0 + Cfg::B_ELEMS;
  if (nslabs <= 0) return;
  load_a.fetch(0);
  load_b.fetch(0);
  load_a.put(As0);
  load_b.put(Bs0);
  __syncthreads();
  for (int s = 0; s < nslabs; ++s) {
    const bool more = s + 1 < nslabs;
    if (more) {
      load_a.fetch(s + 1);
      load_b.fetch(s + 1);
    }
    if (s & 1) acc.slab(As1, Bs1);
    else acc.slab(As0, Bs0);
    if (more) {
      load_a.put((s & 1) ? As0 : As1);
      load_b.put((s & 1) ? Bs0 : Bs1);
    }
    __syncthreads();
  }
}

// Spreads `work` logical tiles over the 8 XCDs in contiguous chunks:
// workgroups are dispatched round-robin over XCDs, so block b runs on XCD
// b % 8; giving each XCD a contiguous range keeps neighbouring tiles (same
// expert, same weight panel) in one L2.  Returns -1 for surplus blocks.
__device__ __forceinline__ int xcd_tile(int b, int work) {
  const int per = (work + 7) / 8;
  const int local = b / 8, xcd = b % 8;
  if (local >= per) return -1;
  const int lin = xcd * per + local;
  return lin < work ? lin : -1;
}

}  // namespace moe
