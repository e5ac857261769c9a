// Backward grouped GEMMs of the minimal-activation backward.
//
// SonicMoE ICLR-2026 notes (papernotes.org), key designs 2 and 3: only X, H
// and the routing metadata survive the forward.  The dH kernel gathers dO
// rows into its operand load and, in its epilogue, reads H (loaded before
// the K loop where the registers allow), recomputes A = SwiGLU(H), and forms
// dS = <dA', A> together with dSwiGLU, so neither Y nor dY is ever needed.  The weight gradients are varlen-K grouped GEMMs:
// the contraction runs over each expert's own (gathered) token rows.
//
//   k_dh    dA' = dO[I_e] W2_e^T; dS, dH, s*A in the epilogue
//   k_dxt   dX~_e = dH_e W1_e^T
//   k_dw1   dW1_e = X[I_e]^T dH_e        (varlen-K)
//   k_dw2   dW2_e = (s*A)_e^T dO[I_e]    (varlen-K)
#include <algorithm>

#include "gemm.hpp"
#include "internal.hpp"
#include "tiles.hpp"

namespace moe {
namespace {

inline unsigned grid_for(int64_t work) { return unsigned(((work + 7) / 8) * 8); }

// BN == n: one workgroup owns whole rows of dA', so the dS row sums stay
// inside the workgroup and are written once, in a fixed order.
// A = gathered dO rows (K-major), B = W2_e rows (K-major, contraction over d).
template <class Cfg, class T = typename Cfg::T>
__global__ __launch_bounds__(Cfg::kThreads) void k_dh(
    const T* __restrict__ dO, const T* __restrict__ W2, const T* __restrict__ H,
    T* __restrict__ dH, T* __restrict__ As, float* __restrict__ dS,
    const int32_t* __restrict__ tile_expert, const int32_t* __restrict__ tile_row,
    const int32_t* __restrict__ slot_token,
    const float* __restrict__ slot_weight, const int32_t* __restrict__ totals, int d, int ntok) {
  __shared__ __attribute__((aligned(1024))) char lds[Cfg::LDS_BYTES];
  constexpr int BM = Cfg::BM, BN = Cfg::BN, WGN = Cfg::WGN;
  constexpr int n = BN, n2 = 2 * BN, SUB = kTileM / BM;
  const int lin = xcd_tile(blockIdx.x, totals[1] * SUB);
  if (lin < 0) return;
  const int mt = lin / SUB;
  const int e = tile_expert[mt], row0 = tile_row[mt] + (lin % SUB) * BM;
  const int rend = tile_end(tile_row, totals, mt, tile_row[mt]);
  if (row0 >= rend) return;
  const int tok0 = slot_token[row0];

  const uint32_t orow = uint32_t(d) * sizeof(T);
  KLoad<Cfg, BM> la;
  la.init(dO, uint32_t(ntok) * orow, [&](int r) {
    const int slot = row0 + r;
    return uint32_t(slot < rend ? slot_token[slot] : tok0) * orow;
  });
  KLoad<Cfg, BN> lb;
  lb.init(W2 + int64_t(e) * n * d, uint32_t(n) * orow, [&](int j) { return uint32_t(j) * orow; });

  Accum<Cfg> acc;
  acc.init();
  // The H values of this lane's accumulator positions (and the gate weights)
  // do not depend on the product: when they fit in 64 registers they are
  // loaded before the main loop, so their latency hides behind it instead of
  // stalling the epilogue.
  constexpr bool kPreH = Cfg::NW == 8 && Cfg::MB * Cfg::NB * 4 * 2 * 4 * int(sizeof(T)) <= 256;
  T hpre[kPreH ? Cfg::MB : 1][kPreH ? Cfg::NB : 1][4][2][4];
  float spre[kPreH ? Cfg::MB : 1];
  if constexpr (kPreH) {
#pragma unroll
    for (int a = 0; a < Cfg::MB; ++a) {
      const int slot = row0 + acc.row(a);
      const int srow = slot < rend ? slot : row0;
      const T* hrow = H + int64_t(srow) * n2;
      spre[a] = slot_weight[srow];
#pragma unroll
      for (int b = 0; b < Cfg::NB; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j = acc.col(b, q);
          __builtin_memcpy(hpre[a][b][q][0], hrow + j, 4 * sizeof(T));
          __builtin_memcpy(hpre[a][b][q][1], hrow + n + j, 4 * sizeof(T));
        }
    }
  }
  pipeline<Cfg, true, true>(acc, lds, d / Cfg::BK, la, lb, NoTail{});

  // Epilogue: per row, dS = <dA', A> (A from the stored H), dH = dSwiGLU and
  // s * A for the dW2 GEMM.  The three outputs are staged per wave and
  // written as whole rows (through three buffers when they fit in LDS, else
  // one after another through one), and the partial row sums of dS meet in
  // LDS past the staging area.
  using St = RowStage<T, Cfg::WTN>;
  constexpr int RED = Cfg::WGN * BM * 4;
  constexpr bool kAll = 3 * St::BYTES * Cfg::NW + RED <= Cfg::LDS_BYTES;
  constexpr int NSB = kAll ? 3 : 1;
  static_assert(NSB * St::BYTES * Cfg::NW + RED <= Cfg::LDS_BYTES, "staging fits");
  char* wbuf = lds + wave_id() * NSB * St::BYTES;
  const St stg[3] = {St{wbuf}, St{wbuf + (kAll ? St::BYTES : 0)},
                     St{wbuf + (kAll ? 2 * St::BYTES : 0)}};
  float* red = reinterpret_cast<float*>(lds + NSB * St::BYTES * Cfg::NW);  // [WGN][BM]
  const int r32 = acc.lane & 31, h = acc.lane >> 5;
  const int cw = Cfg::colblock(acc.wn, 0);  // first column of this wave
#pragma unroll
  for (int a = 0; a < Cfg::MB; ++a) {
    const int i = acc.row(a), slot = row0 + i;
    const bool live = slot < rend;
    const int srow = live ? slot : row0;  // rows past the expert read a valid row
    float s;
    if constexpr (kPreH) s = spre[a];
    else s = slot_weight[srow];
    const T* hrow = H + int64_t(srow) * n2;
    float part = 0.0f;
    const int rb = row0 + acc.wm * Cfg::WTM + a * 32;
    auto flush = [&](int o) {
      T* base = o == 0 ? dH + cw : o == 1 ? dH + n + cw : As + cw;
      const int ld = o == 2 ? n : n2;
      stg[o].flush(
          [&](int r) -> T* { return rb + r < rend ? base + int64_t(rb + r) * ld : nullptr; });
    };
    // output o of the four values at column group (b, q): 0 = dH gate,
    // 1 = dH up, 2 = s * A; o == 0 also accumulates the dS row sum
    auto outputs = [&](int o, int b, int q, T (&v)[4]) {
      const int j = acc.col(b, q);
      T g4[4], u4[4];
      if constexpr (kPreH) {
        __builtin_memcpy(g4, hpre[a][b][q][0], sizeof(g4));
        __builtin_memcpy(u4, hpre[a][b][q][1], sizeof(u4));
      } else {
        __builtin_memcpy(g4, hrow + j, sizeof(g4));
        __builtin_memcpy(u4, hrow + n + j, sizeof(u4));
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float x = acc.acc[a][b][q * 4 + c];  // dA'
        const float g = Elem<T>::load(g4[c]), u = Elem<T>::load(u4[c]);
        const float sg = sigmoidf_(g), silu = g * sg;
        const float av = silu * u;
        const float da = s * x;
        if (o == 0) {
          part += x * av;
          v[c] = Elem<T>::store(da * u * sg * (1.0f + g * (1.0f - sg)));
        } else if (o == 1) {
          v[c] = Elem<T>::store(da * silu);
        } else {
          v[c] = Elem<T>::store(s * av);
        }
      }
    };
    if constexpr (kAll) {
      // three buffers: every value computed once, all three staged together
#pragma unroll
      for (int b = 0; b < Cfg::NB; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int o = 0; o < 3; ++o) {
            T v[4];
            outputs(o, b, q, v);
            stg[o].put(r32, b * 32 + q * 8 + h * 4, v);
          }
#pragma unroll
      for (int o = 0; o < 3; ++o) flush(o);
    } else {
      // one buffer: one output at a time (the small H fragment is reread and
      // the activation recomputed, which keeps the registers in check)
#pragma unroll
      for (int o = 0; o < 3; ++o) {
        __builtin_amdgcn_sched_barrier(0);  // keep the three passes apart in the schedule
#pragma unroll
        for (int b = 0; b < Cfg::NB; ++b)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            T v[4];
            outputs(o, b, q, v);
            stg[o].put(r32, b * 32 + q * 8 + h * 4, v);
          }
        flush(o);
      }
    }
    part += __shfl_xor(part, 32, 64);
    if (acc.lane < 32) red[acc.wn * BM + i] = part;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < BM; i += Cfg::kThreads) {
    const int slot = row0 + i;
    if (slot < rend) {
      float sum = 0.0f;
#pragma unroll
      for (int w = 0; w < WGN; ++w) sum += red[w * BM + i];
      dS[slot] = sum;
    }
  }
}

// A = dH rows (K-major), B = W1_e rows (K-major, contraction over 2n).
template <class Cfg, class T = typename Cfg::T>
__global__ __launch_bounds__(Cfg::kThreads) void k_dxt(
    const T* __restrict__ dH, const T* __restrict__ W1, T* __restrict__ dXt,
    const int32_t* __restrict__ tile_expert, const int32_t* __restrict__ tile_row,
    const int32_t* __restrict__ expert_offsets, const int32_t* __restrict__ totals, int d,
    int n, int nslot) {
  static_assert(Cfg::BM == kTileM, "128-row tiles");
  __shared__ __attribute__((aligned(1024))) char lds[Cfg::LDS_BYTES];
  constexpr int BN = Cfg::BN;
  const int NT = d / BN, n2 = 2 * n;
  const int lin = xcd_tile(blockIdx.x, totals[1] * NT);
  if (lin < 0) return;
  // W1_e is d x 2n (4 MB at d = 4096, n = 256, as large as the L2): walk
  // groups of an expert's M-tiles column tile by column tile
  int mt, nt;
  grouped_tile<8>(lin, NT, tile_expert, tile_row, expert_offsets, mt, nt);
  const int e = tile_expert[mt], row0 = tile_row[mt];
  const int rend = tile_end(tile_row, totals, mt, row0);
  const int j0 = nt * BN;

  const uint32_t hrow = uint32_t(n2) * sizeof(T);
  KLoad<Cfg, kTileM> la;
  la.init(dH, uint32_t(nslot) * hrow, [&](int r) {
    const int slot = row0 + r;
    return uint32_t(slot < rend ? slot : row0) * hrow;
  });
  KLoad<Cfg, BN> lb;
  lb.init(W1 + int64_t(e) * d * n2, uint32_t(d) * hrow,
          [&](int c) { return uint32_t(j0 + c) * hrow; });

  Accum<Cfg> acc;
  acc.init();
  pipeline<Cfg, true, true>(acc, lds, n2 / Cfg::BK, la, lb, NoTail{});

  static_assert(RowStage<T, Cfg::WTN>::BYTES * Cfg::NW <= Cfg::LDS_BYTES, "staging fits");
  store_acc_staged(acc, lds, [&](int r) -> T* {
    return row0 + r < rend ? dXt + int64_t(row0 + r) * d + j0 : nullptr;
  });
}

// dX-tilde as a persistent launch with loader waves (one workgroup per CU,
// Cfg::NPW > 0): the same tiles, in the same grouped order, walked by each
// workgroup in turn, so the next tile's first slabs are in flight while this
// tile's rows are written.
template <class Cfg, class T = typename Cfg::T>
__global__ __launch_bounds__(Cfg::kThreads) void k_dxt_p(
    const T* __restrict__ dH, const T* __restrict__ W1, T* __restrict__ dXt,
    const int32_t* __restrict__ tile_expert, const int32_t* __restrict__ tile_row,
    const int32_t* __restrict__ expert_offsets, const int32_t* __restrict__ totals, int d,
    int n, int nslot) {
  static_assert(Cfg::BM == kTileM && Cfg::NPW > 0, "128-row tiles with loader waves");
  struct Tile {
    int e, row0, rend, j0;
  };
  __shared__ __attribute__((aligned(1024))) char lds[Cfg::LDS_BYTES];
  __shared__ __attribute__((aligned(16))) Tile table[kPersistentTiles];
  constexpr int BN = Cfg::BN;
  const int NT = d / BN, n2 = 2 * n;
  const PersistentShare ps = PersistentShare::make(totals[1] * NT);
  if (ps.ntiles == 0 || ps.ntiles > kPersistentTiles) return;  // the host keeps it in range
  auto describe = [&](int k) {
    int mt, nt;
    grouped_tile<8>(ps.first + k * ps.stride, NT, tile_expert, tile_row, expert_offsets, mt, nt);
    Tile t;
    t.e = tile_expert[mt];
    t.row0 = tile_row[mt];
    t.rend = tile_end(tile_row, totals, mt, t.row0);
    t.j0 = nt * BN;
    return t;
  };
  const uint32_t hrow = uint32_t(n2) * sizeof(T);
  auto loaders = [&](const Tile& t) {
    LoadPair<KLoad<Cfg, kTileM>, KLoad<Cfg, BN>> p;
    p.la.init(dH, uint32_t(nslot) * hrow, [&](int r) {
      const int slot = t.row0 + r;
      return uint32_t(slot < t.rend ? slot : t.row0) * hrow;
    });
    p.lb.init(W1 + int64_t(t.e) * d * n2, uint32_t(d) * hrow,
              [&](int c) { return uint32_t(t.j0 + c) * hrow; });
    return p;
  };
  auto epilogue = [&](const Tile& t, const Accum<Cfg>& acc, char* stage) {
    static_assert(RowStage<T, Cfg::WTN>::BYTES * Cfg::NW <= Cfg::STAGE_BYTES, "staging fits");
    store_acc_staged(acc, stage, [&](int r) -> T* {
      return t.row0 + r < t.rend ? dXt + int64_t(t.row0 + r) * d + t.j0 : nullptr;
    });
  };
  persistent_split<Cfg, true, true>(lds, table, ps.ntiles, n2 / Cfg::BK, describe, loaders,
                                    epilogue);
}

// dX-tilde with the A operand in registers: a persistent launch (one
// workgroup per CU) over whole M tiles.  Each of the four compute waves reads
// its 32 dH rows (all 2n = 64 NSK k-values) once per M tile straight into
// MFMA operand registers, then sweeps the output columns in chunks of BN:
// the loader waves stream only W1_e (BN rows x 128 bytes per slab, K-major)
// through a ring of S stages, so a slab carries B alone and every B byte is
// used by all 128 rows of the tile.  A stage holds SUB consecutive k slabs,
// so the workgroup meets at a barrier once per SUB slabs.  A compute wave
// writes each finished 32 x BN chunk through its own staging buffer beside
// the ring.
template <class Cfg, int NSK, int SUB>
__global__ __launch_bounds__(Cfg::kThreads) void k_dxt_r(
    const bf16_t* __restrict__ dH, const bf16_t* __restrict__ W1, bf16_t* __restrict__ dXt,
    const int32_t* __restrict__ tile_expert, const int32_t* __restrict__ tile_row,
    const int32_t* __restrict__ totals, int d, int n, int nslot) {
  using T = bf16_t;
  static_assert(Cfg::BM == kTileM && Cfg::NPW > 0 && Cfg::WGN == 1 && Cfg::MB == 1,
                "whole 128-row tiles, one 32-row block per compute wave, loader waves");
  static_assert(NSK % SUB == 0, "whole stages per column chunk");
  constexpr int S = Cfg::STAGES, BN = Cfg::BN, SLAB = Cfg::B_BYTES, STAGE = SUB * SLAB;
  constexpr int NST = NSK / SUB;  // stages per column chunk
  using St = RowStage<T, Cfg::WTN>;
  struct Tile {
    int e, row0, rend;
  };
  __shared__ __attribute__((aligned(1024))) char lds[S * STAGE + Cfg::NW * St::BYTES];
  __shared__ Tile table[kPersistentTiles];
  const int n2 = 2 * n, NC = d / BN;
  const PersistentShare ps = PersistentShare::make(totals[1]);
  if (ps.ntiles == 0 || ps.ntiles > kPersistentTiles) return;  // the host keeps it in range
  for (int k = threadIdx.x; k < ps.ntiles; k += Cfg::kThreads) {
    const int mt = ps.first + k * ps.stride;
    Tile t;
    t.e = tile_expert[mt];
    t.row0 = tile_row[mt];
    t.rend = tile_end(tile_row, totals, mt, t.row0);
    table[k] = t;
  }
  __syncthreads();
  const int per_tile = NC * NST;  // stages per M tile
  const int G = ps.ntiles * per_tile;
  const uint32_t hrow = uint32_t(n2) * sizeof(T);
  if (Cfg::loads(wave_id())) {
    // Stage fill g holds k slabs SUB (g % NST) .. of column chunk
    // (g % per_tile) / NST of M tile g / per_tile.  The loader waves read no LDS (an LDS read after a DMA
    // into LDS would wait for every DMA in flight); each M tile's expert
    // comes from a scalar load issued one tile ahead.
    using LB = KLoad<Cfg, BN>;
    constexpr int NI = LB::NI, CPR = Cfg::KB / 16;
    const int lw = Cfg::loader_index(wave_id()), lane = threadIdx.x & 63;
    uint32_t boff[NI];  // W1 row r of the chunk and its swizzled 16-byte chunk
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int idx = (i * Cfg::NLW + lw) * 64 + lane, r = idx / CPR, pos = idx % CPR;
      boff[i] = uint32_t(r) * hrow + uint32_t((pos ^ kswz<Cfg::KB>(r)) << 4);
    }
    auto expert = [&](int k) { return tile_expert[ps.first + min(k, ps.ntiles - 1) * ps.stride]; };
    int kc = 0, ec = expert(0), en = expert(1);
    auto issue = [&](int g) {
      const int k = g / per_tile, c = (g % per_tile) / NST, s = (g % NST) * SUB;
      if (k != kc) {  // the next M tile: its expert was read one tile ago
        kc = k;
        ec = en;
        en = expert(k + 1);
      }
      const rsrc_t rs = make_rsrc(W1 + int64_t(ec) * d * n2, uint32_t(d) * hrow);
      char* stage = lds + (g % S) * STAGE;
#pragma unroll
      for (int u = 0; u < SUB; ++u) {
        const uint32_t add = uint32_t(c * BN) * hrow + uint32_t((s + u) * Cfg::KB);
#pragma unroll
        for (int i = 0; i < NI; ++i)
          dma16(rs, boff[i] + add, stage + u * SLAB + (i * Cfg::NLW + lw) * 1024);
      }
    };
    for (int g = 0; g < S - 1 && g < G; ++g) issue(g);
    for (int g = 0; g < G; ++g) {
      wait_slab<S, NI * SUB>(min(S - 2, G - 1 - g));
      barrier();
      if (g + S - 1 < G) issue(g + S - 1);
    }
    return;
  }
  Accum<Cfg> acc;
  const int lane = threadIdx.x & 63, r32 = lane & 31, h = lane >> 5;
  const int w = wave_id();
  char* stg = lds + S * STAGE;
  for (int k = 0; k < ps.ntiles; ++k) {
    const Tile t = table[k];
    // this lane's dH row (rows past the expert read the tile's first row),
    // k-values 16 c + 8 h .. + 7 of every 16-wide chunk c: the A operand
    const int row = t.row0 + w * 32 + r32;
    const T* src = dH + int64_t(row < t.rend ? row : t.row0) * n2 + 8 * h;
    Oct<T> a[4 * NSK];
#pragma unroll
    for (int c = 0; c < 4 * NSK; ++c) oct_load(a[c], src + 16 * c);
    for (int c = 0; c < NC; ++c) {
      acc.init();
#pragma unroll
      for (int s = 0; s < NST; ++s) {
        barrier();
        const char* B0 = lds + (((k * NC + c) * NST + s) % S) * STAGE;
        // the fragments of k chunk q + 1 are read while chunk q multiplies
        constexpr int NQ = SUB * Cfg::KCH;
        Oct<T> fb[2][Cfg::NB];
#pragma unroll
        for (int nb = 0; nb < Cfg::NB; ++nb) frag_k<T, Cfg::KB>(fb[0][nb], B0, nb * 32 + r32, 0, h);
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          if (q + 1 < NQ) {
            const char* B = B0 + ((q + 1) / Cfg::KCH) * SLAB;
#pragma unroll
            for (int nb = 0; nb < Cfg::NB; ++nb)
              frag_k<T, Cfg::KB>(fb[(q + 1) & 1][nb], B, nb * 32 + r32, (q + 1) % Cfg::KCH, h);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int nb = 0; nb < Cfg::NB; ++nb)
            mma16(acc.acc[0][nb], fb[q & 1][nb], a[s * NQ + q]);
        }
      }
      const int j0 = c * BN;
      store_acc_staged(acc, stg, [&](int r) -> T* {
        return t.row0 + r < t.rend ? dXt + int64_t(t.row0 + r) * d + j0 : nullptr;
      });
    }
  }
}

// Varlen-K scheduling.  The contraction of an expert with more than KC rows
// is cut into chunks of KC rows, so that no single tile can hold up the end
// of the kernel; every other expert is one chunk.  A plan lists the chunks
// ("items") by expert rank (descending slot count, so the largest work starts
// first; an expert without slots is one item whose tiles only write zeros).
// Item i carries its expert, its row range and, when the expert is split,
// the index of its fp32 partial-sum slab.  The PT output tiles of one
// item stay on one XCD (block b runs on XCD b % 8) so that the item's
// gathered rows are fetched into one L2.
struct VarlenItem {
  int e, kb, ke, pslot;  // pslot < 0: the item covers the whole expert
};
struct VarlenSplit {
  int e, pbase, nch, pad;  // expert, first partial slab, number of chunks
};

__device__ __forceinline__ bool varlen_item(int b, int PT, const int* n_items,
                                            const VarlenItem* items, VarlenItem* it,
                                            int* tile) {
  const int xcd = b % 8, local = b / 8;
  const int i = (local / PT) * 8 + xcd;
  if (i >= *n_items) return false;
  *it = items[i];
  *tile = local % PT;
  return true;
}

// One workgroup: the plans of both weight-gradient kernels (chunk sizes kc1,
// kc2).  Thread q handles expert rank q (E <= 1024).
constexpr int kPlanThreads = 1024;

__device__ __forceinline__ void plan_one(const int32_t* offsets, const int32_t* order, int E,
                                         int kc, int* header, VarlenItem* items,
                                         VarlenSplit* splits, int* sh) {
  const int q = threadIdx.x;
  int e = 0, beg = 0, cnt = 0, nch = 0;
  if (q < E) {
    e = order[q];
    beg = offsets[e];
    cnt = offsets[e + 1] - beg;
    nch = cnt > kc ? (cnt + kc - 1) / kc : 1;
  }
  const bool split = nch > 1;
  int n_items, n_part, n_split;
  const int ib = block_excl_scan(nch, sh, &n_items);
  const int pb = block_excl_scan(split ? nch : 0, sh, &n_part);
  const int sj = block_excl_scan(split ? 1 : 0, sh, &n_split);
  for (int c = 0; c < nch; ++c) {
    const int kb = beg + c * kc;
    items[ib + c] = VarlenItem{e, kb, min(kb + kc, beg + cnt), split ? pb + c : -1};
  }
  if (split) splits[sj] = VarlenSplit{e, pb, nch, 0};
  if (q == 0) {
    header[0] = n_items;
    header[1] = n_split;
  }
}

__global__ __launch_bounds__(kPlanThreads) void k_varlen_plan(
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ order, int E, int kc1,
    int kc2, int* header1, VarlenItem* items1, VarlenSplit* splits1, int* header2,
    VarlenItem* items2, VarlenSplit* splits2) {
  __shared__ int sh[kPlanThreads / 64 + 1];
  plan_one(offsets, order, E, kc1, header1, items1, splits1, sh);
  plan_one(offsets, order, E, kc2, header2, items2, splits2, sh);
}

// Schedules of the persistent weight-gradient kernels (one workgroup per
// plan; a plan with cap == 0 has none).  Every (item, tile) pair of a plan
// goes to one of the 256 workgroups, balancing their work by the longest-
// first greedy rule: the items (listed by the plan in descending size) go
// one after another to the XCD with the least work so far, so all tiles of
// an item and its gathered rows stay in one L2; then, per XCD, the PT
// tiles of each item in turn go to its 32 workgroups in ascending order of
// their work so far (tile t to the workgroup of rank t mod 32).  A pair
// costs its slabs plus three for its epilogue (two for a zero tile).  The
// plan needs only the routing, so this runs before dH is ready.
// Workgroup b = x + 8 l (XCD x, local index l) gets the list
// list[b * cap ..] of pair codes item * PT + tile, in item order, and its
// length cnt[b].
constexpr int kSchedThreads = 512;
constexpr int kSchedItems = 1536;  // items of one plan (the host checks)

__device__ __forceinline__ void sched_one(const int* __restrict__ header,
                                          const VarlenItem* __restrict__ items, int PT, int cap,
                                          int* __restrict__ cnt, int* __restrict__ list) {
  __shared__ int cost[kSchedItems];
  __shared__ uint8_t xcd_of[kSchedItems];
  __shared__ int16_t xl[8][kSchedItems];
  __shared__ int xn[8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ni = min(header[0], kSchedItems);
  for (int i = tid; i < ni; i += kSchedThreads) {
    const int r = items[i].ke - items[i].kb;
    cost[i] = r > 0 ? (r + 63) / 64 + 3 : 2;
  }
  __syncthreads();
  if (wave == 0) {  // items to XCDs: one wave, the eight keys (work << 3 | XCD) in scalar registers
    int key[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) key[x] = x;
    for (int i0 = 0; i0 < ni; i0 += 64) {
      const int cv = i0 + lane < ni ? cost[i0 + lane] * PT : 0;
      const int m = min(64, ni - i0);
      int xv = 0;  // lane j: the XCD of item i0 + j
      for (int j = 0; j < m; ++j) {
        const int c8 = __builtin_amdgcn_readlane(cv, j) << 3;
        int best = key[0];  // least work, then lowest XCD
#pragma unroll
        for (int x = 1; x < 8; ++x) best = min(best, key[x]);
        best = __builtin_amdgcn_readfirstlane(best);
#pragma unroll
        for (int x = 0; x < 8; ++x) key[x] += key[x] == best ? c8 : 0;
        xv = lane == j ? (best & 7) : xv;
      }
      if (lane < m) xcd_of[i0 + lane] = uint8_t(xv);
    }
  }
  __syncthreads();
  if (wave < 8) {  // wave x lists XCD x's items in plan order
    const int x = wave;
    int n = 0;
    for (int i0 = 0; i0 < ni; i0 += 64) {
      const bool mine = i0 + lane < ni && xcd_of[i0 + lane] == x;
      const uint64_t bal = __ballot(mine);
      if (mine)
        xl[x][n + __builtin_amdgcn_mbcnt_hi(uint32_t(bal >> 32),
                                            __builtin_amdgcn_mbcnt_lo(uint32_t(bal), 0))] =
            int16_t(i0 + lane);
      n += __popcll(bal);
    }
    if (lane == 0) xn[x] = n;
  }
  __syncthreads();
  if (wave < 8) {  // wave x: XCD x's pairs; lane l < 32 is workgroup b = x + 8 l
    const int x = wave, b = x + 8 * lane, nx = xn[x];
    int key = lane < 32 ? lane : INT_MAX;  // work << 5 | l
    int c = 0;                             // entries of b's list
    int* const mine = list + int64_t(lane < 32 ? b : 0) * cap;  // lanes past 31 write nothing
    for (int k0 = 0; k0 < nx; k0 += 64) {
      const int iv = k0 + lane < nx ? xl[x][k0 + lane] : 0;
      const int cv = k0 + lane < nx ? cost[iv] : 0;
      const int m = min(64, nx - k0);
      for (int j = 0; j < m; ++j) {
        const int i = __builtin_amdgcn_readlane(iv, j), ci = __builtin_amdgcn_readlane(cv, j);
        int r = 0;  // this workgroup's rank by work so far
#pragma unroll
        for (int q = 0; q < 32; ++q) r += __builtin_amdgcn_readlane(key, q) < key ? 1 : 0;
        if (lane < 32) {
          int nt = 0;
          for (int t = r; t < PT && c < cap; t += 32, ++nt) mine[c++] = i * PT + t;
          key += (nt * ci) << 5;
        }
      }
    }
    if (lane < 32) cnt[b] = c;
  }
}

__global__ __launch_bounds__(kSchedThreads) void k_dw_sched(
    const int* __restrict__ header1, const VarlenItem* __restrict__ items1, int PT1, int cap1,
    int* __restrict__ cnt1, int* __restrict__ list1, const int* __restrict__ header2,
    const VarlenItem* __restrict__ items2, int PT2, int cap2, int* __restrict__ cnt2,
    int* __restrict__ list2) {
  if (blockIdx.x == 0 && cap1 > 0) sched_one(header1, items1, PT1, cap1, cnt1, list1);
  if (blockIdx.x == 1 && cap2 > 0) sched_one(header2, items2, PT2, cap2, cnt2, list2);
}

// out_e = sum over the chunks of a split expert of its fp32 partials, in
// chunk order (so the result does not depend on which chunk finished first).
// Work unit u = j * gy + g covers split expert j, elements g*2048 .. +2048
// (eight per thread); the blocks stride over the units that exist, and the
// chunk loads are issued four at a time so that they are in flight together.
template <class T>
__global__ __launch_bounds__(256) void k_varlen_reduce(const int* __restrict__ header,
                                                       const VarlenSplit* __restrict__ splits,
                                                       const float* __restrict__ partials,
                                                       T* __restrict__ out, int64_t mn, int gy) {
  const int units = header[1] * gy;
  for (int u = blockIdx.x; u < units; u += gridDim.x) {
    const VarlenSplit sp = splits[u / gy];
    const int64_t i = (int64_t(u % gy) * 256 + threadIdx.x) * 8;
    if (i >= mn) continue;
    float acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = 0.0f;
    for (int k0 = 0; k0 < sp.nch; k0 += 4) {
      float4 x[4], y[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (k0 + v < sp.nch) {
          const float4* q =
              reinterpret_cast<const float4*>(partials + (sp.pbase + k0 + v) * mn + i);
          x[v] = q[0];
          y[v] = q[1];
        } else {
          x[v] = y[v] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {  // chunk order
        acc[0] += x[v].x; acc[1] += x[v].y; acc[2] += x[v].z; acc[3] += x[v].w;
        acc[4] += y[v].x; acc[5] += y[v].y; acc[6] += y[v].z; acc[7] += y[v].w;
      }
    }
    Oct<T> r;
    oct_from(r, acc);
    oct_store(out + sp.e * mn + i, r);
  }
}

// fp32 partial of one output tile: lane l holds four consecutive columns of
// row l % 32 of each 32 x 32 block, written as one 16-byte store.
template <class Cfg>
__device__ __forceinline__ void store_tile_f32(const Accum<Cfg>& acc, float* out, int ld) {
#pragma unroll
  for (int a = 0; a < Cfg::MB; ++a)
#pragma unroll
    for (int b = 0; b < Cfg::NB; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4_t v = {__float_as_uint(acc.acc[a][b][q * 4 + 0]),
                           __float_as_uint(acc.acc[a][b][q * 4 + 1]),
                           __float_as_uint(acc.acc[a][b][q * 4 + 2]),
                           __float_as_uint(acc.acc[a][b][q * 4 + 3])};
        __builtin_nontemporal_store(
            v, reinterpret_cast<u32x4_t*>(out + int64_t(acc.row(a)) * ld + acc.col(b, q)));
      }
}

// Zeroes a ROWS x COLS weight-gradient tile of an expert that was given no
// slots (its gradient is exactly zero): whole rows of 16-byte non-temporal
// stores by NT threads (thread index tid), without the accumulators and the
// staging round trip.
template <class T, int ROWS, int COLS, int NT>
__device__ __forceinline__ void zero_block(T* out, int ld, int tid) {
  constexpr int CPR = COLS * int(sizeof(T)) / 16;  // chunks per row
  static_assert((ROWS * CPR) % NT == 0, "whole rounds");
  const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll 4
  for (int q = tid; q < ROWS * CPR; q += NT) {
    char* row = reinterpret_cast<char*>(out + int64_t(q / CPR) * ld);
    __builtin_nontemporal_store(z, reinterpret_cast<u32x4_t*>(row + (q % CPR) * 16));
  }
}
template <class Cfg>
__device__ __forceinline__ void zero_tile(typename Cfg::T* out, int ld) {
  zero_block<typename Cfg::T, Cfg::BM, Cfg::BN, Cfg::kThreads>(out, ld, threadIdx.x);
}

// Writes a full weight-gradient tile (rows i0.., columns j0..) through the
// epilogue staging buffers.
template <class Cfg>
__device__ __forceinline__ void store_tile(const Accum<Cfg>& acc, char* lds,
                                           typename Cfg::T* out, int ld) {
  using T = typename Cfg::T;
  static_assert(RowStage<T, Cfg::WTN>::BYTES * Cfg::NW <= Cfg::LDS_BYTES, "staging fits");
  store_acc_staged(acc, lds, [&](int r) -> T* { return out + int64_t(r) * ld; });
}


// dW1_e[i][j] = sum over the expert's slots k of X[tok_k][i] * dH[k][j]:
// both operands MN-major, rows = slots (X rows gathered through slot_token).
template <class Cfg, class T = typename Cfg::T>
__global__ __launch_bounds__(Cfg::kThreads) void k_dw1(
    const T* __restrict__ X, const T* __restrict__ dH, T* __restrict__ dW1,
    float* __restrict__ partials, const int* __restrict__ n_items,
    const VarlenItem* __restrict__ items, const int32_t* __restrict__ slot_token, int d, int n,
    int ntok, int nslot) {
  __shared__ __attribute__((aligned(1024))) char lds[Cfg::LDS_BYTES];
  constexpr int BM = Cfg::BM, BN = Cfg::BN, EPC = 16 / int(sizeof(T));
  const int n2 = 2 * n, TN = n2 / BN, PT = (d / BM) * TN;
  VarlenItem it;
  int tile;
  if (!varlen_item(blockIdx.x, PT, n_items, items, &it, &tile)) return;
  const int i0 = (tile / TN) * BM, j0 = (tile % TN) * BN;
  const int kb = it.kb, ke = it.ke;
  if (ke == kb) {  // an expert without slots (never split)
    zero_tile<Cfg>(dW1 + (int64_t(it.e) * d + i0) * n2 + j0, n2);
    return;
  }
  const int nslabs = (ke - kb + Cfg::BK - 1) / Cfg::BK;

  SlotLoad<Cfg, BM, true> la;
  la.init(X, uint32_t(ntok) * d * sizeof(T), uint32_t(d) * sizeof(T),
          [=](int c) { return int((i0 + c * EPC) * sizeof(T)); }, slot_token, kb, ke);
  SlotLoad<Cfg, BN, false> lb;
  lb.init(dH, uint32_t(nslot) * n2 * sizeof(T), uint32_t(n2) * sizeof(T),
          [=](int c) { return int((j0 + c * EPC) * sizeof(T)); }, nullptr, kb, ke);

  Accum<Cfg> acc;
  acc.init();
  VarlenTail<Cfg, BM, BN> tail{nslabs, ke - kb - (nslabs - 1) * Cfg::BK};
  pipeline<Cfg, false, false>(acc, lds, nslabs, la, lb, tail);
  if (it.pslot < 0)
    store_tile(acc, lds, dW1 + (int64_t(it.e) * d + i0) * n2 + j0, n2);
  else
    store_tile_f32(acc, partials + (int64_t(it.pslot) * d + i0) * n2 + j0, n2);
}

// dW2_e[i][j] = sum over the expert's slots k of As[k][i] * dO[tok_k][j].
template <class Cfg, class T = typename Cfg::T>
__global__ __launch_bounds__(Cfg::kThreads) void k_dw2(
    const T* __restrict__ As, const T* __restrict__ dO, T* __restrict__ dW2,
    float* __restrict__ partials, const int* __restrict__ n_items,
    const VarlenItem* __restrict__ items, const int32_t* __restrict__ slot_token, int d, int n,
    int ntok, int nslot) {
  __shared__ __attribute__((aligned(1024))) char lds[Cfg::LDS_BYTES];
  constexpr int BM = Cfg::BM, BN = Cfg::BN, EPC = 16 / int(sizeof(T));
  const int TN = d / BN, PT = (n / BM) * TN;
  VarlenItem it;
  int tile;
  if (!varlen_item(blockIdx.x, PT, n_items, items, &it, &tile)) return;
  const int i0 = (tile / TN) * BM, j0 = (tile % TN) * BN;
  const int kb = it.kb, ke = it.ke;
  if (ke == kb) {  // an expert without slots (never split)
    zero_tile<Cfg>(dW2 + (int64_t(it.e) * n + i0) * d + j0, d);
    return;
  }
  const int nslabs = (ke - kb + Cfg::BK - 1) / Cfg::BK;

  SlotLoad<Cfg, BM, false> la;
  la.init(As, uint32_t(nslot) * n * sizeof(T), uint32_t(n) * sizeof(T),
          [=](int c) { return int((i0 + c * EPC) * sizeof(T)); }, nullptr, kb, ke);
  SlotLoad<Cfg, BN, true> lb;
  lb.init(dO, uint32_t(ntok) * d * sizeof(T), uint32_t(d) * sizeof(T),
          [=](int c) { return int((j0 + c * EPC) * sizeof(T)); }, slot_token, kb, ke);

  Accum<Cfg> acc;
  acc.init();
  VarlenTail<Cfg, BM, BN> tail{nslabs, ke - kb - (nslabs - 1) * Cfg::BK};
  pipeline<Cfg, false, false>(acc, lds, nslabs, la, lb, tail);
  if (it.pslot < 0)
    store_tile(acc, lds, dW2 + (int64_t(it.e) * n + i0) * d + j0, d);
  else
    store_tile_f32(acc, partials + (int64_t(it.pslot) * n + i0) * d + j0, d);
}

// One MN-major operand of a varlen-K tile as a loader wave issues it: COLS
// columns (from col0) of the source rows of slots s0 .. s0 + BK - 1, where
// slot s reads row slot_token[s] (GATHER) or row s of a buffer of `rows`
// rows of `cols` elements.  Loader wave w fills the tile rows 16 w .. 16 w +
// 15 (BK = 64, four loader waves): lane L of its instruction i fills row
// 16 w + i RPI + L / CH with the logical 16-byte chunk that the swizzle
// places at chunk L % CH.  Slots at or past the item's end ke read row
// `rows`, the first one past the buffer, so the DMA writes zeros to their
// LDS rows.  The 16 gather indices of a wave's rows are one 64-byte scalar
// load, issued a slab ahead of their use (fetch, then issue); scalar loads
// leave the in-order vector-memory counter of the DMA alone.
template <class Cfg, int COLS, bool GATHER>
struct SlotOperand {
  static constexpr int RB = COLS * 2, CH = RB / 16, RPI = 64 / CH;
  static constexpr int NI = 16 * RB / 1024;  // instructions per wave and slab
  static_assert(Cfg::BK == 64 && Cfg::NLW == 4, "four loader waves of 16 rows each");
  static_assert(RPI == 2 || RPI == 4, "rows of 256 or 512 bytes");
  rsrc_t rs;
  uint32_t ld;
  int nrows;
  uint32_t chunk[NI];  // byte offset, within the source row, of the chunk this lane fetches
  int w, q;            // loader wave index; this lane's row among an instruction's RPI rows
  // GATHER: tokens of this wave's 16 slots of the next slab (a vector value,
  // so that selecting one per lane never becomes an indexed memory access)
  typedef int v16i_t __attribute__((ext_vector_type(16)));
  v16i_t t;

  __device__ __forceinline__ void init(const bf16_t* base, int rows, int cols, int w_, int lane) {
    ld = uint32_t(cols) * 2u;
    nrows = rows;
    rs = make_rsrc(base, uint32_t(rows) * ld);
    w = w_;
    q = lane / CH;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int k = 16 * w + i * RPI + q;
      chunk[i] = uint32_t(((lane % CH) ^ mswz<CH>(k)) << 4);
    }
  }
  // The gather indices of the slab at slot s0 (slot_token holds nslot
  // entries; near its end each index is clamped to a slot below ke).
  __device__ __forceinline__ void fetch(int s0, int ke, const int32_t* __restrict__ tok,
                                        int nslot) {
    if constexpr (GATHER) {
      const int b = s0 + 16 * w;
      v16i_t v;
      if (b + 16 <= nslot) {
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = tok[b + j];
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = tok[min(b + j, ke - 1)];
      }
      t = v;
    }
  }
  __device__ __forceinline__ void issue(char* tile, int s0, int ke, int col0) const {
    const uint32_t cb = uint32_t(col0) * 2u;
    const v16i_t tv = t;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int slot = s0 + 16 * w + i * RPI + q;
      int v = slot;
      if constexpr (GATHER) {
        v = tv[i * RPI];
#pragma unroll
        for (int p = 1; p < RPI; ++p) v = q == p ? tv[i * RPI + p] : v;
      }
      const int row = slot < ke ? v : nrows;
      dma16(rs, uint32_t(row) * ld + cb + chunk[i], tile + (w * NI + i) * 1024);
    }
  }
};

// Weight gradients out_e = A_e^T B_e (varlen-K over the expert's slots) in a
// persistent launch with loader waves: workgroup b (one per CU, on XCD b % 8)
// walks the (item, output tile) pairs that k_dw_sched listed for it, pair
// code c = item * PT + tile.  A and B are MN-major with one row per slot:
// token rows read through slot_token when GA / GB, else slot rows.  Loader
// and compute waves pass one barrier per slab and one per tile (items
// without slots have neither: the compute waves write their zero tiles
// directly), so the loader waves run up to S - 1 slabs ahead across tile
// boundaries and the next tile's first slabs land while the compute waves
// write the last one.  Both roles read the list and the items with scalar
// loads.  A split item's tile goes to its fp32 partial slab, reduced
// afterwards.
template <class Cfg, bool GA, bool GB>
__global__ __launch_bounds__(Cfg::kThreads) void k_dw_p(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ B, bf16_t* __restrict__ out,
    float* __restrict__ partials, const VarlenItem* __restrict__ items,
    const int* __restrict__ sched_cnt, const int* __restrict__ sched_list, int cap,
    const int32_t* __restrict__ slot_token, int M, int N, int a_rows, int b_rows, int nslot) {
  using T = bf16_t;
  static_assert(Cfg::NPW > 0 && !Cfg::PAIRED, "loader waves, plain columns");
  constexpr int S = Cfg::STAGES, BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK;
  __shared__ __attribute__((aligned(1024))) char lds[Cfg::LDS_BYTES];
  const int TN = N / BN, PT = (M / BM) * TN;
  const int ntiles = sched_cnt[blockIdx.x];
  const int* __restrict__ mine = sched_list + int64_t(blockIdx.x) * cap;
  // pair k of this workgroup: its item and the output tile's first row / column
  auto pair = [&](int k, VarlenItem& it, int& i0, int& j0) {
    const int c = mine[k], tile = c % PT;
    it = items[c / PT];
    i0 = (tile / TN) * BM;
    j0 = (tile % TN) * BN;
  };

  if (Cfg::loads(wave_id())) {
    const int lw = Cfg::loader_index(wave_id()), lane = threadIdx.x & 63;
    SlotOperand<Cfg, BM, GA> oa;
    oa.init(A, a_rows, M, lw, lane);
    SlotOperand<Cfg, BN, GB> ob;
    ob.init(B, b_rows, N, lw, lane);
    constexpr int NI = SlotOperand<Cfg, BM, GA>::NI + SlotOperand<Cfg, BN, GB>::NI;
    static_assert(S >= 2 && S <= 4 && NI * (S - 2) < 64, "pipeline depth");
    // The issue side walks the same stream of slabs ahead of the barriers:
    // pair ki, its slab si of ns.
    int ki = -1, si = 0, ns = 0, kb = 0, ke = 0, i0 = 0, j0 = 0;
    auto next_pair = [&]() {  // the next pair with slots (ki == ntiles at the end)
      while (++ki < ntiles) {
        VarlenItem it;
        pair(ki, it, i0, j0);
        kb = it.kb;
        ke = it.ke;
        if (ke > kb) {
          ns = (ke - kb + BK - 1) / BK;
          si = 0;
          return;
        }
      }
    };
    auto fetch = [&]() {  // the gather indices of the next slab to issue
      if (ki >= ntiles) return;
      oa.fetch(kb + si * BK, ke, slot_token, nslot);
      ob.fetch(kb + si * BK, ke, slot_token, nslot);
    };
    next_pair();
    fetch();
    int issued = 0;
    auto issue = [&]() {
      if (ki >= ntiles) return;
      char* sp = lds + (issued % S) * Cfg::STAGE_BYTES;
      const int s0 = kb + si * BK;
      oa.issue(sp, s0, ke, i0);
      ob.issue(sp + Cfg::A_BYTES, s0, ke, j0);
      ++issued;
      if (++si == ns) next_pair();
      fetch();
    };
    for (int p = 0; p < S - 1; ++p) issue();
    int g = 0;  // slabs consumed
    for (int k = 0; k < ntiles; ++k) {
      VarlenItem it;
      int pi, pj;
      pair(k, it, pi, pj);
      const int kbk = it.kb, kek = it.ke;
      if (kek == kbk) continue;
      const int nsk = (kek - kbk + BK - 1) / BK;
      for (int j = 0; j < nsk; ++j, ++g) {
        wait_slab<S, NI>(issued - 1 - g);  // slab g landed; later ones may fly
        barrier();
        issue();  // into the stage of slab g - 1, which every compute wave is done with
      }
      barrier();  // the compute waves write tile k
    }
    return;
  }
  Accum<Cfg> acc;
  int g = 0;
  for (int k = 0; k < ntiles; ++k) {
    VarlenItem t;
    int i0, j0;
    pair(k, t, i0, j0);
    if (t.ke == t.kb) {  // an expert without slots (never split)
      zero_block<T, BM, BN, 64 * Cfg::NW>(out + (int64_t(t.e) * M + i0) * N + j0, N,
                                          threadIdx.x);
      continue;
    }
    const int ns = (t.ke - t.kb + BK - 1) / BK;
    acc.init();
    for (int j = 0; j < ns; ++j, ++g) {
      barrier();
      const char* cur = lds + (g % S) * Cfg::STAGE_BYTES;
      if constexpr (Cfg::NW == 8) acc.template slab1<false, false>(cur, cur + Cfg::A_BYTES);
      else acc.template slab<false, false>(cur, cur + Cfg::A_BYTES);
    }
    barrier();  // every compute wave is done with the last slab's stage
    if (t.pslot < 0) {
      static_assert(RowStage<T, Cfg::WTN>::BYTES * Cfg::NW <= Cfg::STAGE_BYTES, "staging fits");
      T* o = out + (int64_t(t.e) * M + i0) * N + j0;
      store_acc_staged(acc, lds + ((g - 1) % S) * Cfg::STAGE_BYTES,
                       [&](int r) -> T* { return o + int64_t(r) * N; });
    } else {
      store_tile_f32(acc, partials + (int64_t(t.pslot) * M + i0) * N + j0, N);
    }
  }
}

template <class Cfg>
void dh_launch(const LayerArgs& a, const void* dO, const void* W2, const void* H, void* dH,
               void* As, float* dS, hipStream_t st) {
  using T = typename Cfg::T;
  hipLaunchKernelGGL((k_dh<Cfg>), dim3(grid_for(a.tile_cap * (kTileM / Cfg::BM))),
                     dim3(Cfg::kThreads), 0, st, static_cast<const T*>(dO),
                     static_cast<const T*>(W2), static_cast<const T*>(H), static_cast<T*>(dH),
                     static_cast<T*>(As), dS, a.tile_expert, a.tile_row,
                     a.slot_token, a.slot_weight, a.totals, a.d, a.T);
}

template <class T>
hipError_t dh_t(const LayerArgs& a, const void* dO, const void* W2, const void* H, void* dH,
                void* As, float* dS, hipStream_t st) {
  switch (a.n) {
    case 64: dh_launch<TileCfg<T, 128, 64, 4, 1, 3>>(a, dO, W2, H, dH, As, dS, st); break;
    case 128: dh_launch<TileCfg<T, 128, 128, 2, 2, 3>>(a, dO, W2, H, dH, As, dS, st); break;
    case 256:
      if constexpr (sizeof(T) == 2) dh_launch<DhWide>(a, dO, W2, H, dH, As, dS, st);
      else dh_launch<TileCfg<T, 128, 256, 2, 2, 3>>(a, dO, W2, H, dH, As, dS, st);
      break;
    case 384: dh_launch<TileCfg<T, 64, 384, 1, 4, 3>>(a, dO, W2, H, dH, As, dS, st); break;
    case 512:
      if constexpr (sizeof(T) == 2) dh_launch<DhWide512>(a, dO, W2, H, dH, As, dS, st);
      else dh_launch<TileCfg<T, 64, 512, 1, 4, 2>>(a, dO, W2, H, dH, As, dS, st);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class Cfg>
void dxt_launch(const LayerArgs& a, const void* dH, const void* W1, void* dXt, hipStream_t st) {
  using T = typename Cfg::T;
  hipLaunchKernelGGL((k_dxt<Cfg>), dim3(grid_for(a.tile_cap * (a.d / Cfg::BN))),
                     dim3(Cfg::kThreads), 0, st, static_cast<const T*>(dH),
                     static_cast<const T*>(W1), static_cast<T*>(dXt), a.tile_expert, a.tile_row,
                     a.expert_offsets, a.totals, a.d, a.n, int(a.slot_cap));
}

// Chunking of one varlen-K kernel: PT output tiles per expert, chunks of kc
// rows, and the capacities of its plan.
struct VarlenDims {
  int PT, kc, max_items, max_split;
  int64_t mn;  // elements of one expert's gradient matrix
  int cap;     // persistent kernel: capacity of each workgroup's pair list (0: per-tile kernel)
};

// kc: one CU's fair share of the kernel's work (in rows of a tile), so that
// no chunk is longer than what every CU has to do anyway; only experts that
// would otherwise hold up the end of the kernel are split (each split costs
// an fp32 partial written and read back).  A multiple of the slab depth, at
// least four slabs.
inline VarlenDims varlen_dims(int64_t slot_cap, int E, int PT, int BK, int64_t mn) {
  int64_t kc = slot_cap * PT / kNumCUs;
  kc = std::max<int64_t>(kc, 4 * BK);
  kc = (kc + BK - 1) / BK * BK;
  VarlenDims v;
  v.PT = PT;
  v.kc = int(std::min<int64_t>(kc, 1 << 30));
  const int64_t chunks = (slot_cap + v.kc - 1) / v.kc;
  v.max_items = int(E + chunks);  // every expert is one item, plus extra chunks
  v.max_split = int(2 * chunks);  // a split expert has r > kc rows and < 2 r / kc chunks
  v.mn = mn;
  v.cap = 0;
  return v;
}

// Tile configurations of the two weight-gradient kernels; f(CfgTag<Cfg>{})
// is called with the one the problem uses (the launchers and the workspace
// sizing share this choice).
template <class C>
struct CfgTag {
  using type = C;
};

// The persistent kernel takes tile Cfg for an M x N gradient when the tile
// divides it and the schedule can list every item of the plan.
template <class Cfg>
bool split_fits(int M, int N, int64_t slot_cap, int E) {
  if (M % Cfg::BM != 0 || N % Cfg::BN != 0) return false;
  const int PT = (M / Cfg::BM) * (N / Cfg::BN);
  return varlen_dims(slot_cap, E, PT, Cfg::BK, 0).max_items <= kSchedItems;
}
// A workgroup gets at most ceil(PT / 32) tiles of each item.
inline int sched_cap(const VarlenDims& v) { return v.max_items * ((v.PT + 31) / 32); }

template <class F>
void dw1_cfg(bool f32, int d, int n, int E, int64_t slot_cap, F&& f) {
  const int n2 = 2 * n;
  if (f32) f(CfgTag<TileCfg<float, 128, 128, 2, 2, 3>>{});
  else if (split_fits<GradSplit256>(d, n2, slot_cap, E)) f(CfgTag<GradSplit256>{});
  else if (split_fits<GradSplit>(d, n2, slot_cap, E)) f(CfgTag<GradSplit>{});
  else if (d % 256 == 0 && n2 % 256 == 0) f(CfgTag<GradSquare>{});
  else if (n2 % 256 == 0) f(CfgTag<GradTall>{});
  else f(CfgTag<GradSmall>{});
}

template <class F>
void dw2_cfg(bool f32, int d, int n, int E, int64_t slot_cap, F&& f) {
  if (f32) {
    if (n % 128 == 0) f(CfgTag<TileCfg<float, 128, 128, 2, 2, 3>>{});
    else f(CfgTag<TileCfg<float, 64, 128, 2, 2, 3>>{});
  } else if (split_fits<GradSplit256>(n, d, slot_cap, E)) {
    f(CfgTag<GradSplit256>{});
  } else if (split_fits<GradSplit>(n, d, slot_cap, E)) {
    f(CfgTag<GradSplit>{});
  } else if (n % 256 == 0 && d % 256 == 0) {
    f(CfgTag<GradSquare>{});
  } else if (n % 128 == 0 && d % 256 == 0) {
    f(CfgTag<GradTall>{});
  } else if (n % 128 == 0) {
    f(CfgTag<GradSmall>{});
  } else {
    f(CfgTag<TileCfg<bf16_t, 64, 128, 2, 2, 3>>{});
  }
}

VarlenDims dw1_dims(bool f32, int d, int n, int E, int64_t slot_cap) {
  VarlenDims v{};
  dw1_cfg(f32, d, n, E, slot_cap, [&](auto tag) {
    using Cfg = typename decltype(tag)::type;
    v = varlen_dims(slot_cap, E, (d / Cfg::BM) * (2 * n / Cfg::BN), Cfg::BK, int64_t(d) * 2 * n);
    if constexpr (Cfg::NPW > 0) v.cap = sched_cap(v);
  });
  return v;
}

VarlenDims dw2_dims(bool f32, int d, int n, int E, int64_t slot_cap) {
  VarlenDims v{};
  dw2_cfg(f32, d, n, E, slot_cap, [&](auto tag) {
    using Cfg = typename decltype(tag)::type;
    v = varlen_dims(slot_cap, E, (n / Cfg::BM) * (d / Cfg::BN), Cfg::BK, int64_t(n) * d);
    if constexpr (Cfg::NPW > 0) v.cap = sched_cap(v);
  });
  return v;
}

// Workspace of the weight-gradient phase: two plans, then the fp32 partial
// slabs (shared: dW2 runs after dW1's reduction).
struct VarlenWs {
  size_t hdr1, items1, splits1, hdr2, items2, splits2, cnt1, list1, cnt2, list2, partials, total;
  static size_t align(size_t x) { return (x + 255) & ~size_t(255); }
  static VarlenWs make(const VarlenDims& v1, const VarlenDims& v2, int E) {
    VarlenWs w;
    size_t o = 0;
    w.hdr1 = o; o = align(o + 16);
    w.items1 = o; o = align(o + size_t(v1.max_items) * sizeof(VarlenItem));
    w.splits1 = o; o = align(o + size_t(E) * sizeof(VarlenSplit));
    w.hdr2 = o; o = align(o + 16);
    w.items2 = o; o = align(o + size_t(v2.max_items) * sizeof(VarlenItem));
    w.splits2 = o; o = align(o + size_t(E) * sizeof(VarlenSplit));
    w.cnt1 = o; o = align(o + (v1.cap > 0 ? kNumCUs * sizeof(int) : 0));
    w.list1 = o; o = align(o + size_t(kNumCUs) * size_t(v1.cap) * sizeof(int));
    w.cnt2 = o; o = align(o + (v2.cap > 0 ? kNumCUs * sizeof(int) : 0));
    w.list2 = o; o = align(o + size_t(kNumCUs) * size_t(v2.cap) * sizeof(int));
    w.partials = o;
    o += std::max(size_t(v1.max_split) * size_t(v1.mn), size_t(v2.max_split) * size_t(v2.mn)) * 4;
    w.total = align(o);
    return w;
  }
};

template <class T>
void reduce_launch(const int* hdr, const VarlenSplit* splits, const float* partials, void* out,
                   const VarlenDims& v, hipStream_t st) {
  const int gy = int((v.mn + 2047) / 2048);  // 2048-element units per expert
  const unsigned grid = unsigned(std::min<int64_t>(int64_t(v.max_split) * gy, 2048));
  hipLaunchKernelGGL((k_varlen_reduce<T>), dim3(grid), dim3(256), 0, st, hdr, splits, partials,
                     static_cast<T*>(out), v.mn, gy);
}

}  // namespace

hipError_t launch_dh(const LayerArgs& a, const void* dO, const void* W2, const void* H, void* dH,
                     void* As, float* dS, hipStream_t st) {
  return a.f32 ? dh_t<float>(a, dO, W2, H, dH, As, dS, st)
               : dh_t<bf16_t>(a, dO, W2, H, dH, As, dS, st);
}

hipError_t launch_dxt(const LayerArgs& a, const void* dH, const void* W1, void* dXt,
                      hipStream_t st) {
  // dH rows in registers (2n <= 512, so they fit in 128 registers per lane),
  // else the persistent 256-wide tiles up to d = 2048, else the per-tile
  // 512-wide ones.
  using R = RowsReg;
  const bool reg_tiles = PersistentShare::max_tiles(a.tile_cap, kNumCUs) <= kPersistentTiles;
  if (!a.f32 && a.d % R::BN == 0 && reg_tiles && (a.n == 64 || a.n == 128 || a.n == 256)) {
    auto go = [&](auto kern) {
      hipLaunchKernelGGL(kern, dim3(kNumCUs), dim3(R::kThreads), 0, st,
                         static_cast<const bf16_t*>(dH), static_cast<const bf16_t*>(W1),
                         static_cast<bf16_t*>(dXt), a.tile_expert, a.tile_row, a.totals, a.d,
                         a.n, int(a.slot_cap));
    };
    if (a.n == 256) go(k_dxt_r<R, 8, 2>);
    else if (a.n == 128) go(k_dxt_r<R, 4, 2>);
    else go(k_dxt_r<R, 2, 2>);
    return hipGetLastError();
  }
  // The persistent tile is 256 columns wide, so every dH row block is read
  // d / 256 times; past 2048 columns that re-reading costs more than the
  // overlap gains (measured at d = 4096), and the 512-wide tiles run instead.
  using P = RowsSplit;
  if (!a.f32 && a.d % P::BN == 0 && a.d <= 2048 && 2 * a.n / P::BK >= P::STAGES - 1 &&
      PersistentShare::max_tiles(a.tile_cap * (a.d / P::BN), kNumCUs) <= kPersistentTiles) {
    hipLaunchKernelGGL((k_dxt_p<P>), dim3(kNumCUs), dim3(P::kThreads), 0, st,
                       static_cast<const bf16_t*>(dH), static_cast<const bf16_t*>(W1),
                       static_cast<bf16_t*>(dXt), a.tile_expert, a.tile_row, a.expert_offsets,
                       a.totals, a.d, a.n, int(a.slot_cap));
  } else if (a.f32) dxt_launch<TileCfg<float, kTileM, 128, 2, 2, 3>>(a, dH, W1, dXt, st);
  else if (a.d % 512 == 0) dxt_launch<RowsWide>(a, dH, W1, dXt, st);
  else if (a.d % 256 == 0) dxt_launch<RowsMid>(a, dH, W1, dXt, st);
  else dxt_launch<RowsNarrow>(a, dH, W1, dXt, st);
  return hipGetLastError();
}

size_t varlen_ws_bytes(bool f32, int d, int n, int E, int64_t slot_cap) {
  return VarlenWs::make(dw1_dims(f32, d, n, E, slot_cap), dw2_dims(f32, d, n, E, slot_cap), E)
      .total;
}

hipError_t launch_dw_plan(const LayerArgs& a, void* vws, hipStream_t st) {
  const VarlenDims v1 = dw1_dims(a.f32, a.d, a.n, a.E, a.slot_cap);
  const VarlenDims v2 = dw2_dims(a.f32, a.d, a.n, a.E, a.slot_cap);
  const VarlenWs L = VarlenWs::make(v1, v2, a.E);
  char* w = static_cast<char*>(vws);
  int* hdr1 = reinterpret_cast<int*>(w + L.hdr1);
  int* hdr2 = reinterpret_cast<int*>(w + L.hdr2);
  auto* items1 = reinterpret_cast<VarlenItem*>(w + L.items1);
  auto* items2 = reinterpret_cast<VarlenItem*>(w + L.items2);
  hipLaunchKernelGGL(k_varlen_plan, dim3(1), dim3(kPlanThreads), 0, st, a.expert_offsets,
                     a.expert_order, a.E, v1.kc, v2.kc, hdr1, items1,
                     reinterpret_cast<VarlenSplit*>(w + L.splits1), hdr2, items2,
                     reinterpret_cast<VarlenSplit*>(w + L.splits2));
  if (v1.cap > 0 || v2.cap > 0)
    hipLaunchKernelGGL(k_dw_sched, dim3(2), dim3(kSchedThreads), 0, st, hdr1, items1, v1.PT,
                       v1.cap, reinterpret_cast<int*>(w + L.cnt1), reinterpret_cast<int*>(w + L.list1),
                       hdr2, items2, v2.PT, v2.cap, reinterpret_cast<int*>(w + L.cnt2),
                       reinterpret_cast<int*>(w + L.list2));
  return hipGetLastError();
}

hipError_t launch_dw1(const LayerArgs& a, const void* X, const void* dH, void* dW1, void* vws,
                      hipStream_t st) {
  const VarlenDims v1 = dw1_dims(a.f32, a.d, a.n, a.E, a.slot_cap);
  const VarlenDims v2 = dw2_dims(a.f32, a.d, a.n, a.E, a.slot_cap);
  const VarlenWs L = VarlenWs::make(v1, v2, a.E);
  char* w = static_cast<char*>(vws);
  int* hdr1 = reinterpret_cast<int*>(w + L.hdr1);
  auto* items1 = reinterpret_cast<VarlenItem*>(w + L.items1);
  auto* splits1 = reinterpret_cast<VarlenSplit*>(w + L.splits1);
  float* partials = reinterpret_cast<float*>(w + L.partials);
  dw1_cfg(a.f32, a.d, a.n, a.E, a.slot_cap, [&](auto tag) {
    using Cfg = typename decltype(tag)::type;
    using T = typename Cfg::T;
    if constexpr (Cfg::NPW > 0)
      hipLaunchKernelGGL((k_dw_p<Cfg, true, false>), dim3(kNumCUs), dim3(Cfg::kThreads), 0, st,
                         static_cast<const T*>(X), static_cast<const T*>(dH),
                         static_cast<T*>(dW1), partials, items1,
                         reinterpret_cast<const int*>(w + L.cnt1),
                         reinterpret_cast<const int*>(w + L.list1), v1.cap, a.slot_token, a.d,
                         2 * a.n, a.T, int(a.slot_cap), int(a.slot_cap));
    else
      hipLaunchKernelGGL((k_dw1<Cfg>), dim3(unsigned(8 * cdiv(v1.max_items, 8) * v1.PT)),
                         dim3(Cfg::kThreads), 0, st, static_cast<const T*>(X),
                         static_cast<const T*>(dH), static_cast<T*>(dW1), partials, hdr1, items1,
                         a.slot_token, a.d, a.n, a.T, int(a.slot_cap));
    reduce_launch<T>(hdr1, splits1, partials, dW1, v1, st);
  });
  return hipGetLastError();
}

hipError_t launch_dw2(const LayerArgs& a, const void* As, const void* dO, void* dW2, void* vws,
                      hipStream_t st) {
  const VarlenDims v1 = dw1_dims(a.f32, a.d, a.n, a.E, a.slot_cap);
  const VarlenDims v2 = dw2_dims(a.f32, a.d, a.n, a.E, a.slot_cap);
  const VarlenWs L = VarlenWs::make(v1, v2, a.E);
  char* w = static_cast<char*>(vws);
  int* hdr2 = reinterpret_cast<int*>(w + L.hdr2);
  auto* items2 = reinterpret_cast<VarlenItem*>(w + L.items2);
  auto* splits2 = reinterpret_cast<VarlenSplit*>(w + L.splits2);
  float* partials = reinterpret_cast<float*>(w + L.partials);
  dw2_cfg(a.f32, a.d, a.n, a.E, a.slot_cap, [&](auto tag) {
    using Cfg = typename decltype(tag)::type;
    using T = typename Cfg::T;
    if constexpr (Cfg::NPW > 0)
      hipLaunchKernelGGL((k_dw_p<Cfg, false, true>), dim3(kNumCUs), dim3(Cfg::kThreads), 0, st,
                         static_cast<const T*>(As), static_cast<const T*>(dO),
                         static_cast<T*>(dW2), partials, items2,
                         reinterpret_cast<const int*>(w + L.cnt2),
                         reinterpret_cast<const int*>(w + L.list2), v2.cap, a.slot_token, a.n,
                         a.d, int(a.slot_cap), a.T, int(a.slot_cap));
    else
      hipLaunchKernelGGL((k_dw2<Cfg>), dim3(unsigned(8 * cdiv(v2.max_items, 8) * v2.PT)),
                         dim3(Cfg::kThreads), 0, st, static_cast<const T*>(As),
                         static_cast<const T*>(dO), static_cast<T*>(dW2), partials, hdr2, items2,
                         a.slot_token, a.d, a.n, a.T, int(a.slot_cap));
    reduce_launch<T>(hdr2, splits2, partials, dW2, v2, st);
  });
  return hipGetLastError();
}

}  // namespace moe
