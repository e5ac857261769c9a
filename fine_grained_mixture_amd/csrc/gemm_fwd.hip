// Forward grouped GEMMs over the token-rounded slot layout.
//
// SonicMoE ICLR-2026 notes (papernotes.org), method > overall framework and
// key design 2: the up-projection gathers each expert's token rows straight
// from X into the GEMM operand (no separate gather pass) and applies SwiGLU
// in its epilogue; the down-projection is a plain varlen-M grouped GEMM.
//
//   k_up_swiglu   H_e = X[I_e] W1_e; A_e = SiLU(H_gate) * H_up  -> H, A
//   k_down        Y_e = A_e W2_e                               -> Y
//
// Both walk the device-side M-tile schedule written by the router (one tile
// = up to 128 slot rows of a single expert); surplus workgroups of the
// capacity-sized grid exit at once.
#include "gemm.hpp"
#include "internal.hpp"
#include "tiles.hpp"

namespace moe {
namespace {

// One workgroup computes a 128-row M tile against BN/2 gate columns and the
// matching BN/2 up columns, so SiLU(gate) * up is formed in registers.
// A = gathered X rows (K-major), B = W1_e columns (MN-major).
template <class Cfg, class T = typename Cfg::T>
__global__ __launch_bounds__(Cfg::kThreads) void k_up_swiglu(
    const T* __restrict__ X, const T* __restrict__ W1, T* __restrict__ H, T* __restrict__ Aact,
    const int32_t* __restrict__ tile_expert, const int32_t* __restrict__ tile_row,
    const int32_t* __restrict__ slot_token,
    const int32_t* __restrict__ totals, int d, int n, int ntok) {
  static_assert(Cfg::PAIRED && Cfg::BM == kTileM, "paired 128-row tiles");
  __shared__ __attribute__((aligned(1024))) char lds[Cfg::LDS_BYTES];
  constexpr int BN = Cfg::BN, HALF = BN / 2, EPC = 16 / int(sizeof(T));
  const int NT = n / HALF;
  const int lin = xcd_tile(blockIdx.x, totals[1] * NT);
  if (lin < 0) return;
  const int mt = lin / NT, nt = lin % NT;
  const int e = tile_expert[mt], row0 = tile_row[mt];
  const int rend = tile_end(tile_row, totals, mt, row0);
  const int j0 = nt * HALF, n2 = 2 * n;
  const int tok0 = slot_token[row0];

  const uint32_t xrow = uint32_t(d) * sizeof(T);
  KLoad<Cfg, kTileM> la;
  la.init(X, uint32_t(ntok) * xrow, [&](int r) {
    const int slot = row0 + r;
    return uint32_t(slot < rend ? slot_token[slot] : tok0) * xrow;
  });
  MNLoad<Cfg, BN> lb;
  lb.init(W1 + int64_t(e) * d * n2, uint32_t(d) * n2 * sizeof(T), uint32_t(n2) * sizeof(T),
          [=](int c) {
    const int ce = c * EPC;
    return int((ce < HALF ? j0 + ce : n + j0 + ce - HALF) * sizeof(T));
  });

  Accum<Cfg> acc;
  acc.init();
  pipeline<Cfg, true, false>(acc, lds, d / Cfg::BK, la, lb, NoTail{});

  // Epilogue: H (gate and up halves, rounded to T) and A = SiLU(g) * u from
  // the rounded values, staged per wave and written as whole rows.
  using St = RowStage<T, Cfg::WTN / 2>;
  static_assert(3 * St::BYTES * Cfg::NW <= Cfg::LDS_BYTES, "epilogue staging fits in LDS");
  char* wbuf = lds + wave_id() * 3 * St::BYTES;
  const St sg{wbuf}, su{wbuf + St::BYTES}, sa{wbuf + 2 * St::BYTES};
  const int r32 = acc.lane & 31, h = acc.lane >> 5;
  const int jw = j0 + Cfg::colblock(acc.wn, 0);  // first gate column of this wave
#pragma unroll
  for (int a = 0; a < Cfg::MB; ++a) {
#pragma unroll
    for (int b = 0; b < Cfg::NB / 2; ++b) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        T hg[4], hu[4], av[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float g = Elem<T>::round(acc.acc[a][b][q * 4 + c]);
          const float u = Elem<T>::round(acc.acc[a][b + Cfg::NB / 2][q * 4 + c]);
          hg[c] = Elem<T>::store(g);
          hu[c] = Elem<T>::store(u);
          av[c] = Elem<T>::store(g * sigmoidf_(g) * u);
        }
        const int col = b * 32 + q * 8 + h * 4;
        sg.put(r32, col, hg);
        su.put(r32, col, hu);
        sa.put(r32, col, av);
      }
    }
    const int rb = row0 + acc.wm * Cfg::WTM + a * 32;  // first slot of the block
    sg.flush([&](int r) -> T* { return rb + r < rend ? H + int64_t(rb + r) * n2 + jw : nullptr; });
    su.flush([&](int r) -> T* {
      return rb + r < rend ? H + int64_t(rb + r) * n2 + n + jw : nullptr;
    });
    sa.flush([&](int r) -> T* { return rb + r < rend ? Aact + int64_t(rb + r) * n + jw : nullptr; });
  }
}

// A = activation rows (K-major), B = W2_e columns (MN-major).
template <class Cfg, class T = typename Cfg::T>
__global__ __launch_bounds__(Cfg::kThreads) void k_down(
    const T* __restrict__ Aact, const T* __restrict__ W2, T* __restrict__ Y,
    const int32_t* __restrict__ tile_expert, const int32_t* __restrict__ tile_row,
    const int32_t* __restrict__ totals, int d,
    int n, int nslot) {
  static_assert(Cfg::BM == kTileM, "128-row tiles");
  __shared__ __attribute__((aligned(1024))) char lds[Cfg::LDS_BYTES];
  constexpr int BN = Cfg::BN, EPC = 16 / int(sizeof(T));
  const int NT = d / BN;
  const int lin = xcd_tile(blockIdx.x, totals[1] * NT);
  if (lin < 0) return;
  const int mt = lin / NT, nt = lin % NT;
  const int e = tile_expert[mt], row0 = tile_row[mt];
  const int rend = tile_end(tile_row, totals, mt, row0);
  const int j0 = nt * BN;

  const uint32_t arow = uint32_t(n) * sizeof(T);
  KLoad<Cfg, kTileM> la;
  la.init(Aact, uint32_t(nslot) * arow, [&](int r) {
    const int slot = row0 + r;
    return uint32_t(slot < rend ? slot : row0) * arow;
  });
  MNLoad<Cfg, BN> lb;
  lb.init(W2 + int64_t(e) * n * d, uint32_t(n) * d * sizeof(T), uint32_t(d) * sizeof(T),
          [=](int c) { return int((j0 + c * EPC) * sizeof(T)); });

  Accum<Cfg> acc;
  acc.init();
  pipeline<Cfg, true, false>(acc, lds, n / Cfg::BK, la, lb, NoTail{});

  static_assert(RowStage<T, Cfg::WTN>::BYTES * Cfg::NW <= Cfg::LDS_BYTES, "staging fits");
  store_acc_staged(acc, lds, [&](int r) -> T* {
    return row0 + r < rend ? Y + int64_t(row0 + r) * d + j0 : nullptr;
  });
}

// The down-projection as a persistent launch with loader waves (one
// workgroup per CU, Cfg::NPW > 0): the same tiles, each workgroup walking its
// share in turn, so the next tile's first slabs land while this tile's rows
// are written.
template <class Cfg, class T = typename Cfg::T>
__global__ __launch_bounds__(Cfg::kThreads) void k_down_p(
    const T* __restrict__ Aact, const T* __restrict__ W2, T* __restrict__ Y,
    const int32_t* __restrict__ tile_expert, const int32_t* __restrict__ tile_row,
    const int32_t* __restrict__ totals, int d, int n, int nslot) {
  static_assert(Cfg::BM == kTileM && Cfg::NPW > 0, "128-row tiles with loader waves");
  struct Tile {
    int e, row0, rend, j0;
  };
  __shared__ __attribute__((aligned(1024))) char lds[Cfg::LDS_BYTES];
  __shared__ __attribute__((aligned(16))) Tile table[kPersistentTiles];
  constexpr int BN = Cfg::BN, EPC = 16 / int(sizeof(T));
  const int NT = d / BN;
  const PersistentShare ps = PersistentShare::make(totals[1] * NT);
  if (ps.ntiles == 0 || ps.ntiles > kPersistentTiles) return;  // the host keeps it in range
  auto describe = [&](int k) {
    const int lin = ps.first + k * ps.stride;
    const int mt = lin / NT, nt = lin % NT;
    Tile t;
    t.e = tile_expert[mt];
    t.row0 = tile_row[mt];
    t.rend = tile_end(tile_row, totals, mt, t.row0);
    t.j0 = nt * BN;
    return t;
  };
  const uint32_t arow = uint32_t(n) * sizeof(T);
  auto loaders = [&](const Tile& t) {
    LoadPair<KLoad<Cfg, kTileM>, MNLoad<Cfg, BN>> p;
    p.la.init(Aact, uint32_t(nslot) * arow, [&](int r) {
      const int slot = t.row0 + r;
      return uint32_t(slot < t.rend ? slot : t.row0) * arow;
    });
    p.lb.init(W2 + int64_t(t.e) * n * d, uint32_t(n) * d * sizeof(T), uint32_t(d) * sizeof(T),
              [&](int c) { return int((t.j0 + c * EPC) * sizeof(T)); });
    return p;
  };
  auto epilogue = [&](const Tile& t, const Accum<Cfg>& acc, char* stage) {
    static_assert(RowStage<T, Cfg::WTN>::BYTES * Cfg::NW <= Cfg::STAGE_BYTES, "staging fits");
    store_acc_staged(acc, stage, [&](int r) -> T* {
      return t.row0 + r < t.rend ? Y + int64_t(t.row0 + r) * d + t.j0 : nullptr;
    });
  };
  persistent_split<Cfg, true, false>(lds, table, ps.ntiles, n / Cfg::BK, describe, loaders,
                                     epilogue);
}

inline unsigned grid_for(int64_t work) { return unsigned(((work + 7) / 8) * 8); }

template <class Cfg>
void up_launch(const LayerArgs& a, const void* X, const void* W1, void* H, void* Aact,
               hipStream_t st) {
  using T = typename Cfg::T;
  const int half = Cfg::BN / 2;
  hipLaunchKernelGGL((k_up_swiglu<Cfg>), dim3(grid_for(a.tile_cap * (a.n / half))),
                     dim3(Cfg::kThreads), 0, st, static_cast<const T*>(X),
                     static_cast<const T*>(W1), static_cast<T*>(H), static_cast<T*>(Aact),
                     a.tile_expert, a.tile_row, a.slot_token, a.totals, a.d,
                     a.n, a.T);
}

template <class Cfg>
void down_launch(const LayerArgs& a, const void* Aact, const void* W2, void* Y, hipStream_t st) {
  using T = typename Cfg::T;
  hipLaunchKernelGGL((k_down<Cfg>), dim3(grid_for(a.tile_cap * (a.d / Cfg::BN))),
                     dim3(Cfg::kThreads), 0, st, static_cast<const T*>(Aact),
                     static_cast<const T*>(W2), static_cast<T*>(Y), a.tile_expert, a.tile_row,
                     a.totals, a.d, a.n, int(a.slot_cap));
}

}  // namespace

hipError_t launch_up_swiglu(const LayerArgs& a, const void* X, const void* W1, void* H,
                            void* Aact, hipStream_t st) {
  if (a.f32) up_launch<TileCfg<float, kTileM, 128, 2, 2, 3, 128, true>>(a, X, W1, H, Aact, st);
  else if (a.n % 256 == 0) up_launch<UpWide>(a, X, W1, H, Aact, st);
  else if (a.n % 128 == 0) up_launch<UpMid>(a, X, W1, H, Aact, st);
  else up_launch<UpNarrow>(a, X, W1, H, Aact, st);
  return hipGetLastError();
}

hipError_t launch_down(const LayerArgs& a, const void* Aact, const void* W2, void* Y,
                       hipStream_t st) {
  using P = RowsSplit;
  if (!a.f32 && a.d % P::BN == 0 && a.n / P::BK >= P::STAGES - 1 &&
      PersistentShare::max_tiles(a.tile_cap * (a.d / P::BN), kNumCUs) <= kPersistentTiles) {
    hipLaunchKernelGGL((k_down_p<P>), dim3(kNumCUs), dim3(P::kThreads), 0, st,
                       static_cast<const bf16_t*>(Aact), static_cast<const bf16_t*>(W2),
                       static_cast<bf16_t*>(Y), a.tile_expert, a.tile_row, a.totals, a.d, a.n,
                       int(a.slot_cap));
  } else if (a.f32) down_launch<TileCfg<float, kTileM, 128, 2, 2, 3>>(a, Aact, W2, Y, st);
  else if (a.d % 512 == 0) down_launch<RowsWide>(a, Aact, W2, Y, st);
  else if (a.d % 256 == 0) down_launch<RowsMid>(a, Aact, W2, Y, st);
  else down_launch<RowsNarrow>(a, Aact, W2, Y, st);
  return hipGetLastError();
}

}  // namespace moe
