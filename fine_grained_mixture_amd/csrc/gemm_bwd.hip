// Backward grouped GEMMs of the minimal-activation backward.
//
// SonicMoE ICLR-2026 notes (papernotes.org), key designs 2 and 3: only X, H
// and the routing metadata survive the forward.  The dH kernel gathers dO
// rows into its operand load and, in its epilogue, reloads H, recomputes
// A = SwiGLU(H), and forms dS = <dA', A> together with dSwiGLU, so neither Y
// nor dY is ever needed.  The weight gradients are varlen-K grouped GEMMs:
// the contraction runs over each expert's own (gathered) token rows.
//
//   k_dh    dA' = dO[I_e] W2_e^T; dS, dH, s*A in the epilogue
//   k_dxt   dX~_e = dH_e W1_e^T
//   k_dw1   dW1_e = X[I_e]^T dH_e        (varlen-K)
//   k_dw2   dW2_e = (s*A)_e^T dO[I_e]    (varlen-K)
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
    const int32_t* __restrict__ expert_offsets, const int32_t* __restrict__ slot_token,
    const float* __restrict__ slot_weight, const int32_t* __restrict__ totals, int d, int ntok) {
  __shared__ __attribute__((aligned(1024))) char lds[Cfg::LDS_BYTES];
  constexpr int BM = Cfg::BM, BN = Cfg::BN, WGN = Cfg::WGN;
  constexpr int n = BN, n2 = 2 * BN, SUB = kTileM / BM;
  const int lin = xcd_tile(blockIdx.x, totals[1] * SUB);
  if (lin < 0) return;
  const int mt = lin / SUB;
  const int e = tile_expert[mt], row0 = tile_row[mt] + (lin % SUB) * BM;
  const int rend = expert_offsets[e + 1];
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
    const float s = slot_weight[srow];
    const T* hrow = H + int64_t(srow) * n2;
    float part = 0.0f;
    T out[3][Cfg::NB][4][4];  // dH gate, dH up, s * A
#pragma unroll
    for (int b = 0; b < Cfg::NB; ++b) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = acc.col(b, q);
        T g4[4], u4[4];
        __builtin_memcpy(g4, hrow + j, sizeof(g4));
        __builtin_memcpy(u4, hrow + n + j, sizeof(u4));
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float x = acc.acc[a][b][q * 4 + c];  // dA'
          const float g = Elem<T>::load(g4[c]), u = Elem<T>::load(u4[c]);
          const float sg = sigmoidf_(g), silu = g * sg;
          const float av = silu * u;
          part += x * av;
          const float da = s * x;
          out[0][b][q][c] = Elem<T>::store(da * u * sg * (1.0f + g * (1.0f - sg)));
          out[1][b][q][c] = Elem<T>::store(da * silu);
          out[2][b][q][c] = Elem<T>::store(s * av);
        }
      }
    }
    const int rb = row0 + acc.wm * Cfg::WTM + a * 32;
    auto flush = [&](int o) {
      T* base = o == 0 ? dH + cw : o == 1 ? dH + n + cw : As + cw;
      const int ld = o == 2 ? n : n2;
      stg[o].flush(
          [&](int r) -> T* { return rb + r < rend ? base + int64_t(rb + r) * ld : nullptr; });
    };
#pragma unroll
    for (int o = 0; o < 3; ++o) {
#pragma unroll
      for (int b = 0; b < Cfg::NB; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q) stg[o].put(r32, b * 32 + q * 8 + h * 4, out[o][b][q]);
      if constexpr (!kAll) flush(o);
    }
    if constexpr (kAll) {
#pragma unroll
      for (int o = 0; o < 3; ++o) flush(o);
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
  const int mt = lin / NT, nt = lin % NT;
  const int e = tile_expert[mt], row0 = tile_row[mt], rend = expert_offsets[e + 1];
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

// Varlen-K scheduling: expert_order lists experts by descending slot count.
// Ranks q are dealt round-robin to the 8 XCDs (block b runs on XCD b % 8),
// and all PT output tiles of one expert stay on one XCD, so its gathered rows
// are fetched into one L2; the largest experts start first.
__device__ __forceinline__ bool varlen_k_tile(int b, int PT, int E, const int32_t* order,
                                              int* e, int* tile) {
  const int xcd = b % 8, local = b / 8;
  const int q = (local / PT) * 8 + xcd;
  if (q >= E) return false;
  *e = order[q];
  *tile = local % PT;
  return true;
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

// Zeroes the rows past the expert's last slot in the final, partial slab of
// a varlen-K contraction (those rows were read from the last valid slot).
template <class Cfg, int ACOLS, int BCOLS>
struct VarlenTail {
  int nslabs, valid;
  __device__ __forceinline__ void operator()(int s, char* stage) const {
    if (s != nslabs - 1 || valid == Cfg::BK) return;
    zero_rows<Cfg, ACOLS>(stage, valid);
    zero_rows<Cfg, BCOLS>(stage + Cfg::A_BYTES, valid);
    wait_lgkm0();
    barrier();
  }
};

// dW1_e[i][j] = sum over the expert's slots k of X[tok_k][i] * dH[k][j]:
// both operands MN-major, rows = slots (X rows gathered through slot_token).
template <class Cfg, class T = typename Cfg::T>
__global__ __launch_bounds__(Cfg::kThreads) void k_dw1(
    const T* __restrict__ X, const T* __restrict__ dH, T* __restrict__ dW1,
    const int32_t* __restrict__ expert_order, const int32_t* __restrict__ expert_offsets,
    const int32_t* __restrict__ slot_token, int E, int d, int n, int ntok, int nslot) {
  __shared__ __attribute__((aligned(1024))) char lds[Cfg::LDS_BYTES];
  constexpr int BM = Cfg::BM, BN = Cfg::BN, EPC = 16 / int(sizeof(T));
  const int n2 = 2 * n, TN = n2 / BN, PT = (d / BM) * TN;
  int e, tile;
  if (!varlen_k_tile(blockIdx.x, PT, E, expert_order, &e, &tile)) return;
  const int i0 = (tile / TN) * BM, j0 = (tile % TN) * BN;
  const int kb = expert_offsets[e], ke = expert_offsets[e + 1];
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
  store_tile(acc, lds, dW1 + (int64_t(e) * d + i0) * n2 + j0, n2);
}

// dW2_e[i][j] = sum over the expert's slots k of As[k][i] * dO[tok_k][j].
template <class Cfg, class T = typename Cfg::T>
__global__ __launch_bounds__(Cfg::kThreads) void k_dw2(
    const T* __restrict__ As, const T* __restrict__ dO, T* __restrict__ dW2,
    const int32_t* __restrict__ expert_order, const int32_t* __restrict__ expert_offsets,
    const int32_t* __restrict__ slot_token, int E, int d, int n, int ntok, int nslot) {
  __shared__ __attribute__((aligned(1024))) char lds[Cfg::LDS_BYTES];
  constexpr int BM = Cfg::BM, BN = Cfg::BN, EPC = 16 / int(sizeof(T));
  const int TN = d / BN, PT = (n / BM) * TN;
  int e, tile;
  if (!varlen_k_tile(blockIdx.x, PT, E, expert_order, &e, &tile)) return;
  const int i0 = (tile / TN) * BM, j0 = (tile % TN) * BN;
  const int kb = expert_offsets[e], ke = expert_offsets[e + 1];
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
  store_tile(acc, lds, dW2 + (int64_t(e) * n + i0) * d + j0, d);
}

template <class Cfg>
void dh_launch(const LayerArgs& a, const void* dO, const void* W2, const void* H, void* dH,
               void* As, float* dS, hipStream_t st) {
  using T = typename Cfg::T;
  hipLaunchKernelGGL((k_dh<Cfg>), dim3(grid_for(a.tile_cap * (kTileM / Cfg::BM))),
                     dim3(Cfg::kThreads), 0, st, static_cast<const T*>(dO),
                     static_cast<const T*>(W2), static_cast<const T*>(H), static_cast<T*>(dH),
                     static_cast<T*>(As), dS, a.tile_expert, a.tile_row, a.expert_offsets,
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

inline unsigned varlen_k_grid(int E, int PT) { return unsigned(8 * ((E + 7) / 8) * PT); }

template <class Cfg>
void dw1_launch(const LayerArgs& a, const void* X, const void* dH, void* dW1, hipStream_t st) {
  using T = typename Cfg::T;
  hipLaunchKernelGGL((k_dw1<Cfg>),
                     dim3(varlen_k_grid(a.E, (a.d / Cfg::BM) * (2 * a.n / Cfg::BN))),
                     dim3(Cfg::kThreads), 0, st, static_cast<const T*>(X),
                     static_cast<const T*>(dH), static_cast<T*>(dW1), a.expert_order,
                     a.expert_offsets, a.slot_token, a.E, a.d, a.n, a.T,
                     int(a.slot_cap));
}

template <class Cfg>
void dw2_launch(const LayerArgs& a, const void* As, const void* dO, void* dW2, hipStream_t st) {
  using T = typename Cfg::T;
  hipLaunchKernelGGL((k_dw2<Cfg>), dim3(varlen_k_grid(a.E, (a.n / Cfg::BM) * (a.d / Cfg::BN))),
                     dim3(Cfg::kThreads), 0, st, static_cast<const T*>(As),
                     static_cast<const T*>(dO), static_cast<T*>(dW2), a.expert_order,
                     a.expert_offsets, a.slot_token, a.E, a.d, a.n, a.T,
                     int(a.slot_cap));
}

}  // namespace

hipError_t launch_dh(const LayerArgs& a, const void* dO, const void* W2, const void* H, void* dH,
                     void* As, float* dS, hipStream_t st) {
  return a.f32 ? dh_t<float>(a, dO, W2, H, dH, As, dS, st)
               : dh_t<bf16_t>(a, dO, W2, H, dH, As, dS, st);
}

hipError_t launch_dxt(const LayerArgs& a, const void* dH, const void* W1, void* dXt,
                      hipStream_t st) {
  if (a.f32) dxt_launch<TileCfg<float, kTileM, 128, 2, 2, 3>>(a, dH, W1, dXt, st);
  else if (a.d % 512 == 0) dxt_launch<RowsWide>(a, dH, W1, dXt, st);
  else if (a.d % 256 == 0) dxt_launch<RowsMid>(a, dH, W1, dXt, st);
  else dxt_launch<RowsNarrow>(a, dH, W1, dXt, st);
  return hipGetLastError();
}

hipError_t launch_dw1(const LayerArgs& a, const void* X, const void* dH, void* dW1,
                      hipStream_t st) {
  const int n2 = 2 * a.n;
  if (a.f32) dw1_launch<TileCfg<float, 128, 128, 2, 2, 3>>(a, X, dH, dW1, st);
  else if (a.d % 256 == 0 && n2 % 256 == 0) dw1_launch<GradSquare>(a, X, dH, dW1, st);
  else if (n2 % 256 == 0) dw1_launch<GradTall>(a, X, dH, dW1, st);
  else dw1_launch<GradSmall>(a, X, dH, dW1, st);
  return hipGetLastError();
}

hipError_t launch_dw2(const LayerArgs& a, const void* As, const void* dO, void* dW2,
                      hipStream_t st) {
  if (a.f32) {
    if (a.n % 128 == 0) dw2_launch<TileCfg<float, 128, 128, 2, 2, 3>>(a, As, dO, dW2, st);
    else dw2_launch<TileCfg<float, 64, 128, 2, 2, 3>>(a, As, dO, dW2, st);
  } else if (a.n % 256 == 0 && a.d % 256 == 0) {
    dw2_launch<GradSquare>(a, As, dO, dW2, st);
  } else if (a.n % 128 == 0 && a.d % 256 == 0) {
    dw2_launch<GradTall>(a, As, dO, dW2, st);
  } else if (a.n % 128 == 0) {
    dw2_launch<GradSmall>(a, As, dO, dW2, st);
  } else {
    dw2_launch<TileCfg<bf16_t, 64, 128, 2, 2, 3>>(a, As, dO, dW2, st);
  }
  return hipGetLastError();
}

}  // namespace moe
