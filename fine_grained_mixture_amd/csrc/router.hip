// Router of the MoE layer: its forward (the scores the routing step reads)
// and its backward (from the gate-weight gradients dS of the layer).
//
// SonicMoE ICLR-2026 notes (papernotes.org), method > overall framework and
// key design 1: every token is routed by its router scores; the notes list
// the router gradients among what the layer's backward produces.  The router
// is a linear map with one row per expert, Wr [E, d]:
//
//   k_router_logits   l = X Wr^T                                  (fp32 out)
//   k_router_dlogits  p = softmax(l); g[t, e] = dS of the slot of (t, e), 0 if
//                     the pair is not kept; dl = p * (g - <p, g>)
//   k_router_dx       dX += dl Wr          (the router's share of the input
//                                           gradient, added to the experts')
//   k_router_dw       fp32 partials of dWr = dl^T X over chunks of tokens
//   k_router_reduce   dWr = sum of the partials, in chunk order
//
// The GEMMs use the same LDS-pipelined MFMA tiles as the expert GEMMs.  dl is
// kept twice: fp32 for the caller, and in the operand type with its rows
// padded by zeros to Ep = E rounded up to 128 for the two GEMMs.
#include "common.hpp"
#include "gemm.hpp"
#include "internal.hpp"

namespace moe {
namespace {

// dX and dWr: two stages (64 KB of LDS), so two workgroups share a CU; the
// dX contraction is only Ep deep and the dWr chunks a few slabs each
template <class T>
using RouterCfg = TileCfg<T, 128, 128, 2, 2, 2, 128>;
// logits: 64-token tiles, so that a 16k-token batch fills every CU
template <class T>
using LogitsCfg = TileCfg<T, 64, 128, 1, 4, 3, 128>;

// l[t, e] = sum_i X[t, i] Wr[e, i]: A = X rows, B = Wr rows (both K-major).
// Rows of Wr past E lie past the end of its buffer and read as zeros.
template <class Cfg, class T = typename Cfg::T>
__global__ __launch_bounds__(Cfg::kThreads) void k_router_logits(
    const T* __restrict__ X, const T* __restrict__ Wr, float* __restrict__ logits, int Tn, int d,
    int E) {
  __shared__ __attribute__((aligned(1024))) char lds[Cfg::LDS_BYTES];
  constexpr int BM = Cfg::BM, BN = Cfg::BN;
  const int NE = (E + BN - 1) / BN;
  const int mt = blockIdx.x / NE, nt = blockIdx.x % NE;
  const int t0 = mt * BM, e0 = nt * BN;
  const uint32_t row = uint32_t(d) * sizeof(T);
  KLoad<Cfg, BM> la;
  la.init(X, uint32_t(Tn) * row, [&](int r) { return uint32_t(min(t0 + r, Tn - 1)) * row; });
  KLoad<Cfg, BN> lb;
  lb.init(Wr, uint32_t(E) * row, [&](int c) { return uint32_t(e0 + c) * row; });
  Accum<Cfg> acc;
  acc.init();
  pipeline<Cfg, true, true>(acc, lds, d / Cfg::BK, la, lb, NoTail{});
#pragma unroll
  for (int a = 0; a < Cfg::MB; ++a) {
    const int t = t0 + acc.row(a);
    if (t >= Tn) continue;
#pragma unroll
    for (int b = 0; b < Cfg::NB; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int e = e0 + acc.col(b, q) + c;
          if (e < E) logits[int64_t(t) * E + e] = acc.acc[a][b][q * 4 + c];
        }
  }
}

// One wave per token; lane l holds experts e = l + 64 j, j < EPL = Ep / 64.
// The slot ids of the token come from the token CSR; the expert of a slot is
// found by binary search in the expert offsets (staged in LDS).  The logits
// are read through a buffer descriptor (positions past E read 0 and are
// masked), so all EPL loads of a lane are in flight together.
constexpr int kDlThreads = 256;

template <class T, int EPL>
__global__ __launch_bounds__(kDlThreads) void k_router_dlogits(
    const float* __restrict__ logits, const float* __restrict__ dS,
    const int32_t* __restrict__ token_offsets, const int32_t* __restrict__ token_slots,
    const int32_t* __restrict__ expert_offsets, float* __restrict__ dlogits,
    T* __restrict__ dlp, int Tn, int E, int Ep) {
  __shared__ int off[1025];
  __shared__ float g[kDlThreads / 64][64 * EPL];
  for (int i = threadIdx.x; i <= E; i += kDlThreads) off[i] = expert_offsets[i];
  // the wave index read into a scalar register, so that the token (and the
  // buffer descriptor over its row) is known to be uniform across the wave
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
  const int t = blockIdx.x * (kDlThreads / 64) + w;
  const bool valid = t < Tn;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(logits + int64_t(valid ? t : 0) * E), 0, E * 4, 0x00020000);
  float x[EPL], p[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    x[j] = finite_logit(
        __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, uint32_t(e) * 4u, 0, 0)));
    g[w][e] = 0.0f;
  }
  __syncthreads();  // off[] staged (g is per wave)
  if (!valid) return;
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    if (lane + 64 * j >= E) x[j] = -INFINITY;
    m = fmaxf(m, x[j]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  float z = 0.0f;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    p[j] = lane + 64 * j < E ? __expf(x[j] - m) : 0.0f;
    z += p[j];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) z += __shfl_xor(z, o, 64);
  const float rz = 1.0f / z;
  asm volatile("" ::: "memory");  // zeros of g before the scatter (one wave, in order)
  const int beg = token_offsets[t], cnt = token_offsets[t + 1] - beg;
  for (int i = lane; i < cnt; i += 64) {
    const int slot = token_slots[beg + i];
    int lo = 0, hi = E;  // the expert e with off[e] <= slot < off[e + 1]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (off[mid] <= slot) lo = mid;
      else hi = mid;
    }
    g[w][lo] = dS[slot];
  }
  asm volatile("" ::: "memory");
  float dot = 0.0f;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    p[j] *= rz;
    dot += p[j] * g[w][lane + 64 * j];  // p = 0 past E
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) dot += __shfl_xor(dot, o, 64);
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    const float v = e < E ? p[j] * (g[w][e] - dot) : 0.0f;  // rows padded with zeros to Ep
    if (e < E) dlogits[int64_t(t) * E + e] = v;
    if (dlp) dlp[int64_t(t) * Ep + e] = Elem<T>::store(v);
  }
}

// dX[t, j] += sum_e dl[t, e] Wr[e, j]: A = padded dl rows (K-major over Ep),
// B = Wr (MN-major, rows e; rows past E read as zeros).
template <class Cfg, class T = typename Cfg::T>
__global__ __launch_bounds__(Cfg::kThreads) void k_router_dx(
    const T* __restrict__ dlp, const T* __restrict__ Wr, T* __restrict__ dX, int Tn, int d, int E,
    int Ep) {
  __shared__ __attribute__((aligned(1024))) char lds[Cfg::LDS_BYTES];
  constexpr int BM = Cfg::BM, BN = Cfg::BN, EPC = 16 / int(sizeof(T));
  const int ND = d / BN;
  const int mt = blockIdx.x / ND, nt = blockIdx.x % ND;
  const int t0 = mt * BM, j0 = nt * BN;
  const uint32_t prow = uint32_t(Ep) * sizeof(T);
  KLoad<Cfg, BM> la;
  la.init(dlp, uint32_t(Tn) * prow, [&](int r) { return uint32_t(min(t0 + r, Tn - 1)) * prow; });
  MNLoad<Cfg, BN> lb;
  lb.init(Wr, uint32_t(E) * d * sizeof(T), uint32_t(d) * sizeof(T),
          [=](int c) { return int((j0 + c * EPC) * sizeof(T)); });
  Accum<Cfg> acc;
  acc.init();
  pipeline<Cfg, true, false>(acc, lds, Ep / Cfg::BK, la, lb, NoTail{});
  // Read-modify-write of dX through the per-wave staging buffer: whole rows
  // in, each lane adds its accumulators to its four columns, whole rows out.
  using St = RowStage<T, Cfg::WTN>;
  static_assert(St::BYTES * Cfg::NW <= Cfg::LDS_BYTES, "staging fits");
  const St stg{lds + wave_id() * St::BYTES};
  const int r32 = acc.lane & 31, h = acc.lane >> 5;
  const int cw = j0 + Cfg::colblock(acc.wn, 0);
#pragma unroll
  for (int a = 0; a < Cfg::MB; ++a) {
    const int rb = t0 + acc.wm * Cfg::WTM + a * 32;
    auto rows = [&](int r) -> T* { return rb + r < Tn ? dX + int64_t(rb + r) * d + cw : nullptr; };
    stg.fill(rows);
#pragma unroll
    for (int b = 0; b < Cfg::NB; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = b * 32 + q * 8 + h * 4;
        T v[4];
        stg.get(r32, col, v);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          v[c] = Elem<T>::store(Elem<T>::load(v[c]) + acc.acc[a][b][q * 4 + c]);
        stg.put(r32, col, v);
      }
    stg.flush(rows);
  }
}

// fp32 partial of dWr[e, i] = sum over tokens t of chunk c of dl[t, e] X[t, i]:
// both operands MN-major with token rows; tile rows e (over Ep), columns i.
template <class Cfg, class T = typename Cfg::T>
__global__ __launch_bounds__(Cfg::kThreads) void k_router_dw(
    const T* __restrict__ dlp, const T* __restrict__ X, float* __restrict__ partials, int Tn,
    int d, int Ep, int kc) {
  __shared__ __attribute__((aligned(1024))) char lds[Cfg::LDS_BYTES];
  constexpr int BM = Cfg::BM, BN = Cfg::BN, EPC = 16 / int(sizeof(T));
  const int TD = d / BN, PT = (Ep / BM) * TD;
  const int chunk = blockIdx.x / PT, tile = blockIdx.x % PT;
  const int i0 = (tile / TD) * BM, j0 = (tile % TD) * BN;
  const int kb = chunk * kc, ke = min(kb + kc, Tn);
  const int nslabs = (ke - kb + Cfg::BK - 1) / Cfg::BK;
  SlotLoad<Cfg, BM, false> la;
  la.init(dlp, uint32_t(Tn) * Ep * sizeof(T), uint32_t(Ep) * sizeof(T),
          [=](int c) { return int((i0 + c * EPC) * sizeof(T)); }, nullptr, kb, ke);
  SlotLoad<Cfg, BN, false> lb;
  lb.init(X, uint32_t(Tn) * d * sizeof(T), uint32_t(d) * sizeof(T),
          [=](int c) { return int((j0 + c * EPC) * sizeof(T)); }, nullptr, kb, ke);
  Accum<Cfg> acc;
  acc.init();
  VarlenTail<Cfg, BM, BN> tail{nslabs, ke - kb - (nslabs - 1) * Cfg::BK};
  pipeline<Cfg, false, false>(acc, lds, nslabs, la, lb, tail);
  float* out = partials + (int64_t(chunk) * Ep + i0) * d + j0;
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
        *reinterpret_cast<u32x4_t*>(out + int64_t(acc.row(a)) * d + acc.col(b, q)) = v;
      }
}

// dWr[e, i] = sum over chunks (in order) of the partials, rows e < E; four
// consecutive elements per thread, four chunks' loads in flight at a time.
template <class T>
__global__ __launch_bounds__(256) void k_router_reduce(const float* __restrict__ partials,
                                                       T* __restrict__ dWr, int E, int Ep, int d,
                                                       int nchunks) {
  const int64_t n4 = int64_t(E) * d / 4, stride = int64_t(Ep) * d;
  for (int64_t i4 = int64_t(blockIdx.x) * 256 + threadIdx.x; i4 < n4;
       i4 += int64_t(gridDim.x) * 256) {
    float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int c0 = 0; c0 < nchunks; c0 += 4) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        v[u] = c0 + u < nchunks ? reinterpret_cast<const float4*>(partials + (c0 + u) * stride)[i4]
                                : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
      for (int u = 0; u < 4; ++u) {  // chunk order
        s[0] += v[u].x; s[1] += v[u].y; s[2] += v[u].z; s[3] += v[u].w;
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) dWr[4 * i4 + c] = Elem<T>::store(s[c]);
  }
}

}  // namespace

RouterDims router_dims(int Tn, int d, int E, bool f32) {
  RouterDims r;
  r.Ep = (E + 127) / 128 * 128;
  const int BK = f32 ? 32 : 64;
  const int tiles = (r.Ep / 128) * (d / 128);          // output tiles of dWr
  int nch = std::max(1, (2 * kNumCUs + tiles - 1) / tiles);  // about two waves of tiles
  nch = std::min(nch, std::max(1, (Tn + 4 * BK - 1) / (4 * BK)));  // at least 4 slabs each
  r.kc = ((Tn + nch - 1) / nch + BK - 1) / BK * BK;
  r.nchunks = (Tn + r.kc - 1) / r.kc;
  const size_t es = f32 ? 4 : 2;
  r.dlp_bytes = (size_t(Tn) * r.Ep * es + 255) & ~size_t(255);
  r.ws_bytes = r.dlp_bytes + size_t(r.nchunks) * r.Ep * d * 4;
  return r;
}

template <class T>
hipError_t router_fwd_t(const void* X, const void* Wr, float* logits, int Tn, int d, int E,
                        hipStream_t st) {
  using Cfg = LogitsCfg<T>;
  const int grid = ((Tn + Cfg::BM - 1) / Cfg::BM) * ((E + Cfg::BN - 1) / Cfg::BN);
  hipLaunchKernelGGL((k_router_logits<Cfg>), dim3(grid), dim3(Cfg::kThreads), 0, st,
                     static_cast<const T*>(X), static_cast<const T*>(Wr), logits, Tn, d, E);
  return hipGetLastError();
}

hipError_t launch_router_fwd(bool f32, const void* X, const void* Wr, float* logits, int Tn,
                             int d, int E, hipStream_t st) {
  return f32 ? router_fwd_t<float>(X, Wr, logits, Tn, d, E, st)
             : router_fwd_t<bf16_t>(X, Wr, logits, Tn, d, E, st);
}

template <class T>
hipError_t router_bwd_t(const RouterBwdArgs& a, hipStream_t st, const TraceHook& tr) {
  using Cfg = RouterCfg<T>;
  const RouterDims r = router_dims(a.T, a.d, a.E, sizeof(T) == 4);
  char* w = static_cast<char*>(a.ws);
  T* dlp = reinterpret_cast<T*>(w);
  float* partials = reinterpret_cast<float*>(w + r.dlp_bytes);
  tr.mark(st, 0);
#define MOE_DLOGITS(EPL)                                                                    \
  hipLaunchKernelGGL((k_router_dlogits<T, EPL>), dim3((a.T + 3) / 4), dim3(kDlThreads), 0, st, \
                     a.logits, a.dS, a.token_offsets, a.token_slots, a.expert_offsets,        \
                     a.dlogits, dlp, a.T, a.E, r.Ep)
  switch (r.Ep / 64) {  // Ep is a multiple of 128, at most 1024
    case 2: MOE_DLOGITS(2); break;
    case 4: MOE_DLOGITS(4); break;
    case 6: MOE_DLOGITS(6); break;
    case 8: MOE_DLOGITS(8); break;
    case 10: MOE_DLOGITS(10); break;
    case 12: MOE_DLOGITS(12); break;
    case 14: MOE_DLOGITS(14); break;
    default: MOE_DLOGITS(16); break;
  }
#undef MOE_DLOGITS
  tr.mark(st, 1);
  hipLaunchKernelGGL((k_router_dx<Cfg>), dim3(((a.T + Cfg::BM - 1) / Cfg::BM) * (a.d / Cfg::BN)),
                     dim3(Cfg::kThreads), 0, st, dlp, static_cast<const T*>(a.Wr),
                     static_cast<T*>(a.dX), a.T, a.d, a.E, r.Ep);
  tr.mark(st, 2);
  hipLaunchKernelGGL((k_router_dw<Cfg>),
                     dim3(r.nchunks * (r.Ep / Cfg::BM) * (a.d / Cfg::BN)), dim3(Cfg::kThreads),
                     0, st, dlp, static_cast<const T*>(a.X), partials, a.T, a.d, r.Ep, r.kc);
  tr.mark(st, 3);
  const int64_t n4 = int64_t(a.E) * a.d / 4;  // d is a multiple of 128
  hipLaunchKernelGGL((k_router_reduce<T>), dim3(unsigned(std::min<int64_t>((n4 + 255) / 256, 4096))),
                     dim3(256), 0, st, partials, static_cast<T*>(a.dWr), a.E, r.Ep, a.d,
                     r.nchunks);
  tr.mark(st, 4);
  return hipGetLastError();
}

hipError_t launch_gate_bwd(const float* logits, const float* dS, const int32_t* token_offsets,
                           const int32_t* token_slots, const int32_t* expert_offsets,
                           float* dlogits, int Tn, int E, hipStream_t st) {
  const int Ep = (E + 127) / 128 * 128;
#define MOE_DLOGITS(EPL)                                                                      \
  hipLaunchKernelGGL((k_router_dlogits<float, EPL>), dim3((Tn + 3) / 4), dim3(kDlThreads), 0, st, \
                     logits, dS, token_offsets, token_slots, expert_offsets, dlogits,           \
                     static_cast<float*>(nullptr), Tn, E, Ep)
  switch (Ep / 64) {  // Ep is a multiple of 128, at most 1024
    case 2: MOE_DLOGITS(2); break;
    case 4: MOE_DLOGITS(4); break;
    case 6: MOE_DLOGITS(6); break;
    case 8: MOE_DLOGITS(8); break;
    case 10: MOE_DLOGITS(10); break;
    case 12: MOE_DLOGITS(12); break;
    case 14: MOE_DLOGITS(14); break;
    default: MOE_DLOGITS(16); break;
  }
#undef MOE_DLOGITS
  return hipGetLastError();
}

hipError_t launch_router_bwd(const RouterBwdArgs& a, hipStream_t st, const TraceHook& tr) {
  return a.f32 ? router_bwd_t<float>(a, st, tr) : router_bwd_t<bf16_t>(a, st, tr);
}

}  // namespace moe
