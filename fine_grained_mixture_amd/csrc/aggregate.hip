// Expert aggregation: O[t] = sum over t's slots of s * Y[slot] (forward), and
// dX[t] = sum over t's slots of dX~[slot] (backward).
//
// SonicMoE ICLR-2026 notes (papernotes.org), method > overall framework: the
// forward ends with an expert-aggregation kernel and the backward has a
// matching aggregation for dX.  Each token reads its slots through the
// token CSR written by the router, accumulates in fp32 and writes its row
// once; a token without slots gets a zero row.  Memory-bound: one wave per
// token, 16-byte loads, the token's slot ids and weights held in lanes and
// broadcast with shuffles so that several row loads are in flight at once.
#include "common.hpp"
#include "internal.hpp"

namespace moe {
namespace {

// One wave per token.  Lane l owns octets o0 + l + 64 i (i < OPL) of the row
// chunk starting at octet o0; the token's slot ids and weights sit in lanes
// (one slot per lane) and are broadcast with shuffles.  All SU x OPL row
// loads of a batch of SU slots are issued before any is used, so a wave has
// SU x OPL x 16 bytes per lane in flight (24 KB per wave for K = 8 and a
// 1536-wide bf16 row).  Each gathered row is read exactly once, so the loads
// are non-temporal.
template <class T, int OPL, int SU>
__global__ __launch_bounds__(256) void k_aggregate(
    const T* __restrict__ rows, const float* __restrict__ w,
    const int32_t* __restrict__ token_offsets, const int32_t* __restrict__ token_slots,
    T* __restrict__ out, int ntok, int width) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= ntok) return;
  const int beg = token_offsets[t], cnt = token_offsets[t + 1] - beg;
  const int nocts = width / 8;
  for (int o0 = 0; o0 < nocts; o0 += 64 * OPL) {
    float acc[OPL][8];
#pragma unroll
    for (int i = 0; i < OPL; ++i)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[i][c] = 0.0f;
    for (int base = 0; base < cnt; base += 64) {
      const int m = min(64, cnt - base);
      const int my_slot = lane < m ? token_slots[beg + base + lane] : 0;
      const float my_w = (lane < m && w) ? w[my_slot] : 1.0f;
      for (int j = 0; j < m; j += SU) {
        Oct<T> v[SU][OPL];
#pragma unroll
        for (int u = 0; u < SU; ++u) {
          const int slot = __shfl(my_slot, j + u, 64);
#pragma unroll
          for (int i = 0; i < OPL; ++i) {
            const int o = o0 + lane + 64 * i;
            if (j + u < m && o < nocts) oct_load_nt(v[u][i], rows + int64_t(slot) * width + o * 8);
            else oct_zero(v[u][i]);
          }
        }
#pragma unroll
        for (int u = 0; u < SU; ++u) {
          const float s = __shfl(my_w, j + u, 64);
          if (j + u < m) {
#pragma unroll
            for (int i = 0; i < OPL; ++i)
#pragma unroll
              for (int c = 0; c < 8; ++c) acc[i][c] += s * oct_get(v[u][i], c);
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < OPL; ++i) {
      const int o = o0 + lane + 64 * i;
      if (o < nocts) {
        Oct<T> r;
        oct_from(r, acc[i]);
        oct_store(out + int64_t(t) * width + o * 8, r);
      }
    }
  }
}

template <class T, int OPL, int SU>
void aggregate_launch(const LayerArgs& a, const void* rows, const float* w, void* out, int width,
                      hipStream_t st) {
  hipLaunchKernelGGL((k_aggregate<T, OPL, SU>), dim3((a.T + 3) / 4), dim3(256), 0, st,
                     static_cast<const T*>(rows), w, a.token_offsets, a.token_slots,
                     static_cast<T*>(out), a.T, width);
}

// Octets per lane from the row width; the slot batch keeps the loads in
// flight per lane near 24 to 32 octets (bf16) or 12 to 16 (fp32).
template <class T>
void aggregate_dispatch(const LayerArgs& a, const void* rows, const float* w, void* out,
                        int width, hipStream_t st) {
  constexpr int F = sizeof(T) == 2 ? 1 : 2;  // fp32 octets are twice as wide
  const int opl = (width / 8 + 63) / 64;
  if (opl <= 1) aggregate_launch<T, 1, 16 / F>(a, rows, w, out, width, st);
  else if (opl == 2) aggregate_launch<T, 2, 8 / F>(a, rows, w, out, width, st);
  else if (opl == 3) aggregate_launch<T, 3, 8 / F>(a, rows, w, out, width, st);
  else if (opl == 4) aggregate_launch<T, 4, 8 / F>(a, rows, w, out, width, st);
  else aggregate_launch<T, 8, 4 / F>(a, rows, w, out, width, st);
}

}  // namespace

hipError_t launch_aggregate(const LayerArgs& a, const void* rows, bool weighted, void* out,
                            int width, hipStream_t st) {
  const float* w = weighted ? a.slot_weight : nullptr;
  if (a.f32) aggregate_dispatch<float>(a, rows, w, out, width, st);
  else aggregate_dispatch<bf16_t>(a, rows, w, out, width, st);
  return hipGetLastError();
}

}  // namespace moe
