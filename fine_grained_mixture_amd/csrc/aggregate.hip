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

constexpr int kAggUnroll = 4;

template <class T>
__global__ __launch_bounds__(256) void k_aggregate(
    const T* __restrict__ rows, const float* __restrict__ w,
    const int32_t* __restrict__ token_offsets, const int32_t* __restrict__ token_slots,
    T* __restrict__ out, int ntok, int width) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= ntok) return;
  const int beg = token_offsets[t], cnt = token_offsets[t + 1] - beg;
  const int nocts = width / 8;
  for (int o = lane; o < nocts; o += 64) {
    float acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = 0.0f;
    for (int base = 0; base < cnt; base += 64) {
      const int m = min(64, cnt - base);
      const int my_slot = lane < m ? token_slots[beg + base + lane] : 0;
      const float my_w = (lane < m && w) ? w[my_slot] : 1.0f;
      for (int j = 0; j < m; j += kAggUnroll) {
        Oct<T> v[kAggUnroll];
        float s[kAggUnroll];
#pragma unroll
        for (int u = 0; u < kAggUnroll; ++u) {
          const int slot = __shfl(my_slot, j + u, 64);
          s[u] = __shfl(my_w, j + u, 64);
          if (j + u < m) oct_load(v[u], rows + int64_t(slot) * width + o * 8);
          else oct_zero(v[u]);
        }
#pragma unroll
        for (int u = 0; u < kAggUnroll; ++u)
          if (j + u < m)
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[c] += s[u] * oct_get(v[u], c);
      }
    }
    Oct<T> r;
    oct_from(r, acc);
    oct_store(out + int64_t(t) * width + o * 8, r);
  }
}

}  // namespace

hipError_t launch_aggregate(const LayerArgs& a, const void* rows, bool weighted, void* out,
                            int width, hipStream_t st) {
  const dim3 grid((a.T + 3) / 4);
  const float* w = weighted ? a.slot_weight : nullptr;
  if (a.f32)
    hipLaunchKernelGGL(k_aggregate<float>, grid, dim3(256), 0, st,
                       static_cast<const float*>(rows), w, a.token_offsets, a.token_slots,
                       static_cast<float*>(out), a.T, width);
  else
    hipLaunchKernelGGL(k_aggregate<bf16_t>, grid, dim3(256), 0, st,
                       static_cast<const bf16_t*>(rows), w, a.token_offsets, a.token_slots,
                       static_cast<bf16_t*>(out), a.T, width);
  return hipGetLastError();
}

}  // namespace moe
