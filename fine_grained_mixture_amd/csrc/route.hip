// Routing kernels: softmax top-K token choice and token rounding.
//
// Method: SonicMoE ICLR-2026 notes (papernotes.org), key design 1 (Token
// Rounding routing), and the arXiv abstract (mlsanity.com).  Token choice is
// run first; each expert's count f_e is rounded to the nearest multiple of
// M_tile (pad when the upward gap is strictly smaller, otherwise drop), and
// the expert keeps the first r_e tokens of its list sorted by router score
// with its token-choice tokens always ahead of the other candidates.
//
// Decisions are taken in the precision the method states for them: top-K on
// the fp32 logits (equal logits go to the lower expert), the token-rounding
// order on fp64 softmax probabilities (equal keys go to the lower token).
//
// Kernels, in launch order on one stream:
//   route_clear   zero the per-expert counters and the token-major bitmap
//   route_topk    per token: top-K, fp64 softmax keys for all experts,
//                 token-choice bitmap and histogram f_e
//   route_round   one workgroup: r_e, expert offsets, tile schedule, order
//   route_select  per expert: token-rounding threshold (radix select on the
//                 64-bit keys), slot list in token order, gate weights
//   route_tscan   one workgroup: per-token slot counts -> CSR offsets
//   route_tslots  per token: its slots in ascending expert order
#include "common.hpp"
#include "internal.hpp"

namespace moe {
namespace {

constexpr int kSelectThreads = 256;
constexpr int kScanThreads = 1024;

__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  return v;
}

// Exclusive scan over the block; returns the exclusive prefix and writes the
// block total to *total.  `sh` needs one int per wave plus one.
__device__ __forceinline__ int block_excl_scan(int v, int* sh, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  int incl = wave_incl_scan(v);
  if (lane == 63) sh[wave] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int i = 0; i < nwaves; ++i) { int x = sh[i]; sh[i] = run; run += x; }
    sh[nwaves] = run;
  }
  __syncthreads();
  int res = sh[wave] + incl - v;
  *total = sh[nwaves];
  __syncthreads();
  return res;
}

__global__ void route_clear(int32_t* __restrict__ tc_counts, int E,
                            uint32_t* __restrict__ bits_t, int64_t nbits_t) {
  int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t j = i; j < E; j += stride) tc_counts[j] = 0;
  for (int64_t j = i; j < nbits_t; j += stride) bits_t[j] = 0u;
}

// Orders fp32 values as unsigned integers (larger float -> larger integer).
// -0.0 is folded into +0.0 so that the two compare equal, as floats do.
__device__ __forceinline__ uint32_t ordered_f32(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unordered_f32(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// Eight lanes per token (lane `sub` owns experts e = sub mod 8), 32 tokens per
// block, so each block fills exactly one bitmap word per expert.
constexpr int kTopkLanes = 8;
constexpr int kTopkTokens = 256 / kTopkLanes;

template <int KMAX>
__device__ __forceinline__ void sort_bitonic_desc(uint64_t (&c)[KMAX]) {
#pragma unroll
  for (int j = KMAX / 2; j >= 1; j >>= 1) {
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
      if ((i & j) == 0) {
        const uint64_t a = c[i], b = c[i + j];
        c[i] = a > b ? a : b;
        c[i + j] = a > b ? b : a;
      }
    }
  }
}

template <int KMAX>
__global__ __launch_bounds__(256) void route_topk(
    const float* __restrict__ logits, int T, int E, int K,
    int32_t* __restrict__ topk_ids, int32_t* __restrict__ tc_counts,
    uint64_t* __restrict__ keys, uint32_t* __restrict__ bits_e) {
  __shared__ uint32_t sbits[1024];
  __shared__ int32_t shist[1024];
  const int tid = threadIdx.x;
  for (int i = tid; i < E; i += 256) { sbits[i] = 0u; shist[i] = 0; }
  __syncthreads();

  const int sub = tid & (kTopkLanes - 1), tl = tid / kTopkLanes;
  const int t = blockIdx.x * kTopkTokens + tl;
  const bool valid = t < T;
  const float* row = logits + int64_t(valid ? t : 0) * E;
  // key = ordered(logit) : (~e), so equal logits rank the lower expert first.
  uint64_t best[KMAX];
#pragma unroll
  for (int i = 0; i < KMAX; ++i) best[i] = 0ull;
  if (valid) {
    for (int e = sub; e < E; e += kTopkLanes) {
      const uint64_t key = (uint64_t(ordered_f32(row[e])) << 32) | uint64_t(0xffffffffu - uint32_t(e));
      if (key > best[KMAX - 1]) {
#pragma unroll
        for (int i = KMAX - 1; i > 0; --i) {
          if (key > best[i - 1]) best[i] = best[i - 1];
          else if (key > best[i]) best[i] = key;
        }
        if (key > best[0]) best[0] = key;
      }
    }
  }
  // Merge the eight partial lists (disjoint expert sets) with bitonic merges.
#pragma unroll
  for (int o = 1; o < kTopkLanes; o <<= 1) {
    uint64_t c[KMAX];
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
      const uint64_t other = __shfl_xor(best[KMAX - 1 - i], o, 64);
      c[i] = best[i] > other ? best[i] : other;
    }
    sort_bitonic_desc<KMAX>(c);
#pragma unroll
    for (int i = 0; i < KMAX; ++i) best[i] = c[i];
  }
  const double m = double(unordered_f32(uint32_t(best[0] >> 32)));
  double z = 0.0;
  if (valid)
    for (int e = sub; e < E; e += kTopkLanes) z += exp(double(row[e]) - m);
#pragma unroll
  for (int o = 1; o < kTopkLanes; o <<= 1) z += __shfl_xor(z, o, 64);
  int ids[KMAX];
#pragma unroll
  for (int i = 0; i < KMAX; ++i) ids[i] = int(0xffffffffu - uint32_t(best[i]));
  if (valid) {
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
      if (i < K && (i % kTopkLanes) == sub) {
        topk_ids[int64_t(t) * K + i] = ids[i];
        atomicAdd(&shist[ids[i]], 1);
        atomicOr(&sbits[ids[i]], 1u << tl);
      }
    }
    for (int e = sub; e < E; e += kTopkLanes) {
      const double p = exp(double(row[e]) - m) / z;
      bool tc = false;
#pragma unroll
      for (int i = 0; i < KMAX; ++i) tc |= (i < K) && (ids[i] == e);
      keys[int64_t(e) * T + t] = (uint64_t(tc) << 63) | uint64_t(__double_as_longlong(p));
    }
  }
  __syncthreads();
  const int nw = (T + 31) >> 5;
  for (int e = tid; e < E; e += 256) {
    bits_e[int64_t(e) * nw + blockIdx.x] = sbits[e];
    if (shist[e]) atomicAdd(&tc_counts[e], shist[e]);
  }
}

// One workgroup of 1024 threads, one expert per thread (E <= 1024).
__global__ __launch_bounds__(kScanThreads) void route_round(
    const int32_t* __restrict__ tc_counts, int E, int T, int M, int mode,
    int32_t* __restrict__ counts, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ expert_order, int32_t* __restrict__ tile_expert,
    int32_t* __restrict__ tile_row, int32_t* __restrict__ totals) {
  __shared__ int sh[kScanThreads / 64 + 1];
  __shared__ int sr[1024];
  const int e = threadIdx.x;
  int r = 0;
  if (e < E) {
    const int f = tc_counts[e];
    r = f;
    if (mode == 1) {
      const int lo = (f / M) * M;
      const int hi = (f % M == 0) ? f : lo + M;
      r = ((hi - f) < (f - lo) && hi <= T) ? hi : lo;
    }
    counts[e] = r;
  }
  sr[e] = r;
  int S, ntiles;
  const int off = block_excl_scan(r, sh, &S);
  const int nt = (r + kTileM - 1) / kTileM;
  const int tbase = block_excl_scan(nt, sh, &ntiles);
  if (e < E) {
    expert_offsets[e] = off;
    for (int i = 0; i < nt; ++i) {
      tile_expert[tbase + i] = e;
      tile_row[tbase + i] = off + i * kTileM;
    }
    // rank among experts by descending count, ties to the lower expert
    int rank = 0;
    for (int j = 0; j < E; ++j) {
      const int rj = sr[j];
      rank += (rj > r) || (rj == r && j < e);
    }
    expert_order[rank] = e;
  }
  if (e == 0) {
    expert_offsets[E] = S;
    totals[0] = S;
    totals[1] = ntiles;
  }
}

// Per expert: keep the r_e best tokens under the key (is-TC, p) descending,
// equal keys to the lower token, then list them in token order as slots.
__global__ __launch_bounds__(kSelectThreads) void route_select(
    int T, int E, const int32_t* __restrict__ tc_counts,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ expert_offsets,
    const uint64_t* __restrict__ keys, uint32_t* __restrict__ bits_e,
    uint32_t* __restrict__ bits_t, int32_t* __restrict__ wbase,
    int32_t* __restrict__ slot_token, float* __restrict__ slot_weight) {
  __shared__ uint32_t hist[16][256];
  __shared__ uint32_t tot[256];
  __shared__ int sh[kSelectThreads / 64 + 1];
  __shared__ uint64_t s_digit_info[3];
  const int e = blockIdx.x, tid = threadIdx.x;
  const int f = tc_counts[e], r = counts[e];
  const int nw = (T + 31) >> 5;
  const int W = (E + 31) >> 5;
  const uint64_t* ke = keys + int64_t(e) * T;
  uint32_t* be = bits_e + int64_t(e) * nw;

  if (r != f) {
    uint64_t prefix = 0ull, mask = 0ull;
    int rem = r;  // rank (from the top, 1-based) still to locate under prefix
    uint32_t cnt_eq = 0;
    if (r > 0) {
      for (int pass = 0; pass < 8; ++pass) {
        const int shift = 56 - 8 * pass;
        for (int i = tid; i < 16 * 256; i += kSelectThreads) (&hist[0][0])[i] = 0u;
        __syncthreads();
        for (int t = tid; t < T; t += kSelectThreads) {
          const uint64_t k = ke[t];
          if ((k & mask) == prefix) atomicAdd(&hist[tid & 15][(k >> shift) & 255u], 1u);
        }
        __syncthreads();
        {
          uint32_t s = 0;
#pragma unroll
          for (int c = 0; c < 16; ++c) s += hist[c][tid];
          tot[tid] = s;
        }
        __syncthreads();
        if (tid < 64) {
          // lane l covers digits 255-4l .. 252-4l (descending)
          uint32_t c[4];
          int s = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) { c[j] = tot[255 - 4 * tid - j]; s += int(c[j]); }
          const int incl = wave_incl_scan(s);
          int excl = incl - s;
          const bool hit = (excl < rem) && (rem <= incl);
          if (hit) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              if (excl + int(c[j]) >= rem) {
                s_digit_info[0] = uint64_t(255 - 4 * tid - j);
                s_digit_info[1] = uint64_t(rem - excl);
                s_digit_info[2] = uint64_t(c[j]);
                break;
              }
              excl += int(c[j]);
            }
          }
        }
        __syncthreads();
        prefix |= s_digit_info[0] << shift;
        mask |= 0xffull << shift;
        rem = int(s_digit_info[1]);
        cnt_eq = uint32_t(s_digit_info[2]);
        __syncthreads();
      }
    }
    // prefix is now the r-th largest key; `rem` of the cnt_eq equal keys are
    // kept, the lowest tokens first.
    const bool all_eq = (r > 0) && (int(cnt_eq) == rem);
    for (int w = tid; w < nw; w += kSelectThreads) {
      uint32_t word = 0u;
      if (r > 0) {
        for (int b = 0; b < 32; ++b) {
          const int t = w * 32 + b;
          if (t < T) {
            const uint64_t k = ke[t];
            if (k > prefix || (all_eq && k == prefix)) word |= 1u << b;
          }
        }
      }
      be[w] = word;
    }
    __syncthreads();
    if (r > 0 && !all_eq) {
      int taken = 0;
      for (int base = 0; base < T; base += kSelectThreads) {
        const int t = base + tid;
        const int flag = (t < T) && (ke[t] == prefix);
        int chunk;
        const int ex = block_excl_scan(flag, sh, &chunk);
        if (flag && taken + ex < rem) atomicOr(&be[t >> 5], 1u << (t & 31));
        taken += chunk;
      }
      __syncthreads();
    }
  }

  // Compaction in token order.
  const int off = expert_offsets[e];
  int carry = 0;
  for (int base = 0; base < nw; base += kSelectThreads) {
    const int w = base + tid;
    const uint32_t word = (w < nw) ? be[w] : 0u;
    int chunk;
    const int ex = block_excl_scan(__popc(word), sh, &chunk);
    if (w < nw) {
      const int wb = carry + ex;
      wbase[int64_t(e) * nw + w] = wb;
      uint32_t m = word;
      int i = 0;
      // never past the expert's own r_e slots, whatever the bitmap holds
      while (m && wb + i < r) {
        const int b = __ffs(m) - 1;
        m &= m - 1;
        const int t = w * 32 + b;
        const int slot = off + wb + i++;
        slot_token[slot] = t;
        const uint64_t k = ke[t] & 0x7fffffffffffffffull;
        slot_weight[slot] = float(__longlong_as_double(int64_t(k)));
        atomicOr(&bits_t[int64_t(t) * W + (e >> 5)], 1u << (e & 31));
      }
    }
    carry += chunk;
  }
}

__global__ __launch_bounds__(kScanThreads) void route_tscan(
    int T, int E, const uint32_t* __restrict__ bits_t, int32_t* __restrict__ token_offsets) {
  __shared__ int sh[kScanThreads / 64 + 1];
  const int W = (E + 31) >> 5;
  int carry = 0;
  for (int base = 0; base < T; base += kScanThreads) {
    const int t = base + threadIdx.x;
    int c = 0;
    if (t < T)
      for (int w = 0; w < W; ++w) c += __popc(bits_t[int64_t(t) * W + w]);
    int chunk;
    const int ex = block_excl_scan(c, sh, &chunk);
    if (t < T) token_offsets[t] = carry + ex;
    carry += chunk;
  }
  if (threadIdx.x == 0) token_offsets[T] = carry;
}

__global__ __launch_bounds__(256) void route_tslots(
    int T, int E, const uint32_t* __restrict__ bits_t, const uint32_t* __restrict__ bits_e,
    const int32_t* __restrict__ wbase, const int32_t* __restrict__ expert_offsets,
    const int32_t* __restrict__ token_offsets, int32_t* __restrict__ token_slots) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  const int W = (E + 31) >> 5, nw = (T + 31) >> 5, tw = t >> 5;
  const uint32_t below = (1u << (t & 31)) - 1u;
  int j = token_offsets[t];
  for (int w = 0; w < W; ++w) {
    uint32_t m = bits_t[int64_t(t) * W + w];
    while (m) {
      const int e = w * 32 + __ffs(m) - 1;
      m &= m - 1;
      const int64_t q = int64_t(e) * nw + tw;
      token_slots[j++] = expert_offsets[e] + wbase[q] + __popc(bits_e[q] & below);
    }
  }
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t st, const TraceHook& tr) {
  const int T = a.T, E = a.E, K = a.K;
  const RouteWs L = RouteWs::make(T, E);
  char* ws = static_cast<char*>(a.ws);
  uint64_t* keys = reinterpret_cast<uint64_t*>(ws + L.keys);
  uint32_t* bits_e = reinterpret_cast<uint32_t*>(ws + L.bits_e);
  uint32_t* bits_t = reinterpret_cast<uint32_t*>(ws + L.bits_t);
  int32_t* wbase = reinterpret_cast<int32_t*>(ws + L.wbase);
  const int W = (E + 31) / 32;
  const int64_t nbits_t = int64_t(T) * W;

  tr.mark(st, 0);
  {
    const int blocks = int(std::min<int64_t>(1024, cdiv<int64_t>(std::max<int64_t>(nbits_t, E), 256)));
    hipLaunchKernelGGL(route_clear, dim3(blocks), dim3(256), 0, st, a.tc_counts, E, bits_t, nbits_t);
  }
  tr.mark(st, 1);
  {
    const dim3 grid(cdiv(T, kTopkTokens));
    if (K <= 2)
      hipLaunchKernelGGL(route_topk<2>, grid, dim3(256), 0, st, a.logits, T, E, K, a.topk_ids,
                         a.tc_counts, keys, bits_e);
    else if (K <= 8)
      hipLaunchKernelGGL(route_topk<8>, grid, dim3(256), 0, st, a.logits, T, E, K, a.topk_ids,
                         a.tc_counts, keys, bits_e);
    else if (K <= 16)
      hipLaunchKernelGGL(route_topk<16>, grid, dim3(256), 0, st, a.logits, T, E, K, a.topk_ids,
                         a.tc_counts, keys, bits_e);
    else
      hipLaunchKernelGGL(route_topk<32>, grid, dim3(256), 0, st, a.logits, T, E, K, a.topk_ids,
                         a.tc_counts, keys, bits_e);
  }
  tr.mark(st, 2);
  hipLaunchKernelGGL(route_round, dim3(1), dim3(kScanThreads), 0, st, a.tc_counts, E, T, a.M,
                     a.mode, a.counts, a.expert_offsets, a.expert_order, a.tile_expert,
                     a.tile_row, a.totals);
  tr.mark(st, 3);
  hipLaunchKernelGGL(route_select, dim3(E), dim3(kSelectThreads), 0, st, T, E, a.tc_counts,
                     a.counts, a.expert_offsets, keys, bits_e, bits_t, wbase, a.slot_token,
                     a.slot_weight);
  tr.mark(st, 4);
  hipLaunchKernelGGL(route_tscan, dim3(1), dim3(kScanThreads), 0, st, T, E, bits_t,
                     a.token_offsets);
  tr.mark(st, 5);
  hipLaunchKernelGGL(route_tslots, dim3(cdiv(T, 256)), dim3(256), 0, st, T, E, bits_t, bits_e,
                     wbase, a.expert_offsets, a.token_offsets, a.token_slots);
  tr.mark(st, 6);
  return hipGetLastError();
}

}  // namespace moe
