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
// Non-finite logits are first brought into the finite range (finite_logit).
//
// Kernels, in launch order on one stream:
//   route_topk    per token: top-K, fp64 softmax keys for all experts, the
//                 token-choice bitmap (expert-major); clears the token-major
//                 bitmap rows of its tokens
//   route_count   per expert: f_e = popcount of its bitmap row, r_e
//   route_select  per expert: token-rounding threshold (radix select on the
//                 64-bit keys), slot list in token order, gate weights, and
//                 the expert's slots added to per-256-token block counts; one
//                 extra workgroup scans the counts: expert offsets, the
//                 M-tile schedule, the expert order by count, the totals
//   route_tslots  per token: CSR offset and its slots in ascending expert order
#include "moe.h"
#include "common.hpp"
#include "internal.hpp"

namespace moe {
namespace {

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

// Sixteen lanes per token (lane `sub` owns experts e = sub + 16 j, j < EPL),
// 32 tokens per 512-thread block, so each block fills exactly one bitmap word
// per expert.  The top-K is taken in K rounds: each lane offers its best
// expert not yet taken, the 16 lanes reduce to the maximum, and the owner
// marks it taken.  Keys are (ordered logit, ~e), so equal logits go to the
// lower expert.
constexpr int kTopkLanes = 16;
constexpr int kTopkTokens = 32;
constexpr int kTopkThreads = kTopkLanes * kTopkTokens;
constexpr int kStageE = 128;  // experts per LDS staging group of the key write-out

template <int EPL>
__global__ __launch_bounds__(kTopkThreads) void route_topk(
    const float* __restrict__ logits, int T, int E, int K,
    int32_t* __restrict__ topk_ids,
    uint64_t* __restrict__ keys, uint32_t* __restrict__ bits_e, uint32_t* __restrict__ bits_t) {
  static_assert(EPL >= 1 && EPL <= 64, "experts per lane");
  __shared__ uint32_t sbits[1024];
  __shared__ uint64_t stage[kStageE][kTopkTokens + 1];
  const int tid = threadIdx.x;
  for (int i = tid; i < E; i += kTopkThreads) sbits[i] = 0u;
  {
    // this block's rows of the token-major bitmap start empty
    const int W = (E + 31) >> 5;
    const int64_t beg = int64_t(blockIdx.x) * kTopkTokens * W;
    const int64_t end = min(int64_t(T), int64_t(blockIdx.x + 1) * kTopkTokens) * W;
    for (int64_t i = beg + tid; i < end; i += kTopkThreads) bits_t[i] = 0u;
  }
  __syncthreads();

  const int sub = tid & (kTopkLanes - 1), tl = tid / kTopkLanes;
  const int t = blockIdx.x * kTopkTokens + tl;
  const bool valid = t < T;
  // the token's logits through a buffer descriptor over its row: positions
  // past E read 0 (and are masked), so all EPL loads are issued together
  const __amdgpu_buffer_rsrc_t rrow = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(logits + int64_t(valid ? t : 0) * E), 0, E * 4, 0x00020000);
  float lv[EPL];     // this lane's logits
  uint32_t ok[EPL];  // ordered logits of this lane's experts (0: none)
#pragma unroll
  for (int j = 0; j < EPL; ++j)
    lv[j] = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(rrow, uint32_t(sub + kTopkLanes * j) * 4u, 0, 0));
#pragma unroll
  for (int j = 0; j < EPL; ++j) lv[j] = finite_logit(lv[j]);
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = sub + kTopkLanes * j;
    ok[j] = (valid && e < E) ? ordered_f32(lv[j]) : 0u;
  }
  uint64_t taken = 0ull;
  double m = 0.0;
  for (int k = 0; k < K; ++k) {
    uint64_t best = 0ull;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const uint32_t e = uint32_t(sub + kTopkLanes * j);
      const uint64_t key = ((taken >> j) & 1ull) ? 0ull
                                                 : ((uint64_t(ok[j]) << 32) | (0xffffffffu - e));
      best = key > best ? key : best;
    }
#pragma unroll
    for (int o = 1; o < kTopkLanes; o <<= 1) {
      const uint64_t other = __shfl_xor(best, o, 64);
      best = other > best ? other : best;
    }
    const int eb = int(0xffffffffu - uint32_t(best));
    if (k == 0) m = double(unordered_f32(uint32_t(best >> 32)));
    if ((eb & (kTopkLanes - 1)) == sub) taken |= 1ull << (eb / kTopkLanes);
    if (valid && (k & (kTopkLanes - 1)) == sub) {
      topk_ids[int64_t(t) * K + k] = eb;
      atomicOr(&sbits[eb], 1u << tl);
    }
  }
  // softmax in fp64: each exponential is evaluated once and kept, and the
  // normalisation is one reciprocal
  double ex[EPL];
  double z = 0.0;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = sub + kTopkLanes * j;
    ex[j] = (valid && e < E) ? exp(double(lv[j]) - m) : 0.0;
    z += ex[j];
  }
#pragma unroll
  for (int o = 1; o < kTopkLanes; o <<= 1) z += __shfl_xor(z, o, 64);
  const double rz = 1.0 / z;
  __syncthreads();  // sbits complete; stage below reuses nothing of it
  // Keys go out expert-major (row e holds all T tokens): staged in LDS per
  // group of kStageE experts so that each row receives the block's 32
  // consecutive tokens as one 256-byte run.
  const int t0 = blockIdx.x * kTopkTokens;
  const int ntok = min(kTopkTokens, T - t0);
#pragma unroll
  for (int g = 0; g < (EPL * kTopkLanes + kStageE - 1) / kStageE; ++g) {
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = sub + kTopkLanes * j;
      if (e / kStageE == g && e < E) {
        const double pe = ex[j] * rz;
        stage[e % kStageE][tl] = (((taken >> j) & 1ull) << 63) | uint64_t(__double_as_longlong(pe));
      }
    }
    __syncthreads();
    const int ne = min(kStageE, E - g * kStageE);
    for (int i = tid; i < ne * kTopkTokens; i += kTopkThreads) {
      const int el = i / kTopkTokens, tt = i % kTopkTokens;
      if (tt < ntok) keys[int64_t(g * kStageE + el) * T + t0 + tt] = stage[el][tt];
    }
    __syncthreads();
  }
  const int nw = (T + 31) >> 5;
  for (int e = tid; e < E; e += kTopkThreads) bits_e[int64_t(e) * nw + blockIdx.x] = sbits[e];
}

// The rounded count r_e of an expert with f token-choice tokens: the nearest
// multiple of M (ties down), always up, always down, or up with probability
// (f mod M) / M against the expert's 32-bit draw; a count is only rounded up
// when that many distinct tokens exist (hi <= T).
__device__ __forceinline__ int rounded_count(int f, int T, int M, int mode,
                                             const uint32_t* __restrict__ round_rand, int e) {
  if (mode == MOE_ROUTE_TC) return f;
  const int lo = (f / M) * M;
  const int hi = (f % M == 0) ? f : lo + M;
  bool up;
  if (mode == MOE_ROUTE_TR) up = (hi - f) < (f - lo);
  else if (mode == MOE_ROUTE_TR_UP) up = hi > f;
  else if (mode == MOE_ROUTE_TR_DOWN) up = false;
  else up = uint64_t(round_rand[e]) * uint64_t(M) < (uint64_t(f - lo) << 32);
  return (up && hi <= T) ? hi : lo;
}

// Per expert: f_e = number of set bits in its row of the token-choice bitmap,
// and the rounded count r_e.
__global__ __launch_bounds__(256) void route_count(
    int T, int M, int mode, const uint32_t* __restrict__ round_rand,
    const uint32_t* __restrict__ bits_e, int32_t* __restrict__ tc_counts,
    int32_t* __restrict__ counts) {
  __shared__ int sh[256 / 64 + 1];
  const int e = blockIdx.x, nw = (T + 31) >> 5;
  const uint32_t* row = bits_e + int64_t(e) * nw;
  int c = 0;
  for (int w = threadIdx.x; w < nw; w += 256) c += __popc(row[w]);
  int f;
  block_excl_scan(c, sh, &f);
  if (threadIdx.x == 0) {
    tc_counts[e] = f;
    counts[e] = rounded_count(f, T, M, mode, round_rand, e);
  }
}

// One workgroup of 1024 threads, one expert per thread (E <= 1024): slot
// offsets, the M-tile schedule and the experts ordered by descending count.
__device__ __forceinline__ void scan_body(int r, int E, int* sh, int* sr,
                                          int32_t* __restrict__ expert_offsets,
                                          int32_t* __restrict__ expert_order,
                                          int32_t* __restrict__ tile_expert,
                                          int32_t* __restrict__ tile_row,
                                          int32_t* __restrict__ totals) {
  const int e = threadIdx.x;
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
    // (four counts per LDS read; entries past E hold 0 and sit above e, so
    // they never count)
    int rank = 0;
#pragma unroll 4
    for (int j = 0; j < E; j += 4) {
      const int4 q = *reinterpret_cast<const int4*>(sr + j);
      rank += (q.x > r) || (q.x == r && j < e);
      rank += (q.y > r) || (q.y == r && j + 1 < e);
      rank += (q.z > r) || (q.z == r && j + 2 < e);
      rank += (q.w > r) || (q.w == r && j + 3 < e);
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
//
// With KPT > 0 each of the 1024 threads holds the keys of tokens
// t = j * 1024 + tid (j < KPT) in registers, so the eight 8-bit radix passes
// need no memory traffic; KPT == 0 reads the keys from memory in every pass
// (any T).
constexpr int kSelThreads = 1024;
// at most this many keys left under the prefix: rank them directly
constexpr int kSelFinish = 256;

template <int KPT>
__global__ __launch_bounds__(kSelThreads) void route_select(
    int T, int E, const int32_t* __restrict__ tc_counts,
    const int32_t* __restrict__ counts, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ expert_order, int32_t* __restrict__ tile_expert,
    int32_t* __restrict__ tile_row, int32_t* __restrict__ totals,
    const uint64_t* __restrict__ keys, uint32_t* __restrict__ bits_e,
    uint32_t* __restrict__ bits_t, int32_t* __restrict__ wbase,
    int32_t* __restrict__ slot_token, float* __restrict__ slot_weight,
    int32_t* __restrict__ block_sum) {
  // 16 copies of the 256-bin histogram; the +1 pad puts the copies of one
  // digit in 16 different banks
  __shared__ uint32_t hist[16][257];
  __shared__ uint32_t tot[256];
  __shared__ int sh[kSelThreads / 64 + 1];
  __shared__ int s_digit_info[3];
  __shared__ uint64_t cand[kSelFinish];  // keys left under the prefix (early finish)
  __shared__ int s_ncand;
  __shared__ uint64_t s_thr;
  __shared__ __attribute__((aligned(16))) int sr[1024];
  const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  if (e == E) {
    // the extra workgroup: offsets, tile schedule, expert order and totals
    scan_body(tid < E ? counts[tid] : 0, E, sh, sr, expert_offsets, expert_order, tile_expert,
              tile_row, totals);
    return;
  }
  // this expert's first slot: the counts of the experts before it
  int off;
  {
    int before;
    block_excl_scan(tid < e ? counts[tid] : 0, sh, &before);
    off = before;
  }
  const int f = tc_counts[e], r = counts[e];
  const int nw = (T + 31) >> 5;
  const int W = (E + 31) >> 5;
  const uint64_t* ke = keys + int64_t(e) * T;
  uint32_t* be = bits_e + int64_t(e) * nw;

  if (r != f) {
    uint64_t kr[KPT > 0 ? KPT : 1];
    if constexpr (KPT > 0) {
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const int t = j * kSelThreads + tid;
        kr[j] = t < T ? ke[t] : 0ull;  // 0 ranks below every real key
      }
    }
    uint64_t prefix = 0ull, mask = 0ull;
    int rem = r;  // rank (from the top, 1-based) still to locate under prefix
    int cnt_eq = 0;
    if (r > 0) {
      for (int pass = 0; pass < 8; ++pass) {
        const int shift = 56 - 8 * pass;
        for (int i = tid; i < 16 * 257; i += kSelThreads) (&hist[0][0])[i] = 0u;
        __syncthreads();
        uint32_t* hc = hist[tid & 15];
        if constexpr (KPT > 0) {
#pragma unroll
          for (int j = 0; j < KPT; ++j) {
            const int t = j * kSelThreads + tid;
            if (t < T && (kr[j] & mask) == prefix) atomicAdd(&hc[(kr[j] >> shift) & 255u], 1u);
          }
        } else {
          for (int t = tid; t < T; t += kSelThreads) {
            const uint64_t k = ke[t];
            if ((k & mask) == prefix) atomicAdd(&hc[(k >> shift) & 255u], 1u);
          }
        }
        __syncthreads();
        if (tid < 256) {
          uint32_t c = 0;
#pragma unroll
          for (int q = 0; q < 16; ++q) c += hist[q][tid];
          tot[tid] = c;
        }
        __syncthreads();
        if (tid < 64) {
          // lane l covers digits 255-4l .. 252-4l (descending)
          uint32_t c[4];
          int sum = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) { c[j] = tot[255 - 4 * tid - j]; sum += int(c[j]); }
          const int incl = wave_incl_scan(sum);
          int excl = incl - sum;
          if (excl < rem && rem <= incl) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              if (excl + int(c[j]) >= rem) {
                s_digit_info[0] = 255 - 4 * tid - j;
                s_digit_info[1] = rem - excl;
                s_digit_info[2] = int(c[j]);
                break;
              }
              excl += int(c[j]);
            }
          }
        }
        __syncthreads();
        prefix |= uint64_t(uint32_t(s_digit_info[0])) << shift;
        mask |= 0xffull << shift;
        rem = s_digit_info[1];
        cnt_eq = s_digit_info[2];
        __syncthreads();
        if (KPT > 0 && pass < 7 && cnt_eq <= kSelFinish) {
          // Few keys left under the prefix: gather them and find the rem-th
          // largest directly, by counting for each candidate the candidates
          // above it (and equal to it).
          if (tid == 0) s_ncand = 0;
          __syncthreads();
          if constexpr (KPT > 0) {
#pragma unroll
            for (int j = 0; j < KPT; ++j) {
              const int t = j * kSelThreads + tid;
              if (t < T && (kr[j] & mask) == prefix) cand[atomicAdd(&s_ncand, 1)] = kr[j];
            }
          }
          __syncthreads();
          const int nc = s_ncand;
          if (tid < nc) {
            const uint64_t mine = cand[tid];
            int gt = 0, ge = 0;
            for (int i = 0; i < nc; ++i) {
              const uint64_t o = cand[i];
              gt += o > mine;
              ge += o >= mine;
            }
            if (gt < rem && rem <= ge) {  // every holder of this key writes the same
              s_thr = mine;
              s_digit_info[1] = rem - gt;
              s_digit_info[2] = ge - gt;
            }
          }
          __syncthreads();
          prefix = s_thr;
          mask = ~0ull;
          rem = s_digit_info[1];
          cnt_eq = s_digit_info[2];
          __syncthreads();
          break;
        }
      }
    }
    // prefix is now the r-th largest key; `rem` of the cnt_eq equal keys are
    // kept, the lowest tokens first.
    const bool all_eq = (r > 0) && (cnt_eq == rem);
    if constexpr (KPT > 0) {
      // one ballot covers 64 consecutive tokens = two bitmap words
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const int t = j * kSelThreads + tid;
        const bool keep = r > 0 && t < T && (kr[j] > prefix || (all_eq && kr[j] == prefix));
        const uint64_t m = __ballot(keep);
        const int w0 = t >> 5;  // even: lane 0 starts a word
        if (lane == 0 && w0 < nw) be[w0] = uint32_t(m);
        if (lane == 32 && w0 < nw) be[w0] = uint32_t(m >> 32);
      }
    } else {
      for (int w = tid; w < nw; w += kSelThreads) {
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
    }
    __syncthreads();
    if (r > 0 && !all_eq) {
      // several tokens share the boundary key: keep the lowest `rem` of them
      int taken = 0;
      for (int base = 0; base < T; base += kSelThreads) {
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

  // Compaction in token order: the word pass lists the kept tokens; a flat
  // pass over the expert's slots then fetches all gate weights in parallel.
  int carry = 0;
  for (int base = 0; base < nw; base += kSelThreads) {
    const int w = base + tid;
    const uint32_t word = (w < nw) ? be[w] : 0u;
    int chunk;
    const int ex = block_excl_scan(__popc(word), sh, &chunk);
    int written = 0;
    if (w < nw) {
      const int wb = carry + ex;
      wbase[int64_t(e) * nw + w] = wb;
      uint32_t m = word;
      int i = 0;
      // never past the expert's own r_e slots, whatever the bitmap holds
      while (m && wb + i < r) {
        const int b = __ffs(m) - 1;
        m &= m - 1;
        slot_token[off + wb + i++] = w * 32 + b;
      }
      written = i;
    }
    // this expert's slots in each block of 256 tokens (8 words, 8
    // consecutive lanes), for the token CSR
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) written += __shfl_xor(written, o, 64);
    if ((lane & 7) == 0 && w < nw) block_sum[int64_t(e) * ((nw + 7) >> 3) + (w >> 3)] = written;
    carry += chunk;
  }
  __syncthreads();
  const int kept = min(carry, r);
#pragma unroll 4
  for (int i = tid; i < kept; i += kSelThreads) {
    const int t = slot_token[off + i];
    const uint64_t k = ke[t] & 0x7fffffffffffffffull;
    slot_weight[off + i] = float(__longlong_as_double(int64_t(k)));
    atomicOr(&bits_t[int64_t(t) * W + (e >> 5)], 1u << (e & 31));
  }
}

// Per token: CSR offset (earlier blocks' slots, summed over the experts'
// per-block counts, + exclusive scan inside the block) and the token's slots
// in ascending expert order.
__global__ __launch_bounds__(256) void route_tslots(
    int T, int E, const uint32_t* __restrict__ bits_t, const uint32_t* __restrict__ bits_e,
    const int32_t* __restrict__ wbase, const int32_t* __restrict__ expert_offsets,
    const int32_t* __restrict__ block_sum, int32_t* __restrict__ token_offsets,
    int32_t* __restrict__ token_slots) {
  // LDS: expert offsets [E]; wbase and bits_e of this block's 8 token words
  // [E][8] each; the block's rows of the token-major bitmap [256][W]
  extern __shared__ int32_t dyn[];
  int32_t* s_off = dyn;
  int32_t* s_wb = s_off + E;
  uint32_t* s_be = reinterpret_cast<uint32_t*>(s_wb + E * 8);
  uint32_t* s_bt = s_be + E * 8;
  __shared__ int sh[256 / 64 + 1];
  const int W = (E + 31) >> 5, nw = (T + 31) >> 5, nblk = (nw + 7) >> 3;
  const int tid = threadIdx.x, t0 = blockIdx.x * 256, t = t0 + tid, tw0 = blockIdx.x * 8;
  // stage the lookups of this block's tokens (coalesced), so that the slot
  // loop below reads LDS only
  for (int i = tid; i < E; i += 256) s_off[i] = expert_offsets[i];
  for (int i = tid; i < E * 8; i += 256) {
    const int e = i >> 3, tw = tw0 + (i & 7);
    s_wb[i] = tw < nw ? wbase[int64_t(e) * nw + tw] : 0;
    s_be[i] = tw < nw ? bits_e[int64_t(e) * nw + tw] : 0u;
  }
  const int nrow = min(256, T - t0);
  for (int i = tid; i < nrow * W; i += 256) s_bt[i] = bits_t[int64_t(t0) * W + i];
  // slots of all earlier blocks: the entries [e][b] with b < this block, read
  // in batches of 8 per thread through a buffer descriptor (positions past
  // the count get an offset past the end and read 0, so no load waits behind
  // a branch)
  const int nb = blockIdx.x, n = E * nb;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t*>(block_sum), 0, E * nblk * 4, 0x00020000);
  int before = 0;
  for (int i0 = 0; i0 < n; i0 += 256 * 8) {
    int v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * 256 + tid;
      const uint32_t off = i < n ? uint32_t((i / nb) * nblk + i % nb) * 4u : 0xfffffff0u;
      v[u] = int(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) before += v[u];
  }
  int base;
  block_excl_scan(before, sh, &base);  // base = sum over all earlier blocks (syncs the LDS)
  int c = 0;
  if (t < T)
    for (int w = 0; w < W; ++w) c += __popc(s_bt[tid * W + w]);
  int total;
  const int j0 = base + block_excl_scan(c, sh, &total);
  if (t < T) token_offsets[t] = j0;
  if (t == T - 1) token_offsets[T] = j0 + c;
  if (t >= T) return;
  const int k = tid >> 5;  // this token's word among the block's 8
  const uint32_t below = (1u << (t & 31)) - 1u;
  int j = j0;
  for (int w = 0; w < W; ++w) {
    uint32_t m = s_bt[tid * W + w];
    while (m) {
      const int e = w * 32 + __ffs(m) - 1;
      m &= m - 1;
      token_slots[j++] = s_off[e] + s_wb[e * 8 + k] + __popc(s_be[e * 8 + k] & below);
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
  int32_t* block_sum = reinterpret_cast<int32_t*>(ws + L.block_sum);

  tr.mark(st, 0);
  {
    const dim3 grid(cdiv(T, kTopkTokens));
    const int epl = (E + kTopkLanes - 1) / kTopkLanes;
#define MOE_TOPK(N)                                                                        \
  hipLaunchKernelGGL(route_topk<N>, grid, dim3(kTopkThreads), 0, st, a.logits, T, E, K,  \
                     a.topk_ids, keys, bits_e, bits_t)
    if (epl <= 1) MOE_TOPK(1);
    else if (epl <= 2) MOE_TOPK(2);
    else if (epl <= 4) MOE_TOPK(4);
    else if (epl <= 8) MOE_TOPK(8);
    else if (epl <= 16) MOE_TOPK(16);
    else if (epl <= 32) MOE_TOPK(32);
    else MOE_TOPK(64);
#undef MOE_TOPK
  }
  tr.mark(st, 1);
  hipLaunchKernelGGL(route_count, dim3(E), dim3(256), 0, st, T, a.M, a.mode, a.round_rand, bits_e,
                     a.tc_counts, a.counts);
  tr.mark(st, 2);
#define MOE_SELECT(N)                                                                        \
  hipLaunchKernelGGL(route_select<N>, dim3(E + 1), dim3(kSelThreads), 0, st, T, E, a.tc_counts, \
                     a.counts, a.expert_offsets, a.expert_order, a.tile_expert, a.tile_row,    \
                     a.totals, keys, bits_e, bits_t, wbase, a.slot_token, a.slot_weight,     \
                     block_sum)
  if (T <= 8 * kSelThreads) MOE_SELECT(8);
  else if (T <= 16 * kSelThreads) MOE_SELECT(16);
  else if (T <= 32 * kSelThreads) MOE_SELECT(32);
  else MOE_SELECT(0);
#undef MOE_SELECT
  tr.mark(st, 3);
  const size_t tslots_lds = size_t(E) * 4 + size_t(E) * 8 * 4 * 2 + size_t(256) * cdiv(E, 32) * 4;
  hipLaunchKernelGGL(route_tslots, dim3(cdiv(T, 256)), dim3(256), tslots_lds, st, T, E, bits_t,
                     bits_e, wbase, a.expert_offsets, block_sum, a.token_offsets, a.token_slots);
  tr.mark(st, 4);
  return hipGetLastError();
}

}  // namespace moe
