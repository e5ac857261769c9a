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
//                 token-choice bitmap (expert-major)
//   route_count   per expert: f_e = popcount of its bitmap row, r_e
//   route_select  per expert: token-rounding threshold (radix select on the
//                 64-bit keys), slot list in token order, gate weights, and
//                 the expert's slots before each bitmap word; one extra
//                 workgroup scans the counts: expert offsets, the M-tile
//                 schedule, the expert order by count, the totals
//   route_tslots  per token: CSR offset and its slots in ascending expert order
#include "moe.h"
#include "common.hpp"
#include "internal.hpp"

namespace moe {
namespace {

constexpr int kScanThreads = 1024;

// All-reduce across each row of 16 lanes with DPP moves (register
// crossbar, no LDS round trip): swap neighbours, swap pairs, mirror inside
// 8 lanes, mirror inside 16 lanes.  After each step every lane combines its
// value with one lane of the other half of a growing group, so after the
// four steps all 16 lanes hold the reduction of the row.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
  return uint32_t(__builtin_amdgcn_mov_dpp(int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
  return uint64_t(dpp32<CTRL>(uint32_t(v))) | (uint64_t(dpp32<CTRL>(uint32_t(v >> 32))) << 32);
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;  // lane i <- lane 7 - i inside 8
constexpr int kDppMirror = 0x140;      // lane i <- lane 15 - i inside 16

// AND and OR of a 64-bit value over the 64 lanes of a wave, valid in lane
// 63: an all-reduce inside each row of 16, then rows 0-2 carried into the
// rows after them with row broadcasts (disabled rows contribute the identity).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp32_or(uint32_t v, uint32_t ident) {
  return uint32_t(__builtin_amdgcn_update_dpp(int(ident), int(v), CTRL, ROW_MASK, 0xF, false));
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ void and_or_step(uint64_t& a, uint64_t& o) {
  a &= uint64_t(dpp32_or<CTRL, ROW_MASK>(uint32_t(a), ~0u)) |
       (uint64_t(dpp32_or<CTRL, ROW_MASK>(uint32_t(a >> 32), ~0u)) << 32);
  o |= uint64_t(dpp32_or<CTRL, ROW_MASK>(uint32_t(o), 0u)) |
       (uint64_t(dpp32_or<CTRL, ROW_MASK>(uint32_t(o >> 32), 0u)) << 32);
}
__device__ __forceinline__ void wave_and_or(uint64_t& a, uint64_t& o) {
  and_or_step<0xB1>(a, o);         // quad_perm [1, 0, 3, 2]
  and_or_step<0x4E>(a, o);         // quad_perm [2, 3, 0, 1]
  and_or_step<0x141>(a, o);        // half mirror
  and_or_step<0x140>(a, o);        // mirror: every lane holds its row's result
  and_or_step<0x142, 0xA>(a, o);   // row_bcast:15 into rows 1 and 3
  and_or_step<0x143, 0xC>(a, o);   // row_bcast:31 into rows 2 and 3
}

__device__ __forceinline__ uint64_t row16_max(uint64_t v) {
  uint64_t o;
  o = dpp64<kDppXor1>(v); v = o > v ? o : v;
  o = dpp64<kDppXor2>(v); v = o > v ? o : v;
  o = dpp64<kDppHalfMirror>(v); v = o > v ? o : v;
  o = dpp64<kDppMirror>(v); v = o > v ? o : v;
  return v;
}
__device__ __forceinline__ double row16_sum(double v) {
  v += __longlong_as_double(int64_t(dpp64<kDppXor1>(uint64_t(__double_as_longlong(v)))));
  v += __longlong_as_double(int64_t(dpp64<kDppXor2>(uint64_t(__double_as_longlong(v)))));
  v += __longlong_as_double(int64_t(dpp64<kDppHalfMirror>(uint64_t(__double_as_longlong(v)))));
  v += __longlong_as_double(int64_t(dpp64<kDppMirror>(uint64_t(__double_as_longlong(v)))));
  return v;
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
    uint64_t* __restrict__ keys, uint32_t* __restrict__ bits_e) {
  static_assert(EPL >= 1 && EPL <= 64, "experts per lane");
  __shared__ uint32_t sbits[1024];
  __shared__ uint64_t stage[kStageE][kTopkTokens + 1];
  const int tid = threadIdx.x;
  for (int i = tid; i < E; i += kTopkThreads) sbits[i] = 0u;
  __syncthreads();

  const int sub = tid & (kTopkLanes - 1), tl = tid / kTopkLanes;
  const int t = blockIdx.x * kTopkTokens + tl;
  const bool valid = t < T;
  // the token's logits through one (wave-uniform) buffer descriptor over the
  // whole array, T E 4 bytes (below 4 GiB, checked on the host): positions
  // past E read the next row or, past the end, 0, and are masked below; all
  // EPL loads are issued together
  const __amdgpu_buffer_rsrc_t rlog = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(logits), 0, int(uint32_t(T) * uint32_t(E) * 4u), 0x00020000);
  const uint32_t rowb = uint32_t(valid ? t : T - 1) * uint32_t(E) * 4u;
  float lv[EPL];     // this lane's logits
  uint32_t ok[EPL];  // ordered logits of this lane's experts (0: none)
#pragma unroll
  for (int j = 0; j < EPL; ++j)
    lv[j] = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(rlog, rowb + uint32_t(sub + kTopkLanes * j) * 4u,
                                                    0, 0));
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
    best = row16_max(best);
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
  z = row16_sum(z);
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
// t = j * 1024 + tid (j < KPT) in registers, so the 8-bit radix passes need
// no memory traffic; KPT == 0 reads the keys from memory in every pass (any
// T).
constexpr int kSelThreads = 1024;
// at most this many keys left under the prefix: rank them directly
constexpr int kSelFinish = 256;

template <int KPT>
__global__ __launch_bounds__(kSelThreads) void route_select(
    int T, int E, const int32_t* __restrict__ tc_counts, const int32_t* __restrict__ counts,
    int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ expert_order, int32_t* __restrict__ tile_expert,
    int32_t* __restrict__ tile_row, int32_t* __restrict__ totals,
    const uint64_t* __restrict__ keys, const uint32_t* __restrict__ bits_e,
    uint32_t* __restrict__ bits_s, int32_t* __restrict__ wbase, int32_t* __restrict__ slot_token,
    float* __restrict__ slot_weight) {
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
  // the expert's selection bitmap while it is built (T <= 32 K tokens; with
  // more, the row of bits_s in global memory serves)
  __shared__ uint32_t s_sel[KPT > 0 ? KPT * kSelThreads / 32 : 1];
  // the kept tokens in slot order (T <= 32 K: 16-bit token ids), so that the
  // gate weights are read in one parallel pass without a global barrier
  __shared__ uint16_t s_list[KPT > 0 ? KPT * kSelThreads : 1];
  const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int nw = (T + 31) >> 5;
  // this thread's expert's count (its load issued before the keys', so the
  // offset scan below does not wait for them)
  const int my_r = tid < E ? counts[tid] : 0;
  if (e == E) {
    // the extra workgroup: offsets, tile schedule, expert order and totals
    scan_body(my_r, E, sh, sr, expert_offsets, expert_order, tile_expert, tile_row, totals);
    return;
  }
  const int f = tc_counts[e], r = counts[e];
  const uint64_t* ke = keys + int64_t(e) * T;
  // The keys of this expert, when rounding moved its count: issued now, so
  // that their latency hides behind the offset scan (whose barriers wait for
  // LDS only).
  uint64_t kr[KPT > 0 ? KPT : 1];
  if constexpr (KPT > 0) {
    if (r != f) {
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const int t = j * kSelThreads + tid;
        kr[j] = t < T ? ke[t] : 0ull;  // 0 ranks below every real key
      }
    }
  }
  // this expert's first slot: the counts of the experts before it
  int off;
  {
    int before;
    block_excl_scan(tid < e ? my_r : 0, sh, &before);
    off = before;
  }
  // this expert's row of the selection bitmap: built in LDS when the keys
  // sit in registers, else directly in bits_s (the token-choice bitmap is
  // read by every workgroup's count above and is left as it is)
  uint32_t* be = bits_s + int64_t(e) * nw;
  uint32_t* sel = KPT > 0 ? s_sel : be;
  auto sel_sync = [&] {
    if constexpr (KPT > 0) lds_barrier();
    else __syncthreads();
  };

  if (r == f) {
    // the expert keeps exactly its token-choice tokens
    const uint32_t* tc = bits_e + int64_t(e) * nw;
    for (int w = tid; w < nw; w += kSelThreads) sel[w] = tc[w];
    sel_sync();
  } else {
    // The r-th largest key lies in one class: among the tokens outside token
    // choice when padding (every token-choice key ranks above them, so it is
    // the (r - f)-th largest of that class), among the token-choice tokens
    // when dropping.  The bits that every key of that class shares (the
    // class bit, usually the top exponent bits too) are fixed first from the
    // AND and OR of the class's keys, so the radix passes start at the
    // highest bit where the class's keys differ.
    const uint64_t cls = r > f ? 0ull : (1ull << 63);
    uint64_t prefix = cls, mask = 1ull << 63;
    int rem = r > f ? r - f : r;  // rank (from the top, 1-based) still to locate under prefix
    int cnt_eq = r > f ? T - f : f;
    int hi = -1;  // highest bit still undecided
    if (r > 0) {
      uint64_t a_and = ~0ull, a_or = 0ull;
      if constexpr (KPT > 0) {
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
          const int t = j * kSelThreads + tid;
          if (t < T && (kr[j] & mask) == prefix) { a_and &= kr[j]; a_or |= kr[j]; }
        }
      } else {
        for (int t = tid; t < T; t += kSelThreads) {
          const uint64_t k = ke[t];
          if ((k & mask) == prefix) { a_and &= k; a_or |= k; }
        }
      }
      wave_and_or(a_and, a_or);  // lane 63 holds the wave's AND and OR
      if (lane == 63) { cand[2 * (tid >> 6)] = a_and; cand[2 * (tid >> 6) + 1] = a_or; }
      lds_barrier();
      a_and = ~0ull;
      a_or = 0ull;
      for (int w = 0; w < kSelThreads / 64; ++w) { a_and &= cand[2 * w]; a_or |= cand[2 * w + 1]; }
      lds_barrier();  // cand is reused below
      const uint64_t diff = (a_and ^ a_or) & ~mask;
      hi = diff ? 63 - __clzll(diff) : -1;
      const uint64_t common = hi >= 0 ? ~((2ull << hi) - 1) : ~0ull;  // bits above hi
      prefix = (a_and & common) | cls;
      mask = common;
      while (hi >= 0) {
        const int shift = hi >= 7 ? hi - 7 : 0;
        const int nbits = hi - shift + 1;
        const uint64_t dmask = (1ull << nbits) - 1;
        for (int i = tid; i < 16 * 257; i += kSelThreads) (&hist[0][0])[i] = 0u;
        lds_barrier();
        uint32_t* hc = hist[tid & 15];
        if constexpr (KPT > 0) {
#pragma unroll
          for (int j = 0; j < KPT; ++j) {
            const int t = j * kSelThreads + tid;
            if (t < T && (kr[j] & mask) == prefix) atomicAdd(&hc[(kr[j] >> shift) & dmask], 1u);
          }
        } else {
          for (int t = tid; t < T; t += kSelThreads) {
            const uint64_t k = ke[t];
            if ((k & mask) == prefix) atomicAdd(&hc[(k >> shift) & dmask], 1u);
          }
        }
        lds_barrier();
        if (tid < 256) {
          uint32_t c = 0;
#pragma unroll
          for (int q = 0; q < 16; ++q) c += hist[q][tid];
          tot[tid] = c;
        }
        lds_barrier();
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
        lds_barrier();
        prefix |= uint64_t(uint32_t(s_digit_info[0])) << shift;
        mask |= dmask << shift;
        rem = s_digit_info[1];
        cnt_eq = s_digit_info[2];
        hi = shift - 1;
        lds_barrier();
        if (KPT > 0 && hi >= 0 && cnt_eq <= kSelFinish) {
          // Few keys left under the prefix: gather them and find the rem-th
          // largest directly, by counting for each candidate the candidates
          // above it (and equal to it).
          if (tid == 0) s_ncand = 0;
          lds_barrier();
          if constexpr (KPT > 0) {
#pragma unroll
            for (int j = 0; j < KPT; ++j) {
              const int t = j * kSelThreads + tid;
              if (t < T && (kr[j] & mask) == prefix) cand[atomicAdd(&s_ncand, 1)] = kr[j];
            }
          }
          lds_barrier();
          const int nc = s_ncand;
          {
            // four threads per candidate (a lane quad), each comparing it
            // with a quarter of the candidates; the quad adds its counts
            const int ci = tid >> 2, qt = tid & 3;
            const uint64_t mine = ci < nc ? cand[ci] : 0ull;
            int gt = 0, ge = 0;
            if (ci < nc)
              for (int i = qt; i < nc; i += 4) {
                const uint64_t o = cand[i];
                gt += o > mine;
                ge += o >= mine;
              }
            gt += dpp_or_zero<0xB1>(gt);  // quad_perm [1, 0, 3, 2]
            gt += dpp_or_zero<0x4E>(gt);  // quad_perm [2, 3, 0, 1]
            ge += dpp_or_zero<0xB1>(ge);
            ge += dpp_or_zero<0x4E>(ge);
            if (ci < nc && qt == 0 && gt < rem && rem <= ge) {
              // every holder of this key writes the same
              s_thr = mine;
              s_digit_info[1] = rem - gt;
              s_digit_info[2] = ge - gt;
            }
          }
          lds_barrier();
          prefix = s_thr;
          mask = ~0ull;
          rem = s_digit_info[1];
          cnt_eq = s_digit_info[2];
          lds_barrier();
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
        if (lane == 0 && w0 < nw) sel[w0] = uint32_t(m);
        if (lane == 32 && w0 < nw) sel[w0] = uint32_t(m >> 32);
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
        sel[w] = word;
      }
    }
    sel_sync();
    if (r > 0 && !all_eq) {
      // several tokens share the boundary key: keep the lowest `rem` of them
      int taken = 0;
      for (int base = 0; base < T; base += kSelThreads) {
        const int t = base + tid;
        const int flag = (t < T) && (ke[t] == prefix);
        int chunk;
        const int ex = block_excl_scan(flag, sh, &chunk);
        if (flag && taken + ex < rem) atomicOr(&sel[t >> 5], 1u << (t & 31));
        taken += chunk;
      }
      sel_sync();
    }
  }

  // Compaction in token order: each thread lists the kept tokens of one
  // bitmap word as slots and records the slots before its word; the row of
  // the selection bitmap goes out for the token CSR.  The gate weights then
  // come from a flat pass over the slots, all loads in flight together.
  int carry = 0;
  for (int base = 0; base < nw; base += kSelThreads) {
    const int w = base + tid;
    const uint32_t word = (w < nw) ? sel[w] : 0u;
    int chunk;
    const int ex = block_excl_scan(__popc(word), sh, &chunk);
    if (w < nw) {
      const int wb = carry + ex;
      wbase[int64_t(e) * nw + w] = wb;
      if constexpr (KPT > 0) be[w] = word;
      uint32_t m = word;
      int i = 0;
      // never past the expert's own r_e slots, whatever the bitmap holds
      while (m && wb + i < r) {
        const int b = __ffs(m) - 1;
        m &= m - 1;
        const int t = w * 32 + b;
        slot_token[off + wb + i] = t;
        if constexpr (KPT > 0) s_list[wb + i] = uint16_t(t);
        ++i;
      }
    }
    carry += chunk;
  }
  const int kept = min(carry, r);
  if constexpr (KPT > 0) lds_barrier();
  else __syncthreads();
#pragma unroll 4
  for (int i = tid; i < kept; i += kSelThreads) {
    const int t = KPT > 0 ? int(s_list[i]) : slot_token[off + i];
    const uint64_t k = ke[t] & 0x7fffffffffffffffull;
    slot_weight[off + i] = float(__longlong_as_double(int64_t(k)));
  }
}

// Per token: CSR offset and the token's slots in ascending expert order,
// from the expert-major selection bitmap.  A block covers 64 tokens (2 bitmap
// words) with 4 threads per token, each walking a contiguous quarter of the
// experts.  It stages, per expert, its slot offset and, for both words, the
// expert's slots before the word (wbase) and the word itself (word-major, so
// that four experts' words are one 16-byte read).  The slots of every token
// before the block are the sum over experts of wbase at the block's first
// word; an exclusive scan over (token, quarter) in thread order then gives
// every thread the position of its first slot.
constexpr int kCsrTokens = 64;
__global__ __launch_bounds__(256) void route_tslots(
    int T, int E, const uint32_t* __restrict__ bits_s, const int32_t* __restrict__ wbase,
    const int32_t* __restrict__ expert_offsets, int32_t* __restrict__ token_offsets,
    int32_t* __restrict__ token_slots) {
  // LDS: expert offsets [E4]; wbase and bits_s of this block's 2 token
  // words, [2][E4] each (E padded to a multiple of 128 with empty experts)
  extern __shared__ int32_t dyn[];
  const int E4 = (E + 127) & ~127;
  int32_t* s_off = dyn;
  int32_t* s_wb = s_off + E4;
  uint32_t* s_be = reinterpret_cast<uint32_t*>(s_wb + 2 * E4);
  __shared__ int sh[256 / 64 + 1];
  const int nw = (T + 31) >> 5;
  const int tid = threadIdx.x, tl = tid >> 2, sub = tid & 3;
  const int t = blockIdx.x * kCsrTokens + tl, tw0 = blockIdx.x * 2;
  int before = 0;
  for (int i = tid; i < E4; i += 256) s_off[i] = i < E ? expert_offsets[i] : 0;
  for (int i = tid; i < E4 * 2; i += 256) {
    const int e = i >> 1, k = i & 1, tw = tw0 + k;
    const bool ok = e < E && tw < nw;
    const int wb = ok ? wbase[int64_t(e) * nw + tw] : 0;
    s_wb[k * E4 + e] = wb;
    s_be[k * E4 + e] = ok ? bits_s[int64_t(e) * nw + tw] : 0u;
    if (k == 0) before += wb;
  }
  int base;
  block_excl_scan(before, sh, &base);  // base = slots before the block (syncs the LDS)
  const int k = tl >> 5;  // this token's word among the block's 2
  const int b = t & 31;
  const uint32_t below = (1u << b) - 1u;
  const uint4* row = reinterpret_cast<const uint4*>(s_be + k * E4);
  const int wpq = E4 / 128;  // words of 32 experts per quarter
  // bit i of word w of this token's expert set: expert 32 w + i holds it
  auto word_of = [&](int w) {
    uint32_t word = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint4 q = row[8 * w + i];
      word |= (((q.x >> b) & 1u) << (4 * i)) | (((q.y >> b) & 1u) << (4 * i + 1)) |
              (((q.z >> b) & 1u) << (4 * i + 2)) | (((q.w >> b) & 1u) << (4 * i + 3));
    }
    return word;
  };
  int c = 0;
  if (t < T)
    for (int w = sub * wpq; w < (sub + 1) * wpq; ++w) c += __popc(word_of(w));
  int total;
  int j = base + block_excl_scan(c, sh, &total);
  if (t < T && sub == 0) token_offsets[t] = j;
  if (t == T - 1 && sub == 3) token_offsets[T] = j + c;
  if (t >= T) return;
  const int32_t* wbk = s_wb + k * E4;
  const uint32_t* bek = s_be + k * E4;
  for (int w = sub * wpq; w < (sub + 1) * wpq; ++w) {
    uint32_t m = word_of(w);
    while (m) {
      const int e = 32 * w + __ffs(m) - 1;
      m &= m - 1;
      token_slots[j++] = s_off[e] + wbk[e] + __popc(bek[e] & below);
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
  uint32_t* bits_s = reinterpret_cast<uint32_t*>(ws + L.bits_s);
  int32_t* wbase = reinterpret_cast<int32_t*>(ws + L.wbase);

  tr.mark(st, 0);
  {
    const dim3 grid(cdiv(T, kTopkTokens));
    const int epl = (E + kTopkLanes - 1) / kTopkLanes;
#define MOE_TOPK(N)                                                                        \
  hipLaunchKernelGGL(route_topk<N>, grid, dim3(kTopkThreads), 0, st, a.logits, T, E, K,  \
                     a.topk_ids, keys, bits_e)
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
                     a.totals, keys, bits_e, bits_s, wbase, a.slot_token, a.slot_weight)
  if (T <= 8 * kSelThreads) MOE_SELECT(8);
  else if (T <= 16 * kSelThreads) MOE_SELECT(16);
  else if (T <= 32 * kSelThreads) MOE_SELECT(32);
  else MOE_SELECT(0);
#undef MOE_SELECT
  tr.mark(st, 3);
  const size_t tslots_lds = size_t((E + 127) & ~127) * 4 * 5;
  hipLaunchKernelGGL(route_tslots, dim3(cdiv(T, kCsrTokens)), dim3(256), tslots_lds, st, T, E,
                     bits_s, wbase, a.expert_offsets, a.token_offsets, a.token_slots);
  tr.mark(st, 4);
  return hipGetLastError();
}

}  // namespace moe
