// Building blocks of the grouped GEMMs on gfx950: LDS tiles filled by
// direct global->LDS DMA with the token gather done per lane, a multi-stage
// DMA pipeline, and bf16/fp32 MFMA fragment reads for both operand layouts.
//
// Operand layouts.  Every GEMM computes C[i][j] = sum_k A[i][k] B[k][j] for
// one BM x BN output tile, KB bytes of k per slab (KB = 64 or 128; BK = KB /
// sizeof(T) k-values).
//   K-major tile   one LDS row of KB bytes per output row (i of A, j of B),
//                  holding that row's BK k-values.  Used where the source
//                  rows hold k contiguously (X, dO, A, dH, and the weights
//                  when the contraction runs along their rows).
//   MN-major tile  one LDS row per k, holding COLS contiguous output
//                  indices.  Used where the source rows are indexed by k:
//                  the weights along their columns, and both operands of the
//                  varlen-K weight-gradient GEMMs (rows = the expert's slots).
//
// DMA.  buffer_load_dwordx4 ... lds copies 16 B per lane and places lane L's
// bytes at LDS base + 16 L, so one wave instruction fills 1 KB of a tile
// contiguously while every lane may read any address of the buffer (the
// gather).
// Tiles are unpadded; bank conflicts are avoided by XOR-swizzling the 16-byte
// chunks of each row (the lane that fills a physical chunk fetches the
// logical chunk that belongs there):
//   K-major:   physical chunk = logical chunk ^ ((row >> 1) & 7)   (KB = 128)
//              physical chunk = logical chunk ^ ((row >> 2) & 3)   (KB = 64)
//   MN-major:  physical chunk = logical chunk ^ ((k & 3) << 2)  (rows >= 256 B)
//              physical chunk = logical chunk ^ (((k >> 1) & 1) << 2)  (128 B)
// The LDS has 64 banks of 4 bytes.  A 16-byte read is serviced 16 lanes at
// a time: the 16 consecutive rows of a K-major fragment land in distinct
// banks.  A transposing 8-byte read is serviced 32 lanes at a time: 4 rows x
// 64 contiguous bytes, and the MN-major swizzle moves whole 64-byte windows
// so those 4 windows cover all 256 bytes of banks.
//
// Fragment reads.  A 32x32x16 bf16 MFMA takes, in lane l, 8 consecutive
// k-values of row l % 32 (k half l / 32).  K-major tiles give them with one
// 16-byte LDS read.  MN-major tiles give them with two ds_read_b64_tr_b16:
// within each group of 16 lanes, lane s points at (k0 + s/4, c0 + 4 (s%4))
// and receives the four k-values k0..k0+3 of column c0 + s.
//
// The MFMA is issued with the B fragment as its first operand, so each
// accumulator block holds C^T: lane l owns output row (l % 32) of the block
// and, for accumulator element r, column (r/4)*8 + (l/32)*4 + r%4 — four
// consecutive r are four consecutive columns of one row.
#pragma once

#include "common.hpp"

namespace moe {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

template <class T_, int BM_, int BN_, int WGM_, int WGN_, int STAGES_, int KB_ = 128,
          bool PAIRED_ = false, int NPW_ = 0>
struct TileCfg {
  using T = T_;
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_, KB = KB_;
  static_assert(KB == 64 || KB == 128, "slab bytes");
  static constexpr bool PAIRED = PAIRED_;  // B columns = [gate half | up half]
  static constexpr int NW = WGM * WGN;  // compute waves (they hold the accumulators)
  // Loader waves.  NPW == 0: the compute waves issue their own share of each
  // slab's DMA.  NPW > 0: waves NW .. NW + NPW - 1 issue all of it and never
  // multiply, so no compute wave stalls behind the address unit.
  static constexpr int NPW = NPW_;
  static constexpr int NLW = NPW > 0 ? NPW : NW;  // waves that issue DMA
  static constexpr int kThreads = 64 * (NW + NPW);
  static_assert(NW == 4 || NW == 8, "four or eight compute waves per workgroup");
  static_assert(NPW == 0 || NPW == 4, "four loader waves beside four or eight compute waves");
  // Wave w's roles.  Waves w, w + 4, w + 8 share a SIMD, so with loader
  // waves every SIMD runs one or two compute waves and one loader wave.
  __device__ static constexpr bool loads(int w) { return NPW == 0 || w >= NW; }
  __device__ static constexpr int loader_index(int w) { return NPW == 0 ? w : w - NW; }
  static constexpr int BK = KB / int(sizeof(T));  // k-values per slab
  static constexpr int WTM = BM / WGM, WTN = BN / WGN;
  static constexpr int MB = WTM / 32, NB = WTN / 32;
  static_assert(MB >= 1 && NB >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
  static_assert(!PAIRED || NB % 2 == 0, "paired tiles split each wave's columns");
  static constexpr int KCH = BK / 16;  // 16-wide k chunks per slab
  static constexpr int A_BYTES = BM * KB, B_BYTES = BN * KB;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  // the requested depth, or the deepest that fits in the 160 KB of LDS
  static constexpr int STAGES =
      STAGES_ * STAGE_BYTES <= 160 * 1024 ? STAGES_ : (160 * 1024) / STAGE_BYTES;
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");

  // Tile column (B-tile output index) of the first column of wave block nb.
  __device__ static constexpr int colblock(int wn, int nb) {
    if constexpr (PAIRED) {
      constexpr int half = BN / 2, per = half / WGN, hb = NB / 2;
      return nb < hb ? wn * per + nb * 32 : half + wn * per + (nb - hb) * 32;
    } else {
      return wn * WTN + nb * 32;
    }
  }
};

// ---------------------------------------------------------------------------
// Low-level helpers
// ---------------------------------------------------------------------------
// Buffer descriptor of `bytes` bytes at the wave-uniform address `base`
// (raw, unswizzled; word 3 is the gfx9-family default).  A load whose offset
// lies at or past `bytes` returns zeros instead of touching memory.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), 0x00020000);
}

// 16 bytes per lane from `rs` at byte offset `voff` straight into LDS: lane
// L of the wave writes lds_wave + 16 L.  The MUBUF form is used rather than
// the global (FLAT-encoded) one: the compiler's wait-counter pass treats a
// FLAT DMA as a possible out-of-order LDS access and would then wait for
// every outstanding fragment read (lgkmcnt(0)) before each MFMA.
__device__ __forceinline__ void dma16(rsrc_t rs, uint32_t voff, char* lds_wave) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)lds_wave, 16, voff, 0, 0, 0);
}

// s_waitcnt vmcnt(N) with expcnt / lgkmcnt left unconstrained.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier that also stops the compiler from moving memory
// operations across it.  Waits for outstanding memory operations are
// explicit (wait_vm / wait_lgkm0) at the call sites.
__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
}

template <int KB>
__device__ __forceinline__ int kswz(int r) {
  if constexpr (KB == 128) return (r >> 1) & 7;
  else return (r >> 2) & 3;
}
template <int CH>  // 16-byte chunks per MN-major row
__device__ __forceinline__ int mswz(int k) {
  static_assert(CH >= 8, "MN-major rows of at least 128 bytes");
  if constexpr (CH >= 16) return (k & 3) << 2;
  else return ((k >> 1) & 1) << 2;
}

// ---------------------------------------------------------------------------
// Loaders (one DMA instruction fills 1 KB of a tile; wave w of NW issues
// instructions i = 0..NI-1 into tile bytes [(NW i + w) KB, (NW i + w + 1) KB)).
// ---------------------------------------------------------------------------

// K-major operand whose ROWS source rows are fixed over the k loop: row r's
// k-values for slab s start at byte rowoff(r) + KB s of a buffer of `bytes`
// bytes at `base`.
template <class Cfg, int ROWS>
struct KLoad {
  static constexpr int KB = Cfg::KB, CPR = KB / 16;  // 16-byte chunks per row
  static_assert((ROWS * KB) % (Cfg::NLW * 1024) == 0, "rows");
  static constexpr int NI = ROWS * KB / (Cfg::NLW * 1024);
  rsrc_t rs;
  uint32_t off[NI];
  int w;  // index among the waves that issue DMA

  template <class RowOff>
  __device__ __forceinline__ void init(const void* base, uint32_t bytes, RowOff rowoff) {
    rs = make_rsrc(base, bytes);
    w = Cfg::loader_index(wave_id());
    const int L = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int idx = (i * Cfg::NLW + w) * 64 + L;
      const int r = idx / CPR, pos = idx % CPR;
      off[i] = uint32_t(rowoff(r)) + uint32_t((pos ^ kswz<KB>(r)) << 4);
    }
  }
  __device__ __forceinline__ void issue(int s, char* tile) const {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      dma16(rs, off[i] + uint32_t(s * KB), tile + (i * Cfg::NLW + w) * 1024);
  }  __device__ __forceinline__ void next(int) const {}
};

// MN-major operand with a fixed row stride (weights): row k of slab s is at
// byte (s*BK + k) * ld_bytes of a buffer of `bytes` bytes at `base`;
// col_bytes(c) is the byte offset of logical 16-byte chunk c of the tile row
// inside a source row.
template <class Cfg, int COLS>
struct MNLoad {
  using T = typename Cfg::T;
  static constexpr int RB = COLS * int(sizeof(T)), CH = RB / 16;
  static constexpr int NI = Cfg::BK * RB / (Cfg::NLW * 1024);
  static_assert(NI >= 1 && (Cfg::BK * RB) % (Cfg::NLW * 1024) == 0, "tile size");
  rsrc_t rs;
  uint32_t off[NI];
  uint32_t step;
  int w;  // index among the waves that issue DMA

  template <class ColBytes>
  __device__ __forceinline__ void init(const void* base, uint32_t bytes, uint32_t ld_bytes,
                                       ColBytes col_bytes) {
    rs = make_rsrc(base, bytes);
    w = Cfg::loader_index(wave_id());
    const int L = threadIdx.x & 63;
    step = uint32_t(Cfg::BK) * ld_bytes;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int idx = (i * Cfg::NLW + w) * 64 + L;
      const int k = idx / CH, pos = idx % CH;
      off[i] = uint32_t(k) * ld_bytes + uint32_t(col_bytes(pos ^ mswz<CH>(k)));
    }
  }
  __device__ __forceinline__ void issue(int s, char* tile) const {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      dma16(rs, off[i] + uint32_t(s) * step, tile + (i * Cfg::NLW + w) * 1024);
  }  __device__ __forceinline__ void next(int) const {}
};

// MN-major operand whose rows are an expert's slots (varlen-K): row k of
// slab s is slot kb + s*BK + k, read from source row idx[slot] (GATHER) or
// row slot of a buffer of `bytes` bytes at `base`; slots past the expert's
// end read its last slot and are zeroed in LDS afterwards.  Each lane's
// source rows are fetched one issue ahead (vector loads that land while the
// previous slab is multiplied), so no DMA waits for its gather index.
// issue(s) then next(s) must be called for s = 0, 1, 2, ... in order.
template <class Cfg, int COLS, bool GATHER>
struct SlotLoad {
  using T = typename Cfg::T;
  static constexpr int RB = COLS * int(sizeof(T)), CH = RB / 16;
  static constexpr int NI = Cfg::BK * RB / (Cfg::kThreads * 16);
  static constexpr int RPI = 64 / CH;  // tile rows per DMA instruction
  static_assert(NI >= 1 && RPI >= 1, "tile size");
  static_assert(Cfg::NPW == 0, "slot-row loads are issued by the compute waves");
  rsrc_t rs;
  const int32_t* idx;
  uint32_t ld_bytes;
  uint32_t colb[NI];
  mutable int row[NI];  // source rows of the next issue
  int kb, klast, w, sub;

  __device__ __forceinline__ void fetch(int s) const {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int slot = min(kb + s * Cfg::BK + (i * Cfg::NW + w) * RPI + sub, klast);
      row[i] = GATHER ? idx[slot] : slot;
    }
  }

  template <class ColBytes>
  __device__ __forceinline__ void init(const void* base, uint32_t bytes, uint32_t ldb,
                                       ColBytes col_bytes, const int32_t* index, int kbeg,
                                       int kend) {
    rs = make_rsrc(base, bytes);
    idx = index;
    ld_bytes = ldb;
    kb = kbeg;
    klast = max(kend - 1, kbeg);
    w = wave_id();
    const int L = threadIdx.x & 63;
    sub = L / CH;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int q = (i * Cfg::NW + w) * 64 + L;
      const int k = q / CH, pos = q % CH;
      colb[i] = uint32_t(col_bytes(pos ^ mswz<CH>(k)));
    }
    fetch(0);
  }
  __device__ __forceinline__ void issue(int s, char* tile) const {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      dma16(rs, uint32_t(row[i]) * ld_bytes + colb[i], tile + (i * Cfg::NW + w) * 1024);
  }
  // after both operands of slab s have been issued: rows of slab s + 1
  __device__ __forceinline__ void next(int s) const { fetch(s + 1); }
};

// Zero rows [valid, BK) of an MN-major tile of COLS elements (tail slab of a
// varlen-K contraction).
template <class Cfg, int COLS>
__device__ __forceinline__ void zero_rows(char* tile, int valid) {
  constexpr int RB = COLS * int(sizeof(typename Cfg::T));
  const int start = valid * RB, end = Cfg::BK * RB;
  for (int o = start + int(threadIdx.x) * 16; o < end; o += Cfg::kThreads * 16)
    *reinterpret_cast<uint4*>(tile + o) = make_uint4(0u, 0u, 0u, 0u);
}

// Zeroes the rows past the last valid row in the final, partial slab of
// a varlen-K contraction (those rows were read from the last valid row).
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

// ---------------------------------------------------------------------------
// Fragment reads
// ---------------------------------------------------------------------------
// K-major: 8 k-values (k = 16 kc + 8 h ..) of tile row r.
template <class T, int KB>
__device__ __forceinline__ void frag_k(Oct<T>& f, const char* tile, int r, int kc, int h) {
  constexpr int CPO = int(sizeof(T)) / 2;  // 16-byte chunks per octet
  const int c0 = (kc * 2 + h) * CPO;
#pragma unroll
  for (int j = 0; j < CPO; ++j) {
    const uint4 v =
        *reinterpret_cast<const uint4*>(tile + r * KB + (((c0 + j) ^ kswz<KB>(r)) << 4));
    f.w[4 * j + 0] = v.x; f.w[4 * j + 1] = v.y; f.w[4 * j + 2] = v.z; f.w[4 * j + 3] = v.w;
  }
}

// MN-major: 8 k-values of column cb + (lane % 32) for the 32-column block at
// cb (bf16: two transposing reads; fp32: eight scalar reads).
template <class T, int COLS>
__device__ __forceinline__ void frag_mn(Oct<T>& f, const char* tile, int cb, int kc, int lane);

template <class T, int COLS>
__device__ __forceinline__ void frag_mn(Oct<T>& f, const char* tile, int cb, int kc, int lane) {
  constexpr int RB = COLS * int(sizeof(T)), CH = RB / 16;
  if constexpr (sizeof(T) == 2) {
    const int g = lane >> 4, s = lane & 15, h = g >> 1;
    const int c = cb + 16 * (g & 1) + 4 * (s & 3);  // column this lane points at
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int k = kc * 16 + h * 8 + half * 4 + (s >> 2);
      const char* a = tile + k * RB + ((((c >> 3) ^ mswz<CH>(k))) << 4) + (c & 7) * 2;
      const v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)a);
      f.w[half * 2 + 0] = uint32_t(uint16_t(v[0])) | (uint32_t(uint16_t(v[1])) << 16);
      f.w[half * 2 + 1] = uint32_t(uint16_t(v[2])) | (uint32_t(uint16_t(v[3])) << 16);
    }
  } else {
    const int col = cb + (lane & 31), h = lane >> 5;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = kc * 16 + h * 8 + j;
      const int byte = col * 4;
      f.w[j] = *reinterpret_cast<const uint32_t*>(tile + k * RB +
                                                  ((((byte >> 4) ^ mswz<CH>(k))) << 4) + (byte & 15));
    }
  }
}

// ---------------------------------------------------------------------------
// Accumulators and the slab computation
// ---------------------------------------------------------------------------
template <class Cfg>
struct Accum {
  using T = typename Cfg::T;
  f32x16_t acc[Cfg::MB][Cfg::NB];
  int wm, wn, lane;

  __device__ __forceinline__ void init() {
    const int wave = wave_id();
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

  // Fragments of k chunk kc: A tile (K-major if AK, else MN-major of BM
  // columns) and B tile (K-major if BKM, else MN-major of BN columns).
  template <bool AK, bool BKM>
  __device__ __forceinline__ void frags(Oct<T> (&fa)[Cfg::MB], Oct<T> (&fb)[Cfg::NB],
                                        const char* As, const char* Bs, int kc) const {
    const int r32 = lane & 31, h = lane >> 5;
#pragma unroll
    for (int a = 0; a < Cfg::MB; ++a) {
      const int rb = wm * Cfg::WTM + a * 32;
      if constexpr (AK) frag_k<T, Cfg::KB>(fa[a], As, rb + r32, kc, h);
      else frag_mn<T, Cfg::BM>(fa[a], As, rb, kc, lane);
    }
#pragma unroll
    for (int b = 0; b < Cfg::NB; ++b) {
      const int cb = Cfg::colblock(wn, b);
      if constexpr (BKM) frag_k<T, Cfg::KB>(fb[b], Bs, cb + r32, kc, h);
      else frag_mn<T, Cfg::BN>(fb[b], Bs, cb, kc, lane);
    }
  }

  // One slab: the fragments of chunk kc + 1 are read while the MFMAs of
  // chunk kc run.
  template <bool AK, bool BKM>
  __device__ __forceinline__ void slab(const char* As, const char* Bs) {
    Oct<T> fa[2][Cfg::MB], fb[2][Cfg::NB];
    frags<AK, BKM>(fa[0], fb[0], As, Bs, 0);
#pragma unroll
    for (int kc = 0; kc < Cfg::KCH; ++kc) {
      if (kc + 1 < Cfg::KCH) frags<AK, BKM>(fa[(kc + 1) & 1], fb[(kc + 1) & 1], As, Bs, kc + 1);
      // keep those reads ahead of this chunk's MFMAs
      __builtin_amdgcn_sched_barrier(0);
      mma(fa[kc & 1], fb[kc & 1]);
    }
  }

  // One slab with a single set of fragment registers: chunk kc's reads,
  // then its MFMAs.  For tiles whose accumulators leave no room for a
  // second set; the SIMD's other compute wave covers the read latency.
  template <bool AK, bool BKM>
  __device__ __forceinline__ void slab1(const char* As, const char* Bs) {
#pragma unroll
    for (int kc = 0; kc < Cfg::KCH; ++kc) {
      Oct<T> fa[Cfg::MB], fb[Cfg::NB];
      frags<AK, BKM>(fa, fb, As, Bs, kc);
      mma(fa, fb);
    }
  }

  // The MFMAs of one k chunk.
  __device__ __forceinline__ void mma(const Oct<T> (&fa)[Cfg::MB], const Oct<T> (&fb)[Cfg::NB]) {
#pragma unroll
    for (int a = 0; a < Cfg::MB; ++a)
#pragma unroll
      for (int b = 0; b < Cfg::NB; ++b) mma16(acc[a][b], fb[b], fa[a]);
  }

  // Tile row of block a for this lane; tile column of the 4-column group q.
  __device__ __forceinline__ int row(int a) const { return wm * Cfg::WTM + a * 32 + (lane & 31); }
  __device__ __forceinline__ int col(int b, int q) const {
    return Cfg::colblock(wn, b) + q * 8 + (lane >> 5) * 4;
  }
};

// One pipeline step: DMA for a later slab into `nxt` while slab s is
// multiplied out of `cur`.  The two stages are distinct restrict pointers so
// that the compiler can tell the DMA writes from the fragment reads (alias
// scopes); otherwise it would wait for every outstanding DMA before the first
// LDS read and the prefetch would be lost.
template <class Cfg, bool AK, bool BKM, class LA, class LB, class Tail>
__device__ __forceinline__ void pipeline_step(Accum<Cfg>& acc, const char* __restrict__ cur,
                                              char* __restrict__ nxt, bool issue, int s_next,
                                              int s, const LA& la, const LB& lb, Tail& tail) {
  if (issue) {
    la.issue(s_next, nxt);
    lb.issue(s_next, nxt + Cfg::A_BYTES);
    la.next(s_next);
    lb.next(s_next);
  }
  tail(s, const_cast<char*>(cur));
  acc.template slab<AK, BKM>(cur, cur + Cfg::A_BYTES);
}

// Multi-stage DMA pipeline over `nslabs` slabs.  Slab s lives in stage s % S;
// at the top of iteration s the wave waits until its own DMA for slab s has
// landed (later slabs may stay in flight), the barrier makes every wave's
// part visible and shows that every wave is done with slab s - 1, and the
// DMA for slab s + S - 1 is issued into that stage, so each slab has S - 1
// slabs of compute to arrive in.  `tail(s, stage)` may patch the stage (it
// must end with its own wait + barrier if it writes LDS).  Ends with a
// barrier, so the caller may reuse the LDS.
template <class Cfg, bool AK, bool BKM, class LA, class LB, class Tail>
__device__ __forceinline__ void pipeline(Accum<Cfg>& acc, char* lds, int nslabs, const LA& la,
                                         const LB& lb, Tail&& tail) {
  constexpr int S = Cfg::STAGES, NI = LA::NI + LB::NI;
  static_assert(S >= 2 && S <= 4 && NI * (S - 2) < 64, "pipeline depth");
  static_assert(Cfg::NPW == 0, "tiles with loader waves run persistent_split");
#pragma unroll
  for (int st = 0; st < S - 1; ++st) {
    if (st < nslabs) {
      char* sp = lds + st * Cfg::STAGE_BYTES;
      la.issue(st, sp);
      lb.issue(st, sp + Cfg::A_BYTES);
      la.next(st);
      lb.next(st);
    }
  }
  for (int s = 0; s < nslabs; ++s) {
    const int ahead = min(S - 2, nslabs - 1 - s);  // slabs issued after slab s
    if constexpr (S >= 4) {
      if (ahead >= 2) wait_vm<2 * NI>();
      else if (ahead == 1) wait_vm<NI>();
      else wait_vm<0>();
    } else if constexpr (S == 3) {
      if (ahead >= 1) wait_vm<NI>();
      else wait_vm<0>();
    } else {
      wait_vm<0>();
    }
    barrier();
    pipeline_step<Cfg, AK, BKM>(acc, lds + (s % S) * Cfg::STAGE_BYTES,
                                lds + ((s + S - 1) % S) * Cfg::STAGE_BYTES, s + S - 1 < nslabs,
                                s + S - 1, s, la, lb, tail);
  }
  barrier();
}

// Slab waits of a wave that issued the DMA for slabs up to s + ahead: its own
// part of slab s has landed once at most `ahead` slabs of NI instructions are
// still outstanding (the vector-memory counter completes in order).
template <int S, int NI>
__device__ __forceinline__ void wait_slab(int ahead) {
  if constexpr (S >= 4) {
    if (ahead >= 2) wait_vm<2 * NI>();
    else if (ahead == 1) wait_vm<NI>();
    else wait_vm<0>();
  } else if constexpr (S == 3) {
    if (ahead >= 1) wait_vm<NI>();
    else wait_vm<0>();
  } else {
    wait_vm<0>();
  }
}

// The two loaders of one tile.
template <class LA, class LB>
struct LoadPair {
  LA la;
  LB lb;
};

// Tiles one workgroup of a persistent launch keeps descriptors for (in LDS).
constexpr int kPersistentTiles = 512;

// A persistent launch runs one workgroup per CU.  Workgroup b is on XCD b % 8
// and takes every (gridDim / 8)-th tile of that XCD's contiguous range,
// starting at b / 8, so the tiles running at once on an XCD are consecutive
// (same expert, same weight columns, one L2).  Tile k of the workgroup is
// first + k * stride.
struct PersistentShare {
  int first, stride, ntiles;
  __device__ static PersistentShare make(int work) {
    const int per = (work + 7) / 8;
    const int xcd = blockIdx.x % 8, local = blockIdx.x / 8, stride = gridDim.x / 8;
    const int beg = xcd * per + local, end = min(xcd * per + per, work);
    PersistentShare p;
    p.first = beg;
    p.stride = stride;
    p.ntiles = beg < end ? (end - beg + stride - 1) / stride : 0;
    return p;
  }
  // Largest ntiles of a launch of `grid` workgroups over at most `work` tiles.
  static int64_t max_tiles(int64_t work, int grid) {
    return ((work + 7) / 8 + grid / 8 - 1) / (grid / 8);
  }
};

// A 16-byte tile descriptor from LDS for a wave that has DMA into LDS in
// flight.  The compiler cannot tell that the descriptor table is never a DMA
// destination, so a plain LDS read would first wait for every DMA of the
// wave; this read waits only for itself.  Its fields are made wave-uniform
// (they are: every lane reads the same entry), so buffer descriptors built
// from them stay in scalar registers.
template <class Tile>
__device__ __forceinline__ Tile lds_tile(const Tile* p) {
  static_assert(sizeof(Tile) == 16, "16-byte descriptors");
  typedef unsigned u32x4v_t __attribute__((ext_vector_type(4)));
  const uint32_t a =
      uint32_t(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)p));
  u32x4v_t v;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
  const uint32_t w[4] = {uint32_t(__builtin_amdgcn_readfirstlane(int(v.x))),
                         uint32_t(__builtin_amdgcn_readfirstlane(int(v.y))),
                         uint32_t(__builtin_amdgcn_readfirstlane(int(v.z))),
                         uint32_t(__builtin_amdgcn_readfirstlane(int(v.w)))};
  Tile t;
  __builtin_memcpy(&t, w, sizeof(t));
  return t;
}

// The slab pipeline of a persistent workgroup with loader waves: its ntiles
// tiles (each of nslabs >= S - 1 slabs) form one stream of slabs.  The loader
// waves issue and wait for every DMA and run ahead across tile boundaries,
// so the first S - 1 slabs of the next tile land while the compute waves
// write the current tile; the compute waves only multiply landed stages and
// write the outputs.  Both roles pass one barrier per slab and one per tile:
// the barrier of slab g tells the compute waves that slab g has landed and
// the loader waves that stage (g - 1) % S is free; the barrier after a
// tile's last slab frees that slab's stage for the epilogue's staging, until
// the next slab's barrier.
//   describe(k)          descriptor of tile k (a 16-byte trivially copyable
//                        struct); all are read once into `table` (LDS)
//   loaders(desc)        the LoadPair of a tile (called in loader waves)
//   epilogue(desc, acc, stage)  writes a finished tile, staging through the
//                        STAGE_BYTES at `stage` (called in compute waves)
template <class Cfg, bool AK, bool BKM, class Tile, class Describe, class Loaders, class Epilogue>
__device__ __forceinline__ void persistent_split(char* lds, Tile* table, int ntiles, int nslabs,
                                                 Describe&& describe, Loaders&& loaders,
                                                 Epilogue&& epilogue) {
  constexpr int S = Cfg::STAGES;
  static_assert(Cfg::NPW > 0, "tiles with loader waves");
  for (int k = threadIdx.x; k < ntiles; k += Cfg::kThreads) table[k] = describe(k);
  __syncthreads();
  const int G = ntiles * nslabs;  // slabs in the stream
  if (Cfg::loads(wave_id())) {
    auto cur = loaders(lds_tile(table));
    auto nxt = loaders(lds_tile(table + (ntiles > 1 ? 1 : 0)));
    using LP = decltype(cur);
    constexpr int NI = decltype(cur.la)::NI + decltype(cur.lb)::NI;
    static_assert(S >= 2 && S <= 4 && NI * (S - 2) < 64, "pipeline depth");
    auto issue = [&](const LP& p, int j, int g) {  // slab j of p's tile is slab g of the stream
      char* sp = lds + (g % S) * Cfg::STAGE_BYTES;
      p.la.issue(j, sp);
      p.lb.issue(j, sp + Cfg::A_BYTES);
    };
    for (int g = 0; g < S - 1 && g < G; ++g) {
      if (g < nslabs) issue(cur, g, g);
      else issue(nxt, g - nslabs, g);
    }
    for (int k = 0; k < ntiles; ++k) {
      for (int j = 0; j < nslabs; ++j) {
        const int g = k * nslabs + j;
        wait_slab<S, NI>(min(S - 2, G - 1 - g));
        barrier();
        if (g + S - 1 < G) {
          if (j + S - 1 < nslabs) issue(cur, j + S - 1, g + S - 1);
          else issue(nxt, j + S - 1 - nslabs, g + S - 1);
        }
      }
      barrier();  // the compute waves write tile k
      if (k + 1 < ntiles) {
        cur = nxt;
        if (k + 2 < ntiles) nxt = loaders(lds_tile(table + k + 2));
      }
    }
    return;
  }
  Accum<Cfg> acc;
  for (int k = 0; k < ntiles; ++k) {
    const Tile desc = table[k];
    acc.init();
    for (int j = 0; j < nslabs; ++j) {
      barrier();
      const char* cur = lds + ((k * nslabs + j) % S) * Cfg::STAGE_BYTES;
      if constexpr (Cfg::NW == 8) acc.template slab1<AK, BKM>(cur, cur + Cfg::A_BYTES);
      else acc.template slab<AK, BKM>(cur, cur + Cfg::A_BYTES);
    }
    barrier();  // every compute wave is done with the last slab's stage
    epilogue(desc, acc, lds + ((k * nslabs + nslabs - 1) % S) * Cfg::STAGE_BYTES);
  }
}

struct NoTail {
  __device__ __forceinline__ void operator()(int, char*) const {}
};

// Epilogue staging.  A wave deposits the values of one 32-row accumulator
// block (lane l: row l % 32, four consecutive columns per MFMA group) into a
// wave-private LDS buffer, then writes whole rows to global memory with
// 16-byte stores, so each store instruction covers several full 128-byte
// lines instead of 32 partial ones.  The stores are non-temporal: every
// output here is read at most once, by a later kernel.  Rows are padded by 8 bytes so that the
// 32 rows written at one column fall in distinct banks.
template <class T, int COLS>
struct RowStage {
  static constexpr int RB = COLS * int(sizeof(T));
  static_assert(RB % 16 == 0, "whole 16-byte chunks per row");
  static constexpr int LDR = RB + 8;
  static constexpr int BYTES = 32 * LDR;
  char* buf;

  __device__ __forceinline__ void put(int row, int col, const T (&v)[4]) const {
    __builtin_memcpy(buf + row * LDR + col * int(sizeof(T)), v, sizeof(v));
  }
  __device__ __forceinline__ void get(int row, int col, T (&v)[4]) const {
    __builtin_memcpy(v, buf + row * LDR + col * int(sizeof(T)), sizeof(v));
  }
  // The inverse of flush: whole rows from global memory into the buffer
  // (rowptr(r) == nullptr leaves row r as it is).
  template <class RowPtr>
  __device__ __forceinline__ void fill(RowPtr rowptr) const {
    constexpr int CPR = RB / 16;
    static_assert((32 * CPR) % 64 == 0, "whole rounds of the wave");
    const int lane = threadIdx.x & 63;
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < 32 * CPR / 64; ++i) {
      const int idx = i * 64 + lane, r = idx / CPR, c = idx % CPR;
      const T* g = rowptr(r);
      if (g) {
        const uint4 v = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(g) + c * 16);
        char* dst = buf + r * LDR + c * 16;
        *reinterpret_cast<uint2*>(dst) = make_uint2(v.x, v.y);
        *reinterpret_cast<uint2*>(dst + 8) = make_uint2(v.z, v.w);
      }
    }
    asm volatile("" ::: "memory");
  }
  // rowptr(r): destination of staged column 0 of block row r, or nullptr.
  template <class RowPtr>
  __device__ __forceinline__ void flush(RowPtr rowptr) const {
    constexpr int CPR = RB / 16;
    static_assert((32 * CPR) % 64 == 0, "whole rounds of the wave");
    const int lane = threadIdx.x & 63;
    asm volatile("" ::: "memory");  // deposits before read-back (LDS keeps wave order)
#pragma unroll
    for (int i = 0; i < 32 * CPR / 64; ++i) {
      const int idx = i * 64 + lane, r = idx / CPR, c = idx % CPR;
      const char* src = buf + r * LDR + c * 16;
      const uint2 lo = *reinterpret_cast<const uint2*>(src);
      const uint2 hi = *reinterpret_cast<const uint2*>(src + 8);
      T* g = rowptr(r);
      if (g) {
        const u32x4_t v = {lo.x, lo.y, hi.x, hi.y};
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(reinterpret_cast<char*>(g) + c * 16));
      }
    }
    asm volatile("" ::: "memory");  // read-back before the next deposits
  }
};

// Writes a plain accumulator tile: wave block rows go to rowptr(tile_row) +
// (wave's first column), via the staging buffer at lds + wave * BYTES.
template <class Cfg, class RowPtr>
__device__ __forceinline__ void store_acc_staged(const Accum<Cfg>& acc, char* lds, RowPtr rowptr) {
  using T = typename Cfg::T;
  using St = RowStage<T, Cfg::WTN>;
  const St st{lds + wave_id() * St::BYTES};
  const int r32 = acc.lane & 31, h = acc.lane >> 5;
  const int c0 = Cfg::colblock(acc.wn, 0);
#pragma unroll
  for (int a = 0; a < Cfg::MB; ++a) {
#pragma unroll
    for (int b = 0; b < Cfg::NB; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        T v[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = Elem<T>::store(acc.acc[a][b][q * 4 + c]);
        st.put(r32, b * 32 + q * 8 + h * 4, v);
      }
    const int rb = acc.wm * Cfg::WTM + a * 32;
    st.flush([&](int r) -> T* {
      T* row = rowptr(rb + r);
      return row ? row + c0 : nullptr;
    });
  }
}

// The end of the rows of M tile mt: the next tile's first row when it exists
// (a later tile of the same expert, or the first row of the next expert that
// has any), else S, capped at the tile's 128 rows.  Equal to the tile's
// expert's end offset (capped), without waiting for the expert id first.
__device__ __forceinline__ int tile_end(const int32_t* __restrict__ tile_row,
                                        const int32_t* __restrict__ totals, int mt, int row0) {
  const int next = mt + 1 < totals[1] ? tile_row[mt + 1] : totals[0];
  return min(row0 + kTileM, next);
}

// M-tile mt and column tile nt of linear tile index lin, in expert-major
// order: an expert with M-tiles [m0, m0 + c) owns the linear range
// [NT m0, NT (m0 + c)); inside it the M-tiles go in groups of up to G, and
// a group is walked column tile by column tile (its M-tiles consecutive).
// The tiles that run at once on one XCD then share the expert's weight
// block of their column, and a group's row blocks stay in the L2 over its
// column sweep: each weight block is fetched once per group, each row
// block once.  The expert of lin is the expert of M-tile lin / NT (inside
// its range); its M-tiles start at slot rows off_e + i kTileM.
template <int G>
__device__ __forceinline__ void grouped_tile(int lin, int NT,
                                             const int32_t* __restrict__ tile_expert,
                                             const int32_t* __restrict__ tile_row,
                                             const int32_t* __restrict__ expert_offsets,
                                             int& mt, int& nt) {
  const int g = lin / NT;
  const int e = tile_expert[g];
  const int off = expert_offsets[e];
  const int m0 = g - (tile_row[g] - off) / kTileM;
  const int c = (expert_offsets[e + 1] - off + kTileM - 1) / kTileM;
  const int r = lin - NT * m0;
  const int grp = r / (G * NT), gm = min(G, c - grp * G);
  const int rr = r - grp * G * NT;
  nt = rr / gm;
  mt = m0 + grp * G + rr % gm;
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
