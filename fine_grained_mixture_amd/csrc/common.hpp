// Shared device-side definitions for the gfx950 MoE kernels: storage types,
// bf16 conversion, MFMA wrappers and the routing-workspace layout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // bf16 storage (upper half of an fp32)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;
constexpr int kTileM = 128;  // rows per M tile of the grouped GEMMs

// ---------------------------------------------------------------------------
// Conversions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round-to-nearest-even (the hardware v_cvt_pk_bf16_f32 conversion).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

template <class T> struct Elem;
template <> struct Elem<bf16_t> {
  __device__ __forceinline__ static float load(bf16_t v) { return bf16_to_f32(v); }
  __device__ __forceinline__ static bf16_t store(float v) { return f32_to_bf16(v); }
  // value after one round trip through storage precision
  __device__ __forceinline__ static float round(float v) { return bf16_to_f32(f32_to_bf16(v)); }
};
template <> struct Elem<float> {
  __device__ __forceinline__ static float load(float v) { return v; }
  __device__ __forceinline__ static float store(float v) { return v; }
  __device__ __forceinline__ static float round(float v) { return v; }
};

// Eight consecutive elements of T ("an octet"): 16 B for bf16, 32 B for fp32.
template <class T> struct Oct {
  static constexpr int kWords = sizeof(T) * 2;  // 32-bit words
  uint32_t w[kWords];
};

template <class T>
__device__ __forceinline__ void oct_zero(Oct<T>& o) {
#pragma unroll
  for (int i = 0; i < Oct<T>::kWords; ++i) o.w[i] = 0u;
}

template <class T>
__device__ __forceinline__ void oct_load(Oct<T>& o, const T* p) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int i = 0; i < Oct<T>::kWords / 4; ++i) {
    uint4 v = q[i];
    o.w[4 * i + 0] = v.x; o.w[4 * i + 1] = v.y; o.w[4 * i + 2] = v.z; o.w[4 * i + 3] = v.w;
  }
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Streaming (non-temporal) load of an octet that is read once: it does not
// displace reusable lines from the caches.
template <class T>
__device__ __forceinline__ void oct_load_nt(Oct<T>& o, const T* p) {
  const u32x4_t* q = reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
  for (int i = 0; i < Oct<T>::kWords / 4; ++i) {
    const u32x4_t v = __builtin_nontemporal_load(q + i);
    o.w[4 * i + 0] = v[0]; o.w[4 * i + 1] = v[1]; o.w[4 * i + 2] = v[2]; o.w[4 * i + 3] = v[3];
  }
}

template <class T>
__device__ __forceinline__ void oct_store(T* p, const Oct<T>& o) {
  uint4* q = reinterpret_cast<uint4*>(p);
#pragma unroll
  for (int i = 0; i < Oct<T>::kWords / 4; ++i)
    q[i] = make_uint4(o.w[4 * i + 0], o.w[4 * i + 1], o.w[4 * i + 2], o.w[4 * i + 3]);
}

template <class T>
__device__ __forceinline__ float oct_get(const Oct<T>& o, int i);
template <>
__device__ __forceinline__ float oct_get<bf16_t>(const Oct<bf16_t>& o, int i) {
  uint32_t w = o.w[i >> 1];
  return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
}
template <>
__device__ __forceinline__ float oct_get<float>(const Oct<float>& o, int i) {
  return __uint_as_float(o.w[i]);
}

// Transpose an 8x8 block: out[c] element k = in[k] element c.
__device__ __forceinline__ void oct_transpose(Oct<bf16_t> (&out)[8], const Oct<bf16_t> (&in)[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
#pragma unroll
    for (int kp = 0; kp < 4; ++kp) {
      const uint32_t a = in[2 * kp].w[c >> 1];
      const uint32_t b = in[2 * kp + 1].w[c >> 1];
      // low half of the output word from row 2kp, high half from row 2kp+1
      out[c].w[kp] = (c & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
  }
}
__device__ __forceinline__ void oct_transpose(Oct<float> (&out)[8], const Oct<float> (&in)[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int k = 0; k < 8; ++k) out[c].w[k] = in[k].w[c];
}

// ---------------------------------------------------------------------------
// MFMA: one 32x32 fp32 accumulator block += 16 k-values.
//
// Lane l supplies 8 k-values of row (l % 32) of each operand; lanes 0-31 and
// 32-63 hold the two halves of the 16-wide k chunk.  The result element r of
// lane l sits at row (r/4)*8 + (l/32)*4 + r%4 of the first operand and
// column l % 32 of the second.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void mma16(f32x16_t& acc, const Oct<bf16_t>& a, const Oct<bf16_t>& b) {
  bf16x8_t va, vb;
  __builtin_memcpy(&va, a.w, 16);
  __builtin_memcpy(&vb, b.w, 16);
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, vb, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x16_t& acc, const Oct<float>& a, const Oct<float>& b) {
#pragma unroll
  for (int k = 0; k < 8; ++k)
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w[k]), __uint_as_float(b.w[k]),
                                                 acc, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Small helpers
// ---------------------------------------------------------------------------
// Logistic function with the hardware exp and reciprocal (about 1 ulp each,
// far below the bf16 rounding of every value it feeds).
__device__ __forceinline__ float sigmoidf_(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

template <class T>
__host__ __device__ constexpr T cdiv(T a, T b) { return (a + b - 1) / b; }

// A router score brought into the finite fp32 range: NaN and -inf become
// -FLT_MAX, +inf becomes +FLT_MAX.  Routing and the gate's backward see the
// logits only through this, so inputs outside the real numbers still get one
// ranking (a NaN below every number) and a finite softmax.
__device__ __forceinline__ float finite_logit(float x) {
  constexpr float kMax = 3.40282347e+38f;
  if (__builtin_isnan(x)) return -kMax;
  return x > kMax ? kMax : (x < -kMax ? -kMax : x);
}

// ---------------------------------------------------------------------------
// Wave and workgroup prefix sums with DPP moves (no LDS round trip inside a
// wave): shifts by 1, 2, 4 and 8 lanes inside each row of 16, then row 0's
// and row 1's totals broadcast into the rows after them (row_bcast, gfx9).
// ---------------------------------------------------------------------------
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_or_zero(int v) {
  // lanes without a source (or outside ROW_MASK) get 0
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dpp_or_zero<0x111>(v);        // row_shr:1
  v += dpp_or_zero<0x112>(v);        // row_shr:2
  v += dpp_or_zero<0x114>(v);        // row_shr:4
  v += dpp_or_zero<0x118>(v);        // row_shr:8
  v += dpp_or_zero<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
  v += dpp_or_zero<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
  return v;
}

// Workgroup barrier for data exchanged through LDS only: waits for this
// wave's own LDS operations, not for its outstanding global loads and
// stores (which __syncthreads would also drain), so loads issued earlier
// stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt left alone
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Exclusive prefix sum over the workgroup (at most 1024 threads, whole
// waves); returns the exclusive prefix and writes the total to *total.
// `sh` (LDS) needs one int per wave plus one.  Every thread must call it.
__device__ __forceinline__ int block_excl_scan(int v, int* sh, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) sh[wave] = incl;
  lds_barrier();
  if (wave == 0) {
    const int x = lane < nwaves ? sh[lane] : 0;
    const int xi = wave_incl_scan(x);
    if (lane < nwaves) sh[lane] = xi - x;
    if (lane == nwaves - 1) sh[nwaves] = xi;
  }
  lds_barrier();
  const int res = sh[wave] + incl - v;
  *total = sh[nwaves];
  lds_barrier();
  return res;
}

// Routing workspace layout (byte offsets), shared by the host code and the
// routing kernels.
struct RouteWs {
  size_t keys;     // uint64 [E][T]  (is-token-choice << 63) | bits(p[t,e])
  size_t bits_e;   // uint32 [E][nw] token-choice bitmap, expert-major (nw = ceil(T/32))
  size_t bits_s;   // uint32 [E][nw] selection bitmap (the tokens each expert keeps)
  size_t wbase;    // int32  [E][nw] slots of expert e in words before w
  size_t total;
  __host__ __device__ static size_t align(size_t x) { return (x + 255) & ~size_t(255); }
  __host__ __device__ static RouteWs make(int64_t T, int64_t E) {
    RouteWs w;
    const int64_t nw = (T + 31) / 32;
    size_t o = 0;
    w.keys = o;   o = align(o + size_t(E) * T * 8);
    w.bits_e = o; o = align(o + size_t(E) * nw * 4);
    w.bits_s = o; o = align(o + size_t(E) * nw * 4);
    w.wbase = o;  o = align(o + size_t(E) * nw * 4);
    w.total = o;
    return w;
  }
};

}  // namespace moe

namespace moe {
template <class T>
__device__ __forceinline__ void oct_from(Oct<T>& o, const float (&v)[8]);
template <>
__device__ __forceinline__ void oct_from<bf16_t>(Oct<bf16_t>& o, const float (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o.w[i] = uint32_t(f32_to_bf16(v[2 * i])) | (uint32_t(f32_to_bf16(v[2 * i + 1])) << 16);
}
template <>
__device__ __forceinline__ void oct_from<float>(Oct<float>& o, const float (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) o.w[i] = __float_as_uint(v[i]);
}
}  // namespace moe
