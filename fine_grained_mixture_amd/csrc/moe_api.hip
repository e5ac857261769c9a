// C ABI of the MoE layer library: argument validation, workspace sizing and
// the launch sequence of each entry point.  Validation and sizing run on the
// host only and touch no HIP API, so a bad call enqueues nothing.
#include "moe.h"

#include <limits.h>

#include <algorithm>
#include <mutex>

#include "common.hpp"
#include "internal.hpp"

// Fixed device scratch for moe_route_noalloc: the routing workspace of
// callers that cannot allocate.  One copy per device, for the life of the
// process.  Host code never passes `scratch` itself to a kernel (on the host
// the name is a stand-in, not a device address): each device's address is
// looked up once with hipGetSymbolAddress, with that device current.
static __device__ __align__(256) char scratch[MOE_NOALLOC_ROUTE_BYTES];

namespace {

using moe::cdiv;

bool aligned16(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int64_t elem_size(const moe_problem* p) { return p->dtype == MOE_F32 ? 4 : 2; }

// Slots any routing of the problem can produce.  Token choice keeps exactly
// T*K pairs; the rounding subroutines move each expert's count to a multiple
// of M_tile: nearest pads only when the upward gap is strictly smaller than
// M_tile/2 (so by at most floor((M_tile-1)/2) slots), up and stochastic pad
// by at most M_tile-1, down never pads.  No expert holds more than T tokens.
int64_t slot_bound(const moe_problem* p) {
  const int64_t tk = p->T * p->K, M = p->M_tile;
  int64_t pad = 0;
  switch (p->mode) {
    case MOE_ROUTE_TR: pad = (M - 1) / 2; break;
    case MOE_ROUTE_TR_UP:
    case MOE_ROUTE_TR_STOCHASTIC: pad = M - 1; break;
    default: pad = 0; break;  // token choice, round down
  }
  return std::min(tk + p->E * pad, p->T * p->E);
}

int check_problem(const moe_problem* p) {
  if (!p) return MOE_ERR_INVALID;
  if (p->T < 1 || p->d < 1 || p->n < 1 || p->E < 1 || p->K < 1 || p->M_tile < 1)
    return MOE_ERR_INVALID;
  if (p->K > p->E) return MOE_ERR_INVALID;
  if (p->dtype != MOE_BF16 && p->dtype != MOE_F32) return MOE_ERR_INVALID;
  if (p->mode < MOE_ROUTE_TC || p->mode > MOE_ROUTE_TR_STOCHASTIC) return MOE_ERR_INVALID;
  if (p->K > 32 || p->E > 1024 || p->M_tile > 1024) return MOE_ERR_UNSUPPORTED;
  if (p->d % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (p->n != 64 && p->n != 128 && p->n != 256 && p->n != 384 && p->n != 512)
    return MOE_ERR_UNSUPPORTED;
  // Kernels index rows with 32-bit element offsets, and the GEMM and routing
  // loads address each array through a buffer descriptor with a 32-bit byte
  // extent: every such array must stay below 4 GiB.
  if (p->T > INT_MAX / 64 || p->E > INT_MAX / p->T) return MOE_ERR_UNSUPPORTED;
  const int64_t slot_cap = slot_bound(p);
  if (p->T * p->d >= INT_MAX || slot_cap * 2 * p->n >= INT_MAX || slot_cap * p->d >= INT_MAX)
    return MOE_ERR_UNSUPPORTED;
  const int64_t es = p->dtype == MOE_F32 ? 4 : 2, lim = int64_t(UINT32_MAX);
  const int64_t Ep = (p->E + 127) / 128 * 128;  // row length of the router's padded dl copy
  const int64_t extents[] = {
      p->T * p->d * es,           // X, dO, O, dX
      slot_cap * 2 * p->n * es,   // H, dH
      slot_cap * p->d * es,       // Y, dX-tilde
      p->d * 2 * p->n * es,       // one expert of W1 / dW1
      p->n * p->d * es,           // one expert of W2 / dW2
      p->E * p->d * es,           // Wr, dWr
      p->T * Ep * es,             // the router's padded dl copy
      p->T * p->E * 4,            // logits, dlogits
  };
  for (int64_t x : extents)
    if (x > lim) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

void sizes_of(const moe_problem* p, moe_sizes_t* s) {
  const int64_t es = elem_size(p);
  s->slot_cap = slot_bound(p);
  s->tile_cap = cdiv<int64_t>(s->slot_cap, moe::kTileM) + p->E;
  s->ws_route = moe::RouteWs::make(p->T, p->E).total;
  // forward transients: A [slot_cap, n], Y [slot_cap, d]
  s->ws_fwd = align256(size_t(s->slot_cap * p->n * es)) + align256(size_t(s->slot_cap * p->d * es));
  // backward transients: dH [slot_cap, 2n], s*A [slot_cap, n], dX~
  // [slot_cap, d], and the weight-gradient chunk plans and fp32 partial sums
  // (their own space: the weight gradients run beside dX~ and its aggregation)
  const size_t vw = moe::varlen_ws_bytes(p->dtype == MOE_F32, int(p->d), int(p->n), int(p->E),
                                         s->slot_cap);
  s->ws_router = moe::router_dims(int(p->T), int(p->d), int(p->E), p->dtype == MOE_F32).ws_bytes;
  s->ws_bwd = align256(size_t(s->slot_cap * 2 * p->n * es)) +
              align256(size_t(s->slot_cap * p->n * es)) +
              align256(size_t(s->slot_cap * p->d * es)) + vw;
}

// A second stream per device for the backward's weight gradients, and the
// events that fork it from and join it to the caller's stream.  Created on
// first use with the device current; kept until the process ends.  Work on
// it is ordered only by those events, so one mutex covers each fork/join
// sequence (the events are shared between calls).  A caller's stream that
// belongs to another device than the current one (or whose device cannot be
// read) gets no side stream (*out = nullptr): the call then runs in order on
// the caller's stream.
constexpr int kMaxDevices = 64;
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, ready = nullptr, join = nullptr;
};
std::mutex g_side_mu;
SideStream g_side[kMaxDevices];

// Caller holds g_side_mu.
hipError_t side_stream(hipStream_t caller, SideStream** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (caller) {
    // a stream whose device cannot be read is treated as another device's
    hipDevice_t sd = 0;
    if (hipStreamGetDevice(caller, &sd) != hipSuccess) {
      (void)hipGetLastError();
      return hipSuccess;
    }
    if (int(sd) != dev) return hipSuccess;
  }
  SideStream& s = g_side[dev];
  if (!s.stream) {
    hipStream_t st = nullptr;
    hipEvent_t f = nullptr, r = nullptr, j = nullptr;
    e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&f, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&r, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&j, hipEventDisableTiming);
    if (e != hipSuccess) {
      if (j) (void)hipEventDestroy(j);
      if (r) (void)hipEventDestroy(r);
      if (f) (void)hipEventDestroy(f);
      if (st) (void)hipStreamDestroy(st);
      return e;
    }
    s.stream = st;
    s.fork = f;
    s.ready = r;
    s.join = j;
  }
  *out = &s;
  return hipSuccess;
}

// The current device's copy of `scratch` is looked up once per device and
// kept in g_scratch_ptr (see the definition of `scratch` above).
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (looked up on its first use).
hipError_t scratch_ptr(void** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

bool routing_ok(const moe_routing* r) {
  return r && aligned16(r->tc_counts) && aligned16(r->counts) && aligned16(r->expert_offsets) &&
         aligned16(r->expert_order) && aligned16(r->topk_ids) && aligned16(r->slot_token) &&
         aligned16(r->slot_weight) && aligned16(r->token_offsets) && aligned16(r->token_slots) &&
         aligned16(r->tile_expert) && aligned16(r->tile_row) && aligned16(r->totals);
}

// A trace must name real events: a NULL handle would make hipEventRecord
// fail and leave an error behind for the next launch check.
bool trace_ok(const moe_trace* t) {
  if (!t || !t->events || t->count <= 0) return true;
  for (int i = 0; i < t->count; ++i)
    if (!t->events[i]) return false;
  return true;
}

moe::TraceHook hook(const moe_trace* t) {
  moe::TraceHook h;
  if (t && t->events && t->count > 0) {
    h.events = t->events;
    h.count = t->count;
  }
  return h;
}

moe::LayerArgs layer_args(const moe_problem* p, const moe_routing* r) {
  moe_sizes_t s;
  sizes_of(p, &s);
  moe::LayerArgs a;
  a.T = int(p->T);
  a.d = int(p->d);
  a.n = int(p->n);
  a.E = int(p->E);
  a.slot_cap = s.slot_cap;
  a.tile_cap = s.tile_cap;
  a.f32 = p->dtype == MOE_F32;
  a.expert_offsets = r->expert_offsets;
  a.expert_order = r->expert_order;
  a.slot_token = r->slot_token;
  a.token_offsets = r->token_offsets;
  a.token_slots = r->token_slots;
  a.tile_expert = r->tile_expert;
  a.tile_row = r->tile_row;
  a.totals = r->totals;
  a.slot_weight = r->slot_weight;
  return a;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported problem";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int moe_sizes(const moe_problem* p, moe_sizes_t* out) {
  const int st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!out) return MOE_ERR_INVALID;
  sizes_of(p, out);
  return MOE_OK;
}

int moe_route_noalloc(const moe_problem* p, const float* logits, const uint32_t* round_rand,
                      const moe_routing* r, void* stream, const moe_trace* trace) {
  // the same validation as moe_route, before any HIP call
  int st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!aligned16(logits) || !routing_ok(r) || !trace_ok(trace)) return MOE_ERR_INVALID;
  if (p->mode == MOE_ROUTE_TR_STOCHASTIC &&
      (!round_rand || reinterpret_cast<uintptr_t>(round_rand) % 4 != 0))
    return MOE_ERR_INVALID;
  moe_sizes_t s;
  sizes_of(p, &s);
  if (s.ws_route > size_t(MOE_NOALLOC_ROUTE_BYTES)) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  if (scratch_ptr(&ws) != hipSuccess) return MOE_ERR_HIP;
  return moe_route(p, logits, round_rand, r, ws, s.ws_route, stream, trace);
}

int moe_route(const moe_problem* p, const float* logits, const uint32_t* round_rand,
              const moe_routing* r, void* ws, size_t ws_bytes, void* stream,
              const moe_trace* trace) {
  int st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!aligned16(logits) || !routing_ok(r) || !aligned16(ws) || !trace_ok(trace))
    return MOE_ERR_INVALID;
  if (p->mode == MOE_ROUTE_TR_STOCHASTIC &&
      (!round_rand || reinterpret_cast<uintptr_t>(round_rand) % 4 != 0))
    return MOE_ERR_INVALID;
  moe_sizes_t s;
  sizes_of(p, &s);
  if (ws_bytes < s.ws_route) return MOE_ERR_WORKSPACE;
  moe::RouteArgs a;
  a.T = int(p->T);
  a.E = int(p->E);
  a.K = int(p->K);
  a.M = int(p->M_tile);
  a.mode = p->mode;
  a.logits = logits;
  a.round_rand = p->mode == MOE_ROUTE_TR_STOCHASTIC ? round_rand : nullptr;
  a.tc_counts = r->tc_counts;
  a.counts = r->counts;
  a.expert_offsets = r->expert_offsets;
  a.expert_order = r->expert_order;
  a.topk_ids = r->topk_ids;
  a.slot_token = r->slot_token;
  a.slot_weight = r->slot_weight;
  a.token_offsets = r->token_offsets;
  a.token_slots = r->token_slots;
  a.tile_expert = r->tile_expert;
  a.tile_row = r->tile_row;
  a.totals = r->totals;
  a.ws = ws;
  return hip_status(moe::launch_route(a, static_cast<hipStream_t>(stream), hook(trace)));
}

int moe_fwd(const moe_problem* p, const void* X, const void* W1, const void* W2,
            const moe_routing* r, void* O, void* H, void* ws, size_t ws_bytes, void* stream,
            const moe_trace* trace) {
  int st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!aligned16(X) || !aligned16(W1) || !aligned16(W2) || !routing_ok(r) || !aligned16(O) ||
      !aligned16(H) || !aligned16(ws) || !trace_ok(trace))
    return MOE_ERR_INVALID;
  moe_sizes_t s;
  sizes_of(p, &s);
  if (ws_bytes < s.ws_fwd) return MOE_ERR_WORKSPACE;
  const moe::LayerArgs a = layer_args(p, r);
  const moe::TraceHook tr = hook(trace);
  hipStream_t sm = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  void* Aact = w;
  void* Y = w + align256(size_t(s.slot_cap * p->n * elem_size(p)));

  tr.mark(sm, 0);
  hipError_t e = moe::launch_up_swiglu(a, X, W1, H, Aact, sm);
  if (e != hipSuccess) return MOE_ERR_HIP;
  tr.mark(sm, 1);
  e = moe::launch_down(a, Aact, W2, Y, sm);
  if (e != hipSuccess) return MOE_ERR_HIP;
  tr.mark(sm, 2);
  e = moe::launch_aggregate(a, Y, true, O, a.d, sm);
  tr.mark(sm, 3);
  return hip_status(e);
}

int moe_bwd(const moe_problem* p, const void* dO, const void* X, const void* H, const void* W1,
            const void* W2, const moe_routing* r, void* dX, void* dW1, void* dW2, float* dS,
            void* ws, size_t ws_bytes, void* stream, const moe_trace* trace) {
  int st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!aligned16(dO) || !aligned16(X) || !aligned16(H) || !aligned16(W1) || !aligned16(W2) ||
      !routing_ok(r) || !aligned16(dX) || !aligned16(dW1) || !aligned16(dW2) || !aligned16(dS) ||
      !aligned16(ws) || !trace_ok(trace))
    return MOE_ERR_INVALID;
  moe_sizes_t s;
  sizes_of(p, &s);
  if (ws_bytes < s.ws_bwd) return MOE_ERR_WORKSPACE;
  const moe::LayerArgs a = layer_args(p, r);
  const moe::TraceHook tr = hook(trace);
  hipStream_t sm = static_cast<hipStream_t>(stream);
  const int64_t es = elem_size(p);
  char* w = static_cast<char*>(ws);
  void* dH = w;
  void* As = w + align256(size_t(s.slot_cap * 2 * p->n * es));
  void* dXt = static_cast<char*>(As) + align256(size_t(s.slot_cap * p->n * es));

  void* vws = static_cast<char*>(dXt) + align256(size_t(s.slot_cap * p->d * es));

  std::unique_lock<std::mutex> lock(g_side_mu, std::defer_lock);
  SideStream* side = nullptr;
  if (tr.count == 0) {
    lock.lock();
    if (side_stream(sm, &side) != hipSuccess) return MOE_ERR_HIP;
    if (!side) lock.unlock();
  }
  if (!side) {
    // traced (or no side stream): every step in order on the caller's
    // stream, so that each segment between two events times one step
    tr.mark(sm, 0);
    hipError_t e = moe::launch_dw_plan(a, vws, sm);
    if (e != hipSuccess) return MOE_ERR_HIP;
    tr.mark(sm, 1);
    e = moe::launch_dh(a, dO, W2, H, dH, As, dS, sm);
    if (e != hipSuccess) return MOE_ERR_HIP;
    tr.mark(sm, 2);
    e = moe::launch_dxt(a, dH, W1, dXt, sm);
    if (e != hipSuccess) return MOE_ERR_HIP;
    tr.mark(sm, 3);
    e = moe::launch_aggregate(a, dXt, false, dX, a.d, sm);
    if (e != hipSuccess) return MOE_ERR_HIP;
    tr.mark(sm, 4);
    e = moe::launch_dw1(a, X, dH, dW1, vws, sm);
    if (e != hipSuccess) return MOE_ERR_HIP;
    tr.mark(sm, 5);
    e = moe::launch_dw2(a, As, dO, dW2, vws, sm);
    tr.mark(sm, 6);
    return hip_status(e);
  }
  // Untraced: the weight-gradient plans, which need only the routing, run
  // on the side stream beside dH.  Then dX~ and its aggregation run on the
  // caller's stream and, beside them, dW1 then dW2 on the side stream.  Both
  // chains need only dH / s*A, and neither writes what the other reads.
  // Running them together keeps the CUs out of step: one kernel's tiles
  // store their outputs while the other's stream operands, instead of every
  // CU storing at once.
  hipError_t e = hipEventRecord(side->fork, sm);
  if (e == hipSuccess) e = hipStreamWaitEvent(side->stream, side->fork, 0);
  if (e != hipSuccess) return MOE_ERR_HIP;
  hipError_t e_side = moe::launch_dw_plan(a, vws, side->stream);
  hipError_t e_main = moe::launch_dh(a, dO, W2, H, dH, As, dS, sm);
  if (e_main == hipSuccess) e_main = hipEventRecord(side->ready, sm);
  // the side stream goes on only once it waits for dH
  if (e_main == hipSuccess && e_side == hipSuccess)
    e_side = hipStreamWaitEvent(side->stream, side->ready, 0);
  else if (e_side == hipSuccess)
    e_side = hipErrorNotReady;
  if (e_main == hipSuccess) e_main = moe::launch_dxt(a, dH, W1, dXt, sm);
  if (e_main == hipSuccess) e_main = moe::launch_aggregate(a, dXt, false, dX, a.d, sm);
  if (e_side == hipSuccess) e_side = moe::launch_dw1(a, X, dH, dW1, vws, side->stream);
  if (e_side == hipSuccess) e_side = moe::launch_dw2(a, As, dO, dW2, vws, side->stream);
  // join whatever was enqueued, so the caller's stream (or its capture) ends
  // after both chains even on an error
  hipError_t e_join = hipEventRecord(side->join, side->stream);
  if (e_join == hipSuccess) e_join = hipStreamWaitEvent(sm, side->join, 0);
  if (e_main != hipSuccess || e_side != hipSuccess || e_join != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}

int moe_gate_bwd(const moe_problem* p, const float* logits, const float* dS, const moe_routing* r,
                 float* dlogits, void* stream, const moe_trace* trace) {
  int st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!aligned16(logits) || !aligned16(dS) || !routing_ok(r) || !aligned16(dlogits) ||
      !trace_ok(trace))
    return MOE_ERR_INVALID;
  hipStream_t sm = static_cast<hipStream_t>(stream);
  const moe::TraceHook tr = hook(trace);
  tr.mark(sm, 0);
  const hipError_t e = moe::launch_gate_bwd(logits, dS, r->token_offsets, r->token_slots,
                                            r->expert_offsets, dlogits, int(p->T), int(p->E), sm);
  tr.mark(sm, 1);
  return hip_status(e);
}

int moe_router_fwd(const moe_problem* p, const void* X, const void* Wr, float* logits,
                   void* stream, const moe_trace* trace) {
  int st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!aligned16(X) || !aligned16(Wr) || !aligned16(logits) || !trace_ok(trace))
    return MOE_ERR_INVALID;
  hipStream_t sm = static_cast<hipStream_t>(stream);
  const moe::TraceHook tr = hook(trace);
  tr.mark(sm, 0);
  const hipError_t e = moe::launch_router_fwd(p->dtype == MOE_F32, X, Wr, logits, int(p->T),
                                              int(p->d), int(p->E), sm);
  tr.mark(sm, 1);
  return hip_status(e);
}

int moe_router_bwd(const moe_problem* p, const void* X, const void* Wr, const float* logits,
                   const float* dS, const moe_routing* r, float* dlogits, void* dWr, void* dX,
                   void* ws, size_t ws_bytes, void* stream, const moe_trace* trace) {
  int st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!aligned16(X) || !aligned16(Wr) || !aligned16(logits) || !aligned16(dS) ||
      !routing_ok(r) || !aligned16(dlogits) || !aligned16(dWr) || !aligned16(dX) ||
      !aligned16(ws) || !trace_ok(trace))
    return MOE_ERR_INVALID;
  moe_sizes_t s;
  sizes_of(p, &s);
  if (ws_bytes < s.ws_router) return MOE_ERR_WORKSPACE;
  moe::RouterBwdArgs a;
  a.T = int(p->T);
  a.d = int(p->d);
  a.E = int(p->E);
  a.f32 = p->dtype == MOE_F32;
  a.X = X;
  a.Wr = Wr;
  a.logits = logits;
  a.dS = dS;
  a.token_offsets = r->token_offsets;
  a.token_slots = r->token_slots;
  a.expert_offsets = r->expert_offsets;
  a.dlogits = dlogits;
  a.dWr = dWr;
  a.dX = dX;
  a.ws = ws;
  return hip_status(moe::launch_router_bwd(a, static_cast<hipStream_t>(stream), hook(trace)));
}

}  // extern "C"
