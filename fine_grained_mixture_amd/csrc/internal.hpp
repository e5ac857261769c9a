// Host-side launcher interfaces between the C ABI (moe_api.hip) and the
// kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace moe {

// Records caller-supplied events between launches (see moe_trace in moe.h).
struct TraceHook {
  void** events = nullptr;
  int count = 0;
  void mark(hipStream_t st, int i) const {
    if (events && i < count) (void)hipEventRecord(static_cast<hipEvent_t>(events[i]), st);
  }
};

struct RouteArgs {
  int T, E, K, M, mode;  // mode: moe_route_mode
  const float* logits;
  const uint32_t* round_rand;  // [E] draws of stochastic rounding, else null
  int32_t *tc_counts, *counts, *expert_offsets, *expert_order, *topk_ids;
  int32_t* slot_token;
  float* slot_weight;
  int32_t *token_offsets, *token_slots, *tile_expert, *tile_row, *totals;
  void* ws;
};

// Everything the grouped GEMMs and aggregation kernels need.
constexpr int kNumCUs = 256;  // compute units of an MI355X

struct LayerArgs {
  int T, d, n, E;
  int64_t slot_cap, tile_cap;
  bool f32;  // element type: fp32 when true, bf16 otherwise
  // routing
  const int32_t *expert_offsets, *expert_order, *slot_token, *token_offsets, *token_slots;
  const int32_t *tile_expert, *tile_row, *totals;
  const float* slot_weight;
};

hipError_t launch_route(const RouteArgs& a, hipStream_t st, const TraceHook& tr);

// Forward: K1 up-proj + SwiGLU, K2 down-proj, K3 aggregation.
hipError_t launch_up_swiglu(const LayerArgs& a, const void* X, const void* W1, void* H,
                            void* Aact, hipStream_t st);
hipError_t launch_down(const LayerArgs& a, const void* Aact, const void* W2, void* Y,
                       hipStream_t st);
// out[t] = sum over t's slots of (weighted ? s : 1) * rows[slot]
hipError_t launch_aggregate(const LayerArgs& a, const void* rows, bool weighted, void* out,
                            int width, hipStream_t st);

// Backward: K4 dH (+dS, dSwiGLU, s*A), K5 dX-tilde, K7 dW1, K8 dW2.
hipError_t launch_dh(const LayerArgs& a, const void* dO, const void* W2, const void* H,
                     void* dH, void* As, float* dS, hipStream_t st);
hipError_t launch_dxt(const LayerArgs& a, const void* dH, const void* W1, void* dXt,
                      hipStream_t st);
// Varlen-K weight gradients.  `vws` is the weight-gradient workspace of
// varlen_ws_bytes() bytes (chunk plans, the persistent kernels' schedules
// and fp32 partial sums).  launch_dw_plan writes the plans and schedules
// from the routing alone and must run before launch_dw1 and launch_dw2.
size_t varlen_ws_bytes(bool f32, int d, int n, int E, int64_t slot_cap);
hipError_t launch_dw_plan(const LayerArgs& a, void* vws, hipStream_t st);
hipError_t launch_dw1(const LayerArgs& a, const void* X, const void* dH, void* dW1, void* vws,
                      hipStream_t st);
hipError_t launch_dw2(const LayerArgs& a, const void* As, const void* dO, void* dW2, void* vws,
                      hipStream_t st);

// Router (linear scores l = X Wr^T and their backward from dS).
struct RouterDims {
  int Ep;            // E rounded up to 128: row length of the padded dl copy
  int kc, nchunks;   // tokens per dWr partial, number of partials
  size_t dlp_bytes;  // padded dl copy in the operand type
  size_t ws_bytes;   // + fp32 partials of dWr
};
RouterDims router_dims(int T, int d, int E, bool f32);
hipError_t launch_router_fwd(bool f32, const void* X, const void* Wr, float* logits, int T,
                             int d, int E, hipStream_t st);
struct RouterBwdArgs {
  int T, d, E;
  bool f32;
  const void *X, *Wr;
  const float *logits, *dS;
  const int32_t *token_offsets, *token_slots, *expert_offsets;
  float* dlogits;
  void *dWr, *dX, *ws;
};
hipError_t launch_router_bwd(const RouterBwdArgs& a, hipStream_t st, const TraceHook& tr);
// dlogits alone (the gate's softmax backward), no workspace.
hipError_t launch_gate_bwd(const float* logits, const float* dS, const int32_t* token_offsets,
                           const int32_t* token_slots, const int32_t* expert_offsets,
                           float* dlogits, int T, int E, hipStream_t st);

}  // namespace moe
