/*
 * moe.h -- C ABI of the MI355X (gfx950) fine-grained MoE layer library.
 *
 * The library computes one fine-grained Mixture-of-Experts layer as described
 * in "SonicMoE: Accelerating MoE with IO and Tile-aware Optimizations"
 * (ICLR-2026 notes on papernotes.org; arXiv abstract on mlsanity.com):
 *
 *   moe_route  top-K token-choice routing on softmax router scores, then
 *              optionally token rounding of every expert's token count to a
 *              multiple of M_tile (notes, key design 1);
 *   moe_fwd    up-projection with the token gather fused into the operand
 *              load and SwiGLU in the epilogue, down-projection, and the
 *              router-weighted aggregation (notes, method > overall
 *              framework, and key design 2);
 *   moe_bwd    the minimal-activation backward: it reads only X, H and the
 *              routing metadata, computes dH and dS = <dA', A> in the
 *              epilogue of the dH grouped GEMM, and forms dW1 / dW2 with
 *              varlen-K grouped GEMMs (notes, key designs 2 and 3).
 *
 * Problem statement (notes, background and key design 3): T tokens, model
 * dim d, expert intermediate dim n, E experts, K experts per token, and the
 * GEMM M tile M_tile that token rounding aligns counts to.
 *   X  [T, d]         W1 [E, d, 2n]  (columns [0, n) gate, [n, 2n) up)
 *   W2 [E, n, d]      O  [T, d]       H  [>= S, 2n]  (pre-activation)
 * All matrices are dense, row-major, with no padding between rows.
 *
 * Conventions for every entry point:
 *   - All buffer pointers are DEVICE pointers, allocated and owned by the
 *     caller.  The library never allocates or frees memory and keeps no
 *     data between calls.  Its only state is, per device, one stream and
 *     two events that moe_bwd creates on first use and keeps until the
 *     process ends, and the fixed scratch array of moe_route_noalloc.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     null stream).  No call synchronises the host or copies device data to
 *     the host.  Untraced, moe_bwd forks part of its work onto its own
 *     stream and joins it back to `stream` (event record + wait) before
 *     returning, so everything it enqueues completes before later work on
 *     `stream`, and a capture of `stream` captures all of it.  Data-dependent sizes (slot count S, tile count) stay on the
 *     device in `moe_routing.totals`; kernels past them exit early.
 *   - Arguments are validated on the host before anything is enqueued; on
 *     failure the call returns a negative moe_status and enqueues nothing.
 *     A HIP launch failure returns MOE_ERR_HIP.
 *   - Pointers must be 16-byte aligned.
 *   - Floating-point inputs and outputs use `dtype` (bf16 or fp32); logits,
 *     gate weights and dS are always fp32; accumulation is always fp32.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 4

/* Rows per M tile of the grouped GEMMs; the tile schedule in moe_routing is
 * expressed in these units. */
#define MOE_GEMM_TILE_M 128

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID = -1,     /* null / misaligned pointer, bad dimension     */
  MOE_ERR_UNSUPPORTED = -2, /* valid problem the library does not handle   */
  MOE_ERR_WORKSPACE = -3,   /* workspace smaller than moe_sizes reports     */
  MOE_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed   */
} moe_status;

typedef enum { MOE_BF16 = 0, MOE_F32 = 1 } moe_dtype;

typedef enum {
  MOE_ROUTE_TC = 0,            /* vanilla top-K token choice                 */
  MOE_ROUTE_TR = 1,            /* token rounding, nearest multiple of M_tile */
  MOE_ROUTE_TR_UP = 2,         /* token rounding, always up (hi)             */
  MOE_ROUTE_TR_DOWN = 3,       /* token rounding, always down (lo)           */
  MOE_ROUTE_TR_STOCHASTIC = 4  /* token rounding, up w.p. (f - lo) / M_tile  */
} moe_route_mode;

typedef struct {
  int64_t T, d, n, E, K, M_tile;
  int32_t dtype; /* moe_dtype      */
  int32_t mode;  /* moe_route_mode */
} moe_problem;

/*
 * slot_cap bounds the slot count S = sum of r_e of every routing of the
 * problem, per mode: TC and TR_DOWN keep at most T*K pairs; TR pads an
 * expert only when the upward gap is below M_tile/2, so by at most
 * floor((M_tile-1)/2) slots; TR_UP and TR_STOCHASTIC pad by at most
 * M_tile-1.  Hence slot_cap = min(T*K + E*pad, T*E) with pad = 0,
 * floor((M_tile-1)/2) or M_tile-1.
 */
typedef struct {
  int64_t slot_cap; /* upper bound on slots S (see above)                      */
  int64_t tile_cap; /* upper bound on M tiles: ceil(slot_cap/TILE_M) + E       */
  size_t ws_route;  /* workspace bytes moe_route needs                         */
  size_t ws_fwd;    /* workspace bytes moe_fwd needs                           */
  size_t ws_bwd;    /* workspace bytes moe_bwd needs                           */
  size_t ws_router; /* workspace bytes moe_router_bwd needs                    */
} moe_sizes_t;

/*
 * Routing metadata (the "routing metadata" the notes' key design 3 keeps
 * for the backward).  Every array is a caller-allocated device buffer.
 * Slots are in canonical order: experts ascending, and tokens ascending
 * inside an expert.  moe_route writes all of it; moe_fwd / moe_bwd read it.
 */
typedef struct {
  int32_t *tc_counts;      /* [E]        f_e, token-choice count per expert  */
  int32_t *counts;         /* [E]        r_e, final count (r_e = f_e for TC)  */
  int32_t *expert_offsets; /* [E+1]      exclusive scan of counts             */
  int32_t *expert_order;   /* [E]        experts by descending r_e (ties: e)  */
  int32_t *topk_ids;       /* [T*K]      token-choice experts, best first     */
  int32_t *slot_token;     /* [slot_cap] token of each slot                   */
  float *slot_weight;      /* [slot_cap] gate weight s = softmax prob p[t,e]  */
  int32_t *token_offsets;  /* [T+1]      CSR offsets of each token's slots    */
  int32_t *token_slots;    /* [slot_cap] a token's slots, ascending expert    */
  int32_t *tile_expert;    /* [tile_cap] expert of each M tile                */
  int32_t *tile_row;       /* [tile_cap] first slot row of each M tile        */
  int32_t *totals;         /* [2]        S, number of M tiles                 */
} moe_routing;

/*
 * Optional per-kernel timing.  When `trace` is non-NULL and trace->count is
 * at least the number of kernels the call launches plus one, the call
 * records trace->events[i] (hipEvent_t, created by the caller) on `stream`
 * before its i-th kernel and trace->events[kernels] after the last one.
 * moe_route launches 4 kernels (top-K, counts, selection with the offset
 * scan, token CSR), moe_fwd 3, moe_bwd 6 segments (the weight-gradient chunk
 * plans and schedules, dH, dX-tilde, dX aggregate, dW1, dW2; the dW segments
 * include the reduction of split experts), moe_router_fwd 1, moe_router_bwd 4
 * (dlogits, router dX, dWr partials, dWr reduction).  NULL disables tracing.
 */
typedef struct {
  void **events;
  int32_t count;
} moe_trace;

/* Host only; touches no device.  Validates `p` and fills `out`.
 * Errors: MOE_ERR_INVALID for null arguments or T, d, n, E, K, M_tile < 1,
 * K > E, unknown dtype/mode; MOE_ERR_UNSUPPORTED for K > 32, E > 1024,
 * d % 128 != 0, n not in {64, 128, 256, 384, 512}, M_tile > 1024, sizes whose
 * slot or element counts overflow 32-bit indexing, or an array that a kernel
 * addresses through a 32-bit byte extent exceeding 4 GiB - 1 bytes: X, dO,
 * O, dX (T x d); H, dH (slot_cap x 2n); Y, dX-tilde (slot_cap x d); one
 * expert of W1 (d x 2n) or W2 (n x d); Wr (E x d); logits (T x E fp32); the
 * router backward's padded copy of dlogits (T x ceil(E/128)*128).
 * Why these limits: the library's tile shapes cover d in multiples of
 * 128 and the listed n (the GEMM tiles take whole 128-column slabs of d and
 * whole gate/up halves of n); the routing kernels keep one token's experts
 * and one expert's ranking state in a workgroup (K <= 32, E <= 1024). */
int moe_sizes(const moe_problem *p, moe_sizes_t *out);

/*
 * Routing (notes, key design 1).  logits: [T, E] fp32 device buffer.
 *   p[t,e]  = softmax over the E logits of token t, evaluated in fp64;
 *   TopK(t) = the K largest fp32 logits, equal logits to the lower expert;
 *   non-finite logits count as finite ones first: NaN and -inf as -FLT_MAX,
 *   +inf as +FLT_MAX (reading: the pages' router scores are real numbers;
 *   this gives such inputs one ranking, a NaN below every number, and a
 *   finite softmax);
 *   f_e     = number of tokens whose TopK holds e;
 *   TC:  r_e = f_e and expert e keeps exactly those tokens;
 *   TR*: lo/hi = the multiples of M_tile just below/above f_e, and r_e is
 *        TR            hi when hi - f_e < f_e - lo, else lo (the notes' rule);
 *        TR_UP         hi;
 *        TR_DOWN       lo;
 *        TR_STOCHASTIC hi when round_rand[e] * M_tile < (f_e - lo) * 2^32
 *                      (integer comparison), else lo, so E[r_e] = f_e
 *                      (notes, key design 1: the expected total count is
 *                      that of token choice; the loss function / training
 *                      strategy section: the subroutine matters little);
 *        every TR mode takes hi only when hi <= T.  Expert e keeps the first
 *        r_e tokens ordered by (e in TopK(t), p[t,e]) descending, equal keys
 *        to the lower token;
 *   s = p[t,e] for every kept pair (no renormalisation).
 * round_rand: [E] uint32 device buffer of uniform draws, one per expert,
 * owned by the caller; required (4-byte aligned) for TR_STOCHASTIC, ignored
 * (may be NULL) otherwise.  MOE_ERR_INVALID if required and NULL.
 * ws: at least sizes.ws_route bytes.  Writes every field of `r`.
 */
int moe_route(const moe_problem *p, const float *logits, const uint32_t *round_rand,
              const moe_routing *r, void *ws, size_t ws_bytes, void *stream,
              const moe_trace *trace);

/*
 * moe_route without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  It computes exactly what moe_route computes, with
 * the same arguments and errors, but its workspace is a fixed array in the
 * library's device memory (one per GPU, MOE_NOALLOC_ROUTE_BYTES = 48 MiB,
 * held until the process ends) instead of a caller buffer; it calls no
 * allocator.  Problems whose sizes.ws_route exceeds MOE_NOALLOC_ROUTE_BYTES
 * (E * T * 8 bytes of sort keys plus about 3%: E * T up to about 6.1M, e.g.
 * T = 16384 tokens with E = 256, or T = 8192 with E = 512) return
 * MOE_ERR_WORKSPACE before anything is enqueued.  Every call on one GPU
 * shares that array: calls that overlap on one GPU (on different streams,
 * or from different threads without ordering) race and must not be made.
 * No part of the array needs to start at zero (each call writes every byte
 * it reads).  The first call on a device looks the array's address up
 * (hipGetSymbolAddress; no allocation) with that device current.
 */
#define MOE_NOALLOC_ROUTE_BYTES (48 * 1024 * 1024)
int moe_route_noalloc(const moe_problem *p, const float *logits, const uint32_t *round_rand,
                      const moe_routing *r, void *stream, const moe_trace *trace);

/*
 * Forward (notes, method > overall framework; key design 2).  For every
 * expert e with kept tokens I_e:
 *   H_e = X[I_e] W1_e          (rows gathered inside the GEMM operand load)
 *   A_e = SiLU(H_e[:, :n]) * H_e[:, n:]   (epilogue, from H rounded to dtype)
 *   Y_e = A_e W2_e
 *   O[t] = sum over t's slots of s * Y   (a token without slots gets 0)
 * Outputs: O [T, d]; H [rows, 2n] with rows >= S (slot_cap always suffices;
 * a caller that has read S = totals[0] back may allocate exactly S rows),
 * saved for moe_bwd.  Only rows [0, S) of H are written or, by moe_bwd,
 * read; the library cannot check `rows` and a smaller H is overrun.
 * ws: at least sizes.ws_fwd bytes (holds the transient A and Y).
 */
int moe_fwd(const moe_problem *p, const void *X, const void *W1,
            const void *W2, const moe_routing *r, void *O, void *H, void *ws,
            size_t ws_bytes, void *stream, const moe_trace *trace);

/*
 * Minimal-activation backward (notes, key designs 2 and 3).  Reads only
 * dO, X, H, W1, W2 and the routing; never Y or a gathered copy of X.
 *   dA'_e = dO[I_e] W2_e^T, A recomputed from H,
 *   dS    = rowsum(dA' * A)          (per slot, fp32, not scaled by s)
 *   dA    = s * dA',  dH = [dA * u * sig(g) * (1 + g (1 - sig(g))),
 *                           dA * SiLU(g)]  with g, u the halves of H
 *   dX[t] = sum over t's slots of dH W1_e^T
 *   dW1_e = X[I_e]^T dH_e,   dW2_e = (s * A_e)^T dO[I_e]   (varlen-K)
 * H: as moe_fwd wrote it (at least S rows).
 * Outputs: dX [T, d], dW1 [E, d, 2n], dW2 [E, n, d] (experts without slots
 * get zeros), dS [slot_cap] fp32 with rows [0, S) valid.
 * ws: at least sizes.ws_bwd bytes.
 * Order: dH first; then dX (dX-tilde, its aggregation) on `stream` and, on
 * the library's second stream of this device, dW1 then dW2, joined back to
 * `stream`.  With a trace, or when `stream` belongs to another device than
 * the current one, all five run in order on `stream` instead.
 * Concurrent calls on one device share that stream (a mutex orders their
 * fork/join); the results do not depend on which path ran.  The first
 * untraced call on a device creates the stream and its two events, so make
 * one such call before capturing `stream` into a graph.
 */
int moe_bwd(const moe_problem *p, const void *dO, const void *X, const void *H,
            const void *W1, const void *W2, const moe_routing *r, void *dX,
            void *dW1, void *dW2, float *dS, void *ws, size_t ws_bytes,
            void *stream, const moe_trace *trace);

/*
 * Backward of the gate weights alone (notes, method > overall framework: the
 * layer's backward yields the router gradients; dS is the layer's
 * router-facing output).  With s = softmax(logits[t])[e] for every kept pair
 * (no renormalisation) and g[t, e] = dS of the slot of (t, e), 0 where the
 * pair is not kept (routing decisions carry no gradient):
 *   dlogits[t] = p[t] * (g[t] - <p[t], g[t]>),  p = softmax(logits[t]) (fp32,
 *                non-finite logits replaced as moe_route does)
 * For callers whose router is not the linear map of moe_router_fwd: they
 * take dlogits into their own router's backward.  Inputs: logits [T, E] fp32
 * (those moe_route read), dS [slot_cap] fp32 from moe_bwd, `r` from
 * moe_route.  Output: dlogits [T, E] fp32.  All device buffers, caller-owned,
 * 16-byte aligned; no workspace; asynchronous on `stream`; a trace records 1
 * kernel.  Errors as moe_sizes, MOE_ERR_INVALID for null or misaligned
 * buffers.
 */
int moe_gate_bwd(const moe_problem *p, const float *logits, const float *dS,
                 const moe_routing *r, float *dlogits, void *stream, const moe_trace *trace);

/*
 * Router forward (notes, method > overall framework and key design 1: tokens
 * are routed by their router scores).  Reading: the router is a linear map
 * with one row per expert.
 *   logits[t, e] = sum_i X[t, i] Wr[e, i]   fp32 result, fp32 accumulation
 * X: [T, d] and Wr: [E, d] in p->dtype; logits: [T, E] fp32 (what moe_route
 * reads).  All device buffers, caller-owned, 16-byte aligned; asynchronous
 * on `stream`.  Errors as moe_sizes, MOE_ERR_INVALID for null or misaligned
 * buffers.
 */
int moe_router_fwd(const moe_problem *p, const void *X, const void *Wr, float *logits,
                   void *stream, const moe_trace *trace);

/*
 * Router backward (notes, method > overall framework: the layer's backward
 * yields the router gradients; dS is what moe_bwd hands to the router).  The
 * gate weight of a kept pair is s = softmax(logits[t])[e], so with g[t, e] =
 * dS of the slot of (t, e) (0 where the pair is not kept; routing decisions
 * carry no gradient):
 *   dlogits[t] = p[t] * (g[t] - <p[t], g[t]>),  p = softmax(logits[t]) (fp32)
 *   dWr        = dlogits^T X                    [E, d], p->dtype
 *   dX        += dlogits Wr                     [T, d], p->dtype, in place:
 *                the router's share of the input gradient is added to the
 *                experts' share that moe_bwd wrote
 * Inputs: X, Wr as in moe_router_fwd; logits [T, E] fp32; dS [slot_cap] fp32
 * from moe_bwd; `r` from moe_route.  Outputs: dlogits [T, E] fp32, dWr, dX.
 * ws: at least sizes.ws_router bytes.
 */
int moe_router_bwd(const moe_problem *p, const void *X, const void *Wr, const float *logits,
                   const float *dS, const moe_routing *r, float *dlogits, void *dWr, void *dX,
                   void *ws, size_t ws_bytes, void *stream, const moe_trace *trace);

/* Static, NUL-terminated description of a moe_status value. */
const char *moe_status_string(int status);

/* MOE_ABI_VERSION of the built library. */
int moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
