"""Benchmark of the MoE layer forward+backward on one MI355X.

A step is one pass of the whole path on one batch of synthetic input:
moe_route (top-K + token rounding) -> moe_fwd (up-proj + SwiGLU, down-proj,
aggregation) -> moe_bwd (dH + dS, dX-tilde, dX aggregation, dW1, dW2).
The step is credited with 6TnKd forward + 12TnKd backward FLOPs.

Prints ONE JSON line.  `roofline` describes the kernel with the largest
average duration, timed live with HIP events recorded on the library's stream
between its launches; `cpu_baseline` times the fp64 oracle on a bounded
sample of the same workload (a subset of the experts) on the host cores.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--config 7b]
                       [--mode tc|tr|tr_up|tr_down|tr_stochastic] [--no-cpu-baseline]
       python bench.py --sweep   (TC vs token rounding at 1, 2, 4, 8 tiles per expert)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from fine_grained_mixture_amd import moe  # noqa: E402
from fine_grained_mixture_amd.inputs import (SHAPES, make_layer_inputs,  # noqa: E402
                                             make_round_rand, make_router_weight,
                                             round_rand_tensor)
from fine_grained_mixture_amd.profiling import kernel_model, read_traffic  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3    # MI355X fp32 (matrix and vector)
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
KERNEL_NAMES = [f"route:{k}" for k in moe.ROUTE_KERNELS] + list(moe.FWD_KERNELS) + \
    list(moe.BWD_KERNELS)


def restrict_routing(rt, keep):
    """Oracle routing restricted to the experts in `keep` (the others empty)."""
    from oracle import moe_oracle as orc

    E = len(rt.counts)
    sel = np.isin(rt.slot_expert, keep)
    slot_token = rt.slot_token[sel]
    slot_expert = rt.slot_expert[sel]
    counts = np.bincount(slot_expert, minlength=E)
    offsets = np.zeros(E + 1, np.int64)
    offsets[1:] = np.cumsum(counts)
    T = len(rt.token_offsets) - 1
    order = np.argsort(slot_token, kind="stable")
    toff = np.zeros(T + 1, np.int64)
    toff[1:] = np.cumsum(np.bincount(slot_token, minlength=T))
    return orc.Routing(rt.topk_ids, rt.tc_counts, counts, offsets, slot_token, slot_expert,
                       rt.slot_weight[sel], toff, order, rt.probs)


def cpu_baseline(sh, inp, mode, target_s=15.0):
    """fp64 oracle on a sample of experts: route (full), forward, backward."""
    from oracle import moe_oracle as orc

    threads, blas = os.cpu_count(), "unknown"
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            threads = sum(i.get("num_threads", 0) for i in libs) or threads
            blas = ", ".join(f"{i.get('internal_api')} {i.get('version')} "
                             f"({i.get('num_threads')} threads)" for i in libs)
    except Exception:  # pragma: no cover
        pass
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    a = {k: v.float().numpy().astype(np.float64) for k, v in inp.items() if k != "logits"}
    logits = inp["logits"].numpy()
    t0 = time.perf_counter()
    modes = {"tc": orc.TC, "tr": orc.TR, "tr_up": orc.TR_UP, "tr_down": orc.TR_DOWN,
             "tr_stochastic": orc.TR_STOCHASTIC}
    rt = orc.route(logits, sh.K, sh.M, modes[mode], make_round_rand(sh.E, 0))
    t_route = time.perf_counter() - t0
    # Grow the expert sample until the timed fwd+bwd takes a few seconds.
    order = np.argsort(-rt.counts, kind="stable")
    n_exp, spent, best = 2, 0.0, None
    while True:
        keep = order[:: max(1, len(order) // n_exp)][:n_exp]
        sub = restrict_routing(rt, keep)
        t0 = time.perf_counter()
        _, c = orc.forward(a["X"], a["W1"], a["W2"], sub)
        orc.backward_minimal(a["dO"], a["X"], c["H"], a["W1"], a["W2"], sub)
        dt = time.perf_counter() - t0
        spent += dt
        best = (sub.S, dt, len(keep))
        if dt > target_s / 3 or n_exp >= len(order) or spent > target_s:
            break
        n_exp = min(len(order), n_exp * 2)
    S_s, dt, ne = best
    flops = 18 * S_s * sh.n * sh.d
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOPS",
        "cores": int(threads),
        "cpu_model": cpu_model,
        "blas": blas,
        "kind": "oracle",
        "sample": f"fp64 numpy oracle: full routing ({t_route:.2f} s) + forward and minimal "
                  f"backward over {ne} of {sh.E} experts ({S_s} of {rt.S} slots, "
                  f"{flops / 1e9:.1f} GFLOP in {dt:.2f} s), scaled to TFLOPS",
    }


def _pct(v):
    v = np.asarray(v)
    return {"median": round(float(np.median(v)), 4), "p10": round(float(np.percentile(v, 10)), 4),
            "p90": round(float(np.percentile(v, 90)), 4)}


def measure(sh, mode, steps, warmup, dev, T=None, stats=False, traced_only=False, cold=False):
    """Times `steps` route+fwd+bwd steps of layer `sh` (T tokens if given) in
    routing mode `mode` after `warmup` untimed ones.  Returns the mean step
    time, the mean time of every kernel (trace events on the stream), the
    slot count S and the number of 128-row M tiles.  The mean step time is
    that of back-to-back steps (`ms_warm`), or with `cold` that of steps each
    timed alone after a 512 MiB buffer was written outside its timing
    (`ms_cold`: no input left in L2 or the Infinity Cache).  With `stats`, also the
    median / p10 / p90 of single steps, warm (back to back) and cold (a
    512 MiB buffer written before each step, outside its timing, so that
    no input is left in L2 or the Infinity Cache).  With `traced_only`, every
    step (warm-up included) is traced and the step time is the traced one:
    the profiler's run, whose per-kernel averages then cover exactly the
    launches that `per_ms` times."""
    inp = make_layer_inputs(sh, dtype=torch.bfloat16, seed=0, T=T)
    T = sh.T if T is None else T
    X, W1, W2, lg, dO = (inp[k].to(dev) for k in ("X", "W1", "W2", "logits", "dO"))
    rr = round_rand_tensor(make_round_rand(sh.E, 0)).to(dev)  # stochastic rounding draws
    p = moe.problem(T, sh.d, sh.n, sh.E, sh.K, sh.M, torch.bfloat16, mode)
    sz = moe.sizes(p)
    rt = moe.alloc_routing(p, dev)
    ws_r = moe.workspace(sz.ws_route, dev)
    ws_f = moe.workspace(sz.ws_fwd, dev)
    ws_b = moe.workspace(sz.ws_bwd, dev)
    O = torch.empty(T, sh.d, dtype=torch.bfloat16, device=dev)
    H = torch.empty(sz.slot_cap, 2 * sh.n, dtype=torch.bfloat16, device=dev)
    grads = (torch.empty_like(X), torch.empty_like(W1), torch.empty_like(W2),
             torch.empty(sz.slot_cap, dtype=torch.float32, device=dev))
    stream = torch.cuda.current_stream(dev)

    def mk(k):
        # torch creates an event's handle on its first record
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(k)]
        for e in evs:
            e.record(stream)
        return evs

    def step(ev=None):
        e_r, e_f, e_b = ev if ev else (None, None, None)
        moe.route(p, lg, rt=rt, ws=ws_r, stream=stream, events=e_r, round_rand=rr)
        moe.forward(p, X, W1, W2, rt, out=(O, H), ws=ws_f, stream=stream, events=e_f)
        moe.backward(p, dO, X, H, W1, W2, rt, out=grads, ws=ws_b, stream=stream, events=e_b)

    def traced_events(k):
        return [(mk(len(moe.ROUTE_KERNELS) + 1), mk(len(moe.FWD_KERNELS) + 1),
                 mk(len(moe.BWD_KERNELS) + 1)) for _ in range(k)]

    if traced_only:
        # every launch traced (a traced backward runs its kernels in order), so
        # a profiler's per-kernel averages cover the same launches as `per_ms`
        for ev in traced_events(warmup):
            step(ev)
        torch.cuda.synchronize()
    else:
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        # The step time comes from steps without trace events (an event record
        # costs GPU time of its own: about 3 us each, 50 us per step); the
        # per-kernel times come from the same number of traced steps right
        # after.
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(steps):
            step()
        stop.record(stream)
        torch.cuda.synchronize()
        ms_warm = start.elapsed_time(stop) / steps
        ms = ms_warm
        if cold:
            scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
            pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                     for _ in range(steps)]
            torch.cuda.synchronize()
            for i, (a, b) in enumerate(pairs):
                scratch.fill_(i & 255)  # evicts L2 and the Infinity Cache, untimed
                a.record(stream)
                step()
                b.record(stream)
            torch.cuda.synchronize()
            ms = float(np.mean([a.elapsed_time(b) for a, b in pairs]))
            del scratch
    evs = traced_events(steps)
    torch.cuda.synchronize()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    if traced_only:
        ms = float(np.mean([e_r[0].elapsed_time(e_b[-1]) for e_r, _, e_b in evs]))
    per = np.zeros(len(KERNEL_NAMES))
    for e_r, e_f, e_b in evs:
        d = [a.elapsed_time(b) for group in (e_r, e_f, e_b) for a, b in zip(group, group[1:])]
        per += np.array(d)
    per /= steps
    out = {"ms": ms, "per_ms": per, "S": int(rt.totals[0].item()),
           "tiles": int(rt.totals[1].item()), "E_act": int(np.count_nonzero(rt.counts.cpu().numpy()))}
    if not traced_only:
        out["ms_warm"] = ms_warm
    if stats:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        for cold in (False, True):
            pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                     for _ in range(steps)]
            torch.cuda.synchronize()
            for i, (a, b) in enumerate(pairs):
                if cold:
                    scratch.fill_(i & 255)
                a.record(stream)
                step()
                b.record(stream)
            torch.cuda.synchronize()
            out["cold" if cold else "warm"] = _pct([a.elapsed_time(b) for a, b in pairs])
        del scratch
    return out


def measure_router(sh, steps, warmup, dev):
    """Router forward (logits = X Wr^T) and backward (dlogits, dX += dl Wr,
    dWr) of layer `sh`, outside the metric's step: dS comes from one layer
    step.  Returns the mean time of each router kernel in ms."""
    inp = make_layer_inputs(sh, dtype=torch.bfloat16, seed=0)
    X, W1, W2, dO = (inp[k].to(dev) for k in ("X", "W1", "W2", "dO"))
    Wr = make_router_weight(sh, torch.bfloat16, seed=0).to(dev)
    p = moe.problem(sh.T, sh.d, sh.n, sh.E, sh.K, sh.M, torch.bfloat16, "tr")
    lg = moe.router_forward(p, X, Wr)
    rt = moe.route(p, lg)
    O, H = moe.forward(p, X, W1, W2, rt)
    dX, dW1, dW2, dS = moe.backward(p, dO, X, H, W1, W2, rt)
    ws = moe.workspace(moe.sizes(p).ws_router, dev)
    out = (torch.empty(sh.T, sh.E, dtype=torch.float32, device=dev),
           torch.empty(sh.E, sh.d, dtype=torch.bfloat16, device=dev))
    stream = torch.cuda.current_stream(dev)

    def mk(k):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(k)]
        for e in evs:
            e.record(stream)
        return evs

    def step(ev=None):
        ef, eb = ev if ev else (None, None)
        moe.router_forward(p, X, Wr, out=lg, stream=stream, events=ef)
        moe.router_backward(p, X, Wr, lg, dS, rt, dX, out=out, ws=ws, stream=stream, events=eb)

    for _ in range(warmup):
        step()
    evs = [(mk(len(moe.ROUTER_FWD_KERNELS) + 1), mk(len(moe.ROUTER_BWD_KERNELS) + 1))
           for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    names = list(moe.ROUTER_FWD_KERNELS) + list(moe.ROUTER_BWD_KERNELS)
    per = np.zeros(len(names))
    for ef, eb in evs:
        per += np.array([a.elapsed_time(b) for g in (ef, eb) for a, b in zip(g, g[1:])])
    return dict(zip(names, per / steps))


def router_line(sh, per_ms):
    """Router kernel times with the FLOPs of the two GEMM-shaped ones."""
    out = {}
    gemm = {"router_logits": 2 * sh.T * sh.d * sh.E, "router_dx": 2 * sh.T * sh.E * sh.d,
            "router_dw": 2 * sh.T * sh.E * sh.d}
    for k, t in per_ms.items():
        out[k] = {"us": round(t * 1e3, 2)}
        if k in gemm:
            out[k]["tflops"] = round(gemm[k] / (t / 1e3) / 1e12, 1)
    out["fwd_us"] = round(per_ms["router_logits"] * 1e3, 2)
    out["bwd_us"] = round(sum(v for k, v in per_ms.items() if k != "router_logits") * 1e3, 2)
    return out


def sweep(dev, steps, warmup):
    """Token choice against every token-rounding subroutine at average
    tokens per expert T_e = T K / E of 1, 2, 4 and 8 M-tiles (the 7B layer's
    width, T varied).  One JSON line per point: step time, slots S, executed
    rows (whole 128-row tiles), padding waste, and TFLOPS counted on the
    slots (useful) and on the executed rows."""
    sh = SHAPES["7b"]
    for ratio in (1, 2, 4, 8):
        T = ratio * sh.M * sh.E // sh.K
        for mode in ("tc", "tr", "tr_up", "tr_down", "tr_stochastic"):
            r = measure(sh, mode, steps, warmup, dev, T=T)
            rows = r["tiles"] * moe.TILE_M
            per_row = 18 * sh.n * sh.d / (r["ms"] / 1e3) / 1e12
            print(json.dumps({"tokens_per_expert_in_tiles": ratio, "T": T, "mode": mode,
                              "ms_per_step": round(r["ms"], 4), "slots": r["S"],
                              "executed_rows": rows,
                              "padding_waste": round((rows - r["S"]) / rows, 4),
                              "useful_tflops": round(r["S"] * per_row, 1),
                              "executed_tflops": round(rows * per_row, 1)}), flush=True)


def requested_bytes(dev):
    """Bytes of live tensors as requested from the torch allocator."""
    return torch.cuda.memory_stats(dev)["requested_bytes.all.current"]


def saved_activation_bytes(sh, mode, dev):
    """Device bytes MoELayerFunction holds for its backward after its forward,
    measured with the torch allocator (bytes of live tensors still requested
    beyond the inputs and the output O): H with exactly S rows, and the routing
    metadata.  X, an input, is kept by reference.  Returns (X bytes, H
    bytes, metadata bytes, measured bytes held, S)."""
    inp = make_layer_inputs(sh, dtype=torch.bfloat16, seed=0)
    X, W1, W2 = (inp[k].to(dev).requires_grad_(True) for k in ("X", "W1", "W2"))
    lg = inp["logits"].to(dev)
    torch.cuda.synchronize()
    before = requested_bytes(dev)
    O = moe.moe_layer(X, W1, W2, lg, sh.K, sh.M, mode)
    torch.cuda.synchronize()
    held = requested_bytes(dev) - before - O.numel() * O.element_size()
    _, H, _, _, _ = O.grad_fn.saved_tensors
    _, rt = O.grad_fn.moe
    meta = sum(t.numel() * t.element_size() for t in rt.tensors.values())
    return (X.numel() * X.element_size(), H.numel() * H.element_size(), meta, held, rt.S)


def granularity_sweep(dev, steps, warmup):
    """Iso-FLOP sweep over granularity G = d/n at d = 1024, T = 16384 and
    sparsity K/E = 1/16, with nK = 1024 fixed (so 18 T n K d is the same at
    every point): G = 2, 4, 8, 16 -> (n, K, E) = (512, 2, 32), (256, 4, 64),
    (128, 8, 128), (64, 16, 256); token rounding.  One JSON line per point:
    step time, TFLOPS, the forward arithmetic intensity, the activation bytes
    the layer's autograd op was measured to hold for its backward (X, H and
    the routing metadata), and, for comparison, what a backward that caches
    every intermediate would keep (the gathered X rows, H, A and Y on top of
    X: a formula, that backward is not built)."""
    from fine_grained_mixture_amd.inputs import LayerShape
    from fine_grained_mixture_amd.profiling import activation_bytes, arithmetic_intensity

    T, d = 16384, 1024
    for G in (2, 4, 8, 16):
        n = d // G
        K = 1024 // n
        E = 16 * K
        sh = LayerShape(f"g{G}", T, d, n, E, K, 128, "fan_in", "normal_bias")
        r = measure(sh, "tr", steps, warmup, dev)
        xb, hb, meta, held, S = saved_activation_bytes(sh, "tr", dev)
        print(json.dumps({"G": G, "n": n, "K": K, "E": E, "T": T, "d": d, "S": S,
                          "ms_per_step": round(r["ms"], 4),
                          "tflops": round(sh.flops / (r["ms"] / 1e3) / 1e12, 1),
                          "arithmetic_intensity": round(arithmetic_intensity(T, d, n, K, E), 1),
                          "saved_bytes_measured": xb + held,
                          "saved_x_h_bytes": xb + hb, "saved_metadata_bytes": meta,
                          "saved_bytes_2Td_4TKn": 2 * T * d + 4 * T * K * n,
                          "saved_bytes_caching_formula":
                              activation_bytes(T, d, n, K, S)["caching"]}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="7b", choices=sorted(SHAPES))
    ap.add_argument("--mode", default="tr", choices=sorted(moe.ROUTE_MODES))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the timed and traced steps of --mode (no single-step statistics, "
                         "no token-choice line): what the profiler runs")
    ap.add_argument("--traced-only", action="store_true",
                    help="every step traced (the backward then runs its kernels in order), "
                         "step time from the traced steps: what the profiler runs, so that its "
                         "per-kernel averages match the per-kernel times printed")
    ap.add_argument("--granularity", action="store_true",
                    help="instead of the benchmark line: iso-FLOP sweep over d/n = 2, 4, 8, 16 "
                         "(one JSON line per point)")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the benchmark line: TC vs token rounding at 1, 2, 4 and 8 "
                         "M-tiles of tokens per expert (one JSON line per point)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (known HBM "
                         "traffic: 1 GiB read + 1 GiB written per launch), to scale the "
                         "FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(collectives and sharding are out of scope); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        src = torch.ones(1 << 29, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 1 << 30, "copy_bytes_written": 1 << 30,
                          "launches": 5}))
        return
    if args.sweep:
        sweep(dev, args.steps, args.warmup)
        return
    if args.granularity:
        granularity_sweep(dev, args.steps, args.warmup)
        return
    sh = SHAPES[args.config]
    r = measure(sh, args.mode, args.steps, args.warmup, dev,
                stats=not (args.no_extras or args.traced_only), traced_only=args.traced_only,
                cold=not args.traced_only)
    ms, per, names = r["ms"], r["per_ms"], KERNEL_NAMES
    S = r["S"]
    flops = sh.flops
    tflops = flops / (ms / 1e3) / 1e12

    # roofline of the dominant kernel
    dom = int(np.argmax(per))
    dname = names[dom]
    E_act = r["E_act"]
    f_k, b_k = kernel_model(dname, sh, S, E_act=E_act) or (0, 0)
    t_mfma, t_hbm = f_k / (PEAK_BF16_TFLOPS * 1e12), b_k / (PEAK_HBM_GBS * 1e9)
    dur = per[dom] / 1e3
    if f_k and t_mfma >= t_hbm:
        roof = {"bound": "mfma", "achieved": f_k / dur / 1e12, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": b_k / dur / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    # HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE summary of
    # this workload, when it was taken on the current kernel sources
    roof["traffic"] = read_traffic(
        os.path.join(ROOT, "profiles", f"hbm_traffic_{sh.name}_{args.mode}.md"), dname)
    roof["algorithmic_bytes"] = b_k
    roof["kernel"] = dname
    roof["avg_us"] = per[dom] * 1e3

    kernels = {}
    for k, t in zip(names, per):
        fk, bk = kernel_model(k, sh, S, E_act=E_act) or (0, 0)
        kernels[k] = {"us": round(t * 1e3, 2)}
        if fk:
            kernels[k]["tflops"] = round(fk / (t / 1e3) / 1e12, 1)
            kernels[k]["mfma_frac"] = round(fk / (t / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 3)
        if bk:
            kernels[k]["gbs"] = round(bk / (t / 1e3) / 1e9, 1)
            kernels[k]["hbm_frac"] = round(bk / (t / 1e3) / 1e9 / PEAK_HBM_GBS, 3)

    out = {
        "metric": "MoE layer fwd+bwd TFLOPS (bf16) + % MFMA peak, T=16k d=1536 E=128 K=8",
        "value": tflops,
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{sh.name} MoE layer fwd+bwd, {args.mode.upper()} routing",
                   "T": sh.T, "d": sh.d, "n": sh.n, "E": sh.E, "K": sh.K, "M_tile": sh.M,
                   "slots": S, "active_experts": E_act, "parallelism": "single GPU"},
        "pct_mfma_peak": 100.0 * tflops / PEAK_BF16_TFLOPS,
        # 18 n d per slot actually routed, and per row executed (whole tiles)
        "useful_tflops": 18 * S * sh.n * sh.d / (ms / 1e3) / 1e12,
        "executed_tflops": 18 * r["tiles"] * moe.TILE_M * sh.n * sh.d / (ms / 1e3) / 1e12,
        # single steps: back to back (warm) and after evicting L2 and the
        # Infinity Cache (cold), ms
        "step_ms": {"warm": r.get("warm"), "cold": r.get("cold")},
        # how ms_per_step was timed: untraced steps (dW1/dW2 beside dX-tilde),
        # each after L2 and the Infinity Cache were evicted (cold), or traced
        # back-to-back ones (every kernel in order, plus the events' own cost)
        "timing": "traced" if args.traced_only else "untraced, cold",
        # the same untraced steps back to back (inputs partly cached)
        "warm": None if args.traced_only else {
            "ms_per_step": r["ms_warm"], "tflops": flops / (r["ms_warm"] / 1e3) / 1e12},
        "roofline": roof,
        "kernels_us": kernels,
    }
    if not args.traced_only:
        # outside the metric's step (its FLOPs are not in 18 T n K d); its set-up
        # runs one untraced layer step, which a profiler would count
        out["router"] = router_line(sh, measure_router(sh, args.steps, args.warmup, dev))
    if args.mode != "tc" and not (args.no_extras or args.traced_only):
        # token choice on the same inputs: the padding its tiles execute
        t = measure(sh, "tc", args.steps, args.warmup, dev, cold=True)
        fl = 18 * sh.n * sh.d / (t["ms"] / 1e3) / 1e12
        out["tc"] = {"ms_per_step": round(t["ms"], 4), "slots": t["S"],
                     "executed_rows": t["tiles"] * moe.TILE_M,
                     "useful_tflops": round(t["S"] * fl, 1),
                     "executed_tflops": round(t["tiles"] * moe.TILE_M * fl, 1)}
    if not args.no_cpu_baseline:
        inp = make_layer_inputs(sh, dtype=torch.bfloat16, seed=0)  # the same seeded inputs
        out["cpu_baseline"] = cpu_baseline(sh, inp, args.mode)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
