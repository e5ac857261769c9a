"""Kernel cost model and rocprofv3 summaries for the MoE layer.

* ``kernel_model``: algorithmic FLOPs and HBM bytes of one launch of each
  kernel, from the layer shape and the slot count.  These are what the method
  has to move: gathered rows once per slot, weights once, each transient
  written once and read once, outputs once, and no padded work.
* ``kernel_sources_sha256``: a digest of the HIP sources and the C header,
  which stamps every counter summary, so that a stale summary (taken on
  kernels that have changed since) is never reported as current.
* Command line: turns the CSV files of rocprofv3 runs into the short text
  summaries kept under ``profiles/``:

    python -m fine_grained_mixture_amd.profiling stats <kernel_stats.csv> <cmd>
    python -m fine_grained_mixture_amd.profiling traffic --fetch F.csv --write W.csv \
        --cal-fetch CF.csv --cal-write CW.csv --config 7b --slots S <cmd>

  ``traffic`` scales the FETCH_SIZE / WRITE_SIZE counters (KiB per dispatch)
  by what the same counters read for a plain 1 GiB device-to-device copy of
  known traffic (1 GiB read and 1 GiB written per launch).

    python -m fine_grained_mixture_amd.profiling mfma <counter_collection.csv> \
        --config 7b --slots S <cmd>

  ``mfma`` reads SQ_VALU_MFMA_BUSY_CYCLES (MFMA-pipe cycles summed over every
  SIMD: a 32x32x16 bf16 MFMA counts 32) and GRBM_GUI_ACTIVE (GPU-busy clock
  cycles summed over the 8 XCDs) of each dispatch, with the dispatch's own
  start and end times: MFMA utilisation is the busy cycles over the SIMD
  cycles the kernel had (GRBM_GUI_ACTIVE / 8 x 1024 SIMDs), and the average
  clock is GRBM_GUI_ACTIVE / 8 over the duration.

    python -m fine_grained_mixture_amd.profiling pipeline --csv C1.csv --csv C2.csv ... <cmd> ...

  ``pipeline`` summarises the vector-memory path of each kernel from the
  counter runs given (any split of the counters over runs): the mean latency
  of an L1 -> L2 read request (TCP_TCC_READ_REQ_LATENCY / TCP_TCC_READ_REQ, in
  cycles), the read requests per CU per cycle, their product (requests in
  flight per CU), the L2 hit rate, the mean latency of an L2 -> memory read
  (TCC_EA0_RDREQ_LEVEL / TCC_EA0_RDREQ), and the busy fractions of the
  address (TA) and data (TD) units, of TD waiting on the L1, and of the L1
  waiting on the L2 (TCP_PENDING_STALL_CYCLES), each per CU over the kernel's
  cycles (GRBM_GUI_ACTIVE / 8).
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import os
import re
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)

# rocprofv3 kernel name -> the name the benchmark and the trace events use
KERNEL_LABELS = {
    "k_up_swiglu": "up_swiglu", "k_down": "down", "k_dh": "dh", "k_dxt": "dxt",
    "k_dw1": "dw1", "k_dw2": "dw2",
    # persistent launches of the same steps
    "k_down_p": "down", "k_dxt_p": "dxt", "k_dxt_r": "dxt",
}
# kernels launched twice per step, labelled by launch order: the aggregation
# (forward O, then backward dX) and the persistent weight-gradient kernel
# (dW1, then dW2) when rocprofv3 truncates its template arguments
AGGREGATE_LABELS = ("aggregate_O", "aggregate_dX")
TWICE = {"k_aggregate": AGGREGATE_LABELS, "k_dw_p": ("dw1", "dw2")}


class _Labeller:
    """Step labels of base kernel names, fed in dispatch order."""

    def __init__(self):
        self.seen = collections.Counter()

    def __call__(self, k):
        if k in TWICE:
            lab = TWICE[k][self.seen[k] % 2]
            self.seen[k] += 1
            return lab
        return KERNEL_LABELS.get(k, k)
COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_BYTES = 1 << 30
NUM_XCD, NUM_SIMD = 8, 1024  # MI355X: 8 XCDs, 256 CUs of 4 SIMDs
PEAK_BF16_FLOPS = 2.5e15


def kernel_model(name, sh, S, esz=2, E_act=None):
    """(FLOPs, bytes) of one launch of kernel `name` for layer shape `sh`
    with S slots (bf16 when esz = 2), or None for kernels without a model.
    E_act is the number of experts given at least one slot (default: all):
    the forward and dH / dX-tilde GEMMs read only those experts' weights,
    while dW1 / dW2 write the gradient of every expert (zero for the rest)."""
    T, d, n, E = sh.T, sh.d, sh.n, sh.E
    Ea = E if E_act is None else E_act
    idx = 4 * S  # one int32 per slot
    m = {
        "up_swiglu": (4 * S * d * n, esz * (S * d + Ea * d * 2 * n + S * 2 * n + S * n) + idx),
        "down": (2 * S * n * d, esz * (S * n + Ea * n * d + S * d)),
        "aggregate_O": (2 * S * d, esz * (S * d + T * d) + 2 * idx + 4 * T),
        "dh": (2 * S * d * n, esz * (S * d + Ea * n * d + S * 2 * n + S * 2 * n + S * n)
               + 4 * S + 2 * idx),
        "dxt": (4 * S * n * d, esz * (S * 2 * n + Ea * d * 2 * n + S * d)),
        "aggregate_dX": (S * d, esz * (S * d + T * d) + idx + 4 * T),
        "dw1": (4 * S * d * n, esz * (S * d + S * 2 * n + E * d * 2 * n) + idx),
        "dw2": (2 * S * n * d, esz * (S * n + S * d + E * n * d) + idx),
    }
    return m.get(name)


def arithmetic_intensity(T, d, n, K, E):
    """Forward arithmetic intensity (FLOP per byte) of a fine-grained MoE
    layer as the notes state it (background and motivation, with G = d/n and
    rho = K/E), in the dimensionally consistent reading
    3 / ((2 + 2G)/d + 3/(T rho)): a byte count of the forward (X_e read, W1,
    A written and read, W2, Y written; the H write-back left out)."""
    G, rho = d / n, K / E
    return 3.0 / ((2.0 + 2.0 * G) / d + 3.0 / (T * rho))


def activation_bytes(T, d, n, K, S, esz=2):
    """Bytes kept from the forward for the backward.  minimal: X and H (S
    rows of 2n) in the operand type (notes, key design 3: 2Td + 4TKn at S =
    TK for bf16).  caching: what a backward that keeps every intermediate
    holds besides: the gathered X_e, A and Y (S rows of d, n and d)."""
    minimal = esz * (T * d + S * 2 * n)
    return {"minimal": minimal, "caching": minimal + esz * (S * d + S * n + S * d)}


def kernel_sources_sha256(root=ROOT):
    """sha256 over the kernel sources (csrc/*.hip, *.hpp) and include/*.h."""
    files = sorted(glob.glob(os.path.join(root, "fine_grained_mixture_amd", "csrc", "*.hip")) +
                   glob.glob(os.path.join(root, "fine_grained_mixture_amd", "csrc", "*.hpp")) +
                   glob.glob(os.path.join(root, "include", "*.h")))
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.relpath(f, root).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _base_name(kernel_name):
    m = re.search(r"(k_\w+|route_\w+|__amd_rocclr_\w+)", kernel_name)
    if not m:
        return kernel_name
    if m.group(1) == "k_dw_p" and "<" in kernel_name:
        # one template for both steps: dW1 gathers A (X), dW2 gathers B (dO)
        return "k_dw1" if re.search(r"k_dw_p<.*,\s*true,\s*false>", kernel_name) else "k_dw2"
    return m.group(1)


def counter_per_dispatch(path, counter):
    """{label: [value per dispatch, in dispatch order]} of one counter."""
    rows = []
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] == counter:
                rows.append((int(r["Dispatch_Id"]), _base_name(r["Kernel_Name"]),
                             float(r["Counter_Value"])))
    rows.sort()
    out = collections.defaultdict(list)
    label = _Labeller()
    for _, k, v in rows:
        out[label(k)].append(v)
    return out


def _mean(v):
    return sum(v) / len(v)


def traffic_table(fetch_csv, write_csv, cal_fetch_csv, cal_write_csv):
    """Per kernel: (launches, HBM bytes read, HBM bytes written) per launch,
    calibrated; plus the two scale factors (counter bytes / true bytes)."""
    cf = counter_per_dispatch(cal_fetch_csv, "FETCH_SIZE")[COPY_KERNEL]
    cw = counter_per_dispatch(cal_write_csv, "WRITE_SIZE")[COPY_KERNEL]
    f_scale = _mean(cf) * 1024 / COPY_BYTES
    w_scale = _mean(cw) * 1024 / COPY_BYTES
    fe = counter_per_dispatch(fetch_csv, "FETCH_SIZE")
    wr = counter_per_dispatch(write_csv, "WRITE_SIZE")
    rows = {}
    for k in fe:
        if k not in wr or k == COPY_KERNEL:
            continue
        rows[k] = (len(fe[k]), _mean(fe[k]) * 1024 / f_scale, _mean(wr[k]) * 1024 / w_scale)
    return rows, f_scale, w_scale


def read_traffic(path, kernel):
    """HBM bytes per launch of `kernel` from a committed traffic summary, or
    None when the summary is missing or was taken on other kernel sources."""
    try:
        with open(path) as fh:
            text = fh.read()
    except OSError:
        return None
    m = re.search(r"kernel-sources-sha256: ([0-9a-f]{64})", text)
    if not m or m.group(1) != kernel_sources_sha256():
        return None
    for line in text.splitlines():
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) >= 5 and cells[0] == kernel:
            try:
                return int(round(float(cells[4]) * 1e6))
            except ValueError:
                return None
    return None


def _stats_md(path, cmd):
    rows = []
    with open(path) as fh:
        for r in csv.DictReader(fh):
            rows.append((r["Name"], int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                         float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
                         float(r["Percentage"])))
    out = ["Command (run from /tmp with TMPDIR=/tmp; $R is the repository root):", "",
           "```", cmd, "```", "",
           "| kernel | calls | avg us | min us | max us | % of GPU time |",
           "|---|---|---|---|---|---|"]
    for name, calls, avg, mn, mx, pct in rows:
        out.append(f"| {name} | {calls} | {avg:.2f} | {mn:.2f} | {mx:.2f} | {pct:.2f} |")
    trace = os.path.join(os.path.dirname(path), "run_kernel_trace.csv")
    split = _split_twice(trace) if os.path.exists(trace) else {}
    if split:
        out += ["", "Kernels launched twice per step, by launch order (from the per-dispatch "
                "trace of the same run):", "",
                "| step | kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|---|"]
        for lab, (k, v) in split.items():
            out.append(f"| {lab} | {k} | {len(v)} | {_mean(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
    return "\n".join(out) + "\n"


def _split_twice(trace_csv):
    """{step label: (kernel, [us per launch])} of the kernels in TWICE."""
    rows = []
    with open(trace_csv) as fh:
        for r in csv.DictReader(fh):
            k = _base_name(r["Kernel_Name"])
            if k in TWICE:
                rows.append((int(r["Dispatch_Id"]), k,
                             (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    rows.sort()
    label = _Labeller()
    out = {}
    for _, k, us in rows:
        out.setdefault(label(k), (k, []))[1].append(us)
    return out


def mfma_table(counters_csv):
    """Per kernel: (launches, mean duration s, mean MFMA busy cycles, mean
    GRBM_GUI_ACTIVE) over the dispatches of a counter run that collected
    SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE."""
    rows = collections.defaultdict(dict)
    with open(counters_csv) as fh:
        for r in csv.DictReader(fh):
            d = rows[int(r["Dispatch_Id"])]
            d["name"] = _base_name(r["Kernel_Name"])
            d["dur"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
            d[r["Counter_Name"]] = float(r["Counter_Value"])
    per = collections.defaultdict(list)
    label = _Labeller()
    for _, d in sorted(rows.items()):
        per[label(d["name"])].append(d)
    out = {}
    for k, ds in per.items():
        out[k] = (len(ds), _mean([d["dur"] for d in ds]),
                  _mean([d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) for d in ds]),
                  _mean([d.get("GRBM_GUI_ACTIVE", 0.0) for d in ds]))
    return out


def _mfma_md(args):
    sys.path.insert(0, ROOT)
    from fine_grained_mixture_amd.inputs import SHAPES

    sh = SHAPES[args.config]
    rows = mfma_table(args.csv)
    out = ["Command (run from /tmp with TMPDIR=/tmp; $R is the repository root):", "",
           "```", args.cmd, "```", "",
           f"kernel-sources-sha256: {kernel_sources_sha256()}", "",
           f"Slots S = {args.slots}.  Durations are the counter run's own (one kernel at a "
           "time).  MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024 "
           "SIMDs); clock = GRBM_GUI_ACTIVE / 8 / duration; TFLOP/s are algorithmic.", "",
           "| kernel | launches | avg us | MFMA busy | clock GHz | TFLOP/s | of 2.5 PF |",
           "|---|---|---|---|---|---|---|"]
    order = ["up_swiglu", "down", "aggregate_O", "dh", "dxt", "aggregate_dX", "dw1", "dw2"]
    names = order + sorted(k for k in rows if k not in order)
    for k in names:
        if k not in rows:
            continue
        n, dur, busy, grbm = rows[k]
        cyc = grbm / NUM_XCD
        util = busy / (cyc * NUM_SIMD) if cyc > 0 else 0.0
        clk = cyc / dur / 1e9 if dur > 0 else 0.0
        model = kernel_model(k, sh, args.slots)
        tf = f"{model[0] / dur / 1e12:.0f}" if model and model[0] and dur > 0 else "-"
        frac = f"{model[0] / dur / PEAK_BF16_FLOPS:.3f}" if model and model[0] and dur > 0 else "-"
        out.append(f"| {k} | {n} | {dur * 1e6:.1f} | {util:.3f} | {clk:.2f} | {tf} | {frac} |")
    return "\n".join(out) + "\n"


def _traffic_md(args):
    sys.path.insert(0, ROOT)
    from fine_grained_mixture_amd.inputs import SHAPES

    sh = SHAPES[args.config]
    rows, fs, ws = traffic_table(args.fetch, args.write, args.cal_fetch, args.cal_write)
    out = ["Commands (run from /tmp with TMPDIR=/tmp; $R is the repository root):", "",
           "```", *args.cmd, "```", "",
           f"Calibration: a 1 GiB device-to-device copy ({COPY_KERNEL}) reads "
           f"FETCH_SIZE = {fs:.3f} x and WRITE_SIZE = {ws:.3f} x its true bytes; the "
           "figures below are divided by those factors.", "",
           f"kernel-sources-sha256: {kernel_sources_sha256()}", "",
           f"Slots S = {args.slots}; experts with at least one slot: "
           f"{sh.E if args.active_experts is None else args.active_experts} of {sh.E}.  "
           "MB = 1e6 bytes per launch.", "",
           "| kernel | launches | read MB | write MB | HBM MB | algorithmic MB | HBM / algorithmic |",
           "|---|---|---|---|---|---|---|"]
    order = ["up_swiglu", "down", "aggregate_O", "dh", "dxt", "aggregate_dX", "dw1", "dw2"]
    names = order + sorted(k for k in rows if k not in order)
    for k in names:
        if k not in rows:
            continue
        n, rd, wr = rows[k]
        model = kernel_model(k, sh, args.slots, E_act=args.active_experts)
        alg = f"{model[1] / 1e6:.1f}" if model else "-"
        ratio = f"{(rd + wr) / model[1]:.2f}" if model else "-"
        out.append(f"| {k} | {n} | {rd / 1e6:.1f} | {wr / 1e6:.1f} | {(rd + wr) / 1e6:.1f} | "
                   f"{alg} | {ratio} |")
    return "\n".join(out) + "\n"


PIPELINE_COUNTERS = (
    "TCP_TCC_READ_REQ_LATENCY_sum", "TCP_TCC_READ_REQ_sum", "TCP_PENDING_STALL_CYCLES_sum",
    "TA_BUSY_avr", "TD_TD_BUSY_sum", "TD_TC_STALL_sum", "TCC_HIT_sum", "TCC_MISS_sum",
    "TCC_EA0_RDREQ_LEVEL_sum", "TCC_EA0_RDREQ_sum", "GRBM_GUI_ACTIVE")


def pipeline_table(csvs):
    """Per kernel label: (launches, mean duration s, {counter: mean value per
    dispatch}) over one or more counter runs of the same program."""
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    durs = collections.defaultdict(list)
    for path in csvs:
        rows = collections.defaultdict(dict)
        with open(path) as fh:
            for r in csv.DictReader(fh):
                d = rows[int(r["Dispatch_Id"])]
                d["name"] = _base_name(r["Kernel_Name"])
                d["dur"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
                d[r["Counter_Name"]] = float(r["Counter_Value"])
        label = _Labeller()
        for _, d in sorted(rows.items()):
            k = label(d["name"])
            durs[k].append(d["dur"])
            for c, v in d.items():
                if c not in ("name", "dur"):
                    per[k][c].append(v)
    return {k: (len(durs[k]) // max(1, len(csvs)), _mean(durs[k]),
                {c: _mean(v) for c, v in per[k].items()}) for k in per}


def _pipeline_md(args):
    rows = pipeline_table(args.csv)
    out = ["Commands (run from /tmp with TMPDIR=/tmp; $R is the repository root):", "",
           "```", *args.cmd, "```", "",
           f"kernel-sources-sha256: {kernel_sources_sha256()}", "",
           "Per launch, averaged over launches; cycles are GPU clock cycles; \"per CU\" "
           "fractions are of the kernel's cycles (GRBM_GUI_ACTIVE / 8) on each of the 256 CUs.",
           "",
           "| kernel | avg us | L2 read latency (cyc) | L2 reads per CU per cyc | "
           "in flight per CU | L2 hit | memory read latency (cyc) | TA busy | TD busy | "
           "TD waits on L1 | L1 waits on L2 |",
           "|---|---|---|---|---|---|---|---|---|---|---|"]
    order = ["up_swiglu", "down", "aggregate_O", "dh", "dxt", "aggregate_dX", "dw1", "dw2"]
    for k in order:
        if k not in rows:
            continue
        _, dur, v = rows[k]
        cyc = v.get("GRBM_GUI_ACTIVE", 0.0) / NUM_XCD
        if not cyc:
            continue
        cu = cyc * (NUM_SIMD // 4)
        lat = v["TCP_TCC_READ_REQ_LATENCY_sum"] / v["TCP_TCC_READ_REQ_sum"]
        rate = v["TCP_TCC_READ_REQ_sum"] / cu
        hit = v["TCC_HIT_sum"] / (v["TCC_HIT_sum"] + v["TCC_MISS_sum"])
        mlat = v["TCC_EA0_RDREQ_LEVEL_sum"] / v["TCC_EA0_RDREQ_sum"]
        out.append(f"| {k} | {dur * 1e6:.1f} | {lat:.0f} | {rate:.3f} | {lat * rate:.0f} | "
                   f"{hit:.2f} | {mlat:.0f} | {v['TA_BUSY_avr'] / cyc:.2f} | "
                   f"{v['TD_TD_BUSY_sum'] / cu:.2f} | {v['TD_TC_STALL_sum'] / cu:.2f} | "
                   f"{v['TCP_PENDING_STALL_CYCLES_sum'] / cu:.2f} |")
    return "\n".join(out) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats", help="kernel-trace statistics table")
    s.add_argument("csv")
    s.add_argument("cmd")
    t = sub.add_parser("traffic", help="HBM traffic table from FETCH_SIZE / WRITE_SIZE")
    for a in ("--fetch", "--write", "--cal-fetch", "--cal-write"):
        t.add_argument(a, required=True)
    t.add_argument("--config", default="7b")
    t.add_argument("--slots", type=int, required=True)
    t.add_argument("--active-experts", type=int, default=None,
                   help="experts given at least one slot (default: all)")
    t.add_argument("cmd", nargs="+", help="the commands that produced the CSV files")
    m = sub.add_parser("mfma", help="MFMA utilisation and clock from SQ / GRBM counters")
    m.add_argument("csv")
    m.add_argument("--config", default="7b")
    m.add_argument("--slots", type=int, required=True)
    m.add_argument("cmd")
    q = sub.add_parser("pipeline", help="vector-memory path summary from counter runs")
    q.add_argument("--csv", action="append", required=True, help="one counter CSV (repeat)")
    q.add_argument("cmd", nargs="+", help="the commands that produced the CSV files")
    args = ap.parse_args(argv)
    if args.what == "stats":
        sys.stdout.write(_stats_md(args.csv, args.cmd))
    elif args.what == "mfma":
        sys.stdout.write(_mfma_md(args))
    elif args.what == "pipeline":
        sys.stdout.write(_pipeline_md(args))
    else:
        sys.stdout.write(_traffic_md(args))


if __name__ == "__main__":
    main()
