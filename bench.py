"""Benchmark: MoE-layer tokens/s on one MI355X for the redundant-expert dispatch path.

Default workload: R=32 simulated ranks, S=4096 tokens/rank, E=256 experts (8 per rank),
K=8, B=8 replica slots, H=7168, H'=2048, bf16, Zipf-skewed routing at maxvio ~8; one step =
the whole hot path on rank 0, forward and backward:
  plan, dispatch layout, slot prefetch (both projections), permute, up/down grouped GEMMs,
  combine; weighted permute, down/up DGRAD and WGRAD, replica-gradient folds.
value = input tokens of rank 0 per second (S / step time), inputs resident in HBM.

Also printed in the same JSON line: routed copies/s, the forward alone, the step replayed from
a HIP graph (captured once; --no-graph skips it), per-kernel times and
roofline fractions, the roofline entry of the dominant kernel (HIP events around every launch
in the timed region), the same step at maxvio 0 and 1 with every rank's share timed at each
point (flatness of rank 0's time and of the slowest rank's time across skews), and the CPU
oracle timed on a bounded sample of the same step on this host.

With --activation swiglu the up projection is the gated unit (2H' columns as (gate, up)
pairs, silu(gate)*up in the GEMM epilogue, its derivative in a row kernel in the backward).

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--no-sweep]
                       [--activation identity|swiglu]
"""
import argparse
import json
import os
import sys
import time
from collections import defaultdict

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s per GPU at maxvio 0/1/8; GEMM MFMA %, permute HBM GB/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class EventTimer:
    """HIP events around every launch, on torch's current stream (the one the library uses)."""

    def __init__(self):
        import torch
        self.torch = torch
        self.events = defaultdict(list)

    def __call__(self, name, fn, *args):
        t = self.torch
        s, e = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        s.record()
        fn(*args)
        e.record()
        self.events[name].append((s, e))

    def ms(self):
        return {k: [s.elapsed_time(e) for s, e in v] for k, v in self.events.items()}


KERNEL_SOURCES = {  # bench kernel name -> (rocprof name prefix, source files that define it)
    "gemm_fwd": ("moe::k_ggemm_bf16<0", ("group_gemm.hip", "common.hpp")),
    "gemm_dgrad": ("moe::k_ggemm_bf16<1", ("group_gemm.hip", "common.hpp")),
    "gemm_wgrad": ("moe::k_ggemm_bf16<2", ("group_gemm.hip", "common.hpp")),
    "gemm_fwd_swiglu": ("moe::k_ggemm_bf16<3", ("group_gemm.hip", "common.hpp")),
    "gemm_fwd_gather": ("moe::k_ggemm_bf16<0, false, 2, true>", ("group_gemm.hip", "common.hpp")),
    "gemm_wgrad_gather": ("moe::k_ggemm_bf16<2, false, 4, true>", ("group_gemm.hip", "common.hpp")),
    "permute": ("moe::k_permute<false>", ("rows.hip", "common.hpp")),
    "permute_weighted": ("moe::k_permute<true>", ("rows.hip", "common.hpp")),
    "combine": ("moe::k_combine<true, true>", ("rows.hip", "common.hpp")),
    "combine_wgrad": ("moe::k_combine_wgrad<true>", ("rows.hip", "common.hpp")),
    "unpermute_reduce": ("moe::k_combine<true, false>", ("rows.hip", "common.hpp")),
    "fold": ("moe::k_fold", ("rows.hip", "common.hpp")),
    "prefetch": ("moe::k_prefetch", ("rows.hip", "common.hpp")),
    "swiglu_bwd": ("moe::k_swiglu_bwd<true>", ("rows.hip", "common.hpp")),
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_skew8_fwdbwd.md")
COPY_BYTES = 1 << 30          # calibration copy: reads and writes exactly this many bytes


def source_hash(kernel):
    """sha256 of the kernel's source files with comments and blank space removed, so that a
    change to the comments alone keeps the recorded counters valid."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel][1]:
        with open(os.path.join(ROOT, "balanced_token_dispatch_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def recorded_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary, if still current."""
    import re
    if not os.path.exists(TRAFFIC_FILE):
        return None
    for line in open(TRAFFIC_FILE):
        m = re.match(r"\| `(\w+)` \| ([0-9a-f]{16}) \| ([0-9.]+) \| ([0-9.]+) \| ([0-9.]+) \|", line)
        if m and m.group(1) == kernel and m.group(2) == source_hash(kernel):
            return float(m.group(5)) * 1e6
    return None


def render_traffic(fetch_csv, write_csv):
    """Summarise two rocprofv3 --pmc runs of `bench.py --probe` (FETCH_SIZE, WRITE_SIZE)."""
    import csv
    import collections

    def per_dispatch(path, counter):
        vals = collections.defaultdict(float)
        names = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            vals[r["Dispatch_Id"]] += float(r["Counter_Value"])
            names[r["Dispatch_Id"]] = r["Kernel_Name"]
        return vals, names

    out = []
    f_vals, names = per_dispatch(fetch_csv, "FETCH_SIZE")
    w_vals, _ = per_dispatch(write_csv, "WRITE_SIZE")
    # the calibration copy is the torch copy kernel dispatched right before the probed step
    copies = [d for d, n in names.items() if "copy" in n.lower() and "moe::" not in n]
    big = max(copies, key=lambda d: f_vals[d])
    kf = COPY_BYTES / (f_vals[big] * 1024.0)
    kw = COPY_BYTES / (w_vals[big] * 1024.0)
    out.append(f"calibration copy ({COPY_BYTES} B read + written): FETCH_SIZE "
               f"{f_vals[big]:.0f} KiB, WRITE_SIZE {w_vals[big]:.0f} KiB -> scale "
               f"fetch x{kf:.4f}, write x{kw:.4f}")
    out.append("")
    out.append("| kernel | source sha256[:16] | fetch MB/launch | write MB/launch | traffic MB/launch |")
    out.append("|---|---|---|---|---|")
    for k, (prefix, _) in KERNEL_SOURCES.items():
        ds = [d for d, n in names.items() if n.startswith(prefix) or n.startswith("void " + prefix)]
        if not ds:
            continue
        ds = sorted(ds, key=int)[len(ds) // 2:]  # the probed step's launches (after the warm-up step)
        fb = sum(f_vals[d] for d in ds) / len(ds) * 1024 * kf / 1e6
        wb = sum(w_vals[d] for d in ds) / len(ds) * 1024 * kw / 1e6
        out.append(f"| `{k}` | {source_hash(k)} | {fb:.1f} | {wb:.1f} | {fb + wb:.1f} |")
    print("\n".join(out))


def render_mfma(csv_path):
    """Summarise a rocprofv3 --pmc run of `bench.py --probe` with SQ_INSTS_VALU_MFMA_MOPS_BF16,
    SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE: matrix-unit work and busy fraction of the
    GEMM launches of the probed step."""
    import csv
    import collections

    vals = collections.defaultdict(lambda: collections.defaultdict(float))
    names, span = {}, {}
    for r in csv.DictReader(open(csv_path)):
        d = r["Dispatch_Id"]
        vals[d][r["Counter_Name"]] += float(r["Counter_Value"])
        names[d] = r["Kernel_Name"]
        span[d] = (int(r["Start_Timestamp"]), int(r["End_Timestamp"]))
    import synth
    dm = synth.WORKLOADS["skew8_large_fwdbwd"].dims
    gemm = 2.0 * dm.S * dm.K * dm.H * dm.Hp
    simds = 256 * 4
    out = ["| kernel | launches | MFMA GFLOP executed / launch | algorithmic GFLOP | MFMA busy, % of SIMD cycles | "
           "clock from GRBM_GUI_ACTIVE, GHz |", "|---|---|---|---|---|---|"]
    for k in ("gemm_fwd", "gemm_dgrad", "gemm_wgrad"):
        prefix = KERNEL_SOURCES[k][0]
        ds = [d for d, n in names.items() if n.startswith(prefix) or n.startswith("void " + prefix)]
        if not ds:
            continue
        ds = sorted(ds, key=int)[len(ds) // 2:]  # the probed step's launches (after the warm-up step)
        fl = sum(vals[d]["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 for d in ds) / len(ds)
        gui = [vals[d]["GRBM_GUI_ACTIVE"] / 8 for d in ds]  # summed over the 8 XCDs
        busy = sum(vals[d]["SQ_VALU_MFMA_BUSY_CYCLES"] / (g * simds) for d, g in zip(ds, gui)) / len(ds)
        clk = sum(g / (span[d][1] - span[d][0]) for d, g in zip(ds, gui)) / len(ds)
        out.append(f"| `{k}` | {len(ds)} | {fl / 1e9:.1f} | {gemm / 1e9:.1f} | {100 * busy:.1f} | "
                   f"{clk:.2f} |")
    print("\n".join(out))


def render_stalls(*csv_paths):
    """Summarise rocprofv3 --pmc runs of `bench.py --probe` on the GEMM launches of the probed
    step: wave states, the vector-memory pipeline (TA, TD, TCP, L2 requests) and LDS.  Each
    figure is computed from whichever run holds its counters.  SQ, TA, TD and TCP values arrive
    summed over the chip's shader engines or CUs; the SQ wave counters are in units of 4 clocks
    per wave; clocks per launch are GRBM_GUI_ACTIVE of one XCD (the run's sum over 8)."""
    import csv
    import collections

    def load(path):
        vals = collections.defaultdict(lambda: collections.defaultdict(float))
        names = {}
        for r in csv.DictReader(open(path)):
            vals[r["Dispatch_Id"]][r["Counter_Name"]] += float(r["Counter_Value"])
            names[r["Dispatch_Id"]] = r["Kernel_Name"]
        return vals, names

    cus = 256
    clk = lambda v: v["GRBM_GUI_ACTIVE"] / 8
    figures = [  # (column, counters needed, value per launch, format)
        ("waves per CU", ("SQ_WAVE_CYCLES",), lambda v: 4 * v["SQ_WAVE_CYCLES"] / clk(v) / cus, "{:.2f}"),
        ("dependency wait, % of wave time", ("SQ_WAIT_ANY",),
         lambda v: 100 * v["SQ_WAIT_ANY"] / v["SQ_WAVE_CYCLES"], "{:.1f}"),
        ("issue wait, %", ("SQ_WAIT_INST_ANY",),
         lambda v: 100 * v["SQ_WAIT_INST_ANY"] / v["SQ_WAVE_CYCLES"], "{:.1f}"),
        ("of it LDS, %", ("SQ_WAIT_INST_LDS",),
         lambda v: 100 * v["SQ_WAIT_INST_LDS"] / v["SQ_WAVE_CYCLES"], "{:.1f}"),
        ("VMEM instruction latency, clk", ("VmemLatency",), lambda v: v["VmemLatency"], "{:.0f}"),
        ("L2 read latency at the TCP, clk", ("TCP_TCC_READ_REQ_LATENCY_sum",),
         lambda v: v["TCP_TCC_READ_REQ_LATENCY_sum"] / v["TCP_TCC_READ_REQ_sum"], "{:.0f}"),
        ("L2 read requests, M", ("TCP_TCC_READ_REQ_sum",),
         lambda v: v["TCP_TCC_READ_REQ_sum"] / 1e6, "{:.1f}"),
        ("TA busy, % of CU clocks", ("TA_TA_BUSY_sum",),
         lambda v: 100 * v["TA_TA_BUSY_sum"] / clk(v) / cus, "{:.1f}"),
        ("TA address FIFO full, %", ("SQ_VMEM_TA_ADDR_FIFO_FULL",),
         lambda v: 100 * v["SQ_VMEM_TA_ADDR_FIFO_FULL"] / clk(v) / cus, "{:.1f}"),
        ("TD busy, %", ("TD_TD_BUSY_sum",), lambda v: 100 * v["TD_TD_BUSY_sum"] / clk(v) / cus, "{:.1f}"),
        ("TCP waiting on L2 data, %", ("TCP_PENDING_STALL_CYCLES_sum",),
         lambda v: 100 * v["TCP_PENDING_STALL_CYCLES_sum"] / clk(v) / cus, "{:.1f}"),
        ("LDS busy, %", ("SQ_LDS_IDX_ACTIVE",),
         lambda v: 100 * v["SQ_LDS_IDX_ACTIVE"] / clk(v) / cus, "{:.1f}"),
        ("LDS instruction latency, clk", ("LdsLatency",), lambda v: v["LdsLatency"], "{:.0f}"),
        ("LDS address conflict clocks", ("SQ_LDS_ADDR_CONFLICT",), lambda v: v["SQ_LDS_ADDR_CONFLICT"], "{:.0f}"),
    ]
    runs = [load(p) for p in csv_paths]
    cols = [f for f in figures if any(all(c in v for c in f[1]) for vals, _ in runs for v in vals.values())]
    out = ["| kernel | launches | " + " | ".join(f[0] for f in cols) + " |",
           "|---|---|" + "---|" * len(cols)]
    for k in ("gemm_fwd", "gemm_dgrad", "gemm_wgrad"):
        prefix = KERNEL_SOURCES[k][0]
        row, n = [], 0
        for name, need, fn, fmt in cols:
            cell = "–"
            for vals, names in runs:
                ds = [d for d, m in names.items() if m.startswith(prefix) or m.startswith("void " + prefix)]
                ds = sorted(ds, key=int)[len(ds) // 2:]  # the probed step's launches
                if ds and all(c in vals[ds[0]] for c in need):
                    cell = fmt.format(sum(fn(vals[d]) for d in ds) / len(ds))
                    n = len(ds)
                    break
            row.append(cell)
        if n:
            out.append(f"| `{k}` | {n} | " + " | ".join(row) + " |")
    print("\n".join(out))


def render_stats(stats_csv, title, command):
    """Markdown table of the library's kernels from a rocprofv3 --kernel-trace --stats run
    (its kernel_stats.csv): calls, average / min / max duration, share of profiled GPU time."""
    import csv
    rows = [r for r in csv.DictReader(open(stats_csv)) if "moe::" in r["Name"]]
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = [f"# rocprofv3 kernel stats: {title}", "", "Command (on the MI355X host, `$REPO` = repository root):",
           "", "```", command, "```", "",
           "Kernels of the library (torch's input generation and copies are omitted):", "",
           "| kernel | calls | avg us | min us | max us | % of profiled GPU time |",
           "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"].split("(")[0].replace("void ", "")
        out.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                   f"{float(r['Percentage']):.2f} |")
    print("\n".join(out))


def render_counters(csv_path, title, command):
    """Markdown table of per-launch counter values (averaged over the probed step's launches of
    each library kernel) from a rocprofv3 --pmc run of `bench.py --probe`."""
    import csv
    import collections
    vals = collections.defaultdict(lambda: collections.defaultdict(float))
    names = {}
    for r in csv.DictReader(open(csv_path)):
        vals[r["Dispatch_Id"]][r["Counter_Name"]] += float(r["Counter_Value"])
        names[r["Dispatch_Id"]] = r["Kernel_Name"].split("(")[0].replace("void ", "")
    counters = sorted({c for v in vals.values() for c in v})
    per = collections.defaultdict(list)
    for d in sorted(vals, key=int):
        if "moe::" in names[d]:
            per[names[d]].append(d)
    out = [f"# rocprofv3 counters per launch: {title}", "", "Command (on the MI355X host, `$REPO` = repository root):",
           "", "```", command, "```", "",
           "`--probe` runs one warm-up step, a 1 GiB copy, then one step; the values average each kernel's "
           "launches in that second step.", "",
           "| kernel | launches | " + " | ".join(f"`{c}`" for c in counters) + " |",
           "|---|---|" + "---|" * len(counters)]
    for n, ds in per.items():
        ds = ds[len(ds) // 2:]
        out.append(f"| `{n}` | {len(ds)} | " +
                   " | ".join(f"{sum(vals[d][c] for d in ds) / len(ds):.0f}" for c in counters) + " |")
    print("\n".join(out))


def algorithmic_work(shape, n_slots_used, gated=False):
    """Minimum bytes (or flops) per launch of each kernel of the step.

    Kernels launched once per projection (prefetch, fold, DGRAD, WGRAD) report the mean over
    the step's launches; with the gated unit the up projection is twice as wide as the down.
    """
    R, S, K, E, H, Hp = shape.R, shape.S, shape.K, shape.E, shape.H, shape.Hp
    SK = S * K
    gemm = 2.0 * SK * H * Hp
    up = 2.0 if gated else 1.0
    both = (1.0 + up) / 2.0
    return {
        "plan": ("hbm", 4.0 * R * SK + 4.0 * R * E),
        "dispatch_layout": ("hbm", 8.0 * R * SK + 4.0 * SK),
        "prefetch": ("hbm", 2.0 * n_slots_used * H * Hp * 2 * both),
        "permute": ("hbm", 2.0 * SK * H * 2 + 4.0 * SK),
        "gemm_fwd": ("mfma", gemm),
        "gemm_fwd_swiglu": ("mfma", 2.0 * gemm),
        "gemm_fwd_gather": ("mfma", gemm),
        "gemm_wgrad_gather": ("mfma", gemm),
        "combine": ("hbm", SK * H * 2.0 + S * H * 2.0 + 8.0 * SK),
        "permute_weighted": ("hbm", 2.0 * SK * H * 2 + 8.0 * SK),
        "gemm_dgrad": ("mfma", gemm * both),
        "gemm_wgrad": ("mfma", gemm * both),
        # home row read and written, slot row read and zeroed (fp32)
        "fold": ("hbm", 4.0 * n_slots_used * H * Hp * 4 * both),
        "combine_wgrad": ("hbm", SK * H * 2.0 + S * H * 2.0 + 8.0 * SK),
        "unpermute_reduce": ("hbm", SK * H * 2.0 + S * H * 2.0 + 4.0 * SK),
        # reads h [SK, 2H'] and dz [SK, H'], writes dh [SK, 2H'] (bf16)
        "swiglu_bwd": ("hbm", SK * Hp * 2.0 * 5),
    }


def setup_layer(wl, target, rank, placement="receiver0", layer=None, activation="identity",
                fused_gather=False):
    import numpy as np
    import torch
    import synth
    from balanced_token_dispatch_amd.layer import LayerStep, Shape
    d = wl.dims
    zipf = synth.zipf_for(wl, target, placement)
    t0 = time.time()
    idx, w = synth.routing(d, zipf, wl.base_seed, placement)
    log(f"routing {wl.name} maxvio target {target}: zipf s={zipf:.4f}, {time.time() - t0:.1f}s")
    if layer is None:
        layer = LayerStep(Shape(d.R, d.S, d.K, d.E, d.B, d.H, d.Hp), rank=rank,
                          activation=activation, backward=wl.backward, fused_gather=fused_gather)
        seed = wl.base_seed
        synth.fill_normal_(layer.x_all, 1.0, seed * 10 + 1)
        synth.fill_normal_(layer.w_up, 0.02, seed * 10 + 2)
        synth.fill_normal_(layer.w_down, 0.02, seed * 10 + 3)
        synth.fill_normal_(layer.y_all, 1.0, seed * 10 + 4)
        if layer.backward_enabled:
            synth.fill_normal_(layer.dout_all, 1.0, seed * 10 + 5)
            synth.fill_normal_(layer.dxp_all, 1.0, seed * 10 + 6)
    layer.topk_idx.copy_(torch.from_numpy(idx))
    layer.topk_w.copy_(torch.from_numpy(w))
    torch.cuda.synchronize()
    info = {"maxvio": synth.realised_maxvio(idx, d.E), "zipf_s": zipf,
            "home_load_ratio": synth.home_load_ratio(idx, d)}
    return layer, idx, w, info


def run_steps(layer, steps, warmup, timer=None, forward_only=False):
    import torch
    fn = layer.forward if forward_only else layer.step
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn(timer)
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def graph_replay_ms(layer, steps):
    """The same step captured once in a HIP graph and replayed: ms per replay."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.step()
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1000.0 / steps
    del g
    return ms


def per_rank_ms(layer, reps=3, warmup=1):
    """Step time of every rank's share (same routing), ms: each rank processes exactly S*K
    copies, so the times should be flat across ranks as well as across skews."""
    orig = layer.rank
    out = []
    for r in range(layer.s.R):
        layer.rank = r
        out.append(run_steps(layer, reps, warmup) * 1000.0 / reps)
    layer.rank = orig
    return out


class _LazyRows:
    """Host copies of selected rows of a device weight tensor, fetched on first use."""

    def __init__(self, dev, prefetch_map):
        self.dev, self.map, self.cache = dev, prefetch_map, {}
        self.shape = tuple(dev.shape)

    def __getitem__(self, rho):
        import numpy as np
        import torch
        rho = int(rho)
        if rho not in self.cache:
            src = self.map.get(rho, rho)
            self.cache[rho] = self.dev[src].view(torch.int16).cpu().numpy().view(np.uint16)
        return self.cache[rho]


def _median_of(n, fn):
    """Run fn() n times; (median wall seconds, the last result)."""
    import statistics
    times, out = [], None
    for _ in range(n):
        t0 = time.perf_counter()
        out = fn()
        times.append(time.perf_counter() - t0)
    return statistics.median(times), out


def cpu_baseline(layer, idx, w, rows_sample, tokens_sample, reps=3):
    """The oracle as it stands, on a bounded sample of the same step, scaled to tokens/s.

    Timed on this host, each part the median of ``reps`` runs: the full plan and layout of all
    R ranks' routing, then permute, both projections forward (with the gated unit, when the
    layer has it), the weighted permute, both DGRADs and WGRADs on the first ``rows_sample``
    rows of rank r's buffer, the combine, router-weight gradient and un-permute reduce of
    ``tokens_sample`` tokens, and the fold on 1/8 of each replica row.  Each part is scaled to
    the full step.
    """
    import numpy as np
    import torch
    import oracle
    s, r = layer.s, layer.rank
    bwd = layer.backward_enabled
    t = {}
    t["plan"], pl = _median_of(reps, lambda: oracle.plan(idx, s.E, s.B))
    t["layout"], (cu, dest, src) = _median_of(reps, lambda: oracle.layout(idx, pl, r))
    n = int(min(rows_sample, cu[-1]))
    se, _, _ = pl.slot_table()
    pmap = {s.E + j: int(se[r, j]) for j in range(s.B) if se[r, j] >= 0}
    wu, wd = _LazyRows(layer.w_up, pmap), _LazyRows(layer.w_down, pmap)
    cu_s = np.minimum(cu, n)
    toks = np.unique(src[:n] // s.K)
    x_rows = layer.x_all[torch.from_numpy(toks).cuda()].view(torch.int16).cpu().numpy().view(np.uint16)
    if bwd:
        g_rows = layer.dout_all[torch.from_numpy(toks).cuda()].view(torch.int16).cpu().numpy().view(np.uint16)
    remap = {int(tk): i for i, tk in enumerate(toks)}
    src_l = np.array([remap[int(c) // s.K] * s.K + int(c) % s.K for c in src[:n]], np.int64)
    w_flat = np.zeros(len(toks) * s.K, np.float32)
    w_all = w.reshape(-1)
    for i, c in enumerate(src[:n]):
        w_flat[src_l[i]] = w_all[c]
    for rho in range(s.G):                       # weight rows fetched outside the timed parts
        if cu_s[rho + 1] > cu_s[rho]:
            wu[rho], wd[rho]
    gated = layer.activation == "swiglu"

    def rows_part():
        xp = oracle.permute(x_rows, src_l.astype(np.int32), s.K)
        if gated:
            z, h = oracle.group_gemm_swiglu(xp, wu, cu_s)
        else:
            z = oracle.group_gemm("fwd", xp, wu, cu_s)
        oracle.group_gemm("fwd", z, wd, cu_s)
        if bwd:
            dy = oracle.permute(g_rows, src_l.astype(np.int32), s.K, row_scale=w_flat)
            dz = oracle.group_gemm("dgrad", dy, wd, cu_s)
            dup = oracle.swiglu_backward(dz, h) if gated else dz
            oracle.group_gemm("dgrad", dup, wu, cu_s)
            act = [rho for rho in range(s.G) if cu_s[rho + 1] > cu_s[rho]]
            for a, b, K_, N_ in ((z, dy, s.Hp, s.H), (xp, dup, s.H, layer.up_cols)):
                for rho in act:                      # wgrad of the sampled segments only
                    lo, hi = cu_s[rho], cu_s[rho + 1]
                    sub = np.array([0, hi - lo])
                    oracle.group_gemm("wgrad", a[lo:hi], b[lo:hi], sub,
                                      out=np.zeros((1, K_, N_), np.float32))

    t["rows"], _ = _median_of(reps, rows_part)
    # combine: tokens_sample tokens of rank r, expert outputs gathered from a staged buffer
    ts = np.arange(min(tokens_sample, s.S))
    need = dest.reshape(s.R, s.S, s.K)[r, ts].reshape(-1)
    need = need[need >= 0]
    y_rows = layer.y_all[torch.from_numpy(need.astype(np.int64)).cuda()].view(torch.int16).cpu().numpy().view(np.uint16)
    ymap = np.full(s.R * s.SK, -1, np.int64)
    ymap[need] = np.arange(need.size)
    dest_l = np.where(dest >= 0, ymap[np.maximum(dest, 0)], -1)
    if bwd:
        g_tok = layer.dout_all[r * s.S:(r + 1) * s.S][torch.from_numpy(ts).cuda()].view(torch.int16).cpu().numpy().view(np.uint16)
        g_full = np.zeros((s.S, s.H), np.uint16)
        g_full[ts] = g_tok
        dxp_rows = layer.dxp_all[torch.from_numpy(need.astype(np.int64)).cuda()].view(torch.int16).cpu().numpy().view(np.uint16)

    def combine_part():
        oracle.combine(y_rows, dest_l, w, r, s.S, s.K, tokens=ts)
        if bwd:
            oracle.combine_weight_grad(y_rows, dest_l, g_full, r, s.S, s.K, tokens=ts)
            oracle.unpermute_reduce(dxp_rows, dest_l, r, s.S, s.K, tokens=ts)

    t["combine"], _ = _median_of(reps, combine_part)
    frac = 8
    t["fold"] = 0.0
    if bwd:
        dw_u = np.zeros((s.G, s.H * layer.up_cols // frac), np.float32)
        dw_d = np.zeros((s.G, s.H * s.Hp // frac), np.float32)

        def fold_part():
            oracle.replica_grad_fold(dw_u, pl, r)
            oracle.replica_grad_fold(dw_d, pl, r)

        tf, _ = _median_of(reps, fold_part)
        t["fold"] = tf * frac
    est = (t["plan"] + t["layout"] + t["rows"] * s.SK / max(n, 1)
           + t["combine"] * s.S / max(len(ts), 1) + t["fold"])
    return est, t, n, len(ts)


def host_cpu():
    """CPU model name, the CPUs this process may run on, and the BLAS thread count."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cpu_model": model, "affinity_cpus": len(os.sched_getaffinity(0)),
            "blas_threads": blas_threads()}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        return max([i.get("num_threads", 1) for i in info] or [1])
    except Exception:
        return 1


# Maxvio points of each workload's sweep: (workload whose calibration gives the routing, target).
# The R32 shape's sweep takes maxvio 0 and 1 from the forward workload of the same shape.
SWEEPS = {
    "skew8_large_fwdbwd": [("skew1_large", 0.0), ("skew1_large", 1.0)],
    "sweep_r64": [("sweep_r64", 0.0), ("sweep_r64", 1.0), ("sweep_r64", 4.0)],
}
SCALE_WORKLOAD = "sweep_r64"


def rank_stats(layer):
    import numpy as np
    t = per_rank_ms(layer)
    return {"max_ms": round(max(t), 4), "min_ms": round(min(t), 4),
            "argmax_rank": int(np.argmax(t)), "max_over_min": round(max(t) / min(t), 4)}


def kernel_fracs(timer, shape, n_slots, steps, gated=False):
    """Per-kernel average launch time and fraction of its roofline from HIP-event timings."""
    import numpy as np
    work = algorithmic_work(shape, n_slots, gated=gated)
    kernels, totals = {}, {}
    for name, times in timer.ms().items():
        bound, amount = work[name]
        avg = float(np.mean(times))
        totals[name] = float(np.sum(times)) / steps
        if bound == "mfma":
            ach = amount / (avg * 1e-3) / 1e12
            kernels[name] = {"avg_ms": round(avg, 4), "launches_per_step": len(times) // steps,
                             "tflops": round(ach, 1), "frac": round(ach / BF16_PEAK_TFLOPS, 4)}
        else:
            ach = amount / (avg * 1e-3) / 1e9 if avg > 0 else 0.0
            kernels[name] = {"avg_ms": round(avg, 4), "launches_per_step": len(times) // steps,
                             "gbs": round(ach, 1), "frac": round(ach / HBM_PEAK_GBS, 4)}
    return kernels, totals


def slots_used(layer):
    s = layer.s
    plan = layer.plan.cpu().numpy()
    off_sexp = 8 + 4 * s.E + 5 * (s.E + s.R)
    slots = plan[off_sexp + layer.rank * s.B: off_sexp + (layer.rank + 1) * s.B]
    return int((slots >= 0).sum())


def maxvio_sweep(layer, wl, info, ms_step, value, args):
    """The step at the workload's other maxvio points on the same buffers, every rank's share
    timed at each point; flatness of rank 0's time and of the slowest rank's across skews."""
    s = layer.s
    sweep = {f"{info['maxvio']:.2f}": {"ms_per_step": round(ms_step, 4),
                                        "tokens_per_s": round(value, 1),
                                        "home_load_ratio": round(info["home_load_ratio"], 3),
                                        "every_rank": rank_stats(layer)}}
    for wname, t in SWEEPS[wl.name]:
        import synth
        layer, _, _, info_t = setup_layer(synth.WORKLOADS[wname], t, args.rank, layer=layer)
        n = max(5, args.steps // 2)
        ms_t = run_steps(layer, n, 2) * 1000.0 / n
        key = f"{info_t['maxvio']:.2f}"
        sweep[key] = {"ms_per_step": round(ms_t, 4), "tokens_per_s": round(s.S / (ms_t * 1e-3), 1),
                      "home_load_ratio": round(info_t["home_load_ratio"], 3),
                      "status": int(layer.status.item()), "every_rank": rank_stats(layer)}
        log(f"sweep maxvio {key}: {ms_t:.3f} ms/step, every rank {sweep[key]['every_rank']}")
    pts = list(sweep.values())
    t_all = [v["ms_per_step"] for v in pts]
    sweep["flatness_max_over_min"] = round(max(t_all) / min(t_all), 4)
    t_max = [v["every_rank"]["max_ms"] for v in pts]
    sweep["flatness_of_slowest_rank"] = round(max(t_max) / min(t_max), 4)
    return sweep


def scale_sweep(args):
    """R64 S8192 E384 K8 B8 H7168 H'2048, forward + backward, at maxvio 0, 1, 4 and 16: rank 0's
    step time, tokens/s and every kernel's roofline fraction at each point, every rank's share
    timed at each point, and the flatness across skews."""
    import synth
    import torch
    wl = synth.WORKLOADS[SCALE_WORKLOAD]
    layer = None
    points = {}
    for t in wl.maxvio_targets:
        layer, _, _, info = setup_layer(wl, t, args.rank, layer=layer,
                                        fused_gather=args.fused_gather)
        n = max(5, args.steps // 2)
        el = run_steps(layer, n, 2)
        ms_t = el * 1000.0 / n
        timer = EventTimer()
        ov, layer.overlap = layer.overlap, False  # each kernel's own event time (see main)
        run_steps(layer, n, 0, timer)
        layer.overlap = ov
        kern, _ = kernel_fracs(timer, layer.s, slots_used(layer), n)
        key = f"{info['maxvio']:.2f}"
        points[key] = {"target": t, "ms_per_step": round(ms_t, 4),
                       "tokens_per_s": round(layer.s.S / (ms_t * 1e-3), 1),
                       "home_load_ratio": round(info["home_load_ratio"], 3),
                       "status": int(layer.status.item()),
                       "replica_slots_used_on_rank": slots_used(layer),
                       "every_rank": rank_stats(layer),
                       "kernels": {k: {kk: v[kk] for kk in ("avg_ms", "frac")} for k, v in kern.items()}}
        log(f"scale sweep maxvio {key}: {ms_t:.3f} ms/step, every rank {points[key]['every_rank']}")
    s = layer.s
    del layer
    torch.cuda.empty_cache()
    t_all = [v["ms_per_step"] for v in points.values()]
    t_max = [v["every_rank"]["max_ms"] for v in points.values()]
    return {"workload": wl.name, "R": s.R, "S": s.S, "K": s.K, "E": s.E, "B": s.B, "H": s.H,
            "H_prime": s.Hp, "step": "forward+backward", "points": points,
            "flatness_max_over_min": round(max(t_all) / min(t_all), 4),
            "flatness_of_slowest_rank": round(max(t_max) / min(t_max), 4)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="skew8_large_fwdbwd")
    ap.add_argument("--rank", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-scale-sweep", action="store_true",
                    help="skip the R64 S8192 E384 sweep over maxvio 0/1/4/16")
    ap.add_argument("--cpu-rows", type=int, default=16384)
    ap.add_argument("--cpu-tokens", type=int, default=2048)
    ap.add_argument("--no-graph", action="store_true", help="skip the graph-replay figure")
    ap.add_argument("--main-only", action="store_true",
                    help="time the main step only: no forward-only, graph-replay or sweep figures "
                         "(keeps a profiler's per-kernel averages to the main step's launches)")
    ap.add_argument("--activation", choices=("identity", "swiglu"), default="identity",
                    help="activation between the projections (swiglu: gated up projection)")
    ap.add_argument("--fused-gather", action="store_true",
                    help="the up projection gathers its rows from the token rows (no permute)")
    ap.add_argument("--probe", action="store_true",
                    help="one warm-up step, a 1 GiB calibration copy, one step (for --pmc runs)")
    ap.add_argument("--render-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--render-mfma", metavar="COUNTER_CSV")
    ap.add_argument("--render-stalls", nargs="+", metavar="COUNTER_CSV")
    ap.add_argument("--render-stats", nargs=3, metavar=("STATS_CSV", "TITLE", "COMMAND"))
    ap.add_argument("--render-counters", nargs=3, metavar=("COUNTER_CSV", "TITLE", "COMMAND"))
    args = ap.parse_args()
    if args.render_traffic:
        render_traffic(*args.render_traffic)
        return
    if args.render_mfma:
        render_mfma(args.render_mfma)
        return
    if args.render_stats:
        render_stats(*args.render_stats)
        return
    if args.render_stalls:
        render_stalls(*args.render_stalls)
        return
    if args.render_counters:
        render_counters(*args.render_counters)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures the one-GPU share of one rank; --gpus {args.gpus} "
              f"(WORLD_SIZE {world}) is not supported: the benchmark has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import synth
    import balanced_token_dispatch_amd as moe  # noqa: F401  (fails loudly if not built)

    wl = synth.WORKLOADS[args.workload]
    target = wl.maxvio_targets[-1] if wl.maxvio_targets[-1] is not None else None
    # a forward-only step runs the permute fused into the up GEMM (measured faster: the
    # step has no weight gradient, whose gathered form pays for scattered token rows)
    if not wl.backward and args.activation == "identity":
        args.fused_gather = True
    layer, idx, w, info = setup_layer(wl, target, args.rank, activation=args.activation,
                                      fused_gather=args.fused_gather)
    s = layer.s
    if args.probe:
        layer.step()
        src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        layer.step()
        torch.cuda.synchronize()
        log("probe done")
        return
    # the timed steps run bare; a second pass of as many steps times every launch with HIP
    # events for the per-kernel figures (the events' own host cost would otherwise stretch
    # the short launches of the small workloads)
    elapsed = run_steps(layer, args.steps, args.warmup)
    # per-kernel figures and the sequential step come from the backward in one stream: the
    # overlapped kernels share CUs with a GEMM, so their own event times would not be theirs
    timer = EventTimer()
    overlap = layer.overlap
    layer.overlap = False
    run_steps(layer, args.steps, 1, timer)
    seq_ms = (run_steps(layer, args.steps, 1) * 1000.0 / args.steps
              if overlap else None)
    layer.overlap = overlap
    status = int(layer.status.item())
    if status != 0:
        log(f"WARNING: plan status {status} (bad ids / slot overflow)")
    n_slots = slots_used(layer)
    ms_step = elapsed * 1000.0 / args.steps
    value = s.S * args.steps / elapsed

    work = algorithmic_work(s, n_slots, gated=args.activation == "swiglu")
    kernels, totals = kernel_fracs(timer, s, n_slots, args.steps,
                                   gated=args.activation == "swiglu")
    # the sum of the kernels' event times against the wall-clock step: the rest is launch gaps
    kern_ms = sum(totals.values())
    dom = max(totals, key=totals.get)
    bound, amount = work[dom]
    avg = kernels[dom]["avg_ms"]
    if bound == "mfma":
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(amount / (avg * 1e-3) / 1e12, 1),
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(amount / (avg * 1e-3) / 1e9, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    tr = recorded_traffic(dom)
    roof["traffic"] = None if tr is None else int(tr)
    if tr is not None:
        roof["traffic_unit"] = "bytes per launch (HBM, FETCH_SIZE+WRITE_SIZE, copy-calibrated)"
    log(f"main: {ms_step:.3f} ms/step, {value:.0f} tokens/s, status {status}, slots used {n_slots}")

    fwd_ms = None
    if not args.main_only:
        fwd_ms = run_steps(layer, args.steps, 2, forward_only=True) * 1000.0 / args.steps
        log(f"forward only: {fwd_ms:.3f} ms/step")
    graph = None
    if not args.no_graph and not args.main_only:
        try:
            g_ms = graph_replay_ms(layer, args.steps)
            graph = {"ms_per_step": round(g_ms, 4), "tokens_per_s": round(s.S / (g_ms * 1e-3), 1)}
            log(f"graph replay: {g_ms:.3f} ms/step")
        except Exception as exc:  # reported, not fatal: the eager figures stand
            graph = {"error": str(exc)[:200]}

    fused = None
    if not args.main_only and not args.fused_gather and args.activation == "identity":
        # the same step with the permute fused into the up projection (its forward GEMM and
        # its weight gradient read the token rows through src_flat)
        layer.fused_gather = True
        el_f = run_steps(layer, args.steps, 2)
        fwd_f = run_steps(layer, args.steps, 2, forward_only=True)
        t_f = EventTimer()
        layer.overlap = False
        run_steps(layer, args.steps, 1, t_f)
        layer.overlap = overlap
        layer.fused_gather = False
        kf, _ = kernel_fracs(t_f, s, n_slots, args.steps)
        fused = {"ms_per_step": round(el_f * 1000.0 / args.steps, 4),
                 "tokens_per_s": round(s.S * args.steps / el_f, 1),
                 "forward_only_ms": round(fwd_f * 1000.0 / args.steps, 4),
                 "forward_only_tokens_per_s": round(s.S * args.steps / fwd_f, 1),
                 "kernels": {k: kf[k] for k in kf if k.endswith("_gather")}}
        log(f"fused gather: {fused['ms_per_step']:.3f} ms/step, forward {fused['forward_only_ms']:.3f} ms")

    sweep = {}
    if not args.no_sweep and not args.main_only and wl.name in SWEEPS:
        sweep = maxvio_sweep(layer, wl, info, ms_step, value, args)
        # restore the headline routing for the CPU baseline below
        layer, idx, w, info = setup_layer(wl, target, args.rank, layer=layer)

    cpu = None
    if not args.no_cpu_baseline:
        t0 = time.time()
        est, parts, n_rows, n_tok = cpu_baseline(layer, idx, w, args.cpu_rows, args.cpu_tokens)
        hc = host_cpu()
        cpu = {"value": round(s.S / est, 2), "unit": "tokens/s", "cores": hc["blas_threads"],
               "kind": "oracle",
               "sample": ((f"plan+layout of all {s.R} ranks' routing in full; permute, fwd up/down, "
                           f"weighted permute, dgrad x2, wgrad x2 on {n_rows} of {s.SK} rows; "
                           f"combine, router-weight gradient and un-permute reduce of {n_tok} of "
                           f"{s.S} tokens; fold on 1/8 of each row; "
                           f"each part timed 3 times (median) and scaled to the full step")
                          if layer.backward_enabled else
                          (f"plan+layout of all {s.R} ranks' routing in full; permute, fwd up/down "
                           f"on {n_rows} of {s.SK} rows; combine of {n_tok} of {s.S} tokens; "
                           f"each part timed 3 times (median) and scaled to the full forward")),
               "cpu_model": hc["cpu_model"], "affinity_cpus": hc["affinity_cpus"],
               "blas_threads": hc["blas_threads"],
               "seconds_measured": round(time.time() - t0, 1),
               "parts_s": {k: round(v, 3) for k, v in parts.items()}}
        log(f"cpu baseline: {cpu['value']} tokens/s ({cpu['seconds_measured']} s, "
            f"{hc['blas_threads']} BLAS threads, {hc['affinity_cpus']} CPUs, {hc['cpu_model']})")

    scale = None
    if not args.no_scale_sweep and not args.main_only and wl.name != SCALE_WORKLOAD:
        # the R64 S8192 E384 sweep needs ~205 GB of the 288 GB: free this layer first
        del layer
        import gc
        gc.collect()
        torch.cuda.empty_cache()
        scale = scale_sweep(args)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "copies_per_s": round(s.SK * args.steps / elapsed, 1),
        "kernel_ms_per_step": round(kern_ms, 4),
        "overlap": None if seq_ms is None else {
            "one_stream_ms_per_step": round(seq_ms, 4), "saved_ms": round(seq_ms - ms_step, 4),
            "second_stream": "router-weight gradient beside the down DGRAD; both folds beside "
                             "the up DGRAD"},
        "forward_only": None if fwd_ms is None else {"ms_per_step": round(fwd_ms, 4),
                                                     "tokens_per_s": round(s.S / (fwd_ms * 1e-3), 1)},
        "graph_replay": graph,
        "fused_gather": fused,
        "data": "synthetic",
        "config": {"workload": wl.name, "R": s.R, "S": s.S, "K": s.K, "E": s.E, "B": s.B,
                   "H": s.H, "H_prime": s.Hp, "activation": args.activation,
                   "dispatch": "permute fused into the up GEMM" if args.fused_gather
                   else "permute, then the up GEMM",
                   "rank": args.rank,
                   "step": "forward+backward" if wl.backward else "forward",
                   "maxvio": round(info["maxvio"], 3), "zipf_s": info["zipf_s"],
                   "plan_status": status, "replica_slots_used_on_rank": n_slots},
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "maxvio_sweep": sweep or None,
        "scale_sweep": scale,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
