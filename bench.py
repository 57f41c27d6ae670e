"""Benchmark: LapSum soft top-k forward + backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c4]

A step is one whole pass of the hot path over one synthetic score vector
already resident in HBM: sample, bracket, streaming pass, the band's
partition refinement (whose steps certify the bracket), p emission with its
fp64 mass partials (forward), then the two VJP kernels (backward).  Steps alternate between two input batches
(the second is the first reversed, in its own memory) so that no step starts
on data the previous one left in the caches.  Prints one JSON line.

`value` is the median step time (ms) on the n = 1e8 U(0,1) workload (k = 1e6,
alpha = 1e-3), the largest configuration the metric is quoted on.  The 1e6
and 1e7 workloads are timed too (warm, where both batches fit in the 256 MB
last-level cache, and with that cache flushed by a 512 MB read between
steps) and reported under "sizes".

"roofline" is measured live: the dominant kernel (most time in a profiled
pre-pass) is bracketed by HIP events on its launch stream during the timed
steps; achieved = its algorithmic bytes per launch / its mean duration.
"traffic" comes from profiles/traffic.json (rocprofv3 FETCH_SIZE + WRITE_SIZE
scaled by a copy kernel of known size) when it was taken from the current
kernel source, else null.  That file is written by

    rocprofv3 --pmc FETCH_SIZE -d <dirF> -o f --output-format csv -- python3 bench.py --profile-run
    rocprofv3 --pmc WRITE_SIZE -d <dirW> -o w --output-format csv -- python3 bench.py --profile-run
    python bench.py --pmc-summary <dirF>/f_counter_collection.csv <dirW>/w_counter_collection.csv

(--profile-run: a few steps of the workload, then a plain device copy of
COPY_BYTES bytes whose counter readings calibrate the two counters).

"rows" times the batched-row operator (one soft top-k per row) forward +
backward on two row workloads, warm and cold, the same way; each carries the
traffic of its two kernels when profiles/traffic.json holds current counter
runs for it (the same three commands with --workload r1 or r2 added to each).

"hbm" gives the step's HBM traffic from the same counter runs: the bytes of
every library kernel of a step (calibrated as above), and that over the median
step time.  "streaming" lists each linear pass with its per-launch time from
an event-instrumented pre-pass (event pairs around each launch, so those
times are a little above the uninstrumented ones and their sum exceeds the
step), its algorithmic rate and its counter-measured rate against the peak.

"verified" times the same steps with the certification pass waited for
(verify_mass = 1: the forward folds the fp64 sum of p and checks it against
k before returning).

"dftopk" times the DFTopK comparator (threshold at the midpoint of the k-th
and (k+1)-th largest scores; forward only) on c1..c4 and reports the mass
sum p it selects and its drift from k.

"cpu_baseline" times the fp64 CPU oracle (forward + backward) once over the
whole workload, on one host thread.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "median ms per soft top-k fwd+bwd at n=1e6/1e7/1e8; achieved HBM GB/s"
PEAK_HBM_GBS = 8000.0
# algorithmic HBM bytes per score of each streaming kernel
ALGO_BYTES = {"pass1": 4, "emit": 8, "vjp_reduce": 8, "vjp_apply": 12}
STEP_BYTES = sum(ALGO_BYTES.values())  # 32 B per score for fwd + bwd
KERNEL_SOURCE = {"pass1": "pass1.hip", "emit": "emit_vjp.hip", "vjp_reduce": "emit_vjp.hip",
                 "vjp_apply": "emit_vjp.hip"}
# device symbols of each streaming step: the score-reading kernel and, from 2^22
# scores on, the variant that uses the emission's saturated-segment record
KERNEL_SYMBOLS = {"pass1": ("stk::pass1_kernel",), "emit": ("stk::emit_kernel", "stk::emit_seg_kernel"),
                  "vjp_reduce": ("stk::vjp_reduce_kernel", "stk::vjp_reduce_seg_kernel"),
                  "vjp_apply": ("stk::vjp_apply_kernel", "stk::vjp_apply_seg_kernel")}
# batched rows: the forward's refinement in lane groups (rows up to 2048
# scores) or by one work-group per row; the backward's lane groups (up to
# 1024), work-groups (up to 8192) and streamed work-groups; algorithmic
# bytes per score
ROWS_ALGO_BYTES = {"rows_forward": 8, "rows_backward": 12}
ROWS_SYMBOLS = {"rows_forward": ("stk::rows_refine_kernel", "stk::rows_refine_wg_kernel"),
                "rows_backward": ("stk::rows_group_backward_kernel", "stk::rows_backward_kernel",
                                  "stk::rows_backward_wg_kernel")}
for _k in ROWS_ALGO_BYTES:
    KERNEL_SOURCE[_k] = "rows.hip"


class Runner:
    """Preallocated buffers + direct C-ABI calls (as a training loop would)."""

    def __init__(self, torch, lib, s, g, k, alpha, params=None):
        self.torch, self.lib = torch, lib
        self.params = params
        self.k, self.alpha = float(k), float(alpha)
        # Two input batches, used in turn: the second is the first reversed
        # (the same values, so every step does the same work) in memory of
        # its own, so a step never starts on data the previous step left in
        # the caches, as a training loop that sees a new batch per step.
        self.batches = [(s, g), (torch.flip(s, [0]).contiguous(), torch.flip(g, [0]).contiguous())]
        self.turn = 0
        self.s, self.g = s, g
        n = s.numel()
        self.n = n
        self.p = torch.empty_like(s)
        self.grad = torch.empty_like(s)
        self.b = torch.empty(1, dtype=torch.float64, device=s.device)
        self.ws_bytes = lib.soft_topk_workspace_bytes(n, None)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=s.device)
        self.bws_bytes = lib.soft_topk_backward_workspace_bytes(n)
        self.bws = torch.empty(self.bws_bytes, dtype=torch.uint8, device=s.device)
        self.stream = ctypes.c_void_p(torch.cuda.current_stream(s.device).cuda_stream)
        from differentiable_soft_top_amd import _lib
        self._lib = _lib
        self.stats = _lib.Stats()
        self._calls = self._calls_stats = None

    def _args(self, stats):
        """The two calls' arguments for each batch, marshalled once (the
        buffers never move), as a C or C++ caller would hold them: the step
        then times the library rather than Python's argument handling."""
        v = ctypes.c_void_p
        prm = ctypes.byref(self.params) if self.params is not None else None
        st = ctypes.byref(self.stats) if stats else None
        out = []
        for s, g in self.batches:
            fwd = (v(s.data_ptr()), self.n, ctypes.c_double(self.k), ctypes.c_double(self.alpha), v(self.p.data_ptr()),
                   v(self.b.data_ptr()), v(self.ws.data_ptr()), self.ws_bytes, self.stream, prm, st)
            bwd = (v(g.data_ptr()), v(s.data_ptr()), self.n, ctypes.c_double(self.alpha), v(self.b.data_ptr()),
                   v(self.grad.data_ptr()), v(self.ws.data_ptr()), self.ws_bytes, v(self.bws.data_ptr()),
                   self.bws_bytes, self.stream)
            out.append((fwd, bwd))
        return out

    def step(self, stats=False):
        """Forward + backward; with stats=True the forward also waits for the
        certification pass and fills self.stats (not used in timed steps).
        self.params (None: the library defaults) goes to every forward."""
        calls = self._calls_stats if stats else self._calls
        if calls is None:
            calls = self._args(stats)
            if stats:
                self._calls_stats = calls
            else:
                self._calls = calls
        fwd, bwd = calls[self.turn]
        self.s, self.g = self.batches[self.turn]
        self.turn ^= 1
        L = self.lib
        rc = L.soft_topk_forward_ex(*fwd)
        if rc:
            self._lib.check(rc, "soft_topk_forward")
        rc = L.soft_topk_backward_ex(*bwd)
        if rc:
            self._lib.check(rc, "soft_topk_backward")


class RowsRunner:
    """Batched rows: preallocated buffers, soft_topk_rows_forward then _backward."""

    # algorithmic bytes per score: read s, write p; read s and g, write grad
    BYTES_PER_SCORE = 20

    def __init__(self, torch, lib, s2d, g2d, k, alpha):
        self.lib = lib
        self.k, self.alpha = float(k), float(alpha)
        self.batches = [(s2d, g2d), (torch.flip(s2d, [1]).contiguous(), torch.flip(g2d, [1]).contiguous())]
        self.turn = 0
        self.rows, self.n_row = s2d.shape
        self.p = torch.empty_like(s2d)
        self.grad = torch.empty_like(s2d)
        self.b = torch.empty(self.rows, dtype=torch.float64, device=s2d.device)
        self.ws_bytes = lib.soft_topk_rows_workspace_bytes(self.rows, self.n_row)
        self.ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=s2d.device)
        self.stream = ctypes.c_void_p(torch.cuda.current_stream(s2d.device).cuda_stream)
        from differentiable_soft_top_amd import _lib
        self._lib = _lib
        self._calls = None

    def step(self):
        if self._calls is None:
            # marshalled once per batch (the buffers never move)
            v, d = ctypes.c_void_p, ctypes.c_double
            self._calls = [((v(s.data_ptr()), self.rows, self.n_row, d(self.k), d(self.alpha), v(self.p.data_ptr()),
                             v(self.b.data_ptr()), v(self.ws.data_ptr()), self.ws_bytes, self.stream),
                            (v(g.data_ptr()), v(s.data_ptr()), self.rows, self.n_row, d(self.alpha),
                             v(self.b.data_ptr()), v(self.grad.data_ptr()), v(self.ws.data_ptr()), self.ws_bytes,
                             self.stream))
                           for s, g in self.batches]
        fwd, bwd = self._calls[self.turn]
        self.turn ^= 1
        L = self.lib
        rc = L.soft_topk_rows_forward(*fwd)
        if rc:
            self._lib.check(rc, "soft_topk_rows_forward")
        rc = L.soft_topk_rows_backward(*bwd)
        if rc:
            self._lib.check(rc, "soft_topk_rows_backward")


def time_steps(torch, runner, steps, flush=None):
    """Per-step HIP events on the launch stream; returns list of ms."""
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        if flush is not None:
            flush.sum()  # evicts the caches by reading only (no dirty lines left behind)
        starts[i].record()
        runner.step()
        ends[i].record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in zip(starts, ends)]


def src_hash(name):
    """Hash of the kernel's source file and the headers that shape its launch."""
    h = hashlib.sha256()
    for fn in (KERNEL_SOURCE[name], "stk_common.hpp", "stk_layout.hpp", "stk_scan.hpp"):
        with open(os.path.join(ROOT, "differentiable_soft_top_amd", "csrc", fn), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def all_src_hash():
    """Hash of every library source (the whole step's kernels and launches)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "differentiable_soft_top_amd", "csrc")
    for fn in sorted(os.listdir(csrc)):
        if fn.endswith((".hip", ".hpp")):
            with open(os.path.join(csrc, fn), "rb") as f:
                h.update(fn.encode())
                h.update(f.read())
    return h.hexdigest()


def step_traffic(workload):
    """Counter-measured HBM bytes of one step, or None when stale or absent."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        tr = json.load(f)
    ent = tr.get(workload, {}).get("kernels", {}).get("_step")
    if not ent or ent.get("source_sha256") != all_src_hash():
        return None
    return ent.get("bytes_per_step")


def traffic_for(kernel, workload):
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        tr = json.load(f)
    ent = tr.get(workload, {}).get("kernels", {}).get(kernel)
    if not ent or ent.get("source_sha256") != src_hash(kernel):
        return None
    return ent.get("bytes_per_launch")


COPY_FLOATS = 100_000_000  # calibration copy: 400 MB read + 400 MB written


def profile_run(torch, steps, warmup, workload):
    """Short run for counter collection: the workload's steps (a single vector
    c1..c5 or a batch of rows r1, r2), then one plain device-to-device copy of
    known size (the calibration kernel)."""
    from differentiable_soft_top_amd import _lib
    from differentiable_soft_top_amd.workloads import ROW_WORKLOADS, draw_grad, make_row_workload, make_workload
    lib = _lib.load()
    dev = torch.device("cuda:0")
    if workload in ROW_WORKLOADS:
        s_np, k, alpha, w = make_row_workload(workload)
        g_np = draw_grad(s_np.size, w.seed).reshape(s_np.shape)
        run = RowsRunner(torch, lib, torch.from_numpy(s_np).to(dev), torch.from_numpy(g_np).to(dev), k, alpha)
    else:
        s_np, k, alpha, w = make_workload(workload)
        s = torch.from_numpy(s_np).to(dev)
        g = torch.from_numpy(draw_grad(s_np.size, w.seed)).to(dev)
        run = Runner(torch, lib, s, g, k, alpha)
    for _ in range(warmup + steps):
        run.step()
    torch.cuda.synchronize()
    src = torch.ones(COPY_FLOATS, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"profile_run": workload, "steps": steps, "warmup": warmup, "copy_bytes": 4 * COPY_FLOATS}))


def _read_counter_csv(path, counter):
    """{kernel name: [value per dispatch]} from a rocprofv3 counter_collection.csv."""
    import csv
    out = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") != counter:
                continue
            out.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return out


def pmc_summary(fetch_csv, write_csv, workload="c4"):
    """Turn the two counter runs of --profile-run into the workload's entry of
    profiles/traffic.json: bytes per launch of each streaming kernel, each
    counter scaled so that the calibration copy reads exactly its known size.
    Other workloads' entries are kept."""
    fetch = _read_counter_csv(fetch_csv, "FETCH_SIZE")
    write = _read_counter_csv(write_csv, "WRITE_SIZE")
    copy_bytes = 4 * COPY_FLOATS

    def copy_value(table):
        vals = [v for name, vs in table.items() if "copyBuffer" in name for v in vs]
        return max(vals) * 1024.0  # KiB -> bytes; the largest copy is the calibration one

    f_scale = copy_bytes / copy_value(fetch)
    w_scale = copy_bytes / copy_value(write)
    from differentiable_soft_top_amd.workloads import ROW_WORKLOADS, WORKLOADS
    if workload in ROW_WORKLOADS:
        n = ROW_WORKLOADS[workload].rows * ROW_WORKLOADS[workload].n_row
        algo, symbols = ROWS_ALGO_BYTES, ROWS_SYMBOLS
    else:
        n = WORKLOADS[workload].n
        algo, symbols = ALGO_BYTES, KERNEL_SYMBOLS
    calib = {"copy_bytes": copy_bytes, "fetch_scale": f_scale, "write_scale": w_scale,
             "fetch_csv": os.path.basename(fetch_csv), "write_csv": os.path.basename(write_csv)}
    ent = {}
    for kname in algo:
        fk = [name for name in fetch if any(sym in name for sym in symbols[kname])]
        wk = [name for name in write if any(sym in name for sym in symbols[kname])]
        if not fk or not wk:
            continue
        fv = [v for name in fk for v in fetch[name]]
        wv = [v for name in wk for v in write[name]]
        fb = sum(fv) / len(fv) * 1024.0 * f_scale
        wb = sum(wv) / len(wv) * 1024.0 * w_scale
        ent[kname] = {"kernels": sorted(set(fk)), "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
                      "bytes_per_launch": fb + wb, "algorithmic_bytes_per_launch": algo[kname] * n,
                      "launches": len(fv), "source_sha256": src_hash(kname)}
    # the whole step: every library kernel, per step (the backward's last
    # kernel runs once per step)
    last = symbols["rows_backward" if workload in ROW_WORKLOADS else "vjp_apply"]
    n_steps = sum(len(vs) for name, vs in write.items() if any(sym in name for sym in last))
    if n_steps:
        fb = sum(v for name, vs in fetch.items() if "stk::" in name for v in vs) * 1024.0 * f_scale
        wb = sum(v for name, vs in write.items() if "stk::" in name for v in vs) * 1024.0 * w_scale
        ent["_step"] = {"fetch_bytes_per_step": fb / n_steps, "write_bytes_per_step": wb / n_steps,
                        "bytes_per_step": (fb + wb) / n_steps, "steps": n_steps,
                        "source_sha256": all_src_hash()}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    result = {}
    if os.path.exists(path):
        with open(path) as f:
            result = json.load(f)
    result.pop("_calibration", None)  # older single-workload layout
    result[workload] = {"calibration": calib, "kernels": ent}
    with open(path, "w") as f:
        json.dump(result, f, indent=1, sort_keys=True)
    print(json.dumps(result, indent=1, sort_keys=True))


def cpu_baseline(s_np, g_np, k, alpha, name):
    """The fp64 CPU oracle (forward then backward) once over the whole
    workload, single-threaded (qsort, scans, closed form, then the VJP)."""
    from oracle import oracle as O
    t0 = time.perf_counter()
    _, b = O.forward(s_np, k, alpha)
    O.backward(g_np, s_np, alpha, b)
    dt = time.perf_counter() - t0
    return {
        "value": dt * 1e3,
        "unit": "ms",
        "cores": 1,
        "kind": "oracle",
        "sample": "one run of the fp64 C oracle (qsort + prefix/suffix scans + closed form, then the VJP) "
                  "over the whole %s workload (n=%d), input conversion included, on one host thread"
                  % (name, s_np.size),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c4")
    ap.add_argument("--sizes", default="c1,c2,c3,c5", help="extra workloads timed (comma list, '' for none)")
    ap.add_argument("--rows", default="r1,r2", help="batched-row workloads timed (comma list, '' for none)")
    ap.add_argument("--dftopk", default="c1,c2,c3,c4",
                    help="workloads timed with the DFTopK comparator, whose mass drift is reported")
    ap.add_argument("--curve", default="c3,c4",
                    help="workloads whose threshold curve (full sort of the scores, then the mass at each) is timed")
    ap.add_argument("--fullsort", default="c2,c3",
                    help="workloads timed forward+backward on the forced full-sort route (the fallback)")
    ap.add_argument("--coverage", default="c1,c2,c3,c4",
                    help="workloads run with 100 sampler seeds each on the bracketed route: how many "
                         "certify on their first round (no widening, no fallback)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-run", action="store_true",
                    help="counter-collection run: a few steps of --workload (c1..c5 or a row workload "
                         "r1, r2), then the calibration copy")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from two rocprofv3 counter CSVs (no GPU needed)")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.workload)
        return
    if args.gpus != 1:
        print("bench.py: the benchmark runs on one GPU only (the operator is single-device); "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    if args.profile_run:
        profile_run(torch, min(args.steps, 5), min(args.warmup, 2), args.workload)
        return

    from differentiable_soft_top_amd import _lib
    from differentiable_soft_top_amd.workloads import draw_grad, make_workload

    lib = _lib.load()
    dev = torch.device("cuda:0")

    def setup(name):
        s_np, k, alpha, w = make_workload(name)
        g_np = draw_grad(s_np.size, w.seed)
        s = torch.from_numpy(s_np).to(dev)
        g = torch.from_numpy(g_np).to(dev)
        return s_np, g_np, k, alpha, w, Runner(torch, lib, s, g, k, alpha)

    s_np, g_np, k, alpha, w, run = setup(args.workload)
    n = s_np.size
    run.step(stats=True)  # route, band size and certified mass of this workload
    for _ in range(args.warmup):
        run.step()
    torch.cuda.synchronize()

    # profiled pre-pass: per-kernel time of every kernel (not the timed region)
    _lib.profile_begin(_lib.kernel_names())
    for _ in range(3):
        run.step()
    torch.cuda.synchronize()
    breakdown = _lib.profile_end()
    per_step = {kname: ms / 3.0 for kname, (ms, cnt) in breakdown.items()}
    streaming = {kname: v for kname, v in per_step.items() if kname in ALGO_BYTES}
    # (a vector short enough for the one-kernel route has no streaming kernel)
    dominant = max(streaming, key=streaming.get) if streaming else None

    # timed region: K steps, the dominant kernel bracketed by events live
    _lib.profile_begin([dominant] if dominant else [])
    times = time_steps(torch, run, args.steps)
    prof = _lib.profile_end()
    if dominant:
        dom_ms, dom_launches = prof[dominant]
        dom_avg_s = dom_ms / dom_launches / 1e3
        algo = ALGO_BYTES[dominant] * n
        achieved = algo / dom_avg_s / 1e9
    else:
        dom_launches, dom_avg_s, algo, achieved = 0, float("nan"), 0, float("nan")
    median = float(np.median(times))
    mean = float(np.mean(times))
    st = run.stats.as_dict()

    # the same steps with the certification pass waited for (fp64 sum of p
    # folded and checked against k inside every forward)
    vprm = _lib.default_params()
    vprm.verify_mass = 1
    vrun = Runner(torch, lib, run.batches[0][0], run.batches[0][1], k, alpha, params=vprm)
    for _ in range(3):
        vrun.step()
    vtimes = time_steps(torch, vrun, args.steps)
    del vrun
    torch.cuda.empty_cache()

    # per streaming kernel: pre-pass event times, algorithmic and counter rates
    streaming_out = {}
    for kname in ALGO_BYTES:
        if kname not in per_step:
            continue
        t_ms = per_step[kname]
        tb = traffic_for(kname, args.workload)
        streaming_out[kname] = {
            "avg_us_event_prepass": t_ms * 1e3,
            "algorithmic_bytes": ALGO_BYTES[kname] * n,
            "algorithmic_GBps": ALGO_BYTES[kname] * n / (t_ms / 1e3) / 1e9,
            "counter_bytes": tb,
            "counter_GBps": (tb / (t_ms / 1e3) / 1e9) if tb else None,
            "counter_frac_of_peak": (tb / (t_ms / 1e3) / 1e9 / PEAK_HBM_GBS) if tb else None,
        }
    step_bytes = step_traffic(args.workload)

    sizes = {}
    for extra in [x for x in args.sizes.split(",") if x]:
        es_np, eg_np, ek, ealpha, ew, erun = setup(extra)
        erun.step(stats=True)
        for _ in range(3):
            erun.step()
        warm = time_steps(torch, erun, 50)
        flush = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
        cold = time_steps(torch, erun, 20, flush=flush)
        del flush
        med = float(np.median(warm))
        sizes[extra] = {
            "workload": ew.description, "n": int(es_np.size), "k": ek, "alpha": ealpha,
            "median_ms": med, "p10_ms": float(np.percentile(warm, 10)), "p90_ms": float(np.percentile(warm, 90)),
            "median_ms_cold": float(np.median(cold)),
            "algorithmic_GBps": STEP_BYTES * es_np.size / (med / 1e3) / 1e9,
            "path": erun.stats.path,
        }
        del erun
        torch.cuda.empty_cache()

    rows_out = {}
    from differentiable_soft_top_amd.workloads import make_row_workload
    for rname in [x for x in args.rows.split(",") if x]:
        s2_np, rk, ralpha, rw = make_row_workload(rname)
        g2_np = draw_grad(s2_np.size, rw.seed).reshape(s2_np.shape)
        rrun = RowsRunner(torch, lib, torch.from_numpy(s2_np).to(dev), torch.from_numpy(g2_np).to(dev), rk, ralpha)
        for _ in range(3):
            rrun.step()
        warm = time_steps(torch, rrun, 50)
        flush = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
        cold = time_steps(torch, rrun, 20, flush=flush)
        del flush
        med = float(np.median(warm))
        rows_out[rname] = {
            "workload": rw.description, "rows": rw.rows, "n_row": rw.n_row,
            "median_ms": med, "p10_ms": float(np.percentile(warm, 10)), "p90_ms": float(np.percentile(warm, 90)),
            "median_ms_cold": float(np.median(cold)),
            "algorithmic_GBps": RowsRunner.BYTES_PER_SCORE * s2_np.size / (med / 1e3) / 1e9,
            # HBM bytes per launch from the counter runs (null when stale)
            "traffic": {kname: traffic_for(kname, rname) for kname in ROWS_ALGO_BYTES},
        }
        del rrun
        torch.cuda.empty_cache()

    # DFTopK comparator: forward only (it has no backward), with its mass
    # drift from k at each workload's alpha
    dft_out = {}
    for dname in [x for x in args.dftopk.split(",") if x]:
        ds_np, dk, dalpha, dw = make_workload(dname)
        ds = torch.from_numpy(ds_np).to(dev)
        dp = torch.empty_like(ds)
        db = torch.empty(1, dtype=torch.float64, device=dev)
        dm = torch.empty(1, dtype=torch.float64, device=dev)
        dws_bytes = lib.soft_topk_dftopk_workspace_bytes(ds.numel())
        dws = torch.empty(dws_bytes, dtype=torch.uint8, device=dev)
        stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        v = ctypes.c_void_p

        class _DftRun:
            def step(self):
                _lib.check(lib.soft_topk_dftopk_forward(v(ds.data_ptr()), ds.numel(), float(int(dk)), dalpha,
                                                        v(dp.data_ptr()), v(db.data_ptr()), v(dm.data_ptr()),
                                                        v(dws.data_ptr()), dws_bytes, stream),
                           "soft_topk_dftopk_forward")

        drun = _DftRun()
        for _ in range(3):
            drun.step()
        dt = time_steps(torch, drun, 20)
        mass = float(dm.item())
        dft_out[dname] = {"workload": dw.description, "n": int(ds_np.size), "k": int(dk), "alpha": dalpha,
                          "forward_median_ms": float(np.median(dt)), "b": float(db.item()), "mass": mass,
                          "drift": mass - int(dk), "drift_rel": (mass - int(dk)) / int(dk)}
        del ds, dp, dws
        torch.cuda.empty_cache()

    # the full-sort route forced (the fallback of the bracketed solver),
    # forward + backward through the same runner
    full_out = {}
    for fname in [x for x in args.fullsort.split(",") if x]:
        fs_np, fk, falpha, fw = make_workload(fname)
        fprm = _lib.default_params()
        fprm.force_path = _lib.PATH_FULLSORT
        frun = Runner(torch, lib, torch.from_numpy(fs_np).to(dev), torch.from_numpy(draw_grad(fs_np.size, fw.seed)).to(dev),
                      fk, falpha, params=fprm)
        frun.step(stats=True)
        for _ in range(3):
            frun.step()
        ft = time_steps(torch, frun, 20)
        full_out[fname] = {"workload": fw.description, "n": int(fs_np.size), "k": fk, "alpha": falpha,
                           "median_ms": float(np.median(ft)), "p10_ms": float(np.percentile(ft, 10)),
                           "p90_ms": float(np.percentile(ft, 90)), "path": frun.stats.path}
        del frun
        torch.cuda.empty_cache()

    # the threshold curve: sorted scores and the mass each selects as a
    # threshold (soft_topk_threshold_curve)
    curve_out = {}
    for cname in [x for x in args.curve.split(",") if x]:
        if cname == args.workload:
            cs, calpha, cw = run.batches[0][0], alpha, w
        else:
            cs_np, _, calpha, cw = make_workload(cname)
            cs = torch.from_numpy(cs_np).to(dev)
        cn = cs.numel()
        c_sorted = torch.empty_like(cs)
        c_mass = torch.empty(cn, dtype=torch.float64, device=dev)
        cws_bytes = lib.soft_topk_workspace_bytes(cn, None)
        cws = torch.empty(cws_bytes, dtype=torch.uint8, device=dev)
        cstream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        cargs = (ctypes.c_void_p(cs.data_ptr()), cn, ctypes.c_double(calpha), ctypes.c_void_p(c_sorted.data_ptr()),
                 ctypes.c_void_p(c_mass.data_ptr()), ctypes.c_void_p(cws.data_ptr()), cws_bytes, cstream)

        class _CurveRun:
            def step(self):
                _lib.check(lib.soft_topk_threshold_curve(*cargs), "soft_topk_threshold_curve")

        crun = _CurveRun()
        for _ in range(3):
            crun.step()
        ct = time_steps(torch, crun, 10)
        curve_out[cname] = {"workload": cw.description, "n": int(cn), "alpha": calpha,
                            "median_ms": float(np.median(ct)), "p10_ms": float(np.percentile(ct, 10)),
                            "p90_ms": float(np.percentile(ct, 90))}
        del c_sorted, c_mass, cws
        torch.cuda.empty_cache()

    # path coverage: 100 Philox seeds per workload on the bracketed route
    # (forced for c1, which would otherwise take the one-kernel route)
    import differentiable_soft_top_amd as stk
    cov_out = {}
    for vname in [x for x in args.coverage.split(",") if x]:
        if vname == args.workload:
            vs, vk, valpha = run.batches[0][0], k, alpha
        else:
            vs_np, vk, valpha, _ = make_workload(vname)
            vs = torch.from_numpy(vs_np).to(dev)
        seeds = [int(x) for x in np.random.default_rng(2024).integers(1, 2 ** 63, 100)]
        first = widened = other = 0
        for seed in seeds:
            vprm_s = _lib.default_params()
            vprm_s.seed = seed
            vprm_s.force_path = _lib.PATH_BRACKET
            _, _, vst = stk.forward(vs, vk, valpha, vprm_s, want_stats=True)
            if vst["path"] == _lib.PATH_BRACKET and vst["rounds"] == 1:
                first += 1
            elif vst["path"] == _lib.PATH_WIDENED:
                widened += 1
            else:
                other += 1
        cov_out[vname] = {"seeds": len(seeds), "certified_first_round": first, "widened": widened,
                          "other_route": other}
        del vs
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(s_np, g_np, k, alpha, args.workload)

    out = {
        "metric": METRIC,
        "value": median,
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": mean,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 io, f64 arithmetic",
        "data": "synthetic (seeded numpy PCG64; recipe in differentiable_soft_top_amd/workloads.py)",
        "config": {"workload": "%s: %s, forward+backward" % (args.workload, w.description),
                   "n": int(n), "k": k, "alpha": alpha},
        "p10_ms": float(np.percentile(times, 10)),
        "p90_ms": float(np.percentile(times, 90)),
        "algorithmic_GBps": STEP_BYTES * n / (median / 1e3) / 1e9,
        "path": st["path"],
        "band": st["n_band"],
        "certified_mass_error": abs(st["mass"] - k),
        "verified": {"median_ms": float(np.median(vtimes)), "p10_ms": float(np.percentile(vtimes, 10)),
                     "p90_ms": float(np.percentile(vtimes, 90)), "verify_mass": 1},
        "hbm": {"bytes_per_step": step_bytes,
                "GBps": (step_bytes / (median / 1e3) / 1e9) if step_bytes else None,
                "frac_of_peak": (step_bytes / (median / 1e3) / 1e9 / PEAK_HBM_GBS) if step_bytes else None,
                "source": "rocprofv3 FETCH_SIZE + WRITE_SIZE over every library kernel of a step, "
                          "calibrated on a device copy (profiles/traffic.json)"},
        "streaming": streaming_out,
        "kernels_ms_event_prepass": {kname: round(v, 5) for kname, v in sorted(per_step.items())},
        "roofline": None if dominant is None else {
            "kernel": dominant,
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": traffic_for(dominant, args.workload) if dominant else None,
            "algorithmic_bytes_per_launch": algo,
            "avg_launch_ms": dom_avg_s * 1e3,
            "launches": dom_launches,
        },
        "sizes": sizes,
        "rows": rows_out,
        "dftopk": dft_out,
        "fullsort": full_out,
        "curve": curve_out,
        "coverage": cov_out,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
