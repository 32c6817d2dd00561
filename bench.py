"""Benchmark of the FP32 NCHW convolution library on one MI355X.

One step = one pass of the whole hot path over the seven shape rows of the
five workloads (grouped 3x3 cpg 4, depthwise 144, grouped 64/128/256 groups,
dense 5x9, fused conv+bias+scale+sigmoid+GroupNorm), one library call per
row, with inputs resident in HBM and rotated over B buffer sets so that
every row streams at least ~512 MB per rotation (cold-cache honesty for
rows that fit the 256 MB Infinity Cache).

Timing boundaries:
  step      K steps launched back to back; HIP events recorded on the launch
            stream around every row give each row's device time per launch.
  graph     per row, R launches captured in one HIP graph by the library's
            gconv_time_graph; device events around each replay, 10 batches
            x 30 samples; time / R.
  sync      per row, host clock around (library call + stream sync),
            10 batches x 30 samples.
Medians come with a 95% bootstrap interval (10,000 resamples).

The printed JSON line's `value` is the geometric mean over the seven rows
of algorithmic GB/s (compulsory bytes x + w + y [+ per-channel vectors],
divided by the step-boundary device time).  `roofline` is reported for the
kernel that takes the most device time per step; `cpu_baseline` times the
CPU oracle on a bounded sample of every row on this host.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "per-shape GB/s + GFLOP/s, % roofline, geomean; hipGraph vs sync-API timing"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP32_MFMA_PEAK_TFLOPS = 157.3  # MI355X dense FP32 matrix, published
FP32_VALU_PEAK_TFLOPS = 157.3  # MI355X FP32 vector, published (non-packed FMA chains measure above the
                               # 78.6 TFLOP/s that one FMA per lane per clock would allow)
COLD_BYTES = 512 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rows", default="", help="comma-separated subset of rows (default: all)")
    ap.add_argument("--batches", type=int, default=10)
    ap.add_argument("--samples", type=int, default=30)
    ap.add_argument("--no-boundaries", action="store_true", help="skip the graph/sync tables")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--warm", action="store_true", help="one buffer set per row (cache-warm)")
    ap.add_argument("--copy-only", action="store_true",
                    help="run only the plain device-copy calibration (known byte count per launch)")
    ap.add_argument("--sweep", action="store_true",
                    help="time the 80-shape grouped 3x3 grid instead of the shape rows: the dispatcher's "
                         "choice against the direct kernel and PyTorch's conv2d, paired batches")
    ap.add_argument("--sweep-shapes", default="",
                    help="comma-separated grid shapes, general-geometry or implicit-GEMM layers "
                         "(default: the 80 grid shapes)")
    ap.add_argument("--sweep-out", default="", help="write the per-shape sweep records to this JSON file")
    ap.add_argument("--sweep-no-torch", action="store_true", help="leave PyTorch's conv2d out of the sweep")
    ap.add_argument("--block", action="store_true",
                    help="block-substitution probe: an inverted-residual block (MobileNetV2 features[3] shape) "
                         "timed as is and with its depthwise conv replaced by the library's, paired batches")
    ap.add_argument("--block-batch", default="1,4", help="comma-separated batch sizes for --block")
    return ap.parse_args()


COPY_BYTES = 256 << 20  # bytes read (and as many written) by one calibration copy


def copy_calibration(torch, gc):
    """The library's own streaming copy (gconv_probe_copy) over COPY_BYTES,
    well beyond the 256 MB last-level cache: the measured HBM rate (bytes
    read + written per second, fastest of five launches).  Its dispatches
    (copy_probe_kernel) are also the reference launch for scaling HBM
    traffic counters: each reads and writes exactly COPY_BYTES."""
    n = COPY_BYTES // 4
    src = torch.empty(n, device="cuda").uniform_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    gbs = gc.gconv_probe_copy(dst, src)
    ok = bool(torch.equal(dst, src))
    del src, dst
    return dict(bytes_per_launch=2 * COPY_BYTES, gbs=gbs, kernel="copy_probe_kernel", copy_equal=ok)


# ------------------------------------------------------------------ work accounting


def row_accounting(wl, ho, wo):
    """Algorithmic bytes and flops of one launch (the method's compulsory traffic)."""
    x = wl.N * wl.C * wl.H * wl.W
    w = wl.K * (wl.C // wl.groups) * wl.R * wl.S
    y = wl.N * wl.K * ho * wo
    vec = 4 * wl.K if wl.fused else 0          # bias, scale, gamma, beta
    macs = y * (wl.C // wl.groups) * wl.R * wl.S
    flops = 2 * macs
    byts = 4 * (x + w + y + vec)
    # dense rows run on FP32 MFMA, grouped rows on the FP32 VALU
    peak = FP32_MFMA_PEAK_TFLOPS if wl.groups == 1 else FP32_VALU_PEAK_TFLOPS
    t_mem, t_cmp = byts / (HBM_PEAK_GBS * 1e9), flops / (peak * 1e12)
    if t_mem >= t_cmp:
        bound = "hbm"
    else:
        bound = "mfma" if wl.groups == 1 else "alu"
    return dict(bytes=byts, flops=flops, bound=bound, floor_s=max(t_mem, t_cmp), compute_peak_tflops=peak)


# Sources each benchmark row's kernels are built from (beside the shared
# headers): a committed HBM-traffic record counts only while they are unchanged.
ROW_SOURCES = {
    "c1_grouped_cpg4": ["k_grouped3x3.hip"],
    "c2_depthwise_144": ["k_grouped3x3.hip"],
    "c3a_grouped_g64": ["k_grouped3x3.hip"],
    "c3b_grouped_g128": ["k_grouped3x3.hip"],
    "c3c_depthwise_g256": ["k_grouped3x3.hip"],
    "c4_dense_5x9": ["k_igemm.hip"],
    "c5_fused_gn": ["k_igemm_res.hip", "gconv_api.cpp"],
}
TRAFFIC_RECORDS = os.path.join(ROOT, "profiles", "hbm_traffic_seven_rows.md")


def row_source_hash(row):
    """sha256 over the sources a row's kernels are built from (+ shared headers)."""
    import hashlib
    csrc = os.path.join(ROOT, "grouped_convolution_conv_amd", "csrc")
    h = hashlib.sha256()
    for f in ROW_SOURCES[row] + ["dev_common.h", "internal.h"]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(row):
    """HBM bytes per launch of a row (every kernel of one library call) from
    the committed counter record.

    profiles/hbm_traffic_seven_rows.md carries one line per row
      traffic-record: row=<row> sha256=<row_source_hash> fetch_kib=F write_kib=W fetch_scale=a write_scale=b
    with the rocprofv3 FETCH_SIZE / WRITE_SIZE averages (KiB per call, summed
    over the row's kernels) and the factors that map the library copy probe's
    counters onto its known size.  Returns None when the row has no record or
    its kernels' sources changed since."""
    import re
    if row not in ROW_SOURCES or not os.path.exists(TRAFFIC_RECORDS):
        return None
    m = re.search(r"traffic-record: row=%s sha256=(\w+) fetch_kib=([\d.]+) write_kib=([\d.]+) "
                  r"fetch_scale=([\d.]+) write_scale=([\d.]+)" % re.escape(row), open(TRAFFIC_RECORDS).read())
    if not m or m.group(1) != row_source_hash(row):
        return None
    f, w, fs, ws = (float(m.group(i)) for i in range(2, 6))
    return (f * fs + w * ws) * 1024.0


def boot_ci(samples, n_boot=10000, seed=0):
    a = np.asarray(samples, dtype=np.float64)
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, a.size, size=(n_boot, a.size))
    meds = np.median(a[idx], axis=1)
    return float(np.median(a)), float(np.percentile(meds, 2.5)), float(np.percentile(meds, 97.5))


def geomean(v):
    v = [x for x in v if x and x > 0]
    return float(math.exp(sum(math.log(x) for x in v) / len(v))) if v else None


# ------------------------------------------------------------------ rows


class Row:
    def __init__(self, name, wl, gc, torch, warm):
        import synth
        self.name, self.wl = name, wl
        self.gc, self.torch = gc, torch
        self.desc = gc.conv_desc_create(wl.N, wl.C, wl.H, wl.W, wl.K, wl.R, wl.S, wl.stride, wl.pad,
                                        wl.dil, wl.groups)
        self.ho, self.wo = gc.conv_desc_get_output_dims(self.desc)
        self.algo = gc.ALGO_NAMES[gc.conv_desc_get_algo(self.desc)]
        self.acct = row_accounting(wl, self.ho, self.wo)
        inp = synth.make_inputs(wl)
        dev = "cuda"
        nsets = 1 if warm else max(1, int(math.ceil(COLD_BYTES / self.acct["bytes"])))
        if self.acct["bytes"] < (1 << 20):
            nsets = 1  # launch-bound row: rotation would not change what is measured
        self.nsets = nsets
        x0 = torch.from_numpy(inp["x"]).to(dev)
        self.x = [x0] + [x0.clone() for _ in range(nsets - 1)]
        self.w = torch.from_numpy(inp["w"]).to(dev)
        self.y = [torch.empty((wl.N, wl.K, self.ho, self.wo), device=dev) for _ in range(nsets)]
        self.vec = {k: (torch.from_numpy(inp[k]).to(dev) if inp.get(k) is not None else None)
                    for k in ("bias", "scale", "gamma", "beta")}
        if wl.fused:
            nb = gc.conv_fused_gn_workspace_size(self.desc, wl.gn_groups)
            self.ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)
        self.inputs_host = inp

    def prepare(self, stream):
        """Raw device addresses and the stream handle, resolved once: the timed
        loop then spends its host time in the library call, not in reading
        tensor attributes."""
        self.px = [t.data_ptr() for t in self.x]
        self.py = [t.data_ptr() for t in self.y]
        self.pw = self.w.data_ptr()
        self.pv = {k: (t.data_ptr() if t is not None else None) for k, t in self.vec.items()}
        self.pws = self.ws.data_ptr() if self.wl.fused else None
        self.ws_bytes = self.ws.numel() if self.wl.fused else 0
        self.stream_handle = stream.cuda_stream

    def launch(self, i, stream=None):
        s = i % self.nsets
        gc = self.gc
        if stream is None and getattr(self, "stream_handle", None) is not None:
            if self.wl.fused:
                v = self.pv
                gc.conv_fused_gn_fwd(self.desc, self.px[s], self.pw, v["bias"], v["scale"], v["gamma"], v["beta"],
                                     self.wl.gn_groups, self.wl.eps, self.py[s], self.pws, self.ws_bytes,
                                     stream=self.stream_handle)
            else:
                gc.conv_fwd(self.desc, self.px[s], self.pw, None, self.py[s], stream=self.stream_handle)
            return
        if self.wl.fused:
            v = self.vec
            gc.conv_fused_gn_fwd(self.desc, self.x[s], self.w, v["bias"], v["scale"], v["gamma"], v["beta"],
                                 self.wl.gn_groups, self.wl.eps, self.y[s], self.ws, stream=stream)
        else:
            gc.conv_fwd(self.desc, self.x[s], self.w, None, self.y[s], stream=stream)

    def figures(self, seconds):
        a = self.acct
        return dict(ms=seconds * 1e3, gbs=a["bytes"] / seconds / 1e9, gflops=a["flops"] / seconds / 1e9,
                    roofline_frac=a["floor_s"] / seconds)


def graph_boundary(row, torch, batches, samples):
    """R launches captured in one HIP graph by the library's gconv_time_graph;
    per-launch device time of each replay (device events around the replay)."""
    per = row.acct["bytes"] / (HBM_PEAK_GBS * 1e9) + row.acct["flops"] / 100e12
    R = int(min(500, max(2, math.ceil(1e-3 / max(per, 2e-6)))))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    gc = row.gc
    fused = None
    if row.wl.fused:
        v = row.vec
        fused = dict(scale=v["scale"], gamma=v["gamma"], beta=v["beta"], gn_groups=row.wl.gn_groups,
                     eps=row.wl.eps, workspace=row.ws)
    out = []
    for _ in range(batches):
        out += [m / 1e3 for m in gc.gconv_time_graph(row.desc, row.x, row.y, row.w, row.vec["bias"], launches=R,
                                                    replays=samples, fused=fused, stream=s)]
    torch.cuda.synchronize()
    return out, R


def sync_boundary(row, torch, batches, samples):
    out = []
    for i in range(3):
        row.launch(i)
    torch.cuda.synchronize()
    k = 0
    for _ in range(batches):
        for _ in range(samples):
            t0 = time.perf_counter()
            row.launch(k)
            torch.cuda.synchronize()
            out.append(time.perf_counter() - t0)
            k += 1
    return out


# ------------------------------------------------------------------ CPU baseline

CPU_ROW_SECONDS = 1.0   # target oracle time per row and run: 7 rows x 3 runs x ~1 s of host work
CPU_RUNS = 3            # timed runs per row; the median is reported


def cpu_threads():
    """Host threads for the oracle: OMP_NUM_THREADS when the environment
    sets it (the CPU share a job on this host is given), else every CPU this
    process may run on."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    return len(os.sched_getaffinity(0))


def cpu_baseline(rows):
    """The CPU oracle (fp64, OpenMP over output planes) timed on this host.

    Each row runs on its first n images, n chosen from a one-image probe so
    that the row takes about CPU_ROW_SECONDS; rows whose whole batch is
    faster than that are repeated within a run.  Every row is timed
    CPU_RUNS times and the median run is reported."""
    import oracle
    threads = cpu_threads()
    per_row = {}
    total = 0.0

    def run(wl, inp, n):
        x = inp["x"][:n]
        t0 = time.perf_counter()
        if wl.fused:
            oracle.fused_gn(x, inp["w"], inp["bias"], inp["scale"], inp["gamma"], inp["beta"], wl.gn_groups,
                            wl.eps, wl.stride, wl.pad, wl.dil, wl.groups, threads=threads)
        else:
            oracle.conv2d(x, inp["w"], None, wl.stride, wl.pad, wl.dil, wl.groups, threads=threads,
                          want_bound=False)
        return time.perf_counter() - t0

    for r in rows:
        wl, inp = r.wl, r.inputs_host
        t1 = run(wl, inp, 1)
        total += t1
        n = int(max(1, min(wl.N, round(CPU_ROW_SECONDS / max(t1, 1e-6)))))
        reps = 1
        if n == wl.N:
            reps = int(max(1, min(1000, round(CPU_ROW_SECONDS / max(t1 * wl.N, 1e-6)))))
        runs = []
        for _ in range(CPU_RUNS):
            dt = 0.0
            for _ in range(reps):
                dt += run(wl, inp, n)
            total += dt
            runs.append(dt / reps)
        dt = float(np.median(runs))
        a = row_accounting(wl.with_(N=n), r.ho, r.wo)
        per_row[r.name] = dict(samples_n=n, repeats=reps, runs_s=runs, seconds=dt, gbs=a["bytes"] / dt / 1e9,
                               gflops=a["flops"] / dt / 1e9)
        log("[cpu] %-20s N=%d x%d  median of %d: %.3f s  %.3f GB/s  %.3f GFLOP/s"
            % (r.name, n, reps, CPU_RUNS, dt, per_row[r.name]["gbs"], per_row[r.name]["gflops"]))
    return dict(value=geomean([v["gbs"] for v in per_row.values()]),
                unit="GB/s (geomean of rows, oracle fp64 on the host)", cores=threads, kind="oracle",
                cpu_model=cpu_model(), host_cpus=os.cpu_count(),
                sample="each row on its first n images (repeated when the whole batch is short), median of %d "
                       "runs: " % CPU_RUNS +
                       ", ".join("%s n=%d x%d" % (k, v["samples_n"], v["repeats"]) for k, v in per_row.items()),
                seconds=total, rows=per_row)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def measured_floor_s(acct, wl, peaks):
    """Floor time against what this GPU sustains: the library's measured copy
    rate and the measured FP32 MFMA (dense rows) or FP32 FMA (grouped rows)
    rate."""
    peak = peaks["fp32_mfma_tflops"] if wl.groups == 1 else peaks["fp32_fma_tflops"]
    return max(acct["bytes"] / (peaks["hbm_copy_gbs"] * 1e9), acct["flops"] / (peak * 1e12))


# ------------------------------------------------------------------ shape sweep

PRACTICAL = 1.05   # a ratio counts only when its whole 95% interval clears 5%


def paired_ratio(base_batches, cand_batches, n_boot=10000, seed=0):
    """base / candidate latency from paired batches (the GroupConv Atlas's
    "ten paired batches, 95% bootstrap intervals, 5% practical threshold").

    Each batch gives the ratio of the two medians; the point estimate is the
    geometric mean over batches and the interval comes from resampling the
    batches.  A shape is a "win" for the candidate when the whole interval lies
    above 1.05, a "loss" when it lies below 1/1.05, and a "tie" otherwise."""
    lr = np.log([np.median(b) / np.median(c) for b, c in zip(base_batches, cand_batches)])
    rng = np.random.default_rng(seed)
    means = lr[rng.integers(0, lr.size, size=(n_boot, lr.size))].mean(axis=1)
    lo, hi = float(np.exp(np.percentile(means, 2.5))), float(np.exp(np.percentile(means, 97.5)))
    cls = "win" if lo > PRACTICAL else ("loss" if hi < 1.0 / PRACTICAL else "tie")
    return dict(ratio=float(np.exp(lr.mean())), ci95=[lo, hi], cls=cls)


def _launches_for(seconds_per_launch, target=0.5e-3):
    return int(min(400, max(2, math.ceil(target / max(seconds_per_launch, 1e-6)))))


class LibCandidate:
    """One library descriptor (AUTO or a forced algorithm) on fixed buffers."""

    def __init__(self, gc, torch, wl, x, w, algo):
        self.gc, self.torch = gc, torch
        self.d = gc.conv_desc_create(wl.N, wl.C, wl.H, wl.W, wl.K, wl.R, wl.S, wl.stride, wl.pad, wl.dil, wl.groups)
        gc.conv_desc_set_algo(self.d, algo)
        self.algo = gc.ALGO_NAMES[gc.conv_desc_get_algo(self.d)]
        ho, wo = gc.conv_desc_get_output_dims(self.d)
        self.x, self.w = x, w
        self.y = torch.full((wl.N, wl.K, ho, wo), float("nan"), device="cuda")
        self.px, self.pw, self.py = x.data_ptr(), w.data_ptr(), self.y.data_ptr()
        self.side = torch.cuda.Stream()
        self.sh = torch.cuda.current_stream().cuda_stream

    def launch(self):
        self.gc.conv_fwd(self.d, self.px, self.pw, None, self.py, stream=self.sh)

    def output(self):
        return self.y

    def graph(self, R, n):
        self.side.wait_stream(self.torch.cuda.current_stream())
        ms = self.gc.gconv_time_graph(self.d, [self.x], [self.y], self.w, None, launches=R, replays=n,
                                      stream=self.side)
        self.torch.cuda.current_stream().wait_stream(self.side)
        return [m / 1e3 for m in ms]


class TorchCandidate:
    """PyTorch's conv2d on ROCm (MIOpen): another system, timed as context."""

    algo = "torch"

    def __init__(self, torch, wl, x, w):
        import torch.nn.functional as F
        self.torch, self.groups = torch, wl.groups
        self.fn = lambda: F.conv2d(x, w, None, wl.stride, wl.pad, wl.dil, wl.groups)
        self.g, self.gR, self.graph_error = None, 0, None

    def launch(self):
        self.fn()

    def output(self):
        return self.fn()

    def graph(self, R, n):
        torch = self.torch
        if self.graph_error is not None:
            return None
        if self.g is None or self.gR != R:
            try:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for _ in range(R):
                        self.fn()
                self.g, self.gR = g, R
            except RuntimeError as e:  # capture not supported for this call
                self.graph_error = str(e).splitlines()[0]
                torch.cuda.synchronize()
                return None
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in ev:
            a.record()
            self.g.replay()
            b.record()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) / 1e3 / R for a, b in ev]


def _event_time(torch, launch, reps=10):
    for _ in range(3):
        launch()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        launch()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / 1e3 / reps


def _sync_samples(torch, launch, n):
    out = []
    for _ in range(n):
        t0 = time.perf_counter()
        launch()
        torch.cuda.synchronize()
        out.append(time.perf_counter() - t0)
    return out


def sweep_shape(wl, gc, torch, args):
    import synth
    inp = synth.make_inputs(wl)
    x = torch.from_numpy(inp["x"]).cuda()
    w = torch.from_numpy(inp["w"]).cuda()
    cands = {"auto": LibCandidate(gc, torch, wl, x, w, gc.ALGO_AUTO),
             "direct": LibCandidate(gc, torch, wl, x, w, gc.ALGO_DIRECT)}
    if not args.sweep_no_torch:
        cands["torch"] = TorchCandidate(torch, wl, x, w)
    ho, wo = gc.conv_desc_get_output_dims(cands["auto"].d)
    acct = row_accounting(wl, ho, wo)
    rec = dict(name=wl.name, N=wl.N, C=wl.C, H=wl.H, W=wl.W, K=wl.K, groups=wl.groups, cpg=wl.C // wl.groups,
               algo=cands["auto"].algo, bytes=acct["bytes"], flops=acct["flops"], floor_us=acct["floor_s"] * 1e6)

    # verify before timing: every candidate's full output against PyTorch's
    # FP32 conv2d, with the bar 1e-4 * sum|x*w| + 1e-6 (sum|x*w| from the same
    # conv of |x| and |w|); the oracle check of the grid is a GPU test
    import torch.nn.functional as F
    ref = F.conv2d(x, w, None, wl.stride, wl.pad, wl.dil, wl.groups)
    A = F.conv2d(x.abs(), w.abs(), None, wl.stride, wl.pad, wl.dil, wl.groups)
    bound = 1e-4 * A + 1e-6
    rec["check"] = {}
    for k, c in cands.items():
        c.launch()
        torch.cuda.synchronize()
        y = c.output()
        ok = k == "torch" or bool(((y - ref).abs() <= bound).all().item())
        rec["check"][k] = ("pass" if ok else "FAIL") if k != "torch" else "reference"
    del ref, A

    # per-candidate launch count for graph replays of ~0.5 ms
    est = {k: _event_time(torch, c.launch) for k, c in cands.items()}
    Rs = {k: _launches_for(t) for k, t in est.items()}
    boundaries = {"graph": {k: [] for k in cands}, "sync": {k: [] for k in cands}}
    keys = list(cands)
    for b in range(args.batches):
        order = keys[b % len(keys):] + keys[:b % len(keys)]
        for k in order:
            g = cands[k].graph(Rs[k], args.samples)
            if g is not None:
                boundaries["graph"][k].append(g)
        for k in order:
            boundaries["sync"][k].append(_sync_samples(torch, cands[k].launch, args.samples))
    rec["launches_per_replay"] = Rs
    for bname, per in boundaries.items():
        out = {}
        for k, batches in per.items():
            if len(batches) != args.batches:
                out[k] = None
                continue
            flat = [v for bt in batches for v in bt]
            m, lo, hi = boot_ci(flat, n_boot=2000)
            out[k] = dict(us=m * 1e6, ci95_us=[lo * 1e6, hi * 1e6])
            if k == "auto":
                out[k].update(gbs=acct["bytes"] / m / 1e9, gflops=acct["flops"] / m / 1e9,
                              roofline_frac=acct["floor_s"] / m)
        for base in keys:
            if base == "auto" or out.get(base) is None or out.get("auto") is None:
                continue
            out[base + "_over_auto"] = paired_ratio(per[base], per["auto"])
        rec[bname] = out
    if "torch" in cands and cands["torch"].graph_error:
        rec["torch_graph_error"] = cands["torch"].graph_error
    del cands, x, w
    return rec


def sweep(args):
    import torch
    import synth
    import grouped_convolution_conv_amd as gc

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    # "tuned PyTorch": MIOpen searches for its fastest solution per shape on
    # the first call (outside every timed region); FP32 arithmetic only
    torch.backends.cudnn.benchmark = True
    torch.backends.cudnn.allow_tf32 = False
    # the 80-shape grid by default; any grid shape or general-geometry layer
    # by name
    known = dict(synth.ATLAS_GRID, **synth.EXTRA_WORKLOADS, **synth.IGEMM_WORKLOADS)
    names = args.sweep_shapes.split(",") if args.sweep_shapes else list(synth.ATLAS_GRID)
    unknown = [n for n in names if n not in known]
    if unknown:
        print("bench.py: unknown sweep shapes %s" % unknown, file=sys.stderr)
        sys.exit(2)
    log("[sweep] device:", torch.cuda.get_device_name(0), " shapes:", len(names))
    t0 = time.perf_counter()
    records = []
    for i, n in enumerate(names):
        rec = sweep_shape(known[n], gc, torch, args)
        records.append(rec)
        g = rec["graph"]
        parts = ["%-26s %-10s auto %8.2f us" % (n, rec["algo"], g["auto"]["us"])]
        for base in ("direct", "torch"):
            r = g.get(base + "_over_auto")
            if r:
                parts.append("%s/auto %6.2fx %-4s" % (base, r["ratio"], r["cls"]))
        s = rec["sync"]
        parts.append("| sync auto %7.2f us" % s["auto"]["us"])
        if s.get("torch_over_auto"):
            parts.append("torch/auto %5.2fx %s" % (s["torch_over_auto"]["ratio"], s["torch_over_auto"]["cls"]))
        parts.append("check %s" % ",".join("%s:%s" % kv for kv in rec["check"].items()))
        log("[sweep %2d/%d] " % (i + 1, len(names)) + "  ".join(parts))
        torch.cuda.empty_cache()
    summary = {}
    for bname in ("graph", "sync"):
        summary[bname] = {}
        for base in ("direct", "torch"):
            rs = [r[bname].get(base + "_over_auto") for r in records]
            rs = [r for r in rs if r]
            if not rs:
                continue
            summary[bname][base + "_over_auto"] = dict(
                geomean=geomean([r["ratio"] for r in rs]), shapes=len(rs),
                win=sum(r["cls"] == "win" for r in rs), tie=sum(r["cls"] == "tie" for r in rs),
                loss=sum(r["cls"] == "loss" for r in rs))
        summary[bname]["auto_gbs_geomean"] = geomean([r[bname]["auto"]["gbs"] for r in records])
        summary[bname]["auto_roofline_frac_geomean"] = geomean([r[bname]["auto"]["roofline_frac"] for r in records])
    by_cpg = {}
    for r in records:
        by_cpg.setdefault(r["cpg"], []).append(r)
    summary["graph_by_cpg"] = {
        str(c): dict(shapes=len(rs), algo=sorted(set(r["algo"] for r in rs)),
                     direct_over_auto=geomean([r["graph"]["direct_over_auto"]["ratio"] for r in rs]),
                     torch_over_auto=geomean([r["graph"]["torch_over_auto"]["ratio"] for r in rs
                                              if r["graph"].get("torch_over_auto")]),
                     auto_roofline_frac=geomean([r["graph"]["auto"]["roofline_frac"] for r in rs]))
        for c, rs in sorted(by_cpg.items())}
    out = dict(metric=("grouped 3x3 shape sweep" if all(n in synth.ATLAS_GRID for n in names) else "shape sweep") +
               ": baseline latency / dispatcher latency (above 1 favours the library), "
                      "geomean over shapes, paired batches with 95% bootstrap intervals and a 5% practical threshold",
               shapes=len(records), batches=args.batches, samples=args.samples,
               checks_failed=[r["name"] for r in records if "FAIL" in r["check"].values()],
               summary=summary, torch_settings=dict(cudnn_benchmark=True, allow_tf32=False),
               seconds=time.perf_counter() - t0)
    if args.sweep_out:
        with open(args.sweep_out, "w") as f:
            json.dump(dict(out, records=records), f, indent=1)
    print(json.dumps(out), flush=True)


# ------------------------------------------------------------------ block substitution probe


def _inverted_residual(torch, seed):
    """The MobileNetV2 inverted-residual block at features[3]'s shape (24
    channels in and out, expansion 6, stride 1, 56x56): 1x1 conv 24->144, BN,
    ReLU6, 3x3 depthwise conv 144 (pad 1), BN, ReLU6, 1x1 conv 144->24, BN,
    plus the input.  Random weights and BN statistics, inference mode."""
    nn = torch.nn
    g = torch.Generator().manual_seed(seed)

    def bn(c):
        m = nn.BatchNorm2d(c)
        with torch.no_grad():
            m.weight.copy_(0.5 + torch.rand(c, generator=g))
            m.bias.copy_(0.1 * torch.randn(c, generator=g))
            m.running_mean.copy_(0.1 * torch.randn(c, generator=g))
            m.running_var.copy_(0.5 + torch.rand(c, generator=g))
        return m

    def conv(cin, cout, k, groups=1):
        m = nn.Conv2d(cin, cout, k, 1, k // 2, groups=groups, bias=False)
        bound = 1.0 / math.sqrt(cin // groups * k * k)
        with torch.no_grad():
            m.weight.copy_((2 * torch.rand(m.weight.shape, generator=g) - 1) * bound)
        return m

    expand = nn.Sequential(conv(24, 144, 1), bn(144), nn.ReLU6())
    dw = conv(144, 144, 3, groups=144)
    rest = nn.Sequential(bn(144), nn.ReLU6(), conv(144, 24, 1), bn(24))
    return [m.cuda().eval() for m in (expand, dw, rest)]


def block_probe(args):
    import torch
    import grouped_convolution_conv_amd as gc

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    torch.backends.cudnn.benchmark = True
    torch.backends.cudnn.allow_tf32 = False
    expand, dw, rest = _inverted_residual(torch, 1234)
    w_dw = dw.weight.detach().contiguous()
    out = dict(metric="block substitution: original block latency / block with the library's depthwise conv "
                      "(above 1 favours the library), paired batches, 95% bootstrap intervals, 5% practical threshold",
               block="inverted residual 24->144->24, 3x3 depthwise 144, 56x56, BN + ReLU6, residual; random weights",
               batches=args.batches, samples=args.samples, results=[])
    for n in [int(v) for v in args.block_batch.split(",")]:
        x = torch.randn(n, 24, 56, 56, device="cuda")
        d = gc.conv_desc_create(n, 144, 56, 56, 144, 3, 3, 1, 1, 1, 144)
        y_buf = torch.empty(n, 144, 56, 56, device="cuda")

        def original():
            return x + rest(dw(expand(x)))

        def substituted():
            # the expansion's output is a fresh contiguous tensor: the
            # library reads it in place, on torch's current stream
            gc.conv_fwd(d, expand(x), w_dw, None, y_buf)
            return x + rest(y_buf)

        with torch.no_grad():
            # verify: the depthwise conv at the block's own activations, and the block output
            h = expand(x).contiguous()
            ref = dw(h)
            gc.conv_fwd(d, h, w_dw, None, y_buf)
            A = torch.nn.functional.conv2d(h.abs(), w_dw.abs(), None, 1, 1, 1, 144)
            conv_ok = bool(((y_buf - ref).abs() <= 1e-4 * A + 1e-6).all().item())
            a, b = original(), substituted()
            torch.cuda.synchronize()
            block_err = float((a - b).abs().max().item())
            cands = {"original": original, "substituted": substituted}
            graphs, graph_error = {}, None
            for k, f in cands.items():
                for _ in range(3):
                    f()
                torch.cuda.synchronize()
                try:
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g):
                        f()
                    graphs[k] = g
                except RuntimeError as e:  # a call in the block that capture does not support
                    graph_error = str(e).splitlines()[0]
                    torch.cuda.synchronize()
                    break
            torch.cuda.synchronize()
            per = {b: {k: [] for k in cands} for b in (("sync",) if graph_error else ("graph", "sync"))}
            keys = list(cands)
            for bt in range(args.batches):
                order = keys[bt % 2:] + keys[:bt % 2]
                for k in (order if not graph_error else []):
                    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                          for _ in range(args.samples)]
                    for e0, e1 in ev:
                        e0.record()
                        graphs[k].replay()
                        e1.record()
                    torch.cuda.synchronize()
                    per["graph"][k].append([e0.elapsed_time(e1) / 1e3 for e0, e1 in ev])
                for k in order:
                    per["sync"][k].append(_sync_samples(torch, cands[k], args.samples))
        rec = dict(N=n, conv_check="pass" if conv_ok else "FAIL", block_max_abs_diff=block_err)
        if graph_error:
            rec["graph_error"] = graph_error
        for bname, pk in per.items():
            r = paired_ratio(pk["original"], pk["substituted"])
            r.update({k + "_us": float(np.median([v for bt in pk[k] for v in bt])) * 1e6 for k in keys})
            rec[bname] = r
            log("[block] N=%d %-5s original %.2f us  substituted %.2f us  ratio %.3fx [%.3f, %.3f] %s"
                % (n, bname, r["original_us"], r["substituted_us"], r["ratio"], r["ci95"][0], r["ci95"][1], r["cls"]))
        out["results"].append(rec)
        log("[block] N=%d  conv %s  block max|diff| %.2e%s" % (n, rec["conv_check"], block_err,
                                                             ("  graph: " + graph_error) if graph_error else ""))
        del graphs
        torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


# ------------------------------------------------------------------ main


def workload_text(names, known):
    if names == [n for n in known if n in names] and all(n in ROW_TEXT for n in names):
        return "one pass over the shape rows " + ", ".join(names) + " (" + "; ".join(ROW_TEXT[n] for n in names) + ")"
    return "one pass over the shape rows " + "; ".join(
        "%s: N%d C%d->%d %dx%d %dx%d stride %d pad %s dil %d groups %d" % (
            n, known[n].N, known[n].C, known[n].K, known[n].H, known[n].W, known[n].R, known[n].S,
            known[n].stride, known[n].pad, known[n].dil, known[n].groups) for n in names)


ROW_TEXT = {
    "c1_grouped_cpg4": "grouped 3x3 cpg4 N1 C8 16x16",
    "c2_depthwise_144": "depthwise N4 C144 56x56",
    "c3a_grouped_g64": "grouped N32 C256 64x64 g64",
    "c3b_grouped_g128": "grouped N32 C256 64x64 g128",
    "c3c_depthwise_g256": "grouped N32 C256 64x64 g256",
    "c4_dense_5x9": "dense N8 C32->64 256x256 5x9",
    "c5_fused_gn": "fused N64 C8->32 256x256 3x3 + bias, scale, sigmoid, GN(8)",
}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this library runs on one GPU; runs on more than one GPU are not supported "
              "(got --gpus %d, WORLD_SIZE=%d)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    if args.sweep:
        sweep(args)
        return
    if args.block:
        block_probe(args)
        return

    import torch
    import synth
    import grouped_convolution_conv_amd as gc

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    copy = copy_calibration(torch, gc)
    log("[bench] library copy of %d MiB: %.1f GB/s (read + write)" % (COPY_BYTES >> 20, copy["gbs"]))
    sink = torch.zeros(4, device="cuda")
    mfma_meas, _ = gc.gconv_probe_peaks(sink)
    fma_meas, fp64_meas = gc.gconv_probe_vector_peaks(sink)
    peaks = dict(fp32_mfma_tflops=mfma_meas, fp32_fma_tflops=fma_meas, fp64_fma_tflops=fp64_meas,
                 hbm_copy_gbs=copy["gbs"])
    log("[bench] measured peaks: FP32 MFMA %.1f TFLOP/s, FP32 FMA %.1f TFLOP/s, FP64 FMA %.1f TFLOP/s"
        % (mfma_meas, fma_meas, fp64_meas))
    if args.copy_only:
        print(json.dumps({"copy_calibration": copy}), flush=True)
        return
    known = dict(synth.WORKLOADS, **synth.EXTRA_WORKLOADS)
    if args.rows:
        names = args.rows.split(",")
        unknown = [n for n in names if n not in known]
        if unknown:
            print("bench.py: unknown rows %s (known: %s)" % (unknown, ", ".join(known)), file=sys.stderr)
            sys.exit(2)
    else:
        names = list(synth.ROW_ORDER)
    log("[bench] device:", torch.cuda.get_device_name(0))
    rows = []
    for n in names:
        rows.append(Row(n, known[n], gc, torch, args.warm))
        log("[bench] row %-20s algo=%-10s sets=%d bytes=%d flops=%d" % (n, rows[-1].algo, rows[-1].nsets,
                                                                      rows[-1].acct["bytes"], rows[-1].acct["flops"]))
    torch.cuda.synchronize()
    step_stream = torch.cuda.current_stream()
    for r in rows:
        r.prepare(step_stream)

    # ---- warmup
    for i in range(args.warmup):
        for r in rows:
            r.launch(i)
    torch.cuda.synchronize()

    # ---- timed steps
    K = args.steps
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in rows]
          for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        for j, r in enumerate(rows):
            ev[i][j][0].record()
            r.launch(i)
            ev[i][j][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / K * 1e3
    step_times = {r.name: [ev[i][j][0].elapsed_time(ev[i][j][1]) / 1e3 for i in range(K)]
                  for j, r in enumerate(rows)}
    log("[bench] %d steps in %.3f s (%.3f ms/step)" % (K, wall, ms_per_step))

    out_rows = []
    for r in rows:
        med = float(np.median(step_times[r.name]))
        rec = dict(name=r.name, algo=r.algo, bound=r.acct["bound"], bytes=r.acct["bytes"], flops=r.acct["flops"],
                   floor_us=r.acct["floor_s"] * 1e6, buffer_sets=r.nsets)
        rec["step"] = r.figures(med)
        rec["step"]["mean_ms"] = float(np.mean(step_times[r.name])) * 1e3
        rec["floor_us_measured_peaks"] = measured_floor_s(r.acct, r.wl, peaks) * 1e6
        tb = measured_traffic(r.name)
        rec["traffic"] = None if tb is None else dict(bytes_per_launch=tb, ratio_to_algorithmic=tb / r.acct["bytes"])
        out_rows.append(rec)
        log("[bench] %-20s step  %.4f ms  %8.1f GB/s  %8.1f GFLOP/s  frac %.3f"
            % (r.name, rec["step"]["ms"], rec["step"]["gbs"], rec["step"]["gflops"], rec["step"]["roofline_frac"]))

    if not args.no_boundaries:
        for r, rec in zip(rows, out_rows):
            gs, R = graph_boundary(r, torch, args.batches, args.samples)
            ss = sync_boundary(r, torch, args.batches, args.samples)
            for key, smp in (("graph", gs), ("sync", ss)):
                m, lo, hi = boot_ci(smp)
                fig = r.figures(m)
                fig.update(ci95_ms=[lo * 1e3, hi * 1e3], samples=len(smp))
                if key == "graph":
                    fig["launches_per_replay"] = R
                rec[key] = fig
            log("[bench] %-20s graph %.4f ms [%.4f, %.4f]  sync %.4f ms [%.4f, %.4f]"
                % (r.name, rec["graph"]["ms"], *rec["graph"]["ci95_ms"], rec["sync"]["ms"], *rec["sync"]["ci95_ms"]))

    for rec in out_rows:
        for key in ("step", "graph", "sync"):
            if key in rec:
                rec[key]["roofline_frac_measured_peaks"] = rec["floor_us_measured_peaks"] / (rec[key]["ms"] * 1e3)
        if "sync" in rec and "graph" in rec:
            # host time of the synchronized call beyond the device time of a
            # graph replay: Python and ctypes marshalling, the HIP launch and
            # the synchronization round trip
            rec["sync_minus_graph_us"] = (rec["sync"]["ms"] - rec["graph"]["ms"]) * 1e3

    # ---- dominant kernel roofline (single-kernel rows: one launch = one kernel)
    single = [(rec, r) for rec, r in zip(out_rows, rows) if not r.wl.fused]
    dom_rec, dom_row = max(single, key=lambda t: t[0]["step"]["mean_ms"]) if single else (None, None)
    roof = None
    if dom_rec is not None:
        t = dom_rec["step"]["mean_ms"] / 1e3
        if dom_rec["bound"] == "mfma":
            achieved = dom_rec["flops"] / t / 1e12
            roof = dict(bound="mfma", achieved=achieved, peak=FP32_MFMA_PEAK_TFLOPS, unit="TFLOP/s",
                        frac=achieved / FP32_MFMA_PEAK_TFLOPS, measured_peak=peaks["fp32_mfma_tflops"],
                        frac_of_measured_peak=achieved / peaks["fp32_mfma_tflops"])
        else:
            achieved = dom_rec["bytes"] / t / 1e9
            roof = dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s", frac=achieved / HBM_PEAK_GBS,
                        measured_peak=peaks["hbm_copy_gbs"], frac_of_measured_peak=achieved / peaks["hbm_copy_gbs"])
        roof.update(traffic=measured_traffic(dom_rec["name"]), traffic_unit="bytes per launch",
                    algorithmic_bytes=dom_rec["bytes"], algorithmic_flops=dom_rec["flops"],
                    kernel=dom_row.algo, row=dom_rec["name"],
                    avg_launch_ms=dom_rec["step"]["mean_ms"])

    # the synchronization round trip alone, on an idle device
    torch.cuda.synchronize()
    idle = []
    for _ in range(200):
        t0 = time.perf_counter()
        torch.cuda.synchronize()
        idle.append(time.perf_counter() - t0)
    host_sync_us = float(np.median(idle)) * 1e6

    value = geomean([rec["step"]["gbs"] for rec in out_rows])
    result = {
        "metric": METRIC,
        "value": value,
        "unit": "GB/s (geomean over shape rows, device time per launch)",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": workload_text(names, known), "cold_buffer_sets": not args.warm},
        "geomean": {
            "step_gbs": value,
            "step_gflops": geomean([r["step"]["gflops"] for r in out_rows]),
            "step_roofline_frac": geomean([r["step"]["roofline_frac"] for r in out_rows]),
        },
        "roofline": roof,
        "hbm_copy_calibration": copy,
        "host_sync_idle_us": host_sync_us,
        "measured_peaks": peaks,
        "rows": out_rows,
    }
    if not args.no_boundaries:
        for key in ("graph", "sync"):
            result["geomean"][key + "_gbs"] = geomean([r[key]["gbs"] for r in out_rows])
            result["geomean"][key + "_roofline_frac"] = geomean([r[key]["roofline_frac"] for r in out_rows])
        bw = [r for r in out_rows if r["bound"] in ("hbm", "alu")]
        if bw:
            result["geomean"]["graph_roofline_frac_bandwidth_rows"] = geomean([r["graph"]["roofline_frac"] for r in bw])
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(rows)
        for rec in out_rows:
            c = result["cpu_baseline"]["rows"][rec["name"]]
            c["gpu_step_speedup"] = rec["step"]["gbs"] / c["gbs"]
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
