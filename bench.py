"""Benchmark of the weight-only quantized linear layer on one MI355X.

A step is one decode step's worth of the hot path: the three W4A16 (INT4, g128)
GEMVs of a single-stream decode at M=1, K=5120, N in {5120, 6144, 1024}, on
inputs resident in HBM. Weights rotate through a pool of distinct copies larger
than 1 GiB so every launch streams them from HBM, not from the 256 MB Infinity
Cache. `value` is the step's algorithmic bytes (packed weights + scales + x + y,
each once) per second.

Timing protocol: every figure is the median of 5 trials; a trial replays a HIP
graph of launches that rotate over the weight copies (at least 200 launches, or
exactly `--steps` decode steps for the headline) after untimed warm-up, timed
with HIP events on the replay stream. Parity against the oracle is checked on
the first and last weight copies of every workload before and after timing.

Also reported (stderr table and the JSON line's "workloads" list): per-kernel
time, GB/s, TFLOP/s and roofline fraction for every named workload (decode,
M=3/5 verify chunks, M=128 batched verify, MXFP8 at M=1/5/128, the vocabulary
heads, G=32/64 variants), each beside a read-only stream probe of the same bytes
in the kernel's own launch shape and in the best of a fixed sweep of shapes
("probe"), a stream probe of >1 GiB ("chip_stream"), the run record (versions,
device, host CPU, input SHA-256 digests), the CPU oracle on every workload
(``cpu_oracle``, bounded column samples scaled to the full width) and on whole
decode steps (``cpu_baseline``), the fused K/V/Q and gate/up projections against
the same projections launched one by one (``fusion``), and the setup-time steps
(``quantizer``, ``ct_ingest``, ``mxfp8_quantizer``).

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--quick] [--no-cpu]
    python bench.py --only decode_n6144,mxfp8_m128   # a few workloads, for profiling runs
    python bench.py --copy-probe    # a plain 1 GiB device copy, to calibrate HBM counters
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, vendor figure
POOL_BYTES = 1.2 * (1 << 30)
TRIALS = 5                      # every figure is the median of this many trials
MIN_LAUNCHES = 200              # launches per trial (or one per weight copy, if more)
METRIC = "W4A16 GEMM µs, weight-stream GB/s and % HBM peak at M=1/5/128; TFLOP/s"
DECODE = ["decode_n5120", "decode_n6144", "decode_n1024"]
DOMINANT = "decode_n6144"
TABLE = ["decode_n5120", "decode_n6144", "decode_n1024", "verify3_up", "verify3_down", "verify5_up",
         "verify5_down", "batch128_up", "batch128_down", "mxfp8_m1", "mxfp8_m5", "mxfp8_m128",
         "vocab_w8_m1", "vocab_w4_m1", "decode_n6144_g32", "decode_n6144_g64", "verify5_up_g32",
         "verify5_up_g64", "batch128_up_g32", "batch128_up_g64"]
OPS = {"w4a16": 1, "mxfp8": 2, "w8a16": 3}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def group(w):
    return 32 if w["op"] == "mxfp8" else w.get("G", 128)


def weight_bytes(w):
    K, N, G = w["K"], w["N"], group(w)
    if w["op"] == "w4a16":
        return K * N // 2 + (K // G) * N * 2
    if w["op"] == "w8a16":
        return K * N + (K // G) * N * 2
    return K * N + (K // 32) * N


def algo_bytes(w):
    return weight_bytes(w) + 2 * w["M"] * w["K"] + 2 * w["M"] * w["N"]


def flops(w):
    return 2.0 * w["M"] * w["N"] * w["K"]


def med(v):
    return statistics.median(v)


def _dev(torch, a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda:0")


class Problem:
    """Device-resident inputs of one workload with a rotation pool of weight copies."""

    def __init__(self, torch, svq, name, pool_bytes):
        self.name = name
        self.w = synth.WORKLOADS[name]
        self.torch, self.svq = torch, svq
        inp = synth.gen_workload(name)
        self.inp = inp
        self.digest = inp.digest()
        M, K, N, G = self.w["M"], self.w["K"], self.w["N"], group(self.w)
        self.G = G
        self.x = _dev(torch, inp.x)
        self.out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
        ncopy = max(2, int(pool_bytes // max(weight_bytes(self.w), 1)))
        op = self.w["op"]
        if op == "w4a16":
            base_w = svq.q4_repack(_dev(torch, inp.qweight))
            base_s = _dev(torch, inp.scales)
        elif op == "w8a16":
            base_w = torch.from_numpy(np.ascontiguousarray(inp.w)).to("cuda:0")
            base_s = _dev(torch, inp.scales)
        else:
            base_w = svq.mxfp8_repack(_dev(torch, inp.w))
            base_s = _dev(torch, inp.scales)
        self.kernel = svq.kernel_name(OPS[op], M, N, K, G)
        self.geometry = svq.launch_geometry(OPS[op], M, N, K, G)
        nb = svq.workspace_bytes(OPS[op], M, N, K, G)
        self.ws = torch.zeros(max(nb, 256), dtype=torch.uint8, device="cuda:0") if nb else None
        self.ws_w = [base_w] + [base_w.clone() for _ in range(ncopy - 1)]
        self.ws_s = [base_s] + [base_s.clone() for _ in range(ncopy - 1)]
        self.i = 0

    def launch(self, i=None):
        i = self.i if i is None else i
        self.i = (self.i + 1) % len(self.ws_w)
        w = self.w
        if w["op"] == "w4a16":
            self.svq.w4a16_gemm(self.x, self.ws_w[i], self.ws_s[i], w["N"], self.G, out=self.out,
                                workspace=self.ws)
        elif w["op"] == "w8a16":
            self.svq.w8a16_gemm(self.x, self.ws_w[i], self.ws_s[i], self.G, out=self.out, workspace=self.ws)
        else:
            self.svq.mxfp8_gemm(self.x, self.ws_w[i], self.ws_s[i], out=self.out, workspace=self.ws)

    def check(self, oracle):
        """Parity of the first and last pool copies against the oracle (sampled)."""
        torch = self.torch
        inp, w = self.inp, self.w
        rng = np.random.default_rng(1)
        rows = rng.integers(0, w["M"], 256)
        cols = rng.integers(0, w["N"], 256)
        for i in (0, len(self.ws_w) - 1):
            self.launch(i)
            torch.cuda.synchronize()
            bits = self.out.view(torch.int16).cpu().numpy().view(np.uint16)[rows, cols]
            if w["op"] == "w4a16":
                y64, _ = oracle.w4a16_points(inp.x, inp.qweight, inp.scales, self.G, rows, cols)
            elif w["op"] == "w8a16":
                y64, _ = oracle.w8a16_points(inp.x, inp.w, inp.scales, self.G, rows, cols)
            else:
                y64, _ = oracle.mxfp8_points(inp.x, inp.w, inp.scales, rows, cols)
            ok, err, rms = oracle.gate(bits, y64)
            if not ok:
                raise SystemExit(f"parity failure in {self.name} copy {i}: err {err} rms {rms}")

    def release(self):
        self.ws_w = self.ws_s = None


def graph_of(torch, fn, n):
    """Capture n calls fn(i) into one HIP graph (no host launch overhead on replay)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(3):          # warm the allocator/caches outside the capture
            fn(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    torch.cuda.synchronize()
    return g


def time_graph(torch, g, reps):
    """Mean seconds per replay of g over reps replays (events on the replay stream)."""
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e-3 / reps


def time_trials(torch, fn, n, trials=TRIALS):
    """µs per call of fn(i), i = 0..n-1 captured in one graph: one value per trial
    (each trial one replay of the n calls, after one untimed replay)."""
    g = graph_of(torch, fn, n)
    out = [time_graph(torch, g, 1) / n * 1e6 for _ in range(trials)]
    del g
    return out


def time_kernel(torch, prob, launches=None):
    """µs per launch of one kernel, one value per trial: graphs of at least
    MIN_LAUNCHES launches (one per weight copy if there are more) rotating over
    the weight pool."""
    n = launches or max(MIN_LAUNCHES, len(prob.ws_w))
    return time_trials(torch, lambda i: prob.launch(i % len(prob.ws_w)), n)


def summary(trials):
    return {"median": round(med(trials), 3), "min": round(min(trials), 3), "max": round(max(trials), 3),
            "trials": [round(t, 3) for t in trials]}


# ---- streaming probe --------------------------------------------------------------------

class ProbePool:
    """Copies of `nbytes` (rounded up to 16) in one device buffer totalling more than
    1 GiB, read in turn by the stream probe, so that each launch reads from HBM."""

    def __init__(self, torch, nbytes, pool_bytes=POOL_BYTES):
        self.torch = torch
        self.nbytes = (nbytes + 15) // 16 * 16
        self.n = max(2, int(pool_bytes // self.nbytes))
        self.buf = torch.randint(-2 ** 31, 2 ** 31 - 1, (self.n * self.nbytes // 4,), dtype=torch.int32,
                                 device="cuda:0")
        self.sink = torch.zeros(1 << 20, dtype=torch.int32, device="cuda:0")

    def time(self, svq, grid, threads):
        view = lambda i: self.buf[(i % self.n) * self.nbytes // 4:]
        fn = lambda i: svq.stream_probe(view(i), self.nbytes, grid, threads, self.sink)
        return time_trials(self.torch, fn, max(MIN_LAUNCHES, self.n))

    def release(self):
        self.buf = self.sink = None


def probe_shapes(cus, nbytes):
    """A fixed sweep of launch shapes for the best-of probe: one to eight workgroups
    per CU of 256..1024 threads, and many small workgroups of ~5 KiB each."""
    shapes = [(cus, 1024), (2 * cus, 512), (4 * cus, 256), (8 * cus, 256), (2 * cus, 1024)]
    small = max(cus, min(1 << 20, nbytes // 5120))
    shapes.append((small, 256))
    return shapes


def probe_workload(torch, svq, prob, cus):
    """Stream-probe µs for the workload's algorithmic bytes: in the GEMM's own launch
    shape, and the best of the fixed sweep."""
    pool = ProbePool(torch, algo_bytes(prob.w))
    grid, threads, _ = prob.geometry
    same = pool.time(svq, grid, threads)
    best, best_shape = None, None
    for g, t in probe_shapes(cus, pool.nbytes):
        v = med(pool.time(svq, g, t))
        if best is None or v < best:
            best, best_shape = v, (g, t)
    pool.release()
    return {"same_shape": [grid, threads], "same_us": round(med(same), 3), "best_us": round(best, 3),
            "best_shape": list(best_shape)}


def chip_stream(torch, svq, cus):
    """The chip's streaming ceiling: the probe over 1 GiB in the sweep's shapes."""
    nbytes = 1 << 30
    buf = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int32, device="cuda:0")
    sink = torch.zeros(1 << 20, dtype=torch.int32, device="cuda:0")
    res = []
    for g, t in probe_shapes(cus, nbytes) + [(16 * cus, 256), (4 * cus, 1024)]:
        us = med(time_trials(torch, lambda i: svq.stream_probe(buf, nbytes, g, t, sink), 20))
        res.append({"shape": [g, t], "us": round(us, 1), "GBps": round(nbytes / (us * 1e-6) / 1e9, 1)})
    best = max(res, key=lambda r: r["GBps"])
    del buf, sink
    return {"bytes": nbytes, "best_GBps": best["GBps"], "best_shape": best["shape"],
            "hbm_frac": round(best["GBps"] / HBM_PEAK_GBS, 4), "shapes": res}


# ---- matrix-core probe ------------------------------------------------------------------

def mfma_floor(torch, svq, w, geometry):
    """MFMA-issue floor of a batched workload: the matrix-core probe in the GEMM's own
    launch shape, with the workload's MFMA count (rows padded to the 16 of one MFMA)
    spread evenly over its waves."""
    grid, threads, _ = geometry
    total = -(-w["M"] // 16) * (w["N"] // 16) * (w["K"] // 32)
    waves = grid * (threads // 64)
    per_wave = -(-total // waves)
    per_wave = -(-per_wave // 8) * 8
    sink = torch.zeros(max(grid, 1), dtype=torch.float32, device="cuda:0")
    us = med(time_trials(torch, lambda i: svq.mfma_probe(grid, threads, per_wave, sink), MIN_LAUNCHES))
    # random activation-like A and 128 + q B operands: the chip clocks lower under real data
    us_r = med(time_trials(torch, lambda i: svq.mfma_probe(grid, threads, per_wave, sink, random_operands=True),
                           MIN_LAUNCHES))
    flop = per_wave * waves * 16 * 16 * 32 * 2
    return {"shape": [grid, threads], "mfma_per_wave": per_wave, "us": round(us, 3),
            "TFLOPs": round(flop / (us * 1e-6) / 1e12, 1), "us_random": round(us_r, 3),
            "TFLOPs_random": round(flop / (us_r * 1e-6) / 1e12, 1)}


def chip_mfma(torch, svq, cus):
    """The chip's sustained bf16 MFMA rate: the probe with two 8-wave workgroups per CU."""
    grid, threads, per_wave = 2 * cus, 512, 4096
    sink = torch.zeros(grid, dtype=torch.float32, device="cuda:0")
    flop = grid * 8 * per_wave * 16 * 16 * 32 * 2
    out = {"shape": [grid, threads], "mfma_per_wave": per_wave}
    for key, rnd in (("", False), ("_random", True)):
        us = med(time_trials(torch, lambda i: svq.mfma_probe(grid, threads, per_wave, sink, random_operands=rnd), 50))
        tfl = flop / (us * 1e-6) / 1e12
        # every CU busy: 4096 bf16 flop per clock per CU at the clock the chip held
        out.update({"us" + key: round(us, 2), "TFLOPs" + key: round(tfl, 1),
                    "mfma_frac" + key: round(tfl / MFMA_BF16_PEAK_TFLOPS, 4),
                    "clock_MHz" + key: round(tfl * 1e12 / (cus * 4096) / 1e6)})
    return out


# ---- run record -----------------------------------------------------------------------------

def _read(path):
    try:
        with open(path) as f:
            return f.read().strip()
    except OSError:
        return None


def host_cpu():
    model = None
    txt = _read("/proc/cpuinfo") or ""
    for line in txt.splitlines():
        if line.startswith("model name"):
            model = line.split(":", 1)[1].strip()
            break
    smt = _read("/sys/devices/system/cpu/smt/active")
    threads = len(os.sched_getaffinity(0))
    # SMT siblings among the usable CPUs: count distinct physical cores
    cores = set()
    for c in os.sched_getaffinity(0):
        sib = _read(f"/sys/devices/system/cpu/cpu{c}/topology/core_id")
        pkg = _read(f"/sys/devices/system/cpu/cpu{c}/topology/physical_package_id")
        if sib is not None:
            cores.add((pkg, sib))
    return {"model": model, "usable_threads": threads, "physical_cores_of_usable": len(cores) or None,
            "smt_active": None if smt is None else smt == "1", "machine": platform.machine()}


def run_record(torch):
    props = torch.cuda.get_device_properties(0)
    rec = {"device": props.name, "gfx_arch": getattr(props, "gcnArchName", None),
           "compute_units": props.multi_processor_count, "torch": torch.__version__,
           "hip": torch.version.hip, "rocm": _read("/opt/rocm/.info/version"),
           "python": platform.python_version(), "host_cpu": host_cpu()}
    clk = getattr(props, "clock_rate", None)
    if clk:
        rec["max_shader_clock_mhz"] = round(clk / 1000.0, 1)
    clocks = gpu_clocks()
    if clocks:
        rec["clocks"] = clocks
    return rec


def gpu_clocks():
    """The first GPU's supported shader and memory clock levels in MHz, as
    rocm-smi lists them (the highest shader level is the peak figures' clock),
    or None where rocm-smi is missing or prints nothing parseable."""
    import re
    import subprocess
    import shutil
    smi = shutil.which("rocm-smi") or "/opt/rocm/bin/rocm-smi"
    if not os.path.exists(smi):
        return None
    try:
        # the script run by this interpreter directly: its "#!/usr/bin/env"
        # line would exec a second program from a process a profiler may have
        # attached to the GPU already
        txt = subprocess.run([sys.executable, os.path.realpath(smi), "--showclkfrq"], capture_output=True,
                             text=True, timeout=20).stdout
    except Exception:
        return None
    out, cur = {}, None
    for line in txt.splitlines():
        if "GPU[0]" not in line:
            continue
        m = re.search(r"Supported (\w+) frequencies", line)
        if m:
            cur = m.group(1)
            continue
        m = re.search(r":\s*\d+:\s*(\d+)\s*Mhz", line)
        if m and cur:
            out.setdefault(cur + "_levels_mhz", []).append(int(m.group(1)))
    return out or None


# ---- CPU oracle --------------------------------------------------------------------------

def _column_slice(inp, op, nc):
    if op == "w4a16":
        return (inp.x, np.ascontiguousarray(inp.qweight[:, :nc]), np.ascontiguousarray(inp.scales[:, :nc]))
    if op == "w8a16":
        return (inp.x, np.ascontiguousarray(inp.w[:nc]), np.ascontiguousarray(inp.scales[:, :nc]))
    return (inp.x, np.ascontiguousarray(inp.w[:nc]), np.ascontiguousarray(inp.scales[:nc]))


def cpu_oracle_rows(oracle, names, gpu_us, budget_s=0.25):
    """The plain oracle (fp64 sums and the fp32-sequential sum, OpenMP over output
    columns) on each workload: timed on the first `columns` output columns (sized
    for about budget_s per run), one warm-up then 3 runs, median, scaled to the full
    width; rates over the workload's algorithmic bytes and flops."""
    rows = []
    for name in names:
        w = synth.WORKLOADS[name]
        inp = INPUTS.get(name) or synth.gen_workload(name)
        op, G = w["op"], group(w)
        fn = {"w4a16": lambda a: oracle.w4a16(*a, G), "w8a16": lambda a: oracle.w8a16(*a, G),
              "mxfp8": lambda a: oracle.mxfp8(*a)}[op]
        nc = min(w["N"], 64)
        a = _column_slice(inp, op, nc)
        t0 = time.perf_counter()
        fn(a)
        per_col = (time.perf_counter() - t0) / nc
        nc = int(min(w["N"], max(16, budget_s / max(per_col, 1e-9))) // 16 * 16) or 16
        a = _column_slice(inp, op, nc)
        fn(a)
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            fn(a)
            ts.append(time.perf_counter() - t0)
        us = med(ts) * w["N"] / nc * 1e6
        r = {"workload": name, "columns": nc, "us": round(us, 1),
             "GBps": round(algo_bytes(w) / (us * 1e-6) / 1e9, 3),
             "GFLOPs": round(flops(w) / (us * 1e-6) / 1e9, 3)}
        if name in gpu_us:
            r["gpu_speedup"] = round(us / gpu_us[name], 1)
        rows.append(r)
        log(f"cpu oracle {name:17s} {nc:6d} cols  {us:12.1f} µs  {r['GBps']:8.3f} GB/s  {r['GFLOPs']:8.3f} GFLOP/s"
            + (f"  GPU x{r['gpu_speedup']}" if "gpu_speedup" in r else ""))
    return rows


def cpu_baseline(budget_s=10.0):
    """The oracle as it stands, timed on this host on a bounded sample of the decode step."""
    import oracle
    probs = [synth.gen_workload(n) for n in DECODE]
    bytes_step = sum(algo_bytes(synth.WORKLOADS[n]) for n in DECODE)
    for p in probs:                              # warm-up
        oracle.w4a16(p.x, p.qweight, p.scales)
    t0 = time.perf_counter()
    steps = 0
    while time.perf_counter() - t0 < budget_s:
        for p in probs:
            oracle.w4a16(p.x, p.qweight, p.scales)
        steps += 1
    dt = time.perf_counter() - t0
    cpu = host_cpu()
    return {"value": round(bytes_step * steps / dt / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{steps} full decode steps (3 GEMVs, M=1, K=5120, N=5120/6144/1024) in {dt:.1f} s",
            "sums": "both the fp64 sum and the fp32-sequential sum of every output (the oracle as it stands)",
            "threads": oracle.num_threads(), "cpu_model": cpu["model"], "smt_active": cpu["smt_active"],
            "physical_cores_of_usable": cpu["physical_cores_of_usable"],
            "ms_per_step": round(dt / steps * 1e3, 3)}


INPUTS = {}   # generated inputs by workload name, reused by the CPU oracle leg


def workload_table(torch, svq, oracle, names, cus, probe=True):
    """µs per launch (median of 5 trials of graphs of >= 200 rotating launches, parity
    checked before and after), derived rates, and the stream probe of the same bytes."""
    log(f"{'workload':17s} {'kernel':22s} {'µs':>8s} {'GB/s':>8s} {'%HBM':>6s} {'probe':>7s} {'%probe':>7s} "
        f"{'best':>7s} {'%best':>6s} {'TFLOP/s':>8s} {'%MFMA':>6s}")
    detail = []
    for n in names:
        p = Problem(torch, svq, n, POOL_BYTES)
        p.check(oracle)
        tr = time_kernel(torch, p)
        p.check(oracle)
        us = med(tr)
        w = p.w
        gbs = algo_bytes(w) / (us * 1e-6) / 1e9
        tfl = flops(w) / (us * 1e-6) / 1e12
        row = {"workload": n, "op": w["op"], "M": w["M"], "K": w["K"], "N": w["N"], "G": group(w),
               "kernel": p.kernel, "launch_shape": list(p.geometry), "us": round(us, 3), "us_trials": summary(tr),
               "GBps": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
               "weight_GBps": round(weight_bytes(w) / (us * 1e-6) / 1e9, 1),
               "TFLOPs": round(tfl, 2), "mfma_frac": round(tfl / MFMA_BF16_PEAK_TFLOPS, 4),
               "bytes": algo_bytes(w), "input_sha256": p.digest, "weight_copies": len(p.ws_w)}
        INPUTS[n] = p.inp
        p.release()
        del p
        torch.cuda.empty_cache()
        if probe:
            view = _ProbeView(w)
            pr = probe_workload(torch, svq, view, cus)
            pr["frac_same"] = round(pr["same_us"] / us, 4)
            pr["frac_best"] = round(pr["best_us"] / us, 4)
            row["probe"] = pr
            if w["M"] > 16:
                mf = mfma_floor(torch, svq, w, view.geometry)
                mf["frac"] = round(mf["us"] / us, 4)
                mf["frac_random"] = round(mf["us_random"] / us, 4)
                row["mfma_probe"] = mf
        detail.append(row)
        pr = row.get("probe", {})
        mf = row.get("mfma_probe")
        log(f"{n:17s} {row['kernel']:22s} {us:8.2f} {gbs:8.1f} {100 * gbs / HBM_PEAK_GBS:6.1f} "
            f"{pr.get('same_us', 0):7.2f} {100 * pr.get('frac_same', 0):7.1f} {pr.get('best_us', 0):7.2f} "
            f"{100 * pr.get('frac_best', 0):6.1f} {tfl:8.2f} {100 * tfl / MFMA_BF16_PEAK_TFLOPS:6.2f}"
            + (f"   MFMA probe {mf['us']:.2f} µs ({100 * mf['frac']:.1f}%), random operands "
               f"{mf['us_random']:.2f} µs ({100 * mf['frac_random']:.1f}%)" if mf else ""))
        torch.cuda.empty_cache()
    return detail


class _ProbeView:
    """The parts of a workload the probe needs: its bytes and the GEMM's launch shape."""

    def __init__(self, w):
        import spec_verify_amd as svq
        self.w = w
        self.geometry = svq.launch_geometry(OPS[w["op"]], w["M"], w["N"], w["K"], group(w))


def time_quantizer(torch, svq, oracle, N=24832, K=5120, G=128, reps=20):
    """The load-time RTN quantizer on a tenth of the vocabulary head (bf16 [N, K]):
    µs per call and GB/s over its bytes (bf16 read, codes and fp16 scales written);
    the codes of the first call are checked against the oracle on sampled rows."""
    wb = synth.gen_dense_bf16(611, N, K)
    w = torch.from_numpy(wb.view(np.int16)).to("cuda:0")
    res = {"N": N, "K": K, "G": G}
    for bits in (8, 4):
        q, s = svq.rtn_quantize(w, bits, G)
        torch.cuda.synchronize()
        rows = np.arange(0, N, 997)
        q_ref, s_ref = oracle.rtn_quantize(wb[rows], bits, G)
        got_s = s.view(torch.int16).cpu().numpy().view(np.uint16)[:, rows]
        got_q = q.cpu().numpy()[rows] if bits == 8 else q.cpu().numpy()[:, rows]
        if not (np.array_equal(got_s, s_ref) and np.array_equal(got_q, q_ref)):
            raise SystemExit(f"quantizer parity failure (int{bits})")
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            svq.rtn_quantize(w, bits, G, codes=q, scales=s)
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / reps
        nbytes = N * K * 2 + N * K * bits // 8 + (K // G) * N * 2
        res[f"us_int{bits}"] = round(us, 2)
        res[f"GBps_int{bits}"] = round(nbytes / (us * 1e-6) / 1e9, 1)
    return res


def time_fusion(torch, svq, oracle, names):
    """Projections fused at setup against the same projections launched one by
    one: µs per fused GEMM and per sequence of separate GEMMs (each a graph of
    100 steps rotating over >1 GiB of weight copies), plus the one-off fusion
    call itself; sampled outputs of both forms are checked against the oracle
    on the concatenated weights."""
    dev = torch.device("cuda:0")

    def d(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(dev)

    rows_out = []
    for name in names:
        f = synth.FUSIONS[name]
        M, K, widths = f["M"], f["K"], f["widths"]
        Nt = sum(widths)
        inp = synth.gen_fusion(f["seed"], M, K, widths, 128, 4)
        parts = [(d(w), d(sc)) for w, sc in inp.parts]
        x = d(inp.x)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        wf, sf = svq.fuse_projections(parts, 4, 128)
        torch.cuda.synchronize()
        a.record()
        for _ in range(5):
            svq.fuse_projections(parts, 4, 128, weight_fused=wf, scales_fused=sf)
        b.record()
        torch.cuda.synchronize()
        us_setup = a.elapsed_time(b) * 1e3 / 5
        wbytes = K * Nt // 2 + (K // 128) * Nt * 2
        ncopy = max(2, int(POOL_BYTES // wbytes))
        fused_pool = [(wf, sf)] + [(wf.clone(), sf.clone()) for _ in range(ncopy - 1)]
        sep0 = [(svq.q4_repack(w), sc) for w, sc in parts]
        sep_pool = [sep0] + [[(w.clone(), sc.clone()) for w, sc in sep0] for _ in range(ncopy - 1)]
        del parts
        out_f = torch.empty((M, Nt), dtype=torch.bfloat16, device=dev)
        outs = [torch.empty((M, n), dtype=torch.bfloat16, device=dev) for n in widths]
        nb = max([svq.w4a16_workspace_bytes(M, Nt, K)] + [svq.w4a16_workspace_bytes(M, n, K) for n in widths])
        ws = torch.zeros(max(nb, 256), dtype=torch.uint8, device=dev) if nb else None

        def fused(i):
            w, sc = fused_pool[i % ncopy]
            svq.w4a16_gemm(x, w, sc, Nt, 128, out=out_f, workspace=ws)

        def separate(i):
            for (w, sc), n, o in zip(sep_pool[i % ncopy], widths, outs):
                svq.w4a16_gemm(x, w, sc, n, 128, out=o, workspace=ws)

        wf_ref, sf_ref = oracle.fuse_projections(inp.parts, 4, 128)
        rng = np.random.default_rng(2)
        rr, cc = rng.integers(0, M, 256), rng.integers(0, Nt, 256)
        y64, _ = oracle.w4a16_points(inp.x, wf_ref, sf_ref, 128, rr, cc)

        def check(label):
            for i in (0, ncopy - 1):
                fused(i)
                separate(i)
                torch.cuda.synchronize()
                yf = out_f.view(torch.int16).cpu().numpy().view(np.uint16)
                ys = np.concatenate([o.view(torch.int16).cpu().numpy().view(np.uint16) for o in outs], axis=1)
                for got, form in ((yf, "fused"), (ys, "separate")):
                    ok, err, rms = oracle.gate(got[rr, cc], y64)
                    if not ok:
                        raise SystemExit(f"parity failure in {name} ({form}, {label}, copy {i}): err {err} rms {rms}")

        check("before")
        g = graph_of(torch, fused, 100)
        us_f = time_graph(torch, g, 3) / 100 * 1e6
        del g
        g = graph_of(torch, separate, 100)
        us_s = time_graph(torch, g, 3) / 100 * 1e6
        del g
        check("after")
        ab = wbytes + 2 * M * K + 2 * M * Nt
        gbs = ab / (us_f * 1e-6) / 1e9
        kern = svq.w4a16_kernel_name(M, Nt, K)
        rows_out.append({"fusion": name, "M": M, "K": K, "widths": widths, "kernel": kern,
                         "us_fused": round(us_f, 3), "us_separate": round(us_s, 3),
                         "speedup": round(us_s / us_f, 3), "GBps_fused": round(gbs, 1),
                         "hbm_frac_fused": round(gbs / HBM_PEAK_GBS, 4), "us_fuse_setup": round(us_setup, 1)})
        log(f"fusion {name:11s} {kern:22s} fused {us_f:8.2f} µs ({gbs:7.1f} GB/s, "
            f"{100 * gbs / HBM_PEAK_GBS:4.1f}%)  separate {us_s:8.2f} µs  x{us_s / us_f:.2f}  "
            f"(fusion call {us_setup:.1f} µs)")
        del fused_pool, sep_pool, sep0, wf, sf, ws
        torch.cuda.empty_cache()
    return rows_out


def time_mxfp8_quantizer(torch, svq, oracle, N=17408, K=5120, reps=10):
    """The MXFP8 quantizer (plain and optimized round-to-nearest) on one
    MLP-sized projection, bf16 [N, K]: µs per call, GB/s over its bytes (bf16
    read, codes and scales written) and the share of blocks that keep the
    doubled scale; sampled rows are checked bit for bit against the oracle."""
    wb = synth.gen_dense_bf16(962, N, K)
    w = torch.from_numpy(wb.view(np.int16)).to("cuda:0")
    res = {"N": N, "K": K}
    rows = np.arange(0, N, 509)
    for opt in (False, True):
        c, sc = svq.mxfp8_quantize(w, opt)
        torch.cuda.synchronize()
        c_ref, s_ref = oracle.mxfp8_quantize(wb[rows], opt)
        if not (np.array_equal(c.cpu().numpy()[rows], c_ref) and np.array_equal(sc.cpu().numpy()[rows], s_ref)):
            raise SystemExit(f"MXFP8 quantizer parity failure (optimized={opt})")
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            svq.mxfp8_quantize(w, opt, codes=c, scales=sc)
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / reps
        key = "opt" if opt else "plain"
        res[f"us_{key}"] = round(us, 1)
        res[f"GBps_{key}"] = round((N * K * 3 + N * K // 32) / (us * 1e-6) / 1e9, 1)
        if opt:
            plain = svq.mxfp8_quantize(w, False)[1]
            res["doubled_scale_frac"] = round(float((sc != plain).float().mean().item()), 5)
    return res


def time_ct_ingest(torch, svq, oracle, N=17408, K=5120, G=128, reps=20):
    """The compressed-tensors ingest (a transpose of words and scales) on one
    MLP-sized projection: µs per call and GB/s over its bytes (read + write),
    the output checked bit for bit against the oracle."""
    wp, ws = synth.gen_ct_w4a16(961, N, K, G)
    d_wp = torch.from_numpy(wp).to("cuda:0")
    d_ws = torch.from_numpy(ws.view(np.int16)).to("cuda:0")
    qw, s = svq.ct_to_gptq(d_wp, d_ws, G)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.ct_to_gptq(wp, ws)
    if not (np.array_equal(qw.cpu().numpy(), q_ref) and
            np.array_equal(s.view(torch.int16).cpu().numpy().view(np.uint16), s_ref)):
        raise SystemExit("compressed-tensors ingest parity failure")
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        svq.ct_to_gptq(d_wp, d_ws, G, qweight=qw, scales=s)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / reps
    nbytes = 2 * (N * K // 2 + N * (K // G) * 2)
    return {"N": N, "K": K, "G": G, "us": round(us, 2), "GBps": round(nbytes / (us * 1e-6) / 1e9, 1)}


def copy_probe(nbytes=1 << 30, reps=5):
    """Plain device-to-device copies of known size: what FETCH_SIZE / WRITE_SIZE
    read for exactly nbytes read and nbytes written per dispatch."""
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").uniform_()
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    log(f"copy probe: {nbytes} bytes read + {nbytes} written per copy, {dt * 1e6:.1f} µs, "
        f"{2 * nbytes / dt / 1e9:.1f} GB/s")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--quick", action="store_true", help="decode step only, no per-workload table")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle legs")
    ap.add_argument("--no-probe", action="store_true", help="skip the stream probes")
    ap.add_argument("--only", default="",
                    help="comma-separated workloads: time just these (per-workload table, no decode "
                         "step, no CPU leg) and print their rows as JSON; for profiling runs")
    ap.add_argument("--launches", type=int, default=0,
                    help="with --only: just launch each workload's GEMM this many times (rotating "
                         "weight copies, parity checked once), untimed; for counter runs")
    ap.add_argument("--record-profile", nargs="+", metavar="DIR",
                    help="write profiles/trace.json and profiles/traffic.json for the dominant kernel from "
                         "the rocprofv3 result databases under these directories, then exit")
    ap.add_argument("--record-command", default="", help="the profiled command, kept with the trace record")
    ap.add_argument("--setup-only", action="store_true",
                    help="time only the setup-time steps (quantizers, ingest) and print them as JSON")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run 5 copies of a 1 GiB device buffer (known bytes for counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe()
        return

    if args.record_profile:
        record_profile(args.record_profile, args.record_command)
        return

    import torch
    import spec_verify_amd as svq
    import oracle

    if not os.path.exists(svq.library_path):
        from spec_verify_amd import build
        build.build()
    svq.lib()
    record = run_record(torch)
    cus = record["compute_units"]
    log(f"device: {record['device']} ({record['gfx_arch']}), CUs {cus}, torch {record['torch']}, "
        f"hip {record['hip']}, rocm {record['rocm']}; host {record['host_cpu']}")
    if args.setup_only:
        print(json.dumps({"quantizer": time_quantizer(torch, svq, oracle),
                          "ct_ingest": time_ct_ingest(torch, svq, oracle),
                          "mxfp8_quantizer": time_mxfp8_quantizer(torch, svq, oracle)}), flush=True)
        return
    if args.only and args.launches > 0:
        for n in [n for n in args.only.split(",") if n in synth.WORKLOADS]:
            p = Problem(torch, svq, n, POOL_BYTES)
            p.check(oracle)
            for _ in range(args.launches):
                p.launch()
            torch.cuda.synchronize()
            log(f"{n}: {args.launches} launches of {p.kernel} {list(p.geometry)}")
            p.release()
            del p
            torch.cuda.empty_cache()
        return
    if args.only:
        names = [n for n in args.only.split(",") if n]
        rows = workload_table(torch, svq, oracle, [n for n in names if n in synth.WORKLOADS], cus,
                              probe=not args.no_probe)
        fus = time_fusion(torch, svq, oracle, [n for n in names if n in synth.FUSIONS])
        print(json.dumps({"workloads": rows, "fusion": fus}), flush=True)
        return

    # ---- the decode step ----------------------------------------------------
    probs = [Problem(torch, svq, n, POOL_BYTES / len(DECODE)) for n in DECODE]
    for p in probs:
        p.check(oracle)
    bytes_step = sum(algo_bytes(p.w) for p in probs)
    dom = probs[DECODE.index(DOMINANT)]
    # one graph = `chunk` decode steps (3 launches each, weights rotating over the
    # pool); a trial replays it until exactly `steps` steps have run
    chunk = next(c for c in range(min(args.steps, 100), 0, -1) if args.steps % c == 0)
    reps = args.steps // chunk

    def step(i):
        for p in probs:
            p.launch(i % len(p.ws_w))
    g = graph_of(torch, step, chunk)
    for _ in range(max(1, -(-args.warmup // chunk))):
        g.replay()
    torch.cuda.synchronize()
    step_trials = [time_graph(torch, g, reps) / chunk * 1e3 for _ in range(TRIALS)]   # ms per step
    ms_step = med(step_trials)
    del g
    dom_trials = time_kernel(torch, dom)
    dom_us = med(dom_trials)
    value = bytes_step / (ms_step * 1e-3) / 1e9
    dom_gbs = algo_bytes(dom.w) / (dom_us * 1e-6) / 1e9
    dom.check(oracle)
    log(f"decode step: {ms_step * 1e3:.2f} µs/step (trials {[round(t * 1e3, 2) for t in step_trials]}), "
        f"{value:.1f} GB/s; {DOMINANT} ({dom.kernel}) {dom_us:.2f} µs/launch = {dom_gbs:.1f} GB/s "
        f"({100 * dom_gbs / HBM_PEAK_GBS:.1f}% of HBM peak)")
    digests = {p.name: p.digest for p in probs}
    for p in probs:
        p.release()
    torch.cuda.empty_cache()
    dom_probe = None if args.no_probe else probe_workload(torch, svq, _ProbeView(dom.w), cus)

    # ---- per-workload table ------------------------------------------------------
    detail = []
    chip = None
    if not args.quick:
        if not args.no_probe:
            chip = chip_stream(torch, svq, cus)
            log(f"chip stream probe, 1 GiB: best {chip['best_GBps']} GB/s ({100 * chip['hbm_frac']:.1f}% of "
                f"8 TB/s) in {chip['best_shape']}")
            chip["mfma"] = chip_mfma(torch, svq, cus)
            log(f"chip MFMA probe, bf16 16x16x32: {chip['mfma']['TFLOPs']} TFLOP/s "
                f"({100 * chip['mfma']['mfma_frac']:.1f}% of 2.5 PFLOP/s) in {chip['mfma']['shape']}")
        detail = workload_table(torch, svq, oracle, TABLE, cus, probe=not args.no_probe)

    quant = None
    if not args.quick:
        quant = time_quantizer(torch, svq, oracle)
        log(f"load-time RTN quantizer, bf16 [{quant['N']}, {quant['K']}]: int8 {quant['us_int8']:.1f} µs "
            f"({quant['GBps_int8']:.1f} GB/s), int4 {quant['us_int4']:.1f} µs ({quant['GBps_int4']:.1f} GB/s)")

    fusion = ct = mxq = None
    if not args.quick:
        fusion = time_fusion(torch, svq, oracle, list(synth.FUSIONS))
        ct = time_ct_ingest(torch, svq, oracle)
        log(f"compressed-tensors ingest [{ct['N']}, {ct['K']}]: {ct['us']:.1f} µs ({ct['GBps']:.1f} GB/s)")
        mxq = time_mxfp8_quantizer(torch, svq, oracle)
        log(f"MXFP8 quantizer [{mxq['N']}, {mxq['K']}]: plain {mxq['us_plain']:.1f} µs ({mxq['GBps_plain']:.1f} GB/s), "
            f"optimized {mxq['us_opt']:.1f} µs ({mxq['GBps_opt']:.1f} GB/s), doubled scale in "
            f"{100 * mxq['doubled_scale_frac']:.2f}% of blocks")

    cpu = cpu_rows = None
    if not args.no_cpu:
        cpu = cpu_baseline()
        log(f"cpu oracle: {cpu['value']} GB/s on {cpu['cores']} threads ({cpu['sample']})")
        gpu_us = {r["workload"]: r["us"] for r in detail}
        gpu_us.setdefault(DOMINANT, dom_us)
        cpu_rows = cpu_oracle_rows(oracle, [r["workload"] for r in detail] or DECODE, gpu_us)

    traffic = measured_traffic()
    trace = measured_trace()
    roofline = {"bound": "hbm", "achieved": round(dom_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(dom_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": dom.kernel, "workload": DOMINANT, "us_per_launch": round(dom_us, 3),
                "us_trials": summary(dom_trials), "bytes_per_launch": algo_bytes(dom.w),
                "timing": "HIP events around graph replays of rotating launches, median of 5 trials"}
    if trace:
        roofline["trace"] = {**trace, "frac_median": round(algo_bytes(dom.w) / (trace["median_us"] * 1e-6) / 1e9
                                                           / HBM_PEAK_GBS, 4)}
    if dom_probe:
        roofline["probe"] = {**dom_probe, "frac_same": round(dom_probe["same_us"] / dom_us, 4),
                             "frac_best": round(dom_probe["best_us"] / dom_us, 4)}
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 6), "steps_timed": args.steps,
        "step_trials_ms": [round(t, 6) for t in step_trials], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "single-stream decode step: three W4A16 g128 GEMVs, M=1, K=5120, "
                               "N=5120/6144/1024, weights rotated over >1 GiB of copies",
                   "M": 1, "K": 5120, "N": [5120, 6144, 1024], "group_size": 128,
                   "bytes_per_step": bytes_step, "input_sha256": digests},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "run_record": record,
        "chip_stream": chip,
        "workloads": detail,
        "cpu_oracle": cpu_rows,
        "quantizer": quant,
        "fusion": fusion,
        "ct_ingest": ct,
        "mxfp8_quantizer": mxq,
    }
    print(json.dumps(line), flush=True)


# sources the dominant kernel is built from: traffic counters taken on other
# sources do not describe it
DOMINANT_SOURCES = ["w4a16_dot2.hip", "dot2_asm.h", "svq_device.h", "svq_streamk.h", "svq_launch.h",
                    "svq_api.cpp"]


def _kernel_source_sha():
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "spec_verify_amd", "csrc")
    for n in DOMINANT_SOURCES:
        with open(os.path.join(csrc, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_trace(path=None):
    """The dominant kernel's rocprofv3 kernel-trace durations (median, mean, count)
    from profiles/trace.json, or None when there is no record or it was taken on
    other sources than the ones built now."""
    path = path or os.path.join(ROOT, "profiles", "trace.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f).get(DOMINANT)
    if not t or t.get("kernel_source_sha") != _kernel_source_sha():
        return None
    return {k: t[k] for k in ("median_us", "mean_us", "dispatches", "command") if k in t}


def measured_traffic(path=None):
    """HBM bytes per launch of the dominant kernel from its recorded FETCH_SIZE /
    WRITE_SIZE counters, or None when there is no record or the record was taken
    on other sources than the ones built now."""
    path = path or os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f).get(DOMINANT)
    if not t or t.get("kernel_source_sha") != _kernel_source_sha():
        return None
    return t.get("bytes_per_launch")


def _rocpd_rows(dirs):
    """(database, kernel dispatches, per-dispatch counter sums) of every rocprofv3
    result database under dirs."""
    import glob
    import sqlite3
    for d in dirs:
        for path in sorted(glob.glob(os.path.join(d, "**", "*.db"), recursive=True)):
            db = sqlite3.connect(path)
            names = {r[0] for r in db.execute("select name from sqlite_master where type in ('table','view')")}
            if "kernels" not in names:
                continue
            disp = {r[0]: (r[1], r[2], r[3] - r[4]) for r in db.execute(
                "select dispatch_id, name, grid_x * grid_y * grid_z, end, start from kernels")}
            pmc = {}
            if "pmc_events" in names:
                for did, cn, cv in db.execute("select dispatch_id, counter_name, counter_value from pmc_events"):
                    pmc.setdefault(did, {}).setdefault(cn, 0.0)
                    pmc[did][cn] += cv
            yield path, disp, pmc


def record_profile(dirs, command):
    """Write profiles/trace.json and profiles/traffic.json for the dominant kernel
    from rocprofv3 result databases: durations from kernel-trace runs (databases
    without counters), FETCH_SIZE / WRITE_SIZE per dispatch from counter runs,
    scaled by what the same counters read for the copy probe's 1 GiB copies."""
    import spec_verify_amd as svq
    w = synth.WORKLOADS[DOMINANT]
    grid, threads, _ = svq.launch_geometry(OPS[w["op"]], w["M"], w["N"], w["K"], group(w))
    kname = svq.kernel_name(OPS[w["op"]], w["M"], w["N"], w["K"], group(w))
    items = grid * threads
    # the kernel's own instantiation: its last template argument is log2(G) (the
    # same launch shape also runs the G = 32 / 64 instantiations)
    inst = ", %d>" % (group(w).bit_length() - 1)
    durs, fetch, write, cfetch, cwrite = [], [], [], [], []
    copy_kib = (1 << 30) / 1024
    for _, disp, pmc in _rocpd_rows(dirs):
        for did, (name, n, dur) in disp.items():
            mine = kname in name and n == items and inst in name
            if did in pmc:
                c = pmc[did]
                if mine:
                    fetch += [c["FETCH_SIZE"]] if "FETCH_SIZE" in c else []
                    write += [c["WRITE_SIZE"]] if "WRITE_SIZE" in c else []
                elif "copyBuffer" in name:
                    cfetch += [c["FETCH_SIZE"]] if "FETCH_SIZE" in c else []
                    cwrite += [c["WRITE_SIZE"]] if "WRITE_SIZE" in c else []
            elif mine:
                durs.append(dur / 1e3)
    sha = _kernel_source_sha()
    out = []
    if durs:
        rec = {"kernel": kname, "kernel_source_sha": sha, "median_us": round(med(durs), 3),
               "mean_us": round(sum(durs) / len(durs), 3), "dispatches": len(durs), "command": command}
        with open(os.path.join(ROOT, "profiles", "trace.json"), "w") as f:
            json.dump({DOMINANT: rec}, f, indent=2)
            f.write("\n")
        out.append(f"trace: {rec}")
    if fetch and write and cfetch and cwrite:
        ff, wf = copy_kib / med(cfetch), copy_kib / med(cwrite)
        fk, wk = sum(fetch) / len(fetch), sum(write) / len(write)
        rec = {"kernel": kname, "kernel_source_sha": sha, "fetch_kib_per_dispatch": round(fk, 1),
               "write_kib_per_dispatch": round(wk, 1), "fetch_factor": round(ff, 5), "write_factor": round(wf, 5),
               "dispatches": len(fetch), "bytes_per_launch": int(round((fk * ff + wk * wf) * 1024))}
        with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
            json.dump({DOMINANT: rec}, f, indent=2)
            f.write("\n")
        out.append(f"traffic: {rec}")
    log("\n".join(out) if out else "no matching dispatches")


if __name__ == "__main__":
    main()
