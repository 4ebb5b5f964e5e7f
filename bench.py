"""Benchmark of the weight-only quantized linear layer on one MI355X.

A step is one decode step's worth of the hot path: the three W4A16 (INT4, g128)
GEMVs of a single-stream decode at M=1, K=5120, N in {5120, 6144, 1024}, on
inputs resident in HBM. Weights rotate through a pool of distinct copies larger
than 1 GiB so every launch streams them from HBM, not from the 256 MB Infinity
Cache. `value` is the step's algorithmic bytes (packed weights + scales + x + y,
each once) per second.

Also reported (stderr table and the JSON line's "workloads" list): per-kernel
time, GB/s, TFLOP/s and roofline fraction for every named workload (decode,
M=3/5 verify chunks, M=128 batched verify, MXFP8 at M=1/5/128), and the CPU
oracle's throughput on a bounded sample (``cpu_baseline``), the fused K/V/Q and
gate/up projections against the same projections launched one by one
(``fusion``), and the setup-time steps (``quantizer``, ``ct_ingest``,
``mxfp8_quantizer``).

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--quick] [--no-cpu]
    python bench.py --copy-probe    # a plain 1 GiB device copy, to calibrate HBM counters
"""
from __future__ import annotations

import argparse
import json
import os
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
METRIC = "W4A16 GEMM µs, weight-stream GB/s and % HBM peak at M=1/5/128; TFLOP/s"
DECODE = ["decode_n5120", "decode_n6144", "decode_n1024"]
DOMINANT = "decode_n6144"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def weight_bytes(w):
    K, N = w["K"], w["N"]
    if w["op"] == "w4a16":
        return K * N // 2 + (K // 128) * N * 2
    if w["op"] == "w8a16":
        return K * N + (K // 128) * N * 2
    return K * N + (K // 32) * N


def algo_bytes(w):
    return weight_bytes(w) + 2 * w["M"] * w["K"] + 2 * w["M"] * w["N"]


class Problem:
    """Device-resident inputs of one workload with a rotation pool of weight copies."""

    def __init__(self, torch, svq, name, pool_bytes):
        self.name = name
        self.w = synth.WORKLOADS[name]
        self.torch, self.svq = torch, svq
        inp = synth.gen_workload(name)
        self.inp = inp
        dev = torch.device("cuda:0")

        def d(a):
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint16:
                a = a.view(np.int16)
            return torch.from_numpy(a).to(dev)

        self.x = d(inp.x)
        M, K, N = self.w["M"], self.w["K"], self.w["N"]
        self.out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ncopy = max(2, int(pool_bytes // max(weight_bytes(self.w), 1)))
        if self.w["op"] == "w4a16":
            base_w = svq.q4_repack(d(inp.qweight))
            base_s = d(inp.scales)
            self.kernel = svq.w4a16_kernel_name(M, N, K)
            nb = svq.w4a16_workspace_bytes(M, N, K)
        elif self.w["op"] == "w8a16":
            base_w = torch.from_numpy(np.ascontiguousarray(inp.w)).to(dev)
            base_s = d(inp.scales)
            self.kernel = svq.w8a16_kernel_name(M, N, K)
            nb = svq.w8a16_workspace_bytes(M, N, K)
        else:
            base_w = d(inp.w)
            base_s = d(inp.scales)
            self.kernel = svq.mxfp8_kernel_name(M, N, K)
            nb = svq.mxfp8_workspace_bytes(M, N, K)
        self.ws = torch.zeros(max(nb, 256), dtype=torch.uint8, device=dev) if nb else None
        self.ws_w = [base_w] + [base_w.clone() for _ in range(ncopy - 1)]
        self.ws_s = [base_s] + [base_s.clone() for _ in range(ncopy - 1)]
        self.i = 0

    def launch(self, i=None):
        i = self.i if i is None else i
        self.i = (self.i + 1) % len(self.ws_w)
        w = self.w
        if w["op"] == "w4a16":
            self.svq.w4a16_gemm(self.x, self.ws_w[i], self.ws_s[i], w["N"], 128, out=self.out,
                                workspace=self.ws)
        elif w["op"] == "w8a16":
            self.svq.w8a16_gemm(self.x, self.ws_w[i], self.ws_s[i], 128, out=self.out, workspace=self.ws)
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
                y64, _ = oracle.w4a16_points(inp.x, inp.qweight, inp.scales, 128, rows, cols)
            elif w["op"] == "w8a16":
                y64, _ = oracle.w8a16_points(inp.x, inp.w, inp.scales, 128, rows, cols)
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


def time_kernel(torch, prob, launches=100, reps=5):
    """Mean µs per launch of one kernel: a graph of `launches` launches that
    rotate over the weight pool, replayed `reps` times."""
    g = graph_of(torch, lambda i: prob.launch(i % len(prob.ws_w)), launches)
    t = time_graph(torch, g, reps)
    del g
    return t / launches * 1e6


def cpu_baseline(budget_s=12.0):
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
    return {"value": round(bytes_step * steps / dt / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{steps} full decode steps (3 GEMVs, M=1, K=5120, N=5120/6144/1024) in {dt:.1f} s; "
                      "fp64 sums plus the fp32-sequential sum, OpenMP over output columns",
            "ms_per_step": round(dt / steps * 1e3, 3)}


def workload_table(torch, svq, oracle, names):
    """µs per launch (graph of 100 rotating launches, parity checked before and
    after) and the derived rates of each named workload."""
    log(f"{'workload':15s} {'kernel':22s} {'µs':>8s} {'GB/s':>8s} {'%HBM':>6s} "
        f"{'TFLOP/s':>8s} {'%MFMA':>6s}")
    detail = []
    for n in names:
        p = Problem(torch, svq, n, POOL_BYTES)
        p.check(oracle)
        us = time_kernel(torch, p, launches=100, reps=3)
        p.check(oracle)
        w = p.w
        gbs = algo_bytes(w) / (us * 1e-6) / 1e9
        tfl = 2.0 * w["M"] * w["N"] * w["K"] / (us * 1e-6) / 1e12
        detail.append({"workload": n, "op": w["op"], "M": w["M"], "K": w["K"], "N": w["N"], "kernel": p.kernel,
                       "us": round(us, 3),
                       "GBps": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                       "weight_GBps": round(weight_bytes(w) / (us * 1e-6) / 1e9, 1),
                       "TFLOPs": round(tfl, 2), "mfma_frac": round(tfl / MFMA_BF16_PEAK_TFLOPS, 4)})
        log(f"{n:15s} {p.kernel:22s} {us:8.2f} {gbs:8.1f} {100 * gbs / HBM_PEAK_GBS:6.1f} "
            f"{tfl:8.2f} {100 * tfl / MFMA_BF16_PEAK_TFLOPS:6.2f}")
        p.release()
        del p
        torch.cuda.empty_cache()
    return detail


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
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only", default="",
                    help="comma-separated workloads: time just these (per-workload table, no decode "
                         "step, no CPU leg) and print their rows as JSON; for profiling runs")
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

    import torch
    import spec_verify_amd as svq
    import oracle

    if not os.path.exists(svq.library_path):
        from spec_verify_amd import build
        build.build()
    svq.lib()
    props = torch.cuda.get_device_properties(0)
    log(f"device: {props.name} ({getattr(props, 'gcnArchName', '?')}), CUs {props.multi_processor_count}, "
        f"torch {torch.__version__}, hip {torch.version.hip}")
    if args.setup_only:
        print(json.dumps({"quantizer": time_quantizer(torch, svq, oracle),
                          "ct_ingest": time_ct_ingest(torch, svq, oracle),
                          "mxfp8_quantizer": time_mxfp8_quantizer(torch, svq, oracle)}), flush=True)
        return
    if args.only:
        names = [n for n in args.only.split(",") if n]
        rows = workload_table(torch, svq, oracle, [n for n in names if n in synth.WORKLOADS])
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
    # pool); it is replayed until `steps` steps have run, after `warmup` steps
    chunk = next(c for c in range(min(args.steps, 100), 0, -1) if args.steps % c == 0)
    reps = args.steps // chunk

    def step(i):
        for p in probs:
            p.launch(i % len(p.ws_w))
    g = graph_of(torch, step, chunk)
    for _ in range(max(1, -(-args.warmup // chunk))):
        g.replay()
    torch.cuda.synchronize()
    sec = time_graph(torch, g, reps)
    steps_run = chunk * reps
    ms_step = sec / chunk * 1e3
    del g
    dom_us = time_kernel(torch, dom, launches=100, reps=5)
    value = bytes_step / (ms_step * 1e-3) / 1e9
    dom_gbs = algo_bytes(dom.w) / (dom_us * 1e-6) / 1e9
    dom.check(oracle)
    log(f"decode step: {ms_step * 1e3:.2f} µs/step, {value:.1f} GB/s; {DOMINANT} ({dom.kernel}) "
        f"{dom_us:.2f} µs/launch = {dom_gbs:.1f} GB/s ({100 * dom_gbs / HBM_PEAK_GBS:.1f}% of HBM peak)")
    for p in probs:
        p.release()
    torch.cuda.empty_cache()

    # ---- per-workload table ------------------------------------------------------
    detail = []
    if not args.quick:
        detail = workload_table(torch, svq, oracle, [
            "decode_n5120", "decode_n6144", "decode_n1024", "verify3_up", "verify3_down", "verify5_up",
            "verify5_down", "batch128_up", "batch128_down", "mxfp8_m1", "mxfp8_m5", "mxfp8_m128",
            "vocab_w8_m1", "vocab_w4_m1"])

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

    cpu = None if args.no_cpu else cpu_baseline()
    if cpu:
        log(f"cpu oracle: {cpu['value']} GB/s on {cpu['cores']} threads ({cpu['sample']})")

    traffic = measured_traffic()

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 6), "steps_timed": steps_run, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "single-stream decode step: three W4A16 g128 GEMVs, M=1, K=5120, "
                               "N=5120/6144/1024, weights rotated over >1 GiB of copies",
                   "M": 1, "K": 5120, "N": [5120, 6144, 1024], "group_size": 128,
                   "bytes_per_step": bytes_step},
        "roofline": {"bound": "hbm", "achieved": round(dom_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dom_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": dom.kernel, "workload": DOMINANT, "us_per_launch": round(dom_us, 3),
                     "bytes_per_launch": algo_bytes(dom.w)},
        "cpu_baseline": cpu,
        "workloads": detail,
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


if __name__ == "__main__":
    main()
