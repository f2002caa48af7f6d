"""Throughput of the MC2 compute core on one MI355X.

Headline step: the large configuration, one pass of its two GEMM launches --
the AllGatherMatmul local share (gathered x of W=8 chunks of (2048, 8192) =
(16384, 8192) @ weight (8192, 3584)) and the simulated W=8
MatmulReduceScatter (8 k-shards (16384, 1024) @ (1024, 8192) summed into 8
row chunks of 2048) -- both bf16 with fp32 accumulation and per-chunk ready
flags, each weight held as an (n, k) Linear weight and passed transposed
(x2_trans). `value` is the step's FLOPs over the mean step time, in TFLOP/s.

Before the timed steps the headline runs untimed for a fixed settle time
(--settle seconds, default 2) so that the clocks have left their ramp; then
--warmup untimed steps and exactly --steps timed steps, run back to back
between two HIP events on the launch stream: their mean is `ms_per_step`.
A second pass of --steps steps brackets every step and every launch with
events for the median and the split between the two launches (an event
between launches leaves the GPU idle for a few microseconds, so that pass is
not used for the mean). The same JSON line carries the other hot-path rows
(the AllGatherMatmul and int8 shares, the MoE expert-parallel local path and
its backward, MatmulAllReduce, the split granularity), each timed the same
way over at least 200 ms of calls, with its mean and median;
the roofline of the headline kernel; the shader clock sampled while it ran;
and the CPU oracle timed on a bounded sample of the headline workload.

Inputs are seeded synthetic data resident in HBM before timing starts.

    python bench.py [--steps K] [--warmup W] [--settle S]
                    [--only c5|c1|c2|c3|c4|c4bwd|split|rows|all] [--no-cpu-baseline]
                    [--calib-copy] [--calib-lds]
"""
from __future__ import annotations

import argparse
import glob
import json
import os
import statistics
import sys
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TFLOP/s and % of MFMA peak, rank-chunked GEMM/GMM on 1 MI355X"
PEAK_BF16 = 2500.0   # TFLOP/s, dense bf16/fp16 MFMA (published)
PEAK_I8 = 5000.0     # TOP/s, dense int8 MFMA (published)
PEAK_HBM = 8000.0    # GB/s, HBM3E (published)

# Sources of the headline kernel (the grouped and MoE kernels live elsewhere):
# the HBM traffic recorded under profiles/ is reported only while their code,
# comments and blank space aside, is unchanged since the counters were taken.
KERNEL_SOURCES = ["gemm_collective_core_amd/csrc/gemm_core.hpp",
                  "gemm_collective_core_amd/csrc/gemm_core_w4.hpp",
                  "gemm_collective_core_amd/csrc/mc2_tiles.hpp",
                  "gemm_collective_core_amd/csrc/mc2_chunked.hpp",
                  "gemm_collective_core_amd/csrc/mc2_gemm.hip",
                  "gemm_collective_core_amd/csrc/mc2_common.hpp",
                  "gemm_collective_core_amd/csrc/mc2_host.hpp"]
TRAFFIC_FILE = "profiles/traffic_c5_ag_mm_sim_rs_bf16.json"
# The headline launches the recorded traffic must belong to.
HEADLINE_LAUNCH = ("c5: ag_mm bf16 16384x8192x3584 W=8 rank 0 + mm_rs nsim=8 bf16 "
                   "16384x(8x1024)x8192 W=8 rank 0, x2 (n, k) with x2_trans, ready flags")

# The headline workload: (m, k, n) of each launch and its FLOPs.
C5A = (16384, 8192, 3584)
C5B = (16384, 8 * 1024, 8192)
FLOP_A = 2.0 * C5A[0] * C5A[1] * C5A[2]
FLOP_B = 2.0 * C5B[0] * C5B[1] * C5B[2]
# Bytes each launch must move at least: its operands read once, its output
# written once (bf16).
BYTES_A = 2 * (C5A[0] * C5A[1] + C5A[1] * C5A[2] + C5A[0] * C5A[2])
BYTES_B = 2 * (C5B[0] * C5B[1] + C5B[1] * C5B[2] + C5B[0] * C5B[2])


def kernel_source_hash():
    """sha256 of the headline kernel's sources with comments removed and
    blank space collapsed, so that a change to comments alone keeps it."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def recorded_traffic():
    """HBM bytes per launch of the headline kernel from the committed counter
    summary, or None when it is missing, the kernel changed since, or it was
    taken on another launch configuration."""
    path = os.path.join(ROOT, TRAFFIC_FILE)
    if not os.path.exists(path):
        return None
    with open(path, encoding="utf-8") as f:
        rec = json.load(f)
    if rec.get("source_sha256") != kernel_source_hash() or rec.get("launch") != HEADLINE_LAUNCH:
        return None
    return rec.get("traffic_bytes_per_launch")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


class ClockSampler:
    """Samples the GPU's current shader clock from sysfs while the headline
    runs (the hwmon freq1_input of the PCI device torch reports, else the
    starred level of pp_dpm_sclk)."""

    def __init__(self, props):
        self.samples = []
        self.source = None
        self._stop = threading.Event()
        dev = "/sys/bus/pci/devices/%04x:%02x:%02x.0" % (
            getattr(props, "pci_domain_id", 0), props.pci_bus_id, props.pci_device_id)
        cands = sorted(glob.glob(dev + "/hwmon/hwmon*/freq1_input"))
        if cands:
            self.source = cands[0]
            self._read = self._read_hwmon
        elif os.path.exists(dev + "/pp_dpm_sclk"):
            self.source = dev + "/pp_dpm_sclk"
            self._read = self._read_dpm
        self._thread = None

    def _read_hwmon(self):
        with open(self.source, encoding="utf-8") as f:
            return int(f.read().strip()) / 1e6

    def _read_dpm(self):
        with open(self.source, encoding="utf-8") as f:
            for line in f:
                if line.strip().endswith("*"):
                    return float(line.split(":")[1].strip().rstrip("*").strip().lower()
                                 .replace("mhz", ""))
        return None

    def _run(self):
        while not self._stop.is_set():
            try:
                v = self._read()
                if v:
                    self.samples.append(v)
            except (OSError, ValueError):
                pass
            self._stop.wait(0.01)

    def start(self):
        if self.source:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()

    def stop(self):
        self._stop.set()
        if self._thread:
            self._thread.join()

    def report(self):
        if not self.samples:
            return {"mhz_median": None, "source": self.source or "no sysfs clock found",
                    "samples": 0}
        s = sorted(self.samples)
        return {"mhz_median": statistics.median(s), "mhz_min": s[0], "mhz_max": s[-1],
                "samples": len(s), "source": self.source}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--settle", type=float, default=2.0,
                   help="seconds of untimed headline steps before the warmup")
    p.add_argument("--only", default="all")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--calib-copy", action="store_true",
                   help="run only a plain 1 GiB device copy (HBM counter calibration)")
    p.add_argument("--calib-lds", action="store_true",
                   help="run only a one-tile GEMM whose operands are read exactly once "
                        "(counter calibration of the loads into LDS)")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the work; runs on more than one GPU are "
              "not part of this build (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as wl
    from gemm_collective_core_amd import mc2

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(a, bf16=False):
        a = np.ascontiguousarray(a)
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if bf16 else torch.from_numpy(a)
        return t.to(dev)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def measure(fn, min_ms=200.0, warmup=10, min_iters=10, max_iters=5000):
        """Mean and median milliseconds per call of fn(), on the current
        stream (the stream every entry point launches on). The mean is over at
        least `min_ms` of calls run back to back between two HIP events; the
        median comes from a second pass of as many calls, each bracketed by
        events (which leave the GPU idle for a few microseconds between calls,
        so that pass does not give the mean)."""
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record()
        for _ in range(3):
            fn()
        b.record()
        torch.cuda.synchronize()
        est = max(a.elapsed_time(b) / 3, 1e-3)
        n = int(min(max(min_iters, np.ceil(min_ms / est)), max_iters))
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        mean = a.elapsed_time(b) / n
        evs = [ev() for _ in range(n + 1)]
        evs[0].record()
        for i in range(n):
            fn()
            evs[i + 1].record()
        torch.cuda.synchronize()
        per = [evs[i].elapsed_time(evs[i + 1]) for i in range(n)]
        return mean, float(np.median(per)), n

    if args.calib_copy:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        ms, _, _ = measure(lambda: b.copy_(a), 0.0, 3, 20, 20)
        log(f"copy 1 GiB: {ms:.3f} ms -> {2 * n / ms / 1e6:.1f} GB/s (read+write)")
        print(json.dumps({"calib_copy_bytes_read": n, "calib_copy_bytes_written": n,
                          "ms": ms, "GBps": 2 * n / ms / 1e6}))
        return
    if args.calib_lds:
        # one 128 x 256 output tile: one workgroup reads each operand element
        # exactly once (no other tile could share it) through the loads into
        # LDS, so the fetch counter of this launch is known in bytes
        m, k, n = 128, 65472, 256
        d = wl.gemm_inputs(77, m, k, n, wl.BF16, std=0.02, x2_trans=True)
        x, w = to_dev(d["x1"], True), to_dev(d["x2"], True)
        out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        ms, _, it = measure(lambda: mc2.mc2_ag_mm_local(x, w, 1, 0, x2_trans=True, out=out),
                            0.0, 2, 10, 10)
        rd = 2 * (m * k + n * k)
        log(f"one-tile GEMM {m}x{k}x{n}: {ms:.3f} ms, reads {rd} bytes once per launch")
        print(json.dumps({"calib_lds_bytes_read": rd, "calib_lds_bytes_written": 2 * m * n,
                          "launches": it + 15, "ms": ms}))
        return

    only = args.only
    rows = {}
    headline = None
    clock = ClockSampler(torch.cuda.get_device_properties(dev))

    # ------------------------------------------------------------- headline (C5)
    if only in ("all", "c5"):
        log("C5: generating inputs")
        c5_kn = wl.c5_inputs()
        a, b = (wl.x2_as_nk(d) for d in c5_kn)
        W = 8
        xa, wa = to_dev(a["x1"], True), to_dev(a["x2"], True)
        xb, wb = to_dev(b["x1"], True), to_dev(b["x2"], True)
        wb_nk = wb
        del a, b
        out_a = torch.empty((C5A[0], C5A[2]), dtype=torch.bfloat16, device=dev)
        out_b = torch.empty((C5B[0], C5B[2]), dtype=torch.bfloat16, device=dev)
        fl_a, cn_a = (torch.zeros(W, dtype=torch.int32, device=dev) for _ in range(2))
        fl_b, cn_b = (torch.zeros(W, dtype=torch.int32, device=dev) for _ in range(2))
        epoch = [0]

        def launch_a():
            mc2.mc2_ag_mm_local(xa, wa, W, 0, x2_trans=True, out=out_a, ready_flags=fl_a,
                                flag_counters=cn_a, epoch=epoch[0])

        def launch_b():
            mc2.mc2_mm_rs_local(xb, wb, W, 0, x2_trans=True, out=out_b, ready_flags=fl_b,
                                flag_counters=cn_b, epoch=epoch[0])

        def step(mid=None):
            epoch[0] += 1
            launch_a()
            if mid is not None:
                mid.record()
            launch_b()

        clock.start()
        t_settle = time.perf_counter()
        n_settle = 0
        while time.perf_counter() - t_settle < args.settle:
            for _ in range(20):
                step()
            n_settle += 20
            torch.cuda.synchronize()
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        K = args.steps
        # the timed steps, back to back between two events
        first, last = ev(), ev()
        t0 = time.perf_counter()
        first.record()
        for i in range(K):
            step()
        last.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        assert fl_a.cpu().tolist() == [epoch[0]] * W and fl_b.cpu().tolist() == [epoch[0]] * W
        ms = first.elapsed_time(last) / K
        # a second pass with every step and launch bracketed: median, launch split
        starts = [ev() for _ in range(K + 1)]
        mids = [ev() for _ in range(K)]
        starts[0].record()
        for i in range(K):
            step(mids[i])
            starts[i + 1].record()
        torch.cuda.synchronize()
        clock.stop()
        assert fl_a.cpu().tolist() == [epoch[0]] * W and fl_b.cpu().tolist() == [epoch[0]] * W
        per_step = [starts[i].elapsed_time(starts[i + 1]) for i in range(K)]
        t_a = [starts[i].elapsed_time(mids[i]) for i in range(K)]
        t_b = [mids[i].elapsed_time(starts[i + 1]) for i in range(K)]
        tf = (FLOP_A + FLOP_B) / ms / 1e9
        ka, kb = float(np.mean(t_a)), float(np.mean(t_b))
        headline = {"ms": ms, "ms_median": float(np.median(per_step)), "tflops": tf,
                    "wall_s": wall, "settle_steps": n_settle,
                    "launch_ms": {"c5a_ag_mm": ka, "c5b_sim_rs": kb},
                    "kernel_tflops": (FLOP_A + FLOP_B) / (ka + kb) / 1e9}
        rows["c5a_ag_mm_bf16"] = {"ms": ka, "ms_median": float(np.median(t_a)),
                                  "TFLOP/s": FLOP_A / ka / 1e9,
                                  "frac_peak": FLOP_A / ka / 1e9 / PEAK_BF16}
        rows["c5b_sim_rs_bf16"] = {"ms": kb, "ms_median": float(np.median(t_b)),
                                   "TFLOP/s": FLOP_B / kb / 1e9,
                                   "frac_peak": FLOP_B / kb / 1e9 / PEAK_BF16}
        log(f"C5 step: {ms * 1e3:.1f} us (median {headline['ms_median'] * 1e3:.1f})  {tf:.1f} "
            f"TFLOP/s ({100 * tf / PEAK_BF16:.1f}% of peak); C5a {ka * 1e3:.1f} us, "
            f"C5b {kb * 1e3:.1f} us; settle {n_settle} steps")
        if only == "all":
            # the same products with x2 given (k, n)
            del wa
            wa, wb = to_dev(c5_kn[0]["x2"], True), to_dev(c5_kn[1]["x2"], True)
            for name, fn, fl in (
                    ("c5a_ag_mm_bf16_x2_kn", lambda: mc2.mc2_ag_mm_local(
                        xa, wa, W, 0, out=out_a, ready_flags=fl_a, flag_counters=cn_a, epoch=1),
                     FLOP_A),
                    ("c5b_sim_rs_bf16_x2_kn", lambda: mc2.mc2_mm_rs_local(
                        xb, wb, W, 0, out=out_b, ready_flags=fl_b, flag_counters=cn_b, epoch=1),
                     FLOP_B)):
                m_, med, it = measure(fn)
                rows[name] = {"ms": m_, "ms_median": med, "iters": it, "TFLOP/s": fl / m_ / 1e9,
                              "frac_peak": fl / m_ / 1e9 / PEAK_BF16}
                log(f"{name}: {m_ * 1e3:.1f} us  {fl / m_ / 1e9:.1f} TFLOP/s")
            # MatmulAllReduce local share on the C5b partials, per rounding model
            del wb
            wb = wb_nk
            ws = torch.empty(mc2.mc2_mm_ar_workspace_size(16384, 8192, W, torch.bfloat16,
                                                          mc2.MC2_AR_HOP_ROUNDED),
                             dtype=torch.uint8, device=dev)
            for mode, name in ((mc2.MC2_AR_ONE_ROUNDING, "one"), (mc2.MC2_AR_RANK_ROUNDED, "rank"),
                               (mc2.MC2_AR_HOP_ROUNDED, "hop")):
                m_, med, it = measure(lambda: mc2.mc2_mm_ar_local(
                    xb, wb, W, rounding=mode, x2_trans=True, out=out_b, workspace=ws))
                rows[f"c5b_mm_ar_{name}_rounding_bf16"] = {
                    "ms": m_, "ms_median": med, "iters": it, "TFLOP/s": FLOP_B / m_ / 1e9,
                    "frac_peak": FLOP_B / m_ / 1e9 / PEAK_BF16}
                log(f"C5b MM-AR ({name} rounding): {m_ * 1e3:.1f} us  {FLOP_B / m_ / 1e9:.1f} TFLOP/s")
            # the combining step alone: W stored partials read, one result written
            parts = ws[: W * 16384 * 8192 * 2].view(torch.bfloat16).view(W, 16384, 8192)
            m_, med, it = measure(lambda: mc2.mc2_ar_sum_local(parts, mc2.MC2_AR_HOP_ROUNDED,
                                                               out=out_b))
            nbytes = (W + 1) * 16384 * 8192 * 2
            rows["c5b_ar_sum_bf16"] = {"ms": m_, "ms_median": med, "iters": it,
                                       "GB/s": nbytes / m_ / 1e6,
                                       "frac_hbm": nbytes / m_ / 1e6 / PEAK_HBM}
            log(f"C5b AR combine: {m_ * 1e3:.1f} us  {nbytes / m_ / 1e6:.0f} GB/s")
            del ws, parts
        del xa, wa, xb, wb, wb_nk, out_a, out_b

    # ---------------------------------------------------------------- C1
    if only in ("all", "rows", "c1"):
        # the page's example shapes: launch-bound, timed for completeness
        d = wl.c1_inputs()
        x1, x2 = to_dev(d["x1"]), to_dev(d["x2"])
        out = torch.empty((128, 64), dtype=torch.float16, device=dev)
        fl1 = 2.0 * 2 * 128 * 512 * 64
        m_, med, it = measure(lambda: mc2.mc2_mm_rs_local(x1, x2, 2, 0, out=out), 50.0)
        rows["c1_sim_rs_fp16"] = {"ms": m_, "ms_median": med, "iters": it,
                                  "TFLOP/s": fl1 / m_ / 1e9}
        log(f"C1 sim-W=2 MM-RS fp16: {m_ * 1e3:.1f} us")
        del x1, x2, out

    # ---------------------------------------------------------------- C2
    if only in ("all", "rows", "c2"):
        log("C2: generating inputs")
        d = wl.c2_inputs()
        x, w = to_dev(d["x1"], True), to_dev(wl.x2_as_nk(d)["x2"], True)
        W = 8
        out = torch.empty((8192, 3072), dtype=torch.bfloat16, device=dev)
        flags = torch.zeros(W, dtype=torch.int32, device=dev)
        cnt = torch.zeros(W, dtype=torch.int32, device=dev)
        flop = 2.0 * 8192 * 3072 * 3072
        inf = torch.full((W,), 1, dtype=torch.int32, device=dev)
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        cases = [
            ("c2_ag_mm_bf16", lambda: mc2.mc2_ag_mm_local(
                x, w, W, 0, x2_trans=True, out=out, ready_flags=flags, flag_counters=cnt,
                epoch=1)),
            # consumer-side input flags, all already raised: the cost of the
            # per-tile wait and its system-scope acquire
            ("c2_ag_mm_bf16_inflags", lambda: mc2.mc2_ag_mm_local_inflags(
                x, w, W, 0, inf, 1, x2_trans=True, out=out, ready_flags=flags,
                flag_counters=cnt, epoch=1, dev_err=err)),
        ]
        for name, fn in cases:
            m_, med, it = measure(fn)
            rows[name] = {"ms": m_, "ms_median": med, "iters": it, "TFLOP/s": flop / m_ / 1e9,
                          "frac_peak": flop / m_ / 1e9 / PEAK_BF16}
            log(f"{name}: {m_ * 1e3:.1f} us  {flop / m_ / 1e9:.1f} TFLOP/s")
        assert err.item() == 0
        del w
        w = to_dev(d["x2"], True)
        m_, med, it = measure(lambda: mc2.mc2_ag_mm_local(x, w, W, 0, out=out, ready_flags=flags,
                                                          flag_counters=cnt, epoch=2))
        rows["c2_ag_mm_bf16_x2_kn"] = {"ms": m_, "ms_median": med, "iters": it,
                                       "TFLOP/s": flop / m_ / 1e9,
                                       "frac_peak": flop / m_ / 1e9 / PEAK_BF16}
        log(f"C2 with x2 given (k, n): {m_ * 1e3:.1f} us  {flop / m_ / 1e9:.1f} TFLOP/s")
        del x, w, out

    # ---------------------------------------------------------------- C3
    if only in ("all", "rows", "c3"):
        log("C3: generating inputs")
        d = wl.c3_inputs()
        s1, s2 = to_dev(d["x1_scale"]), to_dev(d["x2_scale"])
        out = torch.empty((4096, 2048), dtype=torch.bfloat16, device=dev)
        flags = torch.zeros(4, dtype=torch.int32, device=dev)
        cnt = torch.zeros(4, dtype=torch.int32, device=dev)
        x1 = to_dev(d["x1"])
        op = 2.0 * 4096 * 8192 * 2048
        # x2 as a transposed (n, k) weight (the row), then given (k, n)
        for name, dd in (("c3_mm_rs_int8", wl.x2_as_nk(d)), ("c3_mm_rs_int8_x2_kn", d)):
            x2 = to_dev(dd["x2"])
            m_, med, it = measure(lambda: mc2.mc2_mm_rs_local(
                x1, x2, 4, 0, x2_trans=dd["x2_trans"], x1_scale=s1, x2_scale=s2, out=out,
                ready_flags=flags, flag_counters=cnt, epoch=1))
            rows[name] = {"ms": m_, "ms_median": med, "iters": it, "TOP/s": op / m_ / 1e9,
                          "frac_peak": op / m_ / 1e9 / PEAK_I8}
            log(f"{name}: {m_ * 1e3:.1f} us  {op / m_ / 1e9:.1f} TOP/s "
                f"({100 * op / m_ / 1e9 / PEAK_I8:.1f}% of peak)")
            del x2
        del x1, out

    # ---------------------------------------------------------------- C4
    if only in ("all", "rows", "c4"):
        log("C4: generating inputs")
        d = wl.c4_inputs()
        T, K, E, E_l, H, I = d["T"], d["K"], d["E"], d["E_l"], d["H"], d["I"]
        x, sel, probs = to_dev(d["x"], True), to_dev(d["sel"]), to_dev(d["probs"])
        w1, w2 = to_dev(d["w1"], True), to_dev(d["w2"], True)
        counts = torch.empty(E, dtype=torch.int32, device=dev)
        perm = torch.empty((T * K, H), dtype=torch.bfloat16, device=dev)
        sidx = torch.empty(T * K, dtype=torch.int32, device=dev)
        uidx = torch.empty(T * K, dtype=torch.int32, device=dev)
        offs = torch.empty(E + 1, dtype=torch.int32, device=dev)
        ws = torch.empty(mc2.mc2_moe_permute_workspace_size(T, K, E), dtype=torch.uint8, device=dev)
        h = torch.empty((T * K, I), dtype=torch.bfloat16, device=dev)
        buf = torch.zeros((T * K, H), dtype=torch.bfloat16, device=dev)
        y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        recv = counts[:E_l]

        def f_histc():
            mc2.mc2_moe_histc(sel, E, counts=counts, dev_err=err)

        def f_perm():
            mc2.mc2_moe_permute(x, sel, E, permuted=perm, sorted_idx=sidx, unpermute_idx=uidx,
                                expert_offsets=offs, workspace=ws, dev_err=err)

        def f_disp():
            mc2.mc2_gmm_dispatch(perm, counts, recv, w1, ep_rank=0, num_experts=E, h_out=h,
                                 dev_err=err)

        def f_comb():
            mc2.mc2_gmm_combine(h, recv, counts, w2, buf, ep_rank=0, num_experts=E, dev_err=err)

        def f_unperm():
            mc2.mc2_moe_unpermute(buf, uidx, probs, out=y, dev_err=err)

        for f in (f_histc, f_perm, f_disp, f_comb, f_unperm):
            f()
        torch.cuda.synchronize()
        assert err.item() == 0
        n_loc = int(counts[:E_l].sum().item())
        t = {name: measure(f) for name, f in (("histc", f_histc), ("permute", f_perm),
                                              ("fc1", f_disp), ("fc2", f_comb),
                                              ("unpermute", f_unperm))}
        t_all = measure(lambda: [f() for f in (f_histc, f_perm, f_disp, f_comb, f_unperm)])
        # histc alone is two launches of a few microseconds: called one by one
        # from Python they run at the host's launch rate, so it is also timed
        # as a replayed graph of 20 calls (the library records no memset)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            f_histc()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g_histc = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_histc):
            for _ in range(20):
                f_histc()
        t_histc_graph = measure(g_histc.replay)
        torch.cuda.synchronize()
        assert err.item() == 0
        fl1 = 2.0 * n_loc * H * 2 * I
        fl2 = 2.0 * n_loc * I * H
        perm_bytes = T * H * 2 + T * K * 4 + T * K * H * 2 + 2 * T * K * 4
        unperm_bytes = T * K * H * 2 + T * K * 4 + T * K * 4 + T * H * 2
        gmm_tf = (fl1 + fl2) / (t["fc1"][0] + t["fc2"][0]) / 1e9
        rows["c4_moe_ep_local"] = {
            "n_loc": n_loc, "ms_step": t_all[0], "ms_step_median": t_all[1],
            "histc_us": t["histc"][0] * 1e3,
            "histc_us_graph": t_histc_graph[0] / 20 * 1e3,
            "permute_us": t["permute"][0] * 1e3, "permute_us_median": t["permute"][1] * 1e3,
            "permute_GB/s": perm_bytes / t["permute"][0] / 1e6,
            "permute_frac_hbm": perm_bytes / t["permute"][0] / 1e6 / PEAK_HBM,
            "gmm_fc1_swiglu_us": t["fc1"][0] * 1e3, "gmm_fc1_swiglu_us_median": t["fc1"][1] * 1e3,
            "gmm_fc2_us": t["fc2"][0] * 1e3, "gmm_fc2_us_median": t["fc2"][1] * 1e3,
            "gmm_TFLOP/s": gmm_tf, "gmm_frac_peak": gmm_tf / PEAK_BF16,
            "fc1_TFLOP/s": fl1 / t["fc1"][0] / 1e9, "fc2_TFLOP/s": fl2 / t["fc2"][0] / 1e9,
            "unpermute_us": t["unpermute"][0] * 1e3,
            "unpermute_us_median": t["unpermute"][1] * 1e3,
            "unpermute_GB/s": unperm_bytes / t["unpermute"][0] / 1e6,
            "unpermute_frac_hbm": unperm_bytes / t["unpermute"][0] / 1e6 / PEAK_HBM,
        }
        log("C4 MoE:", json.dumps(rows["c4_moe_ep_local"]))
        del x, perm, h, buf, y, w1, w2

    # ---------------------------------------------------------------- C4 backward
    if only in ("all", "rows", "c4bwd"):
        # backward of the local expert FFN on the C4 shapes and router counts;
        # the stored activations and incoming gradients are seeded stand-ins
        log("C4 backward: generating inputs")
        d = wl.c4_inputs()
        E, E_l, H, I = d["E"], d["E_l"], d["H"], d["I"]
        sel = to_dev(d["sel"])
        counts = mc2.mc2_moe_histc(sel, E)
        recv = counts[:E_l].clone()
        n_loc = int(recv.sum().item())
        bi = wl.moe_backward_inputs(1006, n_loc, H, I)
        tt = {k: to_dev(v, True) for k, v in bi.items()}
        w1, w2 = to_dev(d["w1"], True), to_dev(d["w2"], True)
        dgrad = torch.empty((n_loc, 2 * I), dtype=torch.bfloat16, device=dev)
        dw2 = torch.empty((E_l, I, H), dtype=torch.float32, device=dev)
        dx = torch.empty((n_loc, H), dtype=torch.bfloat16, device=dev)
        dw1 = torch.empty((E_l, H, 2 * I), dtype=torch.float32, device=dev)
        ws_c = torch.empty(mc2.mc2_gmm_backward_workspace_size(n_loc, E_l, I, H), dtype=torch.uint8,
                           device=dev)
        ws_d = torch.empty(mc2.mc2_gmm_backward_workspace_size(n_loc, E_l, H, 2 * I),
                           dtype=torch.uint8, device=dev)
        err = torch.zeros(1, dtype=torch.int32, device=dev)

        def f_cb():
            mc2.mc2_gmm_combine_backward(tt["dy"], recv, counts, w2, tt["h"], ep_rank=0,
                                         num_experts=E, act=mc2.MC2_ACT_SWIGLU, g_saved=tt["g"],
                                         dgrad_out=dgrad, dw2_out=dw2, workspace=ws_c, dev_err=err)

        def f_db():
            mc2.mc2_gmm_dispatch_backward(tt["dg"], recv, counts, w1, tt["send"], dx, ep_rank=0,
                                          num_experts=E, dw1_out=dw1, workspace=ws_d, dev_err=err)

        f_cb()
        f_db()
        torch.cuda.synchronize()
        assert err.item() == 0
        t_cb, _, _ = measure(f_cb)
        t_db, _, _ = measure(f_db)
        fl_cb = 4.0 * n_loc * I * H
        fl_db = 4.0 * n_loc * 2 * I * H
        tf = (fl_cb + fl_db) / (t_cb + t_db) / 1e9
        rows["c4_moe_backward"] = {
            "n_loc": n_loc, "fc2_backward_us": t_cb * 1e3, "fc1_backward_us": t_db * 1e3,
            "fc2_backward_TFLOP/s": fl_cb / t_cb / 1e9, "fc1_backward_TFLOP/s": fl_db / t_db / 1e9,
            "TFLOP/s": tf, "frac_peak": tf / PEAK_BF16}
        log("C4 backward:", json.dumps(rows["c4_moe_backward"]))
        del tt, w1, w2, dgrad, dw2, dx, dw1, ws_c, ws_d

    # ---------------------------------------------------------------- split granularity
    if only in ("all", "rows", "split"):
        # comm_turn pieces: cost of the finer flags, and when the host sees the
        # first and the last segment flag (flags in host-pinned memory, polled
        # from the moment the launch call returns; median of `reps` launches)
        def flag_times(launch, hf, reps):
            v = hf.numpy()
            firsts, lasts = [], []
            for r in range(reps):
                torch.cuda.synchronize()
                e = 1000 + r
                launch(e)
                t0 = time.perf_counter()
                seen = np.full(v.size, np.nan)
                while np.isnan(seen).any():
                    now = time.perf_counter()
                    seen[(v == e) & np.isnan(seen)] = now - t0
                    if now - t0 > 2.0:
                        raise RuntimeError("segment flags did not arrive")
                torch.cuda.synchronize()
                firsts.append(np.min(seen))
                lasts.append(np.max(seen))
            return float(np.median(firsts)) * 1e6, float(np.median(lasts)) * 1e6

        log("split: generating inputs")
        d = wl.c2_inputs()
        _, b = wl.c5_inputs()
        W = 8
        cases = {
            "c2_ag_mm": (lambda S, out, fl, cn, e: mc2.mc2_ag_mm_local(
                xc2, wc2, W, 0, x2_trans=True, out=out, ready_flags=fl, flag_counters=cn, epoch=e,
                comm_turn=S),
                (8192, 3072), 2.0 * 8192 * 3072 * 3072),
            "c5b_sim_rs": (lambda S, out, fl, cn, e: mc2.mc2_mm_rs_local(
                x1b, x2b, W, 0, x2_trans=True, out=out, ready_flags=fl, flag_counters=cn, epoch=e,
                comm_turn=S),
                (16384, 8192), FLOP_B),
        }
        xc2, wc2 = to_dev(d["x1"], True), to_dev(wl.x2_as_nk(d)["x2"], True)
        x1b, x2b = to_dev(b["x1"], True), to_dev(wl.x2_as_nk(b)["x2"], True)
        del d, b
        split = {}
        for name, (call, shape, flop) in cases.items():
            out = torch.empty(shape, dtype=torch.bfloat16, device=dev)
            for S in (1, 2, 4, 8):
                fl = torch.zeros(W * S, dtype=torch.int32, device=dev)
                cn = torch.zeros(W * S, dtype=torch.int32, device=dev)
                ep = [0]

                def step():
                    ep[0] += 1
                    call(S, out, fl, cn, ep[0])
                m_, med, _ = measure(step, 100.0)
                hf = torch.zeros(W * S, dtype=torch.int32, pin_memory=True)
                first, last = flag_times(lambda e: call(S, out, hf, cn, e), hf, 15)
                split[f"{name}_comm_turn{S}"] = {
                    "ms": m_, "ms_median": med, "TFLOP/s": flop / m_ / 1e9,
                    "first_flag_us": first, "last_flag_us": last}
                log(f"split {name} comm_turn={S}: {m_ * 1e3:.1f} us {flop / m_ / 1e9:.1f} TFLOP/s;"
                    f" host sees first/last flag at {first:.0f}/{last:.0f} us")
        rows["split"] = split
        del xc2, wc2, x1b, x2b, out

    # ---------------------------------------------------------------- CPU oracle
    cpu = None
    if headline is not None and not args.no_cpu_baseline:
        from oracle import gemm as og
        try:
            from threadpoolctl import threadpool_info
            threads = max([i.get("num_threads", 1) for i in threadpool_info()
                           if i.get("user_api") == "blas"] or [1])
        except Exception:  # pragma: no cover - informational only
            threads = len(os.sched_getaffinity(0))
        a, b = c5_kn
        done_a = done_b = 0
        t0 = time.perf_counter()
        # whole 2048-row chunks of both launches of the headline workload,
        # alternating, until ~10 s of work
        while time.perf_counter() - t0 < 10.0:
            if done_a <= done_b:
                c = done_a % 8
                og.ag_mm(a["x1"], a["x2"], world_size=8, in_dtype="bf16",
                         rows=np.arange(c * 2048, (c + 1) * 2048))
                done_a += 1
            else:
                c = done_b % 8
                og.mm_rs(b["x1"], b["x2"], world_size=8, in_dtype="bf16", nsim=8,
                         rows=np.arange(c * 2048, (c + 1) * 2048))
                done_b += 1
        dt = time.perf_counter() - t0
        flop = (done_a * FLOP_A + done_b * FLOP_B) / 8
        cpu = {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
               "cpu_model": cpu_model(),
               "sample": f"oracle.gemm.ag_mm and oracle.gemm.mm_rs (float64 NumPy BLAS) on "
                         f"{done_a} + {done_b} whole 2048-row output chunks of the headline "
                         f"workload's two launches (1/8 of each launch per chunk), {dt:.1f} s"}
        log("CPU oracle:", json.dumps(cpu))

    if headline is None:
        print(json.dumps({"rows": rows}))
        return
    kt = headline["kernel_tflops"]
    line = {
        "metric": METRIC,
        "value": headline["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": headline["ms"],
        "ms_per_step_median": headline["ms_median"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0, 0.02) bf16 inputs resident in HBM)",
        "config": {"workload": "large configuration, both launches per step: AllGatherMatmul "
                               "local share, gathered x of W=8 chunks (16384, 8192) @ weight "
                               "(8192, 3584), and the simulated W=8 MatmulReduceScatter of 8 "
                               "k-shards (16384, 1024) @ (1024, 8192) into 8 chunks of 2048 "
                               "rows; bf16, fp32 accumulation, rank 0, per-chunk ready flags, "
                               "each weight held (n, k) and passed transposed (x2_trans); "
                               "*_x2_kn rows time x2 given (k, n)",
                   "world_size": 8, "flop_per_step": FLOP_A + FLOP_B,
                   "settle_s": args.settle, "settle_steps": headline["settle_steps"]},
        "roofline": {"bound": "mfma", "achieved": kt, "peak": PEAK_BF16, "unit": "TFLOP/s",
                     "frac": kt / PEAK_BF16, "traffic": recorded_traffic(),
                     "kernel": "chunked_gemm_kernel (bf16, x2 (n, k), 256 x 256 tiles); "
                               "achieved = mean FLOPs per launch / mean launch time of its "
                               "two launches per step",
                     "launch_ms": headline["launch_ms"],
                     "algorithmic_bytes_per_launch": (BYTES_A + BYTES_B) / 2},
        "sclk": clock.report(),
        "cpu_baseline": cpu,
        "rows": rows,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
