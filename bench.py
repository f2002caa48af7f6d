"""Throughput of the MC2 compute core on one MI355X.

Headline step: the AllGatherMatmul local share in bf16 -- gathered x of W=8
chunks of (1024, 3072) = (8192, 3072) @ weight (3072, 3072), chunks computed in
rank order with per-chunk ready flags -- reported as TFLOP/s of the rank-chunked
GEMM kernel. The weight is held as an (n, k) Linear weight and passed
transposed (x2_trans), which the operator's x2 argument allows; the same
products with x2 given (k, n) are reported as the *_x2_kn rows. The same JSON line carries the other hot-path rows measured the
same way (int8 quantized MatmulReduceScatter, the MoE expert-parallel local
path, the large AllGatherMatmul and the simulated W=8 MatmulReduceScatter),
the roofline of the dominant kernel and the CPU oracle timed on a bounded
sample of the headline workload.

Inputs are seeded synthetic data resident in HBM before timing starts. Times
come from HIP events on the stream the kernels are launched on.

    python bench.py [--steps K] [--warmup W] [--only c2|c3|c4|c4bwd|c5a|c5b|split|all]
                    [--no-cpu-baseline] [--calib-copy]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
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
                  "gemm_collective_core_amd/csrc/mc2_tiles.hpp",
                  "gemm_collective_core_amd/csrc/mc2_chunked.hpp",
                  "gemm_collective_core_amd/csrc/mc2_gemm.hip",
                  "gemm_collective_core_amd/csrc/mc2_common.hpp",
                  "gemm_collective_core_amd/csrc/mc2_host.hpp"]
TRAFFIC_FILE = "profiles/traffic_ag_mm_bf16_8192x3072x3072.json"
# The headline launch the recorded traffic must belong to.
HEADLINE_LAUNCH = "ag_mm bf16 8192x3072x3072 W=8 rank 0, x2 (n, k) with x2_trans, ready flags"


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


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=500)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--only", default="all")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--calib-copy", action="store_true",
                   help="run only a plain 1 GiB device copy (HBM counter calibration)")
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

    def timed(fn, iters, warmup):
        """Mean milliseconds per call of fn() over `iters` calls, HIP events on
        the current stream (the stream every entry point launches on)."""
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(iters):
            fn()
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / iters

    if args.calib_copy:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        ms = timed(lambda: b.copy_(a), 20, 3)
        log(f"copy 1 GiB: {ms:.3f} ms -> {2 * n / ms / 1e6:.1f} GB/s (read+write)")
        print(json.dumps({"calib_copy_bytes_read": n, "calib_copy_bytes_written": n,
                          "ms": ms, "GBps": 2 * n / ms / 1e6}))
        return

    only = args.only
    rows = {}
    headline = None

    # ---------------------------------------------------------------- C2
    if only in ("all", "c2"):
        log("C2: generating inputs")
        d = wl.c2_inputs()
        # the weight held as an (n, k) Linear weight and passed transposed
        x, w = to_dev(d["x1"], True), to_dev(wl.x2_as_nk(d)["x2"], True)
        W = 8
        out = torch.empty((8192, 3072), dtype=torch.bfloat16, device=dev)
        flags = torch.zeros(W, dtype=torch.int32, device=dev)
        cnt = torch.zeros(W, dtype=torch.int32, device=dev)
        ep = [0]

        def step():
            ep[0] += 1
            mc2.mc2_ag_mm_local(x, w, W, 0, x2_trans=True, out=out, ready_flags=flags,
                                flag_counters=cnt, epoch=ep[0])
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        start.record()
        for _ in range(args.steps):
            step()
        end.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = start.elapsed_time(end) / args.steps
        assert flags.cpu().tolist() == [ep[0]] * W
        flop = 2.0 * 8192 * 3072 * 3072
        tf = flop / ms / 1e9
        headline = {"ms": ms, "tflops": tf, "wall_s": wall, "flop": flop}
        rows["c2_ag_mm_bf16"] = {"ms": ms, "TFLOP/s": tf, "frac_peak": tf / PEAK_BF16}
        log(f"C2 AG-MM bf16: {ms * 1e3:.1f} us  {tf:.1f} TFLOP/s  ({100 * tf / PEAK_BF16:.1f}% of peak)")
        # The same launch with consumer-side input flags (all already raised):
        # the cost of the per-tile wait and its system-scope acquire.
        inf = torch.full((W,), 1, dtype=torch.int32, device=dev)
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        ms_w = timed(lambda: mc2.mc2_ag_mm_local_inflags(
            x, w, W, 0, inf, 1, x2_trans=True, out=out, ready_flags=flags, flag_counters=cnt,
            epoch=1, dev_err=err), 200, 20)
        assert err.item() == 0
        rows["c2_ag_mm_bf16_inflags"] = {"ms": ms_w, "TFLOP/s": flop / ms_w / 1e9,
                                         "frac_peak": flop / ms_w / 1e9 / PEAK_BF16}
        log(f"C2 with input flags: {ms_w * 1e3:.1f} us  {flop / ms_w / 1e9:.1f} TFLOP/s")
        # the same launch with x2 given (k, n)
        del w
        w = to_dev(d["x2"], True)
        ms_kn = timed(lambda: mc2.mc2_ag_mm_local(x, w, W, 0, out=out, ready_flags=flags,
                                                  flag_counters=cnt, epoch=2), 200, 20)
        rows["c2_ag_mm_bf16_x2_kn"] = {"ms": ms_kn, "TFLOP/s": flop / ms_kn / 1e9,
                                       "frac_peak": flop / ms_kn / 1e9 / PEAK_BF16}
        log(f"C2 with x2 given (k, n): {ms_kn * 1e3:.1f} us  {flop / ms_kn / 1e9:.1f} TFLOP/s")
        del x, w, out

    # ---------------------------------------------------------------- C3
    if only in ("all", "c3"):
        log("C3: generating inputs")
        d = wl.c3_inputs()
        s1, s2 = to_dev(d["x1_scale"]), to_dev(d["x2_scale"])
        out = torch.empty((4096, 2048), dtype=torch.bfloat16, device=dev)
        flags = torch.zeros(4, dtype=torch.int32, device=dev)
        cnt = torch.zeros(4, dtype=torch.int32, device=dev)
        x1 = to_dev(d["x1"])
        # x2 as a transposed (n, k) weight (the row), then given (k, n)
        for name, dd in (("c3_mm_rs_int8", wl.x2_as_nk(d)), ("c3_mm_rs_int8_x2_kn", d)):
            x2 = to_dev(dd["x2"])
            ms = timed(lambda: mc2.mc2_mm_rs_local(x1, x2, 4, 0, x2_trans=dd["x2_trans"],
                                                   x1_scale=s1, x2_scale=s2, out=out,
                                                   ready_flags=flags, flag_counters=cnt, epoch=1),
                       1000, 50)
            top = 2.0 * 4096 * 8192 * 2048 / ms / 1e9
            rows[name] = {"ms": ms, "TOP/s": top, "frac_peak": top / PEAK_I8}
            log(f"{name}: {ms * 1e3:.1f} us  {top:.1f} TOP/s  ({100 * top / PEAK_I8:.1f}% of peak)")
            del x2
        del x1, out

    # ---------------------------------------------------------------- C4
    if only in ("all", "c4"):
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
        t_h = timed(f_histc, 500, 20)
        t_p = timed(f_perm, 200, 10)
        t_d = timed(f_disp, 200, 10)
        t_c = timed(f_comb, 200, 10)
        t_u = timed(f_unperm, 200, 10)
        t_all = timed(lambda: [f() for f in (f_histc, f_perm, f_disp, f_comb, f_unperm)], 100, 5)
        gmm_flop = 2.0 * n_loc * H * 2 * I + 2.0 * n_loc * I * H
        perm_bytes = T * H * 2 + T * K * 4 + T * K * H * 2 + 2 * T * K * 4
        unperm_bytes = T * K * H * 2 + T * K * 4 + T * K * 4 + T * H * 2
        gmm_tf = gmm_flop / (t_d + t_c) / 1e9
        rows["c4_moe_ep_local"] = {
            "n_loc": n_loc, "ms_step": t_all,
            "histc_us": t_h * 1e3,
            "permute_us": t_p * 1e3, "permute_GB/s": perm_bytes / t_p / 1e6,
            "permute_frac_hbm": perm_bytes / t_p / 1e6 / PEAK_HBM,
            "gmm_fc1_swiglu_us": t_d * 1e3, "gmm_fc2_us": t_c * 1e3,
            "gmm_TFLOP/s": gmm_tf, "gmm_frac_peak": gmm_tf / PEAK_BF16,
            "fc1_TFLOP/s": 2.0 * n_loc * H * 2 * I / t_d / 1e9,
            "fc2_TFLOP/s": 2.0 * n_loc * I * H / t_c / 1e9,
            "unpermute_us": t_u * 1e3, "unpermute_GB/s": unperm_bytes / t_u / 1e6,
            "unpermute_frac_hbm": unperm_bytes / t_u / 1e6 / PEAK_HBM,
        }
        log("C4 MoE:", json.dumps(rows["c4_moe_ep_local"]))
        del x, perm, h, buf, y, w1, w2

    # ---------------------------------------------------------------- C4 backward
    if only in ("all", "c4bwd"):
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
        t = {k: to_dev(v, True) for k, v in bi.items()}
        w1, w2 = to_dev(d["w1"], True), to_dev(d["w2"], True)
        dgrad = torch.empty((n_loc, 2 * I), dtype=torch.bfloat16, device=dev)
        dw2 = torch.empty((E_l, I, H), dtype=torch.float32, device=dev)
        dx = torch.empty((n_loc, H), dtype=torch.bfloat16, device=dev)
        dw1 = torch.empty((E_l, H, 2 * I), dtype=torch.float32, device=dev)
        ws_c = torch.empty(mc2.mc2_gmm_backward_workspace_size(n_loc, E_l, I, H), dtype=torch.uint8,
                           device=dev)
        ws_d = torch.empty(mc2.mc2_gmm_backward_workspace_size(n_loc, E_l, H, 2 * I), dtype=torch.uint8,
                           device=dev)
        err = torch.zeros(1, dtype=torch.int32, device=dev)

        def f_cb():
            mc2.mc2_gmm_combine_backward(t["dy"], recv, counts, w2, t["h"], ep_rank=0,
                                         num_experts=E, act=mc2.MC2_ACT_SWIGLU, g_saved=t["g"],
                                         dgrad_out=dgrad, dw2_out=dw2, workspace=ws_c, dev_err=err)

        def f_db():
            mc2.mc2_gmm_dispatch_backward(t["dg"], recv, counts, w1, t["send"], dx, ep_rank=0,
                                          num_experts=E, dw1_out=dw1, workspace=ws_d, dev_err=err)

        f_cb()
        f_db()
        torch.cuda.synchronize()
        assert err.item() == 0
        t_cb = timed(f_cb, 100, 10)
        t_db = timed(f_db, 100, 10)
        fl_cb = 4.0 * n_loc * I * H
        fl_db = 4.0 * n_loc * 2 * I * H
        tf = (fl_cb + fl_db) / (t_cb + t_db) / 1e9
        rows["c4_moe_backward"] = {
            "n_loc": n_loc, "fc2_backward_us": t_cb * 1e3, "fc1_backward_us": t_db * 1e3,
            "fc2_backward_TFLOP/s": fl_cb / t_cb / 1e9, "fc1_backward_TFLOP/s": fl_db / t_db / 1e9,
            "TFLOP/s": tf, "frac_peak": tf / PEAK_BF16}
        log("C4 backward:", json.dumps(rows["c4_moe_backward"]))
        del t, w1, w2, dgrad, dw2, dx, dw1, ws_c, ws_d

    # ---------------------------------------------------------------- C5
    if only in ("all", "c5a", "c5b"):
        log("C5: generating inputs")
        a, b = wl.c5_inputs()
        W = 8
        if only in ("all", "c5a"):
            x = to_dev(a["x1"], True)
            out = torch.empty((16384, 3584), dtype=torch.bfloat16, device=dev)
            flags = torch.zeros(W, dtype=torch.int32, device=dev)
            cnt = torch.zeros(W, dtype=torch.int32, device=dev)
            # x2 as a transposed (n, k) weight (the row), then given (k, n)
            for name, aa in (("c5a_ag_mm_bf16", wl.x2_as_nk(a)), ("c5a_ag_mm_bf16_x2_kn", a)):
                w = to_dev(aa["x2"], True)
                ms = timed(lambda: mc2.mc2_ag_mm_local(x, w, W, 0, x2_trans=aa["x2_trans"],
                                                       out=out, ready_flags=flags,
                                                       flag_counters=cnt, epoch=1), 100, 10)
                tf = 2.0 * 16384 * 8192 * 3584 / ms / 1e9
                rows[name] = {"ms": ms, "TFLOP/s": tf, "frac_peak": tf / PEAK_BF16}
                log(f"{name}: {ms * 1e3:.1f} us  {tf:.1f} TFLOP/s")
                del w
            del x, out
        if only in ("all", "c5b"):
            x1 = to_dev(b["x1"], True)
            out = torch.empty((16384, 8192), dtype=torch.bfloat16, device=dev)
            flags = torch.zeros(W, dtype=torch.int32, device=dev)
            cnt = torch.zeros(W, dtype=torch.int32, device=dev)
            x2 = to_dev(b["x2"], True)
            ms = timed(lambda: mc2.mc2_mm_rs_local(x1, x2, W, 0, out=out, ready_flags=flags,
                                                   flag_counters=cnt, epoch=1), 50, 5)
            tf = 2.0 * 8 * 16384 * 1024 * 8192 / ms / 1e9
            rows["c5b_sim_rs_bf16_x2_kn"] = {"ms": ms, "TFLOP/s": tf, "frac_peak": tf / PEAK_BF16}
            log(f"C5b sim-W=8 MM-RS, x2 given (k, n): {ms * 1e3:.1f} us  {tf:.1f} TFLOP/s")
            # the row and everything after it: x2 shards as transposed (n, k) weights
            del x2
            x2 = to_dev(wl.x2_as_nk(b)["x2"], True)
            ms = timed(lambda: mc2.mc2_mm_rs_local(x1, x2, W, 0, x2_trans=True, out=out,
                                                   ready_flags=flags, flag_counters=cnt, epoch=1),
                       50, 5)
            tf = 2.0 * 8 * 16384 * 1024 * 8192 / ms / 1e9
            rows["c5b_sim_rs_bf16"] = {"ms": ms, "TFLOP/s": tf, "frac_peak": tf / PEAK_BF16}
            log(f"C5b sim-W=8 MM-RS: {ms * 1e3:.1f} us  {tf:.1f} TFLOP/s")
            # MatmulAllReduce local share on the same partials, per rounding model
            ws = torch.empty(mc2.mc2_mm_ar_workspace_size(16384, 8192, W, torch.bfloat16,
                                                          mc2.MC2_AR_HOP_ROUNDED),
                             dtype=torch.uint8, device=dev)
            for mode, name in ((mc2.MC2_AR_ONE_ROUNDING, "one"), (mc2.MC2_AR_RANK_ROUNDED, "rank"),
                               (mc2.MC2_AR_HOP_ROUNDED, "hop")):
                ms = timed(lambda: mc2.mc2_mm_ar_local(x1, x2, W, rounding=mode, x2_trans=True,
                                                       out=out, workspace=ws), 30, 3)
                tf = 2.0 * 8 * 16384 * 1024 * 8192 / ms / 1e9
                rows[f"c5b_mm_ar_{name}_rounding_bf16"] = {"ms": ms, "TFLOP/s": tf,
                                                           "frac_peak": tf / PEAK_BF16}
                log(f"C5b MM-AR ({name} rounding): {ms * 1e3:.1f} us  {tf:.1f} TFLOP/s")
            # the combining step alone: W stored partials read, one result written
            parts = ws[: W * 16384 * 8192 * 2].view(torch.bfloat16).view(W, 16384, 8192)
            ms = timed(lambda: mc2.mc2_ar_sum_local(parts, mc2.MC2_AR_HOP_ROUNDED, out=out), 50, 5)
            nbytes = (W + 1) * 16384 * 8192 * 2
            rows["c5b_ar_sum_bf16"] = {"ms": ms, "GB/s": nbytes / ms / 1e6,
                                       "frac_hbm": nbytes / ms / 1e6 / PEAK_HBM}
            log(f"C5b AR combine: {ms * 1e3:.1f} us  {nbytes / ms / 1e6:.0f} GB/s")
            del x1, x2, out, ws, parts

    # ---------------------------------------------------------------- split granularity
    if only in ("all", "split"):
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
                (8192, 3072), 2.0 * 8192 * 3072 * 3072, 200),
            "c5b_sim_rs": (lambda S, out, fl, cn, e: mc2.mc2_mm_rs_local(
                x1b, x2b, W, 0, x2_trans=True, out=out, ready_flags=fl, flag_counters=cn, epoch=e,
                comm_turn=S),
                (16384, 8192), 2.0 * 8 * 16384 * 1024 * 8192, 30),
        }
        xc2, wc2 = to_dev(d["x1"], True), to_dev(wl.x2_as_nk(d)["x2"], True)
        x1b, x2b = to_dev(b["x1"], True), to_dev(wl.x2_as_nk(b)["x2"], True)
        split = {}
        for name, (call, shape, flop, iters) in cases.items():
            out = torch.empty(shape, dtype=torch.bfloat16, device=dev)
            for S in (1, 2, 4, 8):
                fl = torch.zeros(W * S, dtype=torch.int32, device=dev)
                cn = torch.zeros(W * S, dtype=torch.int32, device=dev)
                ep = [0]

                def step():
                    ep[0] += 1
                    call(S, out, fl, cn, ep[0])
                ms = timed(step, iters, max(iters // 10, 2))
                hf = torch.zeros(W * S, dtype=torch.int32, pin_memory=True)
                first, last = flag_times(lambda e: call(S, out, hf, cn, e), hf, 15)
                split[f"{name}_comm_turn{S}"] = {
                    "ms": ms, "TFLOP/s": flop / ms / 1e9, "first_flag_us": first,
                    "last_flag_us": last}
                log(f"split {name} comm_turn={S}: {ms * 1e3:.1f} us {flop / ms / 1e9:.1f} TFLOP/s;"
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
        d = wl.c2_inputs()
        done, t0 = 0, time.perf_counter()
        # whole row chunks of the headline workload, repeated until ~10 s of work
        while time.perf_counter() - t0 < 10.0 and done < 1024:
            c = done % 8
            og.ag_mm(d["x1"], d["x2"], world_size=8, in_dtype="bf16",
                     rows=np.arange(c * 1024, (c + 1) * 1024))
            done += 1
        dt = time.perf_counter() - t0
        cpu = {"value": 2.0 * 1024 * done * 3072 * 3072 / dt / 1e12, "unit": "TFLOP/s",
               "cores": threads, "kind": "oracle",
               "sample": f"oracle.gemm.ag_mm (float64 NumPy BLAS) on {done} row chunks "
                         f"(1024 x 3072 @ 3072 x 3072 each, the headline workload's chunks "
                         f"cycled), {dt:.1f} s"}
        log("CPU oracle:", json.dumps(cpu))

    if headline is None:
        print(json.dumps({"rows": rows}))
        return
    line = {
        "metric": METRIC,
        "value": headline["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": headline["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0, 0.02) bf16 inputs resident in HBM)",
        "config": {"workload": "AllGatherMatmul local share: gathered x of W=8 chunks "
                               "(8192, 3072) @ weight (3072, 3072) bf16, the weight held as an "
                               "(n, k) Linear weight and passed transposed (x2_trans), fp32 "
                               "accumulation, chunks in rank order from rank 0, per-chunk ready "
                               "flags; rows c2_ag_mm_bf16_x2_kn and *_x2_kn time x2 given (k, n)",
                   "world_size": 8, "m": 8192, "k": 3072, "n": 3072, "x2_layout": "(n, k), x2_trans"},
        "roofline": {"bound": "mfma", "achieved": headline["tflops"], "peak": PEAK_BF16,
                     "unit": "TFLOP/s", "frac": headline["tflops"] / PEAK_BF16,
                     "traffic": recorded_traffic()},
        "cpu_baseline": cpu,
        "rows": rows,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
