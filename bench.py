#!/usr/bin/env python3
"""Benchmark of the W8A8 dynamic-quant linear on one MI355X.

Workload (the wq_a-shaped decode linear of "DeepSeek-V4 W8A8 性能分析", section 三):
X bf16 [M, 4096] ~ N(0,1) with 0.5% outliers x30, M in {1,2,4,7,8,16,32,64}, against
W int8 [4096 -> 1024] with f32 per-channel scales.  One step = the fused quant+GEMM
linear (one launch) once at every M of the sweep.  Inputs are resident in HBM and rotate
over enough distinct copies (>= 512 MiB) that neither L2 nor the 256 MB Infinity Cache
holds the weights between calls.  Each step is captured in a HIP graph so the host launch
rate does not bound the measurement.

Printed: one JSON line with the metric (mean us per fused call over the sweep), the
per-M sweep (fused and standalone quant+GEMM, GB/s, fraction of the 8 TB/s HBM peak),
the M=8192 wide-linear prefill point (int8 TOPS against 5.0 POPS), the roofline object
for the dominant kernel and the CPU oracle baseline.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
INT8_PEAK_TOPS = 5000.0
SWEEP = (1, 2, 4, 7, 8, 16, 32, 64)
K_A, N_A = 4096, 1024
ROTATE_BYTES = 512 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fused_decode_wq_a.json")


def fused_bytes(M, K=K_A, N=N_A):
    """Algorithmic HBM bytes of one fused call: X bf16 in, W int8, w_scale f32, Y bf16 out."""
    return 2 * M * K + K * N + 4 * N + 2 * M * N


def standalone_bytes(M, K=K_A, N=N_A):
    """Quant (read X, write x_q and x_scale) + GEMM (read x_q, x_scale, W, w_scale, write Y)."""
    return fused_bytes(M, K, N) + 2 * M * K + 8 * M


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("k_decode.hip", "k_quant.hip", "wq_device.h", "wq_api.hip"):
        with open(os.path.join(ROOT, "fp8_dynamic_quant_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def cpu_baseline(budget_s=10.0):
    """Time the CPU oracle (as it stands) on the same workload: the full fused chain at
    every M of the sweep, repeated until about budget_s seconds have passed."""
    import numpy as np

    import synthetic as syn
    from oracle import int8_linear as il

    try:
        from threadpoolctl import threadpool_info

        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    data = {M: syn.wq_a_linear(M) for M in SWEEP}
    calls, t0 = 0, time.perf_counter()
    while True:
        for M in SWEEP:
            x, w, sw = data[M]
            il.linear_w8a8(x, w, sw)
            calls += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {
        "value": el / calls * 1e6,
        "unit": "us per fused W8A8 linear call (mean over the M sweep)",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{calls} oracle calls ({calls // len(SWEEP)} passes over M in {list(SWEEP)}, K=4096, N=1024) in "
                  f"{el:.1f} s",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-sweep", action="store_true", help="skip the per-M breakdown and the floors")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the kernels run on one MI355X and the "
              f"multi-GPU sharding is described, not run.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fp8_dynamic_quant_amd as wq
    import synthetic as syn

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    wq.lib()

    # ---- inputs: R rotating copies of W / w_scale / X / Y per M --------------------------
    R = max(2, ROTATE_BYTES // (K_A * N_A))
    x_host = {M: syn.wq_a_linear(M)[0] for M in SWEEP}
    w_host, sw_host = syn.int8_weights((2, 21, 1), N_A, K_A)
    w0 = torch.from_numpy(w_host).to(dev)
    sw0 = torch.from_numpy(sw_host).to(dev)
    ws = [w0.clone() for _ in range(R)]
    sws = [sw0.clone() for _ in range(R)]
    xs = {M: [torch.from_numpy(x_host[M].view(np.int16)).to(dev).view(torch.bfloat16).clone() for _ in range(R)]
          for M in SWEEP}
    ys = {M: [torch.empty((M, N_A), dtype=torch.bfloat16, device=dev) for _ in range(R)] for M in SWEEP}
    xq = {M: [torch.empty((M, K_A), dtype=torch.int8, device=dev) for _ in range(R)] for M in SWEEP}
    xsc = {M: [torch.empty((M,), dtype=torch.float32, device=dev) for _ in range(R)] for M in SWEEP}

    # one correctness check against the oracle before timing (the full parity suite is in tests/)
    from oracle import int8_linear as il  # noqa: E402  (checker only; not on the timed path)

    for M in (1, 64):
        y = wq.wq_fused_quant_matmul(xs[M][0], ws[0], sws[0])
        ref = il.linear_w8a8(x_host[M], w_host, sw_host)["y"]
        got = y.view(torch.int16).cpu().numpy().view(np.uint16)
        from oracle.numerics import bf16_ulp_distance

        assert bf16_ulp_distance(got, ref).max() <= 1, "fused linear disagrees with the oracle"

    stream = torch.cuda.Stream()

    def graph_len(steps):
        """Steps per captured graph: the largest divisor of `steps` not above R, so the
        timed region is a whole number of replays and each step uses its own copy."""
        for g in range(min(steps, R), 0, -1):
            if steps % g == 0:
                return g
        return 1

    def capture(fn, n):
        """One graph running fn(r) for r = 0..n-1 back to back (one rotation slot each), so
        the GPU runs the kernels without host gaps between them."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            for r in range(min(n, 2)):
                fn(r)  # eager warm calls on the side stream
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=stream):
                for r in range(n):
                    fn(r)
        torch.cuda.synchronize()
        return g

    def fused_step(r, Ms=SWEEP):
        for M in Ms:
            wq.wq_fused_quant_matmul(xs[M][r], ws[r], sws[r], y=ys[M][r])

    def standalone_step(r, Ms=SWEEP):
        for M in Ms:
            wq.wq_dynamic_quant(xs[M][r], x_q=xq[M][r], x_scale=xsc[M][r])
            wq.wq_quant_matmul(xq[M][r], xsc[M][r], ws[r], sws[r], y=ys[M][r])

    def time_graph(g, n_per_graph, steps, warmup):
        """Replay g (n_per_graph steps each) to cover `warmup`, then exactly `steps` steps
        between two events on the replay stream; returns us per step."""
        reps = max(1, steps // n_per_graph)
        with torch.cuda.stream(stream):
            for _ in range(max(1, -(-warmup // n_per_graph))):
                g.replay()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                g.replay()
            b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / (reps * n_per_graph)

    # ---- headline: fused decode linear over the sweep -------------------------------------
    G = graph_len(args.steps)
    g_all = capture(lambda r: fused_step(r), G)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    us_step = time_graph(g_all, G, args.steps, args.warmup)
    wall = time.perf_counter() - t0
    us_per_call = us_step / len(SWEEP)
    del g_all

    # ---- per-M: fused and standalone ------------------------------------------------------
    sweep = []
    for M in ([] if args.no_sweep else SWEEP):
        gf = capture(lambda r, M=M: fused_step(r, (M,)), R)
        us_f = time_graph(gf, R, 4 * R, R)
        del gf
        gs = capture(lambda r, M=M: standalone_step(r, (M,)), R)
        us_s = time_graph(gs, R, 4 * R, R)
        del gs
        bf, bs = fused_bytes(M), standalone_bytes(M)
        sweep.append({
            "M": M,
            "us_fused": round(us_f, 3),
            "us_standalone_quant_plus_gemm": round(us_s, 3),
            "fused_GBps": round(bf / us_f / 1e3, 1),
            "fused_frac_hbm": round(bf / us_f / 1e3 / HBM_PEAK_GBS, 4),
            "algorithmic_bytes": bf,
            "standalone_bytes": bs,
            "TOPS": round(2 * M * K_A * N_A / us_f / 1e6, 3),
        })
        torch.cuda.synchronize()

    # reference floors: an empty-ish launch and a plain same-size device copy
    tiny = torch.zeros(1, device=dev)
    src = torch.empty(K_A * N_A, dtype=torch.uint8, device=dev)
    dst_bufs = [torch.empty_like(src) for _ in range(R)]

    def floor_step(r):
        for _ in SWEEP:
            tiny.add_(1.0)

    def copy_step(r):
        dst_bufs[r].copy_(ws[r].view(-1))

    launch_floor = copy_us = float("nan")
    if not args.no_sweep:
        g_floor = capture(floor_step, R)
        launch_floor = time_graph(g_floor, R, 4 * R, R) / len(SWEEP)
        g_copy = capture(copy_step, R)
        copy_us = time_graph(g_copy, R, 4 * R, R)
        del g_floor, g_copy

    # ---- prefill point: wq_b-shaped M=8192, K=1024, N=32768 -----------------------------
    prefill = None
    if not args.no_prefill:
        Mp, Kp, Np = 8192, 1024, 32768
        xp = torch.from_numpy(syn.wq_b_x(Mp).view(np.int16)).to(dev).view(torch.bfloat16)
        wp_h, swp_h = syn.wq_b_w()
        wp = [torch.from_numpy(wp_h).to(dev) for _ in range(2)]
        swp = torch.from_numpy(swp_h).to(dev)
        xqp, xsp = wq.wq_dynamic_quant(xp)
        yp = torch.empty((Mp, Np), dtype=torch.bfloat16, device=dev)
        for i in range(3):
            wq.wq_quant_matmul(xqp, xsp, wp[i % 2], swp, y=yp)
        torch.cuda.synchronize()
        n_it = 10
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(n_it):
            wq.wq_quant_matmul(xqp, xsp, wp[i % 2], swp, y=yp)
        b.record()
        torch.cuda.synchronize()
        us_p = a.elapsed_time(b) / n_it * 1e3
        tops = 2 * Mp * Np * Kp / us_p / 1e6
        prefill = {"workload": "wq_b wide linear GEMM (x_q given): M=8192, K=1024, N=32768, bf16 out",
                   "us": round(us_p, 2), "TOPS": round(tops, 1), "frac_int8_peak": round(tops / INT8_PEAK_TOPS, 4)}
        del xp, wp, yp, xqp

    # ---- roofline of the dominant kernel (the fused decode launch), over the sweep -------
    total_bytes = sum(fused_bytes(M) for M in SWEEP)
    achieved = total_bytes / us_step / 1e3  # GB/s
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        try:
            tr = json.load(open(TRAFFIC_FILE))
            if tr.get("kernel_source_hash") == kernel_source_hash():
                traffic = tr.get("bytes_per_step")
        except Exception:
            traffic = None

    out = {
        "metric": "W8A8 linear us & % HBM roofline at M=1..64 (K4096,N1024); int8 TOPS at M=8192",
        "value": round(us_per_call, 3),
        "unit": "us per fused W8A8 linear call (mean over M in 1,2,4,7,8,16,32,64)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_step / 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "wq_a decode linear, fused quant+GEMM: X bf16 [M,4096] x W int8 [4096->1024], "
                               "M in 1,2,4,7,8,16,32,64",
                   "K": K_A, "N": N_A, "M_sweep": list(SWEEP), "rotating_copies": R},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "k_decode<MT,NT,FUSED,A_LDS> (wq_fused_quant_matmul; M > 8 adds k_dynamic_quant)",
                     "bytes_per_step": total_bytes, "us_per_step_events": round(us_step, 3)},
        "sweep": sweep,
        "prefill_m8192": prefill,
        "floors": {"graph_launch_us_per_tiny_kernel": round(launch_floor, 3),
                   "copy_4MiB_us": round(copy_us, 3), "copy_4MiB_GBps": round(2 * K_A * N_A / copy_us / 1e3, 1)},
        "timed_wall_s": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
