#!/usr/bin/env python3
"""Benchmark of the W8A8 dynamic-quant linear on one MI355X.

Workload (the wq_a-shaped decode linear of "DeepSeek-V4 W8A8 性能分析", section 三):
X bf16 [M, 4096] ~ N(0,1) with 0.5% outliers x30, M in {1,2,4,7,8,16,32,64}, against
W int8 [4096 -> 1024] with f32 per-channel scales.  One step = the fused quant+GEMM
linear once at every M of the sweep.  Inputs are resident in HBM and rotate over enough
distinct copies (>= 512 MiB) that neither L2 nor the 256 MB Infinity Cache holds the
weights between calls.  Steps are captured in HIP graphs so the host launch rate does not
bound the measurement.

Printed: one JSON line with the metric (mean us per fused call over the sweep), the
per-M sweep (fused and standalone quant+GEMM, GB/s, fraction of the 8 TB/s HBM peak),
the roofline object of the dominant kernel, and one measurement per remaining step of the
path: the M=8192 wide-linear prefill GEMM (int8 TOPS), the standalone quant, the FP8
per-token-group quant with packed UE8M0 scales and the grouped FP8 contraction, and the
expert-sorted MoE block; then the CPU oracle baseline.

--traffic-probe runs only the roofline kernel's launches (plus a copy kernel of known
size that calibrates the counters) for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs;
--traffic-summary FETCH_DIR WRITE_DIR PROBE_LOG turns the two runs' counter CSVs (and the
probe's printed line) into the JSON the roofline object reads its `traffic` from.
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
FP8_PEAK_TOPS = 5000.0
SWEEP = (1, 2, 4, 7, 8, 16, 32, 64)
K_A, N_A = 4096, 1024
ROTATE_BYTES = 512 << 20
ROOFLINE_KERNEL = "k_fused_decode"  # the one-launch fused kernel on fragment-order weights, every <R, CT> instance
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_k_fused_decode_wq_a.json")
TRACE_FILE = os.path.join(ROOT, "profiles", "kernel_trace_k_fused_decode_wq_a.json")
KERNEL_SOURCES = ("k_fused.hip", "wq_device.h", "wq_kernels.h")  # the roofline kernel and the headers it includes


def fused_bytes(M, K=K_A, N=N_A):
    """Algorithmic HBM bytes of one fused call: X bf16 in, W int8, w_scale f32, Y bf16 out."""
    return 2 * M * K + K * N + 4 * N + 2 * M * N


def standalone_bytes(M, K=K_A, N=N_A):
    """Quant (read X, write x_q and x_scale) + GEMM (read x_q, x_scale, W, w_scale, write Y)."""
    return fused_bytes(M, K, N) + 2 * M * K + 8 * M


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "fp8_dynamic_quant_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_summary(fetch_dir, write_dir, probe_log):
    """HBM bytes per roofline-kernel launch from two rocprofv3 --pmc runs of --traffic-probe
    (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by what the same counter
    reads for the probe's final 64 MiB device copy."""
    import csv

    probe = None
    for line in open(probe_log):
        line = line.strip()
        if line.startswith("{") and "traffic_probe" in line:
            probe = json.loads(line)["traffic_probe"]
    if probe is None:
        raise SystemExit(f"no traffic_probe line in {probe_log}")

    def dispatches(d):
        rows = list(csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))))
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        fused = [float(r["Counter_Value"]) for r in rows if ROOFLINE_KERNEL in r["Kernel_Name"]]
        copies = [float(r["Counter_Value"]) for r in rows if r["Kernel_Name"] == "__amd_rocclr_copyBuffer"]
        return fused, copies[-1]

    fetch, fetch_cal = dispatches(fetch_dir)
    write, write_cal = dispatches(write_dir)
    ms, per = probe["roofline_ms"], probe["launches_per_m"]
    if len(fetch) != len(ms) * per or len(write) != len(ms) * per:
        raise SystemExit(f"expected {len(ms) * per} roofline launches, got {len(fetch)} / {len(write)}")
    nbytes = probe["calibration_copy_bytes"]
    ff, wf = nbytes / 1024 / fetch_cal, nbytes / 1024 / write_cal  # true KiB per counted KiB
    per_m = {}
    for i, M in enumerate(ms):
        fk = sum(fetch[i * per:(i + 1) * per]) / per
        wk = sum(write[i * per:(i + 1) * per]) / per
        per_m[str(M)] = {"fetch_kib_raw": round(fk, 2), "write_kib_raw": round(wk, 2),
                         "hbm_bytes": round((fk * ff + wk * wf) * 1024), "algorithmic_bytes": fused_bytes(M)}
    return {
        "kernel": ROOFLINE_KERNEL,
        "workload": f"wq_fused_quant_matmul X bf16 [M,4096] x W int8 [4096->1024], M in {ms}, {per} launches "
                    "per M, each on a cold weight copy",
        "commands": [
            "rocprofv3 --pmc FETCH_SIZE -d gpurun_out/tr_fetch -o run --output-format csv -- python bench.py "
            "--traffic-probe > gpurun_out/tr_fetch.log",
            "rocprofv3 --pmc WRITE_SIZE -d gpurun_out/tr_write -o run --output-format csv -- python bench.py "
            "--traffic-probe > gpurun_out/tr_write.log",
            "python bench.py --traffic-summary gpurun_out/tr_fetch gpurun_out/tr_write gpurun_out/tr_fetch.log "
            "> profiles/traffic_k_fused_decode_wq_a.json",
        ],
        "calibration": {"kernel": "__amd_rocclr_copyBuffer (torch copy_ of 64 MiB)", "bytes_read": nbytes,
                        "bytes_written": nbytes, "fetch_size_kib_read": fetch_cal, "write_size_kib_read": write_cal,
                        "fetch_factor": round(ff, 4), "write_factor": round(wf, 4)},
        "per_M": per_m,
        "hbm_bytes_per_launch_mean": round(sum(v["hbm_bytes"] for v in per_m.values()) / len(per_m)),
        "algorithmic_bytes_per_launch_mean": round(sum(v["algorithmic_bytes"] for v in per_m.values()) / len(per_m)),
        "kernel_source_hash": probe["kernel_source_hash"],
    }


def trace_summary(stats_csv, probe_log, bench_log=None):
    """Per-launch duration of the roofline kernel (fragment-order instances) from a
    rocprofv3 --kernel-trace --stats run of the headline (bench.py --no-rows --no-cpu-baseline
    --no-sweep), next to the event-timed per-launch figure of an unprofiled bench run
    (bench_log) and of the profiled run itself (whose graph replays the tracer slows)."""
    import csv

    line = [ln for ln in open(probe_log) if ln.startswith("{")][-1]
    run = json.loads(line)
    plain = None
    if bench_log:
        bl = [ln for ln in open(bench_log) if ln.startswith("{")][-1]
        plain = json.loads(bl)["roofline"]
    rows = [r for r in csv.DictReader(open(stats_csv)) if ROOFLINE_KERNEL in r["Name"] and "true>" in r["Name"]]
    calls = sum(int(r["Calls"]) for r in rows)
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    return {
        "kernel": ROOFLINE_KERNEL + "<R, CT, false, true>",
        "command": "rocprofv3 --kernel-trace --stats -d gpurun_out/kt_head -o run --output-format csv -- python bench.py "
                   "--no-rows --no-cpu-baseline --no-sweep > gpurun_out/kt_head.log; python bench.py --no-sweep --no-cpu-baseline > "
                   "gpurun_out/bench_plain.log; python bench.py --trace-summary gpurun_out/kt_head/run_kernel_stats.csv "
                   "gpurun_out/kt_head.log gpurun_out/bench_plain.log > profiles/kernel_trace_k_fused_decode_wq_a.json",
        "instances": {r["Name"].split("(")[0].replace("void ", ""): {"calls": int(r["Calls"]),
                                                                   "mean_us": round(float(r["AverageNs"]) / 1e3, 3)}
                      for r in rows},
        "trace_us_per_launch_mean": round(total / calls / 1e3, 3),
        "event_us_per_launch_unprofiled_run": plain["us_per_launch_mean"] if plain else None,
        "event_us_per_launch_by_M_unprofiled_run": plain["us_per_launch"] if plain else None,
        "event_us_per_launch_same_run_under_the_tracer": run["roofline"]["us_per_launch_mean"],
        "kernel_source_hash": kernel_source_hash(),
    }


# kernels of the row probe: (label, kernel-name fragment, algorithmic bytes, algorithmic ops)
def _row_kernels():
    Mp, Kp, Np = 8192, 1024, 32768
    G8, D8, N8 = 8, 4096, 1024
    out = [("prefill GEMM M=8192 K=1024 N=32768", "k_gemm_i8_big", Mp * Kp + Np * Kp + 4 * (Mp + Np) + 2 * Mp * Np,
            2 * Mp * Np * Kp)]
    T = 512
    PH, TA = 8, 512
    out.append(("FP8 group quant T=512 (X bf16 [512, 8, 4096])", "k_group_quant_fp8",
                3 * T * G8 * D8 + 4 * G8 * PH * TA, 0))
    for T, name in ((64, "k_fp8_decode32"), (512, "k_gemm_tile<true>")):
        TA = (T + 3) // 4 * 4
        out.append((f"FP8 contraction T={T}", name,
                    T * G8 * D8 + 4 * G8 * PH * TA + G8 * N8 * D8 + 4 * G8 * (N8 // 128) * (D8 // 128) + 2 * T * G8 * N8,
                    2 * T * G8 * N8 * D8))
    out.append(("MoE gate/up, small experts (fragment order)", "k_seg_decode<2", None, None))
    out.append(("MoE gate/up, large experts (fragment order)", "k_gemm_seg<2>", None, None))
    out.append(("MoE down, small experts", "k_seg_decode<1", None, None))
    out.append(("MoE down, large experts", "k_gemm_seg<1>", None, None))
    return out


def rows_probe(wq, syn, dev):
    """Two launches of each row kernel on cold copies of its inputs, then a 64 MiB device
    copy for the counter calibration (the shapes and data of the bench rows)."""
    import numpy as np
    import torch

    Mp, Kp, Np = 8192, 1024, 32768
    xp = torch.from_numpy(syn.wq_b_x(Mp).view(np.int16)).to(dev).view(torch.bfloat16)
    wp_h, swp_h = syn.wq_b_w()
    wp = [torch.from_numpy(wp_h).to(dev) for _ in range(2)]
    swp = torch.from_numpy(swp_h).to(dev)
    xqp, xsp = wq.wq_dynamic_quant(xp)
    yp = torch.empty((Mp, Np), dtype=torch.bfloat16, device=dev)
    for r in range(2):
        wq.wq_quant_matmul(xqp, xsp, wp[r], swp, y=yp)
    torch.cuda.synchronize()
    del wp, yp, xp
    G8, D8, N8, R8 = 8, 4096, 1024, 4
    wq8_h, ws8_h = syn.fp8_weights(42, G=G8, N=N8, D=D8)
    wq8 = [torch.from_numpy(wq8_h).to(dev) for _ in range(R8)]
    ws8 = torch.from_numpy(ws8_h).to(dev)
    for T in (64, 512):
        x8h = torch.from_numpy(syn.fp8_group_x(T, G=G8, D=D8).view(np.int16)).to(dev).view(torch.bfloat16)
        x8 = [x8h.clone() for _ in range(2)]
        outs = [wq.wq_group_quant_fp8_ue8m0(x8[r]) for r in range(2)]
        y8 = torch.empty((T, G8, N8), dtype=torch.bfloat16, device=dev)
        for r in range(2):
            q8, _, st8 = outs[r]
            wq.wq_quant_matmul(q8, st8, wq8[r], ws8, y=y8, fp8_groups=G8)
        torch.cuda.synchronize()
    del wq8
    T, H, I, E, topk = 256, 4096, 2048, 256, 8
    d = syn.moe_inputs(seed=51, T=T, H=H, I=I, E=E, TOPK=topk, weights=False)
    gen = torch.Generator(device=dev)
    gen.manual_seed(5151)
    w13 = wq.wq_pack_weight_i8(torch.randint(-127, 128, (E, 2 * I, H), generator=gen, device=dev, dtype=torch.int8))
    w2 = wq.wq_pack_weight_i8(torch.randint(-127, 128, (E, H, I), generator=gen, device=dev, dtype=torch.int8))
    sw13 = torch.rand((E, 2 * I), generator=gen, device=dev) * 9e-3 + 1e-3
    sw2 = torch.rand((E, H), generator=gen, device=dev) * 9e-3 + 1e-3
    ids = torch.from_numpy(d["ids"]).to(dev)
    h = torch.from_numpy(d["h"].view(np.int16)).to(dev).view(torch.bfloat16)
    gamma = torch.from_numpy(d["gamma"].view(np.int16)).to(dev).view(torch.bfloat16)
    for _ in range(2):
        perm, row_token, offsets = wq.wq_moe_sort(ids, E)
        q1, s1 = wq.wq_dynamic_quant(h, rms_gamma=gamma, row_index=row_token)
        hmid = wq.wq_quant_matmul(q1, s1, w13, sw13, seg_offsets=offsets, epilogue=wq.WQ_EPI_SWIGLU_F32, b_fragment=True)
        q2, s2 = wq.wq_dynamic_quant(hmid)
        wq.wq_quant_matmul(q2, s2, w2, sw2, seg_offsets=offsets, b_fragment=True)
    torch.cuda.synchronize()
    counts = np.bincount(d["ids"].reshape(-1), minlength=E)
    src = torch.ones(64 << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"rows_probe": {"launches_per_kernel": 2, "calibration_copy_bytes": 64 << 20,
                                     "moe_active_experts": int((counts > 0).sum()),
                                     "kernel_source_hash": kernel_source_hash()}}))


def counter_summary(fetch_dir, write_dir, sq_dir, probe_log):
    """Markdown table of per-kernel counters (second of the two launches of each kernel)
    from three rocprofv3 --pmc runs of --rows-probe: FETCH_SIZE, WRITE_SIZE (scaled by the
    64 MiB copy calibration) and the SQ / GRBM set."""
    import csv

    probe = None
    for line in open(probe_log):
        if line.startswith("{") and "rows_probe" in line:
            probe = json.loads(line)["rows_probe"]
    if probe is None:
        raise SystemExit(f"no rows_probe line in {probe_log}")

    def load(d):
        rows = list(csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))))
        by = {}
        for r in rows:
            key = (int(r["Dispatch_Id"]), r["Kernel_Name"])
            by.setdefault(key, {})[r["Counter_Name"]] = float(r["Counter_Value"])
        return sorted(by.items())

    fetch, write, sq = load(fetch_dir), load(write_dir), load(sq_dir)
    nbytes = probe["calibration_copy_bytes"]
    cal_f = [v["FETCH_SIZE"] for (i, n), v in fetch if n == "__amd_rocclr_copyBuffer"][-1]
    cal_w = [v["WRITE_SIZE"] for (i, n), v in write if n == "__amd_rocclr_copyBuffer"][-1]
    ff, wf = nbytes / 1024 / cal_f, nbytes / 1024 / cal_w

    def last(rows, frag, ctr):
        vals = [v[ctr] for (i, n), v in rows if frag in n and ctr in v]
        return vals[-1] if vals else None

    lines = ["| Kernel (workload) | HBM fetch (MB) | HBM write (MB) | algorithmic (MB) | traffic / algorithmic | "
             "MFMA instructions | SQ_VALU_MFMA_BUSY_CYCLES / (1024 x GRBM_GUI_ACTIVE / 8) |",
             "|---|---|---|---|---|---|---|"]
    for label, frag, alg, ops in _row_kernels():
        f, w = last(fetch, frag, "FETCH_SIZE"), last(write, frag, "WRITE_SIZE")
        if f is None or w is None:
            lines.append(f"| {label} (`{frag}`) | not dispatched | | | | | |")
            continue
        fb, wb = f * ff * 1024, w * wf * 1024
        busy = last(sq, frag, "SQ_VALU_MFMA_BUSY_CYCLES")
        gui = last(sq, frag, "GRBM_GUI_ACTIVE")
        mf = last(sq, frag, "SQ_INSTS_MFMA")
        ratio = f"{busy / (1024 * gui / 8):.3f}" if busy is not None and gui else "-"
        alg_s = f"{alg / 1e6:.1f}" if alg else "-"
        tr = f"{(fb + wb) / alg:.2f}" if alg else "-"
        lines.append(f"| {label} (`{frag}`) | {fb / 1e6:.1f} | {wb / 1e6:.1f} | {alg_s} | {tr} | "
                     f"{int(mf) if mf is not None else '-'} | {ratio} |")
    lines.append("")
    lines.append(f"Calibration: FETCH_SIZE x {ff:.3f}, WRITE_SIZE x {wf:.3f} (the counters' KiB for a 64 MiB "
                 f"device copy).  MoE active experts: {probe['moe_active_experts']}.  Kernel sources: "
                 f"{probe['kernel_source_hash']}.")
    return "\n".join(lines)


def cpu_baseline(budget_s=10.0):
    """Time the CPU oracle (as it stands) on the same workload: the full fused chain at
    every M of the sweep, repeated until about budget_s seconds have passed."""
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
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {
        "value": el / calls * 1e6,
        "unit": "us per fused W8A8 linear call (mean over the M sweep)",
        "cores": int(threads),
        "cpu": model,
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
    ap.add_argument("--no-rows", action="store_true", help="skip the prefill / FP8 / MoE measurements")
    ap.add_argument("--no-sweep", action="store_true", help="skip the standalone sweep and the floors")
    ap.add_argument("--traffic-probe", action="store_true", help="only the roofline kernel's launches, for counters")
    ap.add_argument("--traffic-summary", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "PROBE_LOG"),
                    help="write the traffic JSON from two --traffic-probe counter runs (no GPU)")
    ap.add_argument("--trace-summary", nargs="+", metavar="FILE",
                    help="STATS_CSV RUN_LOG [BENCH_LOG]: write the kernel-trace JSON from a rocprofv3 --stats run of the headline, against an unprofiled bench line (no GPU)")
    ap.add_argument("--prefill-probe", action="store_true",
                    help="only two launches of the M=8192 prefill GEMM on random operands, for counters")
    ap.add_argument("--rows-probe", action="store_true",
                    help="only the row kernels (prefill GEMM, FP8 group quant and contraction, MoE block), two "
                         "launches each on cold copies, then a 64 MiB copy, for counters")
    ap.add_argument("--counter-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "SQ_DIR", "PROBE_LOG"),
                    help="write the per-kernel counter table from three rocprofv3 --pmc runs of --rows-probe (no GPU)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the kernels run on one MI355X and the "
              f"multi-GPU sharding is described, not run.", file=sys.stderr)
        sys.exit(2)
    if args.traffic_summary:
        print(json.dumps(traffic_summary(*args.traffic_summary), indent=1))
        return
    if args.trace_summary:
        print(json.dumps(trace_summary(*args.trace_summary), indent=1))
        return
    if args.counter_summary:
        print(counter_summary(*args.counter_summary))
        return

    import numpy as np
    import torch

    import fp8_dynamic_quant_amd as wq
    import synthetic as syn

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    wq.lib()
    stream = torch.cuda.Stream()

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
    paths = {M: wq.wq_fused_path(M, K_A, N_A) for M in SWEEP}
    roof_ms = [M for M in SWEEP if paths[M] == 2]
    if roof_ms != list(SWEEP):
        raise SystemExit(f"the packed fused call needs the one-launch MFMA path at every M; paths {paths}")

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

    # the weights as a deployment stores them: cast once at load time, untimed, into the
    # fragment order the MFMA kernel reads (wq_pack_weight_i8), one packed copy per slot
    wps = [wq.wq_pack_weight_i8(ws[r]) for r in range(R)]

    def fused_step(r, Ms=SWEEP):
        for M in Ms:
            wq.wq_fused_quant_matmul_packed(xs[M][r], wps[r], sws[r], N_A, y=ys[M][r])

    def fused_call(slot, M):
        wq.wq_fused_quant_matmul_packed(xs[M][slot], wps[slot], sws[slot], N_A, y=ys[M][slot])

    def fused_plain_step(r, Ms=SWEEP):
        for M in Ms:
            wq.wq_fused_quant_matmul(xs[M][r], ws[r], sws[r], y=ys[M][r])

    def time_cycle(cycle, P, steps, warmup, make_partial):
        """`cycle` runs P steps; replay it to cover `warmup` steps, then time exactly `steps`
        steps between two events on the replay stream: whole cycles, then a graph of the
        remaining steps (make_partial(n) captures the first n steps of a cycle, whose copies
        were last used a whole cycle earlier).  Returns us per step."""
        rest = steps % P
        part = make_partial(rest) if rest else None
        with torch.cuda.stream(stream):
            for _ in range(-(-warmup // P)):
                cycle.replay()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(steps // P):
                cycle.replay()
            if part is not None:
                part.replay()
            b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / steps

    def time_in_graph(fn, n=64):
        """Mean us per call of fn(r) over replays of a graph of n back-to-back calls
        r = 0..n-1 (for calls of a few us, where eager launches would time the host)."""
        g = capture(fn, n)
        us = time_graph(g, n, 4 * n, n)
        del g
        return us

    def time_events(fn, n, warm=3):
        """Mean us per call of fn() over n eager calls on the side stream (launch-bound
        work is not timed this way: every call here runs for tens of us or more)."""
        with torch.cuda.stream(stream):
            for _ in range(warm):
                fn()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(n):
                fn()
            b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / n

    if args.prefill_probe:
        g = torch.Generator(device="cpu").manual_seed(0)
        Mp, Kp, Np = 8192, 1024, 32768
        a = torch.randint(-127, 128, (Mp, Kp), dtype=torch.int8, generator=g).to(dev)
        s = (torch.rand(Mp, generator=g) * 0.01).to(dev)
        w = torch.randint(-127, 128, (Np, Kp), dtype=torch.int8, generator=g).to(dev)
        sw = (torch.rand(Np, generator=g) * 0.01).to(dev)
        y = torch.empty((Mp, Np), dtype=torch.bfloat16, device=dev)
        for _ in range(2):
            wq.wq_quant_matmul(a, s, w, sw, y=y)
        torch.cuda.synchronize()
        print(json.dumps({"prefill_probe": {"M": Mp, "K": Kp, "N": Np, "launches": 2}}))
        return

    if args.rows_probe:
        rows_probe(wq, syn, dev)
        return

    if args.traffic_probe:
        # eager launches of the roofline kernel, each on a cold weight copy, then one copy
        # kernel of exactly 64 MiB read + 64 MiB written for the counter calibration
        with torch.cuda.stream(stream):
            for M in roof_ms:
                for r in range(8):
                    fused_step(r, (M,))
            src = torch.ones(64 << 20, dtype=torch.uint8, device=dev)
            dst = torch.empty_like(src)
            torch.cuda.synchronize()
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"traffic_probe": {"roofline_ms": roof_ms, "launches_per_m": 8, "calibration_copy_bytes": 64 << 20,
                                            "kernel_source_hash": kernel_source_hash()}}))
        return

    # one correctness check against the oracle before timing (the full parity suite is in tests/)
    from oracle import int8_linear as il  # noqa: E402  (checker only; not on the timed path)
    from oracle.numerics import bf16_ulp_distance  # noqa: E402

    for M in (1, 8, 64):
        ref = il.linear_w8a8(x_host[M], w_host, sw_host)["y"]
        for y in (wq.wq_fused_quant_matmul_packed(xs[M][0], wps[0], sws[0], N_A),
                  wq.wq_fused_quant_matmul(xs[M][0], ws[0], sws[0])):
            got = y.view(torch.int16).cpu().numpy().view(np.uint16)
            assert bf16_ulp_distance(got, ref).max() <= 1, "fused linear disagrees with the oracle"

    # ---- headline: fused decode linear over the sweep -------------------------------------
    # Every call reads its own weight copy: step p of a cycle of R / len(SWEEP) steps runs
    # the sweep's M values on copies len(SWEEP) p .. len(SWEEP) p + len(SWEEP) - 1, one graph
    # per step, so the timed region cycles through all R copies (>= 512 MiB, past L2 and the
    # Infinity Cache) whatever --steps is, and a copy comes back only after R other calls.
    n_m = len(SWEEP)
    P = R // n_m  # steps per cycle through all R copies
    cycle = capture(lambda c: fused_call(c, SWEEP[c % n_m]), P * n_m)
    t0 = time.perf_counter()
    us_step = time_cycle(cycle, P, args.steps, args.warmup,
                         lambda n: capture(lambda c: fused_call(c, SWEEP[c % n_m]), n * n_m))
    wall = time.perf_counter() - t0
    us_per_call = us_step / n_m
    del cycle

    # ---- per-M: fused (always, for the roofline) and standalone -----------------------------
    xq = {M: [torch.empty((M, K_A), dtype=torch.int8, device=dev) for _ in range(R)] for M in SWEEP}
    xsc = {M: [torch.empty((M,), dtype=torch.float32, device=dev) for _ in range(R)] for M in SWEEP}

    def standalone_step(r, Ms=SWEEP):
        # the two-launch form on the same fragment-order weights as the headline
        for M in Ms:
            wq.wq_dynamic_quant(xs[M][r], x_q=xq[M][r], x_scale=xsc[M][r])
            wq.wq_quant_matmul(xq[M][r], xsc[M][r], wps[r], sws[r], y=ys[M][r], b_fragment=True, n=N_A)

    sweep, us_fused = [], {}
    for M in SWEEP:
        gf = capture(lambda r, M=M: fused_step(r, (M,)), R)
        us_fused[M] = time_graph(gf, R, 4 * R, R)
        del gf
        row = {"M": M, "path": wq.FUSED_PATHS[paths[M]] + ", fragment-order weights", "us_fused": round(us_fused[M], 3)}
        if not args.no_sweep:
            gs = capture(lambda r, M=M: standalone_step(r, (M,)), R)
            row["us_standalone_quant_plus_gemm"] = round(time_graph(gs, R, 4 * R, R), 3)
            del gs
            # the same call on the plain [N, K] weights
            gp = capture(lambda r, M=M: fused_plain_step(r, (M,)), R)
            row["us_fused_plain_weights"] = round(time_graph(gp, R, 4 * R, R), 3)
            del gp
        bf = fused_bytes(M)
        row.update({"fused_GBps": round(bf / us_fused[M] / 1e3, 1),
                    "fused_frac_hbm": round(bf / us_fused[M] / 1e3 / HBM_PEAK_GBS, 4),
                    "algorithmic_bytes": bf, "standalone_bytes": standalone_bytes(M),
                    "TOPS": round(2 * M * K_A * N_A / us_fused[M] / 1e6, 3)})
        sweep.append(row)
        torch.cuda.synchronize()

    # reference floors: a tiny launch and a plain same-size device copy, in the same graphs
    floors = None
    if not args.no_sweep:
        tiny = torch.zeros(1, device=dev)
        src = torch.empty(K_A * N_A, dtype=torch.uint8, device=dev)
        dst_bufs = [torch.empty_like(src) for _ in range(R)]
        g_floor = capture(lambda r: tiny.add_(1.0), R)
        launch_floor = time_graph(g_floor, R, 4 * R, R)
        g_copy = capture(lambda r: dst_bufs[r].copy_(ws[r].view(-1)), R)
        copy_us = time_graph(g_copy, R, 4 * R, R)
        del g_floor, g_copy, dst_bufs
        floors = {"graph_launch_us_per_tiny_kernel": round(launch_floor, 3), "copy_4MiB_us": round(copy_us, 3),
                  "copy_4MiB_GBps": round(2 * K_A * N_A / copy_us / 1e3, 1)}

    # ---- roofline of the dominant kernel: the one-launch fused kernel ----------------------
    roofline = None
    if roof_ms:
        b_sum = sum(fused_bytes(M) for M in roof_ms)
        t_sum = sum(us_fused[M] for M in roof_ms)
        achieved = b_sum / t_sum / 1e3
        traffic = None
        if os.path.exists(TRAFFIC_FILE):
            try:
                tr = json.load(open(TRAFFIC_FILE))
                if tr.get("kernel_source_hash") == kernel_source_hash():
                    traffic = tr.get("hbm_bytes_per_launch_mean")
            except Exception:
                traffic = None
        trace = None
        if os.path.exists(TRACE_FILE):
            try:
                tf = json.load(open(TRACE_FILE))
                if tf.get("kernel_source_hash") == kernel_source_hash():
                    trace = tf.get("trace_us_per_launch_mean")
            except Exception:
                trace = None
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                    "duration_source": "HIP events around graph replays of cold calls on the replay stream; "
                                       "the rocprofv3 kernel trace of the same workload reads longer per launch "
                                       "(its per-dispatch cost weighs most on these few-us launches)",
                    "trace_us_per_launch_mean": trace,
                    "kernel": ROOFLINE_KERNEL + "<R, CT, false, true> (fragment-order weights)",
                    "launches": f"one per fused call at M in {roof_ms} (K=4096, N=1024)",
                    "bytes_per_launch_mean": round(b_sum / len(roof_ms)),
                    "us_per_launch_mean": round(t_sum / len(roof_ms), 3),
                    "us_per_launch": {str(M): round(us_fused[M], 3) for M in roof_ms}}

    rows = {}
    if not args.no_rows:
        # ---- more decode shapes of the same projection family: wkv (K=4096, N=512) over the
        # sweep's M values, and wq_a at M=128 (one launch: the fused kernel takes M < 256) -----
        Nk = 512
        Rk = max(2, ROTATE_BYTES // (K_A * Nk))
        wk_h, swk_h = syn.int8_weights((2, 22, 1), Nk, K_A)
        wk0 = torch.from_numpy(wk_h).to(dev)
        wkp = [wq.wq_pack_weight_i8(wk0) for _ in range(Rk)]
        swk = torch.from_numpy(swk_h).to(dev)
        wkv = {}
        for M in (1, 8, 64):
            xk = [xs[M][r % R] for r in range(Rk)]
            yk = torch.empty((M, Nk), dtype=torch.bfloat16, device=dev)
            us = time_in_graph(lambda r, M=M: wq.wq_fused_quant_matmul_packed(xk[r], wkp[r], swk, Nk, y=yk), Rk)
            b = fused_bytes(M, K_A, Nk)
            wkv[str(M)] = {"us": round(us, 3), "GBps": round(b / us / 1e3, 1), "frac_hbm": round(b / us / 1e3 / HBM_PEAK_GBS, 4)}
        rows["wkv_decode"] = {"workload": "wkv-shaped fused decode linear: X bf16 [M,4096] x W int8 [4096->512], "
                                          "fragment-order weights, cold (rotating copies)",
                              "kernel": "k_fused_decode<R, CT, false, true>", "by_M": wkv}
        del wkp
        x128 = [torch.from_numpy(syn.wq_a_linear(128)[0].view(np.int16)).to(dev).view(torch.bfloat16) for _ in range(R)]
        y128 = torch.empty((128, N_A), dtype=torch.bfloat16, device=dev)
        q128 = torch.empty((128, K_A), dtype=torch.int8, device=dev)
        s128 = torch.empty((128,), dtype=torch.float32, device=dev)
        us128 = time_in_graph(lambda r: wq.wq_fused_quant_matmul(x128[r], ws[r], sws[r], y=y128, x_q_out=q128,
                                                                 x_scale_out=s128), R)
        b128 = standalone_bytes(128)
        rows["wq_a_m128"] = {"workload": "wq_a linear at M=128: fused call, plain [N,K] weights, cold",
                             "path": wq.FUSED_PATHS[wq.wq_fused_path(128, K_A, N_A)],
                             "us": round(us128, 3), "GBps": round(b128 / us128 / 1e3, 1),
                             "frac_hbm": round(b128 / us128 / 1e3 / HBM_PEAK_GBS, 4)}
        del x128

        # ---- expert-local row-count sweep of the segmented gate/up GEMM (SwiGLU epilogue):
        # 32 experts of W13 [4096 -> 2 x 2048] (512 MiB, fragment order), each with M_e rows;
        # M_e <= 16 goes to the weight-streaming kernel, larger M_e to the tiled one ----------
        Ee, He, Ie = 32, 4096, 2048
        gen_e = torch.Generator(device=dev)
        gen_e.manual_seed(7070)
        w13e = wq.wq_pack_weight_i8(torch.randint(-127, 128, (Ee, 2 * Ie, He), generator=gen_e, device=dev,
                                                  dtype=torch.int8))
        sw13e = torch.rand((Ee, 2 * Ie), generator=gen_e, device=dev) * 9e-3 + 1e-3
        me_rows = {}
        me_list = (1, 2, 4, 8, 16, 17, 32, 64, 96, 127, 128, 129, 160, 192, 256)
        me_cases = {}
        for Me in me_list:
            Mt = Ee * Me
            qe = torch.randint(-127, 128, (Mt, He), generator=gen_e, device=dev, dtype=torch.int8)
            se = torch.rand((Mt,), generator=gen_e, device=dev) * 0.05 + 0.01
            offe = torch.arange(0, Ee + 1, device=dev, dtype=torch.int64) * Me
            he = torch.empty((Mt, Ie), dtype=torch.float32, device=dev)
            me_cases[Me] = (qe, se, offe, he)
        # the sizes alternate over 5 rounds of 10 calls each, with and without the hint
        # expected_rows = M_e; each figure is the median round (the spread between rounds,
        # from clocks and the memory system, is a few per cent)
        me_us = {Me: ([], []) for Me in me_list}
        for _ in range(5):
            for Me, (qe, se, offe, he) in me_cases.items():
                for hint, out in ((0, me_us[Me][0]), (Me, me_us[Me][1])):
                    out.append(time_events(lambda: wq.wq_quant_matmul(qe, se, w13e, sw13e, seg_offsets=offe, y=he,
                                                                      epilogue=wq.WQ_EPI_SWIGLU_F32, b_fragment=True,
                                                                      expected_rows=hint), 10, warm=2))
        for Me in me_list:
            Mt = Ee * Me
            us, us_h = float(np.median(me_us[Me][0])), float(np.median(me_us[Me][1]))
            wb = Ee * 2 * Ie * He
            me_rows[str(Me)] = {"us": round(us, 1), "us_with_hint": round(us_h, 1), "us_per_expert": round(us / Ee, 2),
                                "weight_GBps": round(wb / us / 1e3, 1), "TOPS": round(2 * Mt * 2 * Ie * He / us / 1e6, 1),
                                "kernel": ("k_seg_decode<2, 8, true>" if Me <= 16 else
                                           "k_gemm_seg<2>, 128-row tiles" if Me <= 128 else
                                           "k_gemm_seg<2>, 256-row tiles" + (" + 128-row tiles" if Me % 256 and Me % 256 <= 128 else ""))}
        del me_cases
        steps = {}
        for lo_, hi_ in ((16, 17), (128, 129)):
            for key, name in (("us", ""), ("us_with_hint", "_with_hint")):
                steps[f"{lo_}_to_{hi_}{name}"] = round(me_rows[str(hi_)][key] / me_rows[str(lo_)][key] - 1, 4)
        rows["moe_expert_rows_sweep"] = {
            "workload": "segmented gate/up GEMM + SwiGLU, 32 experts x W13 int8 [4096 -> 2x2048] (fragment order), "
                        "M_e rows per expert; us_with_hint: expected_rows = M_e; medians of 5 alternating rounds",
            "steps": steps, "by_M_e": me_rows}
        del w13e

        # ---- prefill GEMM: wq_b-shaped M=8192, K=1024, N=32768 -----------------------------
        Mp, Kp, Np = 8192, 1024, 32768
        xp = torch.from_numpy(syn.wq_b_x(Mp).view(np.int16)).to(dev).view(torch.bfloat16)
        wp_h, swp_h = syn.wq_b_w()
        wp = [torch.from_numpy(wp_h).to(dev) for _ in range(2)]
        swp = torch.from_numpy(swp_h).to(dev)
        xqp, xsp = wq.wq_dynamic_quant(xp)
        yp = torch.empty((Mp, Np), dtype=torch.bfloat16, device=dev)
        it = iter(range(1 << 30))
        # three runs of ten launches back to back (sustained load lowers the clock); the
        # median run is the row's figure
        runs = [time_events(lambda: wq.wq_quant_matmul(xqp, xsp, wp[next(it) % 2], swp, y=yp), 10) for _ in range(3)]
        us_p = sorted(runs)[1]
        tops = 2 * Mp * Np * Kp / us_p / 1e6
        rows["prefill_gemm_m8192"] = {
            "workload": "wq_b wide linear INT8 GEMM (x_q given): M=8192, K=1024, N=32768, bf16 out; "
                        "median of 3 runs of 10 launches back to back",
            "kernel": "k_gemm_i8_big", "us": round(us_p, 2), "us_runs": [round(u, 2) for u in runs],
            "TOPS": round(tops, 1), "frac_int8_peak": round(tops / INT8_PEAK_TOPS, 4)}
        # ---- standalone per-token quant at the prefill shape (HBM bound): 24 rotating copies of
        # X (16 MiB) and of its outputs (8 MiB + 32 KiB), 576 MiB in all, so every call is cold
        del wp, yp
        Rq = 24
        xps = [xp.clone() for _ in range(Rq)]
        xqs = [torch.empty_like(xqp) for _ in range(Rq)]
        xss = [torch.empty_like(xsp) for _ in range(Rq)]
        us_q = time_in_graph(lambda r: wq.wq_dynamic_quant(xps[r], x_q=xqs[r], x_scale=xss[r]), Rq)
        qb = 2 * Mp * Kp + Mp * Kp + 4 * Mp
        rows["int8_quant_m8192"] = {"workload": f"per-token INT8 quant X bf16 [8192, 1024], {Rq} rotating copies of "
                                                "inputs and outputs (cold)", "kernel": "k_dynamic_quant",
                                    "us": round(us_q, 2), "GBps": round(qb / us_q / 1e3, 1),
                                    "frac_hbm": round(qb / us_q / 1e3 / HBM_PEAK_GBS, 4)}
        del xp, xqp, xps, xqs, xss

        # ---- FP8 per-token-group quant (packed UE8M0) and the grouped contraction ----------
        # 16 rotating copies of the 32 MiB weight and of the activations (>= 512 MiB in all
        # at T = 512) keep each call's inputs out of L2 and the Infinity Cache
        G8, D8, N8, R8 = 8, 4096, 1024, 16
        wq8_h, ws8_h = syn.fp8_weights(42, G=G8, N=N8, D=D8)
        wq8 = [torch.from_numpy(wq8_h).to(dev) for _ in range(R8)]
        ws8 = torch.from_numpy(ws8_h).to(dev)
        fp8 = {}
        for T in (1, 64, 512):
            x8h = torch.from_numpy(syn.fp8_group_x(T, G=G8, D=D8).view(np.int16)).to(dev).view(torch.bfloat16)
            x8 = [x8h.clone() for _ in range(R8)]
            _, PH, TA = wq.packed_scale_dims(T, D8)
            q8 = [torch.empty((T, G8, D8), dtype=torch.uint8, device=dev) for _ in range(R8)]
            st8 = [torch.empty((G8, PH, TA), dtype=torch.int32, device=dev) for _ in range(R8)]
            us_gq = time_in_graph(lambda r: wq.wq_group_quant_fp8_ue8m0(x8[r], x_q=q8[r], storage=st8[r]), R8)
            # the MX-like 32-element blocks: same payload size, 4x the scale bytes
            _, PHm, TAm = wq.packed_scale_dims(T, D8, 32)
            stm = [torch.empty((G8, PHm, TAm), dtype=torch.int32, device=dev) for _ in range(R8)]
            us_mx = time_in_graph(lambda r: wq.wq_group_quant_fp8_ue8m0(x8[r], x_q=q8[r], storage=stm[r], group=32), R8)
            mx_bytes = 2 * T * G8 * D8 + T * G8 * D8 + 4 * G8 * PHm * TAm
            del stm
            y8 = torch.empty((T, G8, N8), dtype=torch.bfloat16, device=dev)
            us_c = time_in_graph(lambda r: wq.wq_quant_matmul(q8[r], st8[r], wq8[r], ws8, y=y8, fp8_groups=G8), R8)
            del x8, q8, st8
            gq_bytes = 2 * T * G8 * D8 + T * G8 * D8 + 4 * G8 * PH * TA
            c_bytes = T * G8 * D8 + 4 * G8 * PH * TA + G8 * N8 * D8 + 4 * G8 * (N8 // 128) * (D8 // 128) + 2 * T * G8 * N8
            c_ops = 2 * T * G8 * N8 * D8
            fp8[str(T)] = {"group_quant_us": round(us_gq, 3), "group_quant_GBps": round(gq_bytes / us_gq / 1e3, 1),
                           "mx32_group_quant_us": round(us_mx, 3), "mx32_group_quant_GBps": round(mx_bytes / us_mx / 1e3, 1),
                           "contraction_us": round(us_c, 3), "contraction_GBps": round(c_bytes / us_c / 1e3, 1),
                           "contraction_frac_hbm": round(c_bytes / us_c / 1e3 / HBM_PEAK_GBS, 4),
                           "contraction_TOPS": round(c_ops / us_c / 1e6, 2)}
        # the MX-like 32-element blocks on both operands (decode-sized T)
        wmx_h, wbx_h = syn.mx_weights(44, G=G8, N=N8, D=D8)
        wmx = [torch.from_numpy(wmx_h).to(dev) for _ in range(R8)]
        wbx = torch.from_numpy(wbx_h).to(dev)
        mxc = {}
        for T in (1, 64, 512):
            x8h = torch.from_numpy(syn.fp8_group_x(T, G=G8, D=D8).view(np.int16)).to(dev).view(torch.bfloat16)
            qm, _, stmx = wq.wq_group_quant_fp8_ue8m0(x8h, group=32)
            ym = torch.empty((T, G8, N8), dtype=torch.bfloat16, device=dev)
            us = time_in_graph(lambda r: wq.wq_quant_matmul(qm, stmx, wmx[r], wbx, y=ym, fp8_groups=G8, mx=True), R8)
            b = T * G8 * D8 + 4 * stmx.numel() + G8 * N8 * D8 + G8 * N8 * (D8 // 32) + 2 * T * G8 * N8
            mxc[str(T)] = {"us": round(us, 3), "GBps": round(b / us / 1e3, 1), "frac_hbm": round(b / us / 1e3 / HBM_PEAK_GBS, 4)}
        del wmx
        rows["mx32_contraction"] = {"workload": "MX-like FP8: X E4M3 [T, 8, 4096] with 32-element UE8M0 scales (packed) x "
                                                "W_g E4M3 [1024, 4096] with 32-element UE8M0 scales, bf16 out",
                                    "kernels": "k_fp8_decode<TPW, true> (T <= 64), k_gemm_tile<true> with MX scales (T > 64)",
                                    "by_T": mxc}
        rows["fp8_wo_a"] = {"workload": "X bf16 [T, 8, 4096] -> E4M3 + packed UE8M0 [8, 8, align4(T)]; "
                                        "out[T,g,:] = x_q[T,g,:] W_g^T, W_g E4M3 [1024, 4096], 128x128 pow2 scales",
                            "kernels": "k_group_quant_fp8 (k_group_quant_mx for 32-element blocks); k_fp8_decode (T <= 16), k_fp8_decode32 (16 < T <= 64), k_gemm_tile<FP8> (T > 64)", "by_T": fp8}
        del wq8

        # ---- MoE block: T=256, hidden 4096, 256 experts of 2x2048, top-8 Zipf(1.1) ----------
        T, H, I, E, topk = 256, 4096, 2048, 256, 8
        d = syn.moe_inputs(seed=51, T=T, H=H, I=I, E=E, TOPK=topk, weights=False)
        gen = torch.Generator(device=dev)
        gen.manual_seed(5151)
        w13 = torch.randint(-127, 128, (E, 2 * I, H), generator=gen, device=dev, dtype=torch.int8)
        w2 = torch.randint(-127, 128, (E, H, I), generator=gen, device=dev, dtype=torch.int8)
        sw13 = torch.rand((E, 2 * I), generator=gen, device=dev) * 9e-3 + 1e-3
        sw2 = torch.rand((E, H), generator=gen, device=dev) * 9e-3 + 1e-3
        ids = torch.from_numpy(d["ids"]).to(dev)
        h = torch.from_numpy(d["h"].view(np.int16)).to(dev).view(torch.bfloat16)
        gamma = torch.from_numpy(d["gamma"].view(np.int16)).to(dev).view(torch.bfloat16)

        def moe_block():
            perm, row_token, offsets = wq.wq_moe_sort(ids, E)
            q1, s1 = wq.wq_dynamic_quant(h, rms_gamma=gamma, row_index=row_token)
            hmid = wq.wq_quant_matmul(q1, s1, w13, sw13, seg_offsets=offsets, epilogue=wq.WQ_EPI_SWIGLU_F32)
            q2, s2 = wq.wq_dynamic_quant(hmid)
            return wq.wq_quant_matmul(q2, s2, w2, sw2, seg_offsets=offsets)

        us_moe_plain = time_events(moe_block, 5, warm=2)
        # the expert weights as a deployment stores them: cast once at load (untimed) to the
        # fragment order, read by both segment kernels
        w13, w2 = wq.wq_pack_weight_i8(w13), wq.wq_pack_weight_i8(w2)

        def moe_block():  # noqa: F811  (the same block on the cast weights)
            perm, row_token, offsets = wq.wq_moe_sort(ids, E)
            q1, s1 = wq.wq_dynamic_quant(h, rms_gamma=gamma, row_index=row_token)
            hmid = wq.wq_quant_matmul(q1, s1, w13, sw13, seg_offsets=offsets, epilogue=wq.WQ_EPI_SWIGLU_F32,
                                      b_fragment=True)
            q2, s2 = wq.wq_dynamic_quant(hmid)
            return wq.wq_quant_matmul(q2, s2, w2, sw2, seg_offsets=offsets, b_fragment=True)

        us_moe = time_events(moe_block, 5, warm=2)
        counts = np.bincount(d["ids"].reshape(-1), minlength=E)
        active = int((counts > 0).sum())
        wbytes = active * (2 * I * H + I * H) + active * 4 * (2 * I + H)
        rows["moe_block"] = {
            "workload": "T=256, hidden 4096, E=256 experts (W13 4096->2x2048, W2 2048->4096 int8), top-8 Zipf(1.1): "
                        "sort, RMSNorm+quant+gather, gate/up segmented GEMM + SwiGLU, requant, down segmented GEMM",
            "kernels": "k_moe_sort, k_dynamic_quant x2, k_seg_decode<2> + k_gemm_seg<2> (gate/up), k_seg_decode<1> + k_gemm_seg<1> (down)",
            "active_experts": active,
            "weights": "int8 per expert, cast once at load (untimed) to fragment order (wq_pack_weight_i8)",
            "us": round(us_moe, 1), "us_plain_weights": round(us_moe_plain, 1),
            "weight_bytes": wbytes, "weight_GBps": round(wbytes / us_moe / 1e3, 1),
            "frac_hbm": round(wbytes / us_moe / 1e3 / HBM_PEAK_GBS, 4)}
        del w13, w2

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
                   "K": K_A, "N": N_A, "M_sweep": list(SWEEP), "rotating_copies": R,
                   "weights": "int8, cast once at load (untimed) to the MFMA fragment order (wq_pack_weight_i8); "
                              "plain [N, K] times in sweep[].us_fused_plain_weights"},
        "roofline": roofline,
        "sweep": sweep,
        "floors": floors,
        "rows": rows,
        "timed_wall_s": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
