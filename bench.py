"""Benchmark of the dequantizing GEMV hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload decode] [--no-cpu]

One step = one pass of the decode workload: every (format, shape, lanes)
matvec of the decode configuration, each reading its own copy of the weights
so that no call finds its weights in the 256 MB Infinity Cache:

    formats  affine4_g64 and q6_k
    shapes   17408 x 5120 (gate/up) and 5120 x 17408 (down, + bf16 residual)
    lanes    M = 1, 2, 4
    inputs   weights N(0, 0.02) quantized, activations/residual N(0, 1) bf16

value = weight bytes (codes + scales) read per step / step time, in GB/s.
Prints one JSON line.  The oracle (CPU, float64) is timed on a bounded sample
of the same workload for the cpu_baseline field.
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

HBM_PEAK_GBS = 8000.0
METRIC = "dequant-GEMV weight GB/s (% of HBM peak) at M=1..4; prefill TFLOP/s"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode", choices=["decode"])
    ap.add_argument("--no-cpu", action="store_true", help="skip the cpu_baseline leg")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    return ap.parse_args()


def decode_cases():
    from synth import formats as F
    cases = []
    for fmt in (F.AFFINE4_G64, F.Q6_K):
        for (n, k, res, tag) in ((17408, 5120, False, "gate_up"), (5120, 17408, True, "down")):
            for m in (1, 2, 4):
                cases.append(dict(fmt=fmt, n=n, k=k, m=m, residual=res, tag=tag))
    return cases


def algorithmic_bytes(w_bytes, c):
    """Bytes a launch must move at minimum: weights + x + y (+ residual)."""
    b = w_bytes + c["m"] * c["k"] * 2 + c["m"] * c["n"] * 4
    if c["residual"]:
        b += c["m"] * c["n"] * 2
    return b


def measured_read_peak(q, torch, dev, gib=1.0, reps=10):
    """Achievable HBM read bandwidth: qbench_stream_read over a buffer far
    larger than the caches, median of `reps` launches."""
    buf = torch.empty(int(gib * 2**30) // 4, dtype=torch.int32, device=dev).fill_(1)
    sink = torch.zeros(64, dtype=torch.int32, device=dev)
    best = None
    for blocks in (256, 512):
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            q.bench_stream_read(buf, sink, blocks)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        gbs = buf.numel() * 4 / (float(np.median(ts)) * 1e-3) / 1e9
        if best is None or gbs > best[0]:
            best = (gbs, blocks)
    del buf
    torch.cuda.empty_cache()
    return {"GBps": round(best[0], 1), "blocks": best[1], "bytes": int(gib * 2**30),
            "kernel": "stream_read_kernel (16-byte non-temporal loads)"}


def traffic_from_profile():
    """HBM bytes per GEMV launch measured with rocprofv3 counters, if the
    committed measurement was taken on the current kernel source."""
    import hashlib
    src = os.path.join(ROOT, "gemm_dequant_gemv_amd", "csrc", "gemv.hip")
    prof = os.path.join(ROOT, "profiles", "gemv_decode_traffic.json")
    if not os.path.exists(prof):
        return None
    with open(prof) as f:
        rec = json.load(f)
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    return rec.get("hbm_bytes_per_launch") if rec.get("gemv_source_sha256") == sha else None


def cpu_baseline(cases, seconds):
    """The oracle as it stands, on sampled rows of the same matrices."""
    import oracle
    from synth import quant
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = 1
    t_total, bytes_total, rows_done = 0.0, 0, 0
    rows = 256
    t_start = time.perf_counter()
    for c in cases:
        if time.perf_counter() - t_start > seconds:
            break
        name = f"bench/{c['tag']}/{c['fmt']}"
        p = quant.synthetic_weight(c["fmt"], rows, c["k"], name=name + "/cpu")
        x = quant.synthetic_bf16(c["m"], c["k"], name=name + "/x")
        r = quant.synthetic_bf16(c["m"], rows, name=name + "/r") if c["residual"] else None
        t0 = time.perf_counter()
        oracle.gemv(p, x, r)
        t_total += time.perf_counter() - t0
        bytes_total += p.nbytes()
        rows_done += rows
    gbs = bytes_total / t_total / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{rows} rows of each decode matrix ({rows_done} rows, "
                      f"{bytes_total / 1e6:.1f} MB of packed weights), float64 numpy oracle, "
                      f"{t_total:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); the sharded path "
              "is described in DESIGN.md and not launched.", file=sys.stderr)
        sys.exit(2)
    import torch

    import gemm_dequant_gemv_amd as q
    from synth import quant

    dev = "cuda:0"
    torch.cuda.set_device(0)
    cases = decode_cases()
    # distinct weights per case (one per lane count) -> 12 matrices, ~740 MB
    setup = []
    for c in cases:
        name = f"bench/{c['tag']}/{c['fmt']}"
        p = quant.synthetic_weight(c["fmt"], c["n"], c["k"], name=f"{name}/W{c['m']}")
        w = q.Weight.from_host(p, dev)
        x = torch.from_numpy(quant.synthetic_bf16(c["m"], c["k"], name=name + "/x").view(np.int16)
                             ).view(torch.bfloat16).to(dev)
        r = None
        if c["residual"]:
            r = torch.from_numpy(quant.synthetic_bf16(c["m"], c["n"], name=name + "/r")
                                 .view(np.int16)).view(torch.bfloat16).to(dev)
        y = torch.empty((c["m"], c["n"]), dtype=torch.float32, device=dev)
        ws = q.new_workspace(q.gemv_workspace_size(w, c["m"]), dev)
        call = q.PreparedGemv(w, x, y, r, ws)
        setup.append((c, w, x, r, y, ws, w.nbytes(), call))
    torch.cuda.synchronize()

    def step(events=None):
        # arguments are marshalled once (PreparedGemv), so the host enqueues
        # far faster than the GPU drains and the events bracket kernel time
        for i, item in enumerate(setup):
            if events is not None:
                events[i][0].record()
            item[7]()
            if events is not None:
                events[i][1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K steps, per-launch HIP events on the launch stream
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in setup] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    read_peak = measured_read_peak(q, torch, dev)

    per_case = []
    tot_w, tot_alg, tot_kt = 0, 0, 0.0
    for i, (c, w, x, r, y, ws, wb, _) in enumerate(setup):
        ts = [evs[s][i][0].elapsed_time(evs[s][i][1]) for s in range(args.steps)]
        med = float(np.median(ts))
        mean = float(np.mean(ts))
        alg = algorithmic_bytes(wb, c)
        tot_w += wb * args.steps
        tot_alg += alg * args.steps
        tot_kt += sum(ts)
        per_case.append({"format": {1: "affine4_g64", 4: "q6_k"}[c["fmt"]],
                         "shape": f"{c['n']}x{c['k']}", "m": c["m"], "residual": c["residual"],
                         "us_median": round(med * 1e3, 2),
                         "weight_GBps": round(wb / (med * 1e-3) / 1e9, 1),
                         "pct_hbm_peak": round(100 * wb / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 1)})
    step_s = wall / args.steps
    value = tot_w / args.steps / step_s / 1e9
    achieved = tot_alg / (tot_kt * 1e-3) / 1e9

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "decode matvecs, affine4_g64 and q6_k, 17408x5120 and "
                               "5120x17408 (+bf16 residual), M=1,2,4, cold weights",
                   "calls_per_step": len(setup),
                   "weight_bytes_per_step": tot_w // args.steps},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profile(),
                     "kernel": "gemv_kernel (all instances of the step)",
                     "algorithmic_bytes_per_launch": int(tot_alg / (args.steps * len(setup))),
                     "mean_launch_us": round(tot_kt / (args.steps * len(setup)) * 1e3, 2),
                     "measured_read_peak": read_peak,
                     "frac_of_measured_read_peak": round(achieved / read_peak["GBps"], 4)},
        "detail": per_case,
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(cases, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
