"""Benchmark of the dequantizing matmul hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--no-cpu] [--sections decode,prefill,mid,moe,fp4,hadamard]
    python bench.py --record-traffic FETCH.csv WRITE.csv   (no GPU work; see below)

One step = one pass of the decode workload: every (format, shape, lanes)
matvec of the decode configuration, each reading its own copy of the weights
so that no call finds its weights in the 256 MB Infinity Cache:

    formats  affine4_g64 and q6_k
    shapes   17408 x 5120 (gate/up) and 5120 x 17408 (down, + bf16 residual)
    lanes    M = 1, 2, 4
    inputs   weights N(0, 0.02) quantized, activations/residual N(0, 1) bf16

value = weight bytes (codes + scales) read per step / step time, in GB/s.
The timed region is K steps back to back, bracketed by one HIP event pair on
the launch stream (events between launches add their own packets to every
kernel boundary, about 8 us a launch here); the per-case detail comes from a
later pass in which one case per step is event-bracketed.

After the timed steps the other rows of the hot path are measured on their
own configurations and reported under "sections" (each with its own unit):

    prefill  X [M][5120] x W 17408 x 5120, affine4_g64 and nvfp4,
             M in 128, 512, 2048, 8192 -> TFLOP/s (2 M N K per launch);
             and W4A4: the same matrix in mxfp4 against activations
             quantized to mxfp4 on the GPU (against the FP4 MFMA peak)
    mid      17408 x 5120 at 5, 8 (row-streaming GEMV) and 16 rows (MFMA
             tiles), affine4_g64 and nvfp4 -> us per call
    moe      512 routed + 1 shared expert, hidden 2048, intermediate 512,
             nvfp4, top-10 of N(0, 1) logits by the library's router, T = 4
             (warm and cold) and 8192
    fp4      mxfp4 and nvfp4 matvecs (1% outliers at 8x), 5120 x 5120,
             5120 x 6144 and 248320 x 5120, M = 1..4 -> weight GB/s
    hadamard qgemv_hadamard (prepare, GEMV, finish in one call) against
             the three calls and the GEMV alone, 17408 x 5120 affine4_g64,
             M = 1 and 4 -> us per call

Prints one JSON line.  The oracle (CPU, float64) is timed on bounded samples
of the decode, prefill and MoE workloads for the cpu_baseline field (all BLAS
threads and one thread; the host's core count and CPU model are recorded).

--record-traffic turns two rocprofv3 counter CSVs (FETCH_SIZE, then
WRITE_SIZE, each from `rocprofv3 --pmc <counter> --output-format csv -- python3
bench.py --steps 2 --warmup 1 --no-cpu --sections decode`) into
profiles/gemv_decode_traffic.json: HBM bytes per GEMV launch, calibrated by
the same counters on the benchmark's own 1 GiB read and torch's 1 GiB fill.
"""

from __future__ import annotations

import argparse
import csv
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
FP4_MFMA_PEAK_TFLOPS = 10100.0
METRIC = "dequant-GEMV weight GB/s (% of HBM peak) at M=1..4; prefill TFLOP/s"
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "gemv_decode_traffic.json")
GEMV_SOURCES = ("gemv.hip", "gemv_rows.hip", "gemv_step.h", "qmm_device.h")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the cpu_baseline leg")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--sections", default="decode,prefill,mid,moe,fp4,hadamard")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    return ap.parse_args()


def gemv_sources_sha():
    h = hashlib.sha256()
    for name in GEMV_SOURCES:
        with open(os.path.join(ROOT, "gemm_dequant_gemv_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


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


def dev_bf16(torch, bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def timed(torch, fn, reps, warm=2, batches=3):
    """Median and mean milliseconds per launch of `fn`: `batches` runs of
    `reps` back-to-back launches, each run bracketed by one HIP event pair on
    the current stream (an event between every two launches would add its own
    packets to each kernel boundary and inflate short kernels)."""
    for _ in range(warm):
        fn()
    ts = []
    for _ in range(batches):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) / reps)
    return float(np.median(ts)), float(np.mean(ts))


def measured_read_peak(q, torch, dev, gib=1.0, reps=10):
    """Achievable HBM read bandwidth: qbench_stream_read over a buffer far
    larger than the caches, median of `reps` launches; then torch fills the
    same buffer once (the write calibration of the traffic counters)."""
    buf = torch.empty(int(gib * 2**30) // 4, dtype=torch.int32, device=dev).fill_(1)
    sink = torch.zeros(64, dtype=torch.int32, device=dev)
    best = None
    for blocks in (256, 512):
        med, _ = timed(torch, lambda: q.bench_stream_read(buf, sink, blocks), reps, warm=1)
        gbs = buf.numel() * 4 / (med * 1e-3) / 1e9
        if best is None or gbs > best[0]:
            best = (gbs, blocks)
    del buf
    torch.cuda.empty_cache()
    return {"GBps": round(best[0], 1), "blocks": best[1], "bytes": int(gib * 2**30),
            "kernel": "stream_read_kernel (16-byte non-temporal loads)"}


def measured_mfma_peak(q, torch, dev, reps=10):
    """Achievable dense bf16 MFMA rate: qbench_mfma_peak (random register
    operands, 4 independent accumulators per wave), median of `reps` launches,
    best of 2, 4 and 8 waves per SIMD."""
    sink = torch.zeros(64, dtype=torch.int32, device=dev)
    iters = 2000
    best = None
    for blocks in (512, 1024, 2048):
        flops = [0.0]

        def launch():
            flops[0] = q.bench_mfma_peak(iters, blocks, sink)

        med, _ = timed(torch, launch, reps, warm=1)
        tf = flops[0] / (med * 1e-3) / 1e12
        if best is None or tf > best[0]:
            best = (tf, blocks)
    return {"TFLOPs": round(best[0], 1), "blocks": best[1], "waves_per_block": 4, "iters": iters,
            "kernel": "mfma_peak_kernel (v_mfma_f32_32x32x16_bf16, random register operands)"}


def traffic_from_profile():
    """HBM bytes per GEMV launch measured with rocprofv3 counters, if the
    committed measurement was taken on the current kernel sources."""
    if not os.path.exists(TRAFFIC_JSON):
        return None
    with open(TRAFFIC_JSON) as f:
        rec = json.load(f)
    if rec.get("gemv_sources_sha256") != gemv_sources_sha():
        return None
    return rec.get("hbm_bytes_per_launch")


def record_traffic(fetch_csv, write_csv):
    """Parse two rocprofv3 --pmc CSVs (KiB per dispatch) into the traffic record."""
    def per_kernel(path, counter):
        out = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"].replace("(anonymous namespace)::", "").replace("void ", "")
            name = name.split("(")[0].replace("qmm::", "")
            out.setdefault(name, []).append(float(r["Counter_Value"]))
        return {k: float(np.mean(v)) for k, v in out.items()}
    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")
    gib_kib = 2**30 / 1024
    read_k = [v for k, v in fetch.items() if k.startswith("stream_read_kernel")]
    fill_k = [v for k, v in write.items() if "FillFunctor" in k or "fill" in k.lower()]
    f_factor = gib_kib / max(read_k) if read_k else None
    w_factor = gib_kib / max(fill_k) if fill_k else None
    gemv = sorted(k for k in fetch if k.startswith("gemv"))
    per = {k: {"FETCH_SIZE_KiB": round(fetch[k], 1), "WRITE_SIZE_KiB": round(write.get(k, 0.0), 1)}
           for k in gemv}
    tot = [fetch[k] * f_factor + write.get(k, 0.0) * w_factor for k in gemv]
    rec = {
        "gemv_sources_sha256": gemv_sources_sha(),
        "hbm_bytes_per_launch": int(np.mean(tot) * 1024) if tot else None,
        "fetch_factor": round(f_factor, 3) if f_factor else None,
        "write_factor": round(w_factor, 3) if w_factor else None,
        "commands": [
            "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out> -o run -- python3 bench.py "
            "--steps 2 --warmup 1 --no-cpu --sections decode",
            "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out> -o run -- python3 bench.py "
            "--steps 2 --warmup 1 --no-cpu --sections decode",
            "python3 bench.py --record-traffic <fetch csv> <write csv>"],
        "calibration": "FETCH_SIZE of stream_read_kernel over the bench's 1 GiB buffer and "
                       "WRITE_SIZE of torch's fill of that buffer",
        "per_kernel": per,
    }
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        return 1


def _decode_leg(cases, seconds, tag):
    """Oracle GEMVs on 1024-row blocks of the decode matrices (a new block
    each pass) until `seconds` of oracle time: (GB/s of packed weights,
    calls, rows, bytes, time)."""
    import oracle
    from synth import quant
    t_total, bytes_total, rows_done, calls, p_idx, rows = 0.0, 0, 0, 0, 0, 1024
    while t_total < seconds:
        for c in cases:
            name = f"bench/{c['tag']}/{c['fmt']}"
            p = quant.synthetic_weight(c["fmt"], rows, c["k"], name=f"{name}/cpu{tag}{p_idx}")
            x = quant.synthetic_bf16(c["m"], c["k"], name=name + "/x")
            r = quant.synthetic_bf16(c["m"], rows, name=name + "/r") if c["residual"] else None
            t0 = time.perf_counter()
            oracle.gemv(p, x, r)
            t_total += time.perf_counter() - t0
            bytes_total += p.nbytes()
            rows_done += rows
            calls += 1
            if t_total >= seconds:
                break
        p_idx += 1
    return bytes_total / t_total / 1e9, calls, rows_done, bytes_total, t_total


def _prefill_leg(seconds):
    """Oracle GEMM of 128 activation rows against 256-row blocks of the
    17408 x 5120 affine prefill matrix: GFLOP/s."""
    import oracle
    from synth import formats as F
    from synth import quant
    m, rows, k = 128, 256, 5120
    x = quant.synthetic_bf16(m, k, name="bench/prefill/x128")
    t_total, flops, blocks = 0.0, 0.0, 0
    while t_total < seconds:
        p = quant.synthetic_weight(F.AFFINE4_G64, rows, k, name=f"bench/prefill/cpu{blocks}")
        t0 = time.perf_counter()
        oracle.gemm(p, x)
        t_total += time.perf_counter() - t0
        flops += 2.0 * m * rows * k
        blocks += 1
    return flops / t_total / 1e9, blocks, t_total


def _moe_leg(seconds):
    """The oracle's MoE layer on 4 tokens, top-10 routed + 1 shared expert of
    the hidden 2048 / intermediate 512 NVFP4 shape, over a pool of 32 routed
    experts (the per-token work is the full layer's; only the pool of
    weights it draws from is smaller): tokens/s."""
    import oracle
    from synth import formats as F
    from synth import quant, routing
    E, S, H, I, T, topk = 32, 1, 2048, 512, 4, 10
    gu = quant.synthetic_weight(F.NVFP4, 2 * I, H, batch=E + S, name="bench/moe/cpu_gu")
    dn = quant.synthetic_weight(F.NVFP4, H, I, batch=E + S, name="bench/moe/cpu_dn")
    t_total, tokens, calls = 0.0, 0, 0
    while t_total < seconds:
        x = quant.synthetic_bf16(T, H, name=f"bench/moe/cpu_x{calls}")
        ids, w = oracle.router(routing.router_logits(T, E, name=f"bench/moe/cpu_r{calls}"), topk)
        t0 = time.perf_counter()
        oracle.moe(gu, dn, x, ids, w.astype(np.float32), E, S)
        t_total += time.perf_counter() - t0
        tokens += T
        calls += 1
    return tokens / t_total, calls, t_total


def cpu_baseline(cases, seconds):
    """The oracle as it stands (float64 numpy; its matrix products use the
    BLAS thread pool), timed on bounded samples of the workloads, on this
    host's cores.  value = the decode leg's GB/s of packed weights with every
    BLAS thread; beside it the same leg on one thread, a prefill GEMM leg and
    an MoE layer leg."""
    threads = _blas_threads()
    gbs, calls, rows_done, bytes_total, t_dec = _decode_leg(cases, 0.45 * seconds, "a")
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            gbs1, calls1, _, _, t1 = _decode_leg(cases, 0.2 * seconds, "b")
    except Exception:
        gbs1, calls1, t1 = None, 0, 0.0
    gf, blocks, t_pre = _prefill_leg(0.15 * seconds)
    tok, mcalls, t_moe = _moe_leg(0.2 * seconds)
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"decode leg: 1024-row blocks of the decode matrices ({calls} oracle calls, "
                      f"{rows_done} rows, {bytes_total / 1e6:.1f} MB of packed weights, "
                      f"{t_dec:.1f} s), float64 numpy oracle, {threads} BLAS threads",
            "nproc": os.cpu_count(), "cpu_model": _cpu_model(),
            "one_thread": {"value": None if gbs1 is None else round(gbs1, 4), "unit": "GB/s",
                           "sample": f"decode leg again on 1 thread ({calls1} calls, {t1:.1f} s)"},
            "prefill": {"value": round(gf, 3), "unit": "GFLOP/s",
                        "sample": f"128 x 5120 bf16 activations against {blocks} blocks of 256 rows "
                                  f"of the 17408 x 5120 affine4_g64 matrix ({t_pre:.1f} s)"},
            "moe": {"value": round(tok, 2), "unit": "tokens/s",
                    "sample": f"{mcalls} layers of 4 tokens, top-10 of 32 routed + 1 shared "
                              f"NVFP4 experts, hidden 2048, intermediate 512 ({t_moe:.1f} s)"}}


FMT_NAME = {1: "affine4_g64", 2: "mxfp4", 3: "nvfp4", 4: "q6_k"}


def prefill_section(q, torch, dev):
    from synth import formats as F
    from synth import quant
    out = []
    n, k = 17408, 5120
    for fmt in (F.AFFINE4_G64, F.NVFP4):
        w = q.Weight.from_host(quant.synthetic_weight(fmt, n, k, name=f"bench/prefill/{fmt}"), dev)
        for m in (128, 512, 2048, 8192):
            x = dev_bf16(torch, quant.synthetic_bf16(m, k, name=f"bench/prefill/x{m}"), dev)
            y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            call = q.prepare_gemm(w, x, y)
            reps = 20 if m <= 512 else 8
            med, _ = timed(torch, call, reps)
            tf = 2.0 * m * n * k / (med * 1e-3) / 1e12
            out.append({"format": FMT_NAME[fmt], "m": m, "shape": f"{n}x{k}", "ms": round(med, 4),
                        "TFLOPs": round(tf, 1),
                        "frac_bf16_mfma_peak": round(tf / BF16_MFMA_PEAK_TFLOPS, 4)})
            del x, y, call
        del w
        torch.cuda.empty_cache()
    big = [c for c in out if c["m"] >= 2048]
    best = max(big, key=lambda c: c["TFLOPs"])
    mfma_peak = measured_mfma_peak(q, torch, dev)
    for c in out:
        c["frac_measured_mfma_peak"] = round(c["TFLOPs"] / mfma_peak["TFLOPs"], 4)
    # W4A4: the same 17408 x 5120 matrix in MXFP4 against activations
    # quantized to MXFP4 on the GPU (qquant_mxfp4 + FP4 MFMA GEMM, both timed)
    w4 = []
    w = q.Weight.from_host(quant.synthetic_weight(F.MXFP4, n, k, name="bench/prefill/w4a4"), dev)
    for m in (128, 512, 2048, 8192):
        x = dev_bf16(torch, quant.synthetic_bf16(m, k, name=f"bench/prefill/x{m}"), dev)
        y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        call = q.prepare_gemm_w4a4(w, x, y)
        med, _ = timed(torch, call, 20 if m <= 512 else 8)
        tf = 2.0 * m * n * k / (med * 1e-3) / 1e12
        w4.append({"format": "mxfp4 weights x mxfp4 activations", "m": m, "shape": f"{n}x{k}",
                   "ms": round(med, 4), "TFLOPs": round(tf, 1),
                   "frac_fp4_mfma_peak": round(tf / FP4_MFMA_PEAK_TFLOPS, 4),
                   "frac_bf16_mfma_peak": round(tf / BF16_MFMA_PEAK_TFLOPS, 4)})
        del x, y, call
    del w
    torch.cuda.empty_cache()
    return {"unit": "TFLOP/s", "kernel": "gemm_big_kernel (dequant in registers, bf16 MFMA)",
            "peak_TFLOPs": BF16_MFMA_PEAK_TFLOPS, "measured_mfma_peak": mfma_peak,
            "best_at_M_ge_2048": best, "cases": out,
            "w4a4": {"kernel": "quant_mxfp4_kernel + gemm_w4a4_kernel "
                               "(v_mfma_scale_f32_32x32x64_f8f6f4)",
                     "peak_TFLOPs": FP4_MFMA_PEAK_TFLOPS, "cases": w4}}


def mid_section(q, torch, dev):
    """qgemm at 5 and 8 rows (the mid band: the row-streaming GEMV) and 16
    rows (MFMA tiles) on 17408 x 5120, cold weights: microseconds and weight
    GB/s."""
    from synth import formats as F
    from synth import quant
    out = []
    n, k = 17408, 5120
    for fmt in (F.AFFINE4_G64, F.NVFP4):
        p = quant.synthetic_weight(fmt, n, k, name=f"bench/mid/{fmt}")
        w0 = q.Weight.from_host(p, dev)
        copies = max(2, int(np.ceil(800e6 / w0.nbytes())))
        ws_ = [w0] + [q.Weight.from_host(p, dev) for _ in range(copies - 1)]
        del p
        for m in (5, 8, 16):
            x = dev_bf16(torch, quant.synthetic_bf16(m, k, name=f"bench/mid/x{m}"), dev)
            y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            calls = [q.prepare_gemm(w, x, y) for w in ws_]
            it = iter(range(1 << 30))
            med, _ = timed(torch, lambda: calls[next(it) % copies](), 4 * copies)
            out.append({"format": FMT_NAME[fmt], "m": m, "shape": f"{n}x{k}",
                        "us": round(med * 1e3, 2),
                        "path": "row-streaming GEMV" if m <= 8 else "MFMA tiles",
                        "weight_GBps": round(w0.nbytes() / (med * 1e-3) / 1e9, 1)})
            del x, y, calls
        del ws_, w0
        torch.cuda.empty_cache()
    return {"unit": "us per call", "cases": out}


def moe_section(q, torch, dev):
    """The MoE layer on the GPU.  Routing comes from the library's own router
    (qmoe_router) on N(0, 1) logits, as a model would run it.

    T = 4 is timed two ways: warm (the same call back to back, so the ~72 MB
    of touched experts can stay in the 256 MB Infinity Cache) and cold (calls
    rotate over 8 device copies of the layer's weights and 16 routings, so
    that about 500 MB of other expert weights pass between two reads of the
    same bytes)."""
    from synth import formats as F
    from synth import quant, routing
    E, S, H, I, topk = 512, 1, 2048, 512, 10
    gu_p = quant.synthetic_weight(F.NVFP4, 2 * I, H, batch=E + S, name="bench/moe/gate_up")
    dn_p = quant.synthetic_weight(F.NVFP4, H, I, batch=E + S, name="bench/moe/down")
    gu, dn = q.Weight.from_host(gu_p, dev), q.Weight.from_host(dn_p, dev)
    del gu_p, dn_p
    per_expert = (gu.nbytes() + dn.nbytes()) / (E + S)
    copies, n_route = 8, 16

    def clone(w):
        return q.Weight(w.fmt, w.n, w.k, w.batch, w.codes.clone(), w.scales.clone(), None, None,
                        w.tensor_scale.clone())

    out = []
    for T, ydt in ((4, torch.float32), (8192, torch.bfloat16)):
        x = dev_bf16(torch, quant.synthetic_bf16(T, H, name=f"bench/moe/x{T}"), dev)
        lg = torch.from_numpy(routing.router_logits(T, E, name=f"bench/moe/r{T}")).to(dev)
        ids, wts = q.moe_router(lg, topk)
        y = torch.empty((T, H), dtype=ydt, device=dev)
        call = q.prepare_moe(gu, dn, x, ids, wts, E, S, y)
        med, _ = timed(torch, call, 20 if T == 4 else 8)
        layout = q.moe_workspace_layout(gu, dn, E, S, T, topk)
        decode_form = layout["slot_rows"] == 1
        if decode_form:
            launches = 2
        else:
            launches = 3 + (1 if T * topk <= 16384 else 3)  # route, gate/up, down, combine
        rows = T * (topk + S)
        flops = 2.0 * rows * (2 * I * H + H * I)
        active = len(np.unique(ids.cpu().numpy())) + S
        c = {"tokens": T, "ms": round(med, 4), "rows": rows, "active_experts": int(active),
             "TFLOPs": round(flops / (med * 1e-3) / 1e12, 2),
             "active_weight_GBps": round(active * per_expert / (med * 1e-3) / 1e9, 1),
             "y_dtype": "bf16" if ydt == torch.bfloat16 else "f32",
             "form": "decode (grouped GEMV over token slots)" if decode_form else
                     "grouped (route, gate/up GEMM, down GEMM, combine)",
             "launches": launches, "routing": "qmoe_router on N(0, 1) logits"}
        # the router's top-k and softmax on the GPU (qmoe_router) for the same
        # tokens, timed alone, and the layer from router logits (router + layer)
        rid = torch.empty((T, topk), dtype=torch.int32, device=dev)
        rw = torch.empty((T, topk), dtype=torch.float32, device=dev)
        rmed, _ = timed(torch, lambda: q.moe_router(lg, topk, rid, rw), 20)
        c["router_us"] = round(rmed * 1e3, 2)
        ws = torch.empty(q.moe_workspace_size(gu, dn, E, S, T, topk), dtype=torch.uint8, device=dev)
        lmed, _ = timed(torch, lambda: q.moe_from_logits(gu, dn, x, lg, topk, E, S, y_dtype=ydt,
                                                         out=y, workspace=ws), 20 if T == 4 else 8)
        c["ms_from_logits"] = round(lmed, 4)
        if T == 4:
            c["ms_warm"] = c["ms"]
            wcopies = [(gu, dn)] + [(clone(gu), clone(dn)) for _ in range(copies - 1)]
            lgs = [torch.from_numpy(routing.router_logits(T, E, name=f"bench/moe/cold{j}")).to(dev)
                   for j in range(n_route)]
            routes = [q.moe_router(g, topk) for g in lgs]
            calls = [q.prepare_moe(wcopies[j % copies][0], wcopies[j % copies][1], x, routes[j][0],
                                   routes[j][1], E, S, y) for j in range(n_route)]
            it = iter(range(1 << 30))
            cmed, _ = timed(torch, lambda: calls[next(it) % n_route](), 4 * n_route)
            it2 = iter(range(1 << 30))
            ws2 = torch.empty(q.moe_workspace_size(gu, dn, E, S, T, topk), dtype=torch.uint8,
                              device=dev)

            def from_logits_cold():
                j = next(it2) % n_route
                q.moe_from_logits(wcopies[j % copies][0], wcopies[j % copies][1], x, lgs[j], topk,
                                  E, S, y_dtype=ydt, out=y, workspace=ws2)

            clmed, _ = timed(torch, from_logits_cold, 4 * n_route)
            act = [len(np.unique(r[0].cpu().numpy())) + S for r in routes]
            c["ms_cold"] = round(cmed, 4)
            c["ms_from_logits_cold"] = round(clmed, 4)
            c["active_weight_GBps_cold"] = round(float(np.mean(act)) * per_expert / (cmed * 1e-3) / 1e9, 1)
            c["cold_rotation"] = (f"{copies} device copies of the layer's weights x {n_route} "
                                  "routings, one call each in turn")
            del wcopies, calls, routes, lgs, ws2
            torch.cuda.empty_cache()
        out.append(c)
        del x, y, call, lg, ws
    return {"unit": "ms per layer",
            "config": "512 routed + 1 shared experts, hidden 2048, intermediate 512, nvfp4, top-10",
            "cases": out}


def fp4_section(q, torch, dev):
    from synth import formats as F
    from synth import quant
    out = []
    for fmt in (F.MXFP4, F.NVFP4):
        for n, k in ((5120, 5120), (5120, 6144), (248320, 5120)):
            p = quant.synthetic_weight(fmt, n, k, outlier_rate=0.01, name=f"bench/fp4/{fmt}/{n}x{k}")
            w0 = q.Weight.from_host(p, dev)
            copies = max(2, int(np.ceil(1.0e9 / w0.nbytes())))
            ws_ = [w0] + [q.Weight.from_host(p, dev) for _ in range(copies - 1)]
            del p
            for m in (1, 2, 3, 4):
                x = dev_bf16(torch, quant.synthetic_bf16(m, k, name=f"bench/fp4/x{m}/{k}"), dev)
                y = torch.empty((m, n), dtype=torch.float32, device=dev)
                need = q.gemv_workspace_size(w0, m)
                wsp = q.new_workspace(need, dev) if need else None
                calls = [q.PreparedGemv(w, x, y, None, wsp) for w in ws_]
                it = iter(range(1 << 30))
                med, _ = timed(torch, lambda: calls[next(it) % copies](), 4 * copies if copies > 2 else 10)
                gbs = w0.nbytes() / (med * 1e-3) / 1e9
                out.append({"format": FMT_NAME[fmt], "shape": f"{n}x{k}", "m": m,
                            "us": round(med * 1e3, 2), "weight_GBps": round(gbs, 1),
                            "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1)})
            del ws_, w0
            torch.cuda.empty_cache()
    return {"unit": "GB/s", "cases": out}


def hadamard_section(q, torch, dev):
    """qgemv_hadamard (prepare, GEMV and finish in one call) against the
    three calls (qhadamard_prepare, qgemv, qhadamard_finish) and the GEMV
    alone, on the 17408 x 5120 affine matrix, cold weights, float32 y."""
    from synth import formats as F
    from synth import quant
    out = []
    n, k = 17408, 5120
    p = quant.synthetic_weight(F.AFFINE4_G64, n, k, name="bench/had/w")
    w0 = q.Weight.from_host(p, dev)
    copies = max(2, int(np.ceil(800e6 / w0.nbytes())))
    ws_ = [w0] + [q.Weight.from_host(p, dev) for _ in range(copies - 1)]
    del p
    g = torch.Generator().manual_seed(7)
    si = (torch.rand(k, generator=g) * 4 - 2).to(torch.float16).to(dev)
    so = (torch.rand(n, generator=g) * 4 - 2).to(torch.float16).to(dev)
    for m in (1, 4):
        x = dev_bf16(torch, quant.synthetic_bf16(m, k, name=f"bench/had/x{m}"), dev)
        y = torch.empty((m, n), dtype=torch.float32, device=dev)
        xp = torch.empty_like(x)
        ylin = torch.empty((m, n), dtype=torch.float32, device=dev)
        it = iter(range(1 << 30))
        # argument checks done once: plain C calls in the timed loops
        q.gemv_hadamard(w0, x, si, so, out=y)
        lib = q.lib_handle()
        P = lambda t: ctypes.c_void_p(t.data_ptr())
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        px, pxp, py, pyl, psi, pso = P(x), P(xp), P(y), P(ylin), P(si), P(so)
        need = int(lib.qgemv_hadamard_workspace_size(w0.c, m, q.F32))
        wsh = q.new_workspace(need, dev)
        pws = P(wsh)

        def fused():
            rc = lib.qgemv_hadamard(ws_[next(it) % copies].c, px, m, psi, pso, py, q.F32, pws,
                                    need, st)
            assert rc == 0, rc

        def plain():
            rc = lib.qgemv(ws_[next(it) % copies].c, pxp, m, None, pyl, q.F32, None, 0, st)
            assert rc == 0, rc

        def staged():
            rc = lib.qhadamard_prepare(px, m, k, psi, pxp, st)
            rc |= lib.qgemv(ws_[next(it) % copies].c, pxp, m, None, pyl, q.F32, None, 0, st)
            rc |= lib.qhadamard_finish(pyl, m, n, pso, py, q.F32, st)
            assert rc == 0, rc

        fm, _ = timed(torch, fused, 4 * copies)
        sm, _ = timed(torch, staged, 4 * copies)
        gm, _ = timed(torch, plain, 4 * copies)
        out.append({"format": "affine4_g64", "shape": f"{n}x{k}", "m": m,
                    "us_one_call": round(fm * 1e3, 2), "us_three_calls": round(sm * 1e3, 2),
                    "us_gemv_alone": round(gm * 1e3, 2)})
    del ws_, w0
    torch.cuda.empty_cache()
    return {"unit": "us per call", "cases": out}


def main():
    args = parse()
    if args.record_traffic:
        record_traffic(*args.record_traffic)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); no multi-GPU run is "
              "made.", file=sys.stderr)
        sys.exit(2)
    import torch

    import gemm_dequant_gemv_amd as q
    from synth import quant

    sections = set(s for s in args.sections.split(",") if s)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    cases = decode_cases()
    # distinct weights per case (one per lane count) -> 12 matrices, ~740 MB
    setup = []
    for c in cases:
        name = f"bench/{c['tag']}/{c['fmt']}"
        p = quant.synthetic_weight(c["fmt"], c["n"], c["k"], name=f"{name}/W{c['m']}")
        w = q.Weight.from_host(p, dev)
        x = dev_bf16(torch, quant.synthetic_bf16(c["m"], c["k"], name=name + "/x"), dev)
        r = dev_bf16(torch, quant.synthetic_bf16(c["m"], c["n"], name=name + "/r"), dev) \
            if c["residual"] else None
        y = torch.empty((c["m"], c["n"]), dtype=torch.float32, device=dev)
        need = q.gemv_workspace_size(w, c["m"])
        ws = q.new_workspace(need, dev) if need else None
        call = q.PreparedGemv(w, x, y, r, ws)
        setup.append((c, w, w.nbytes(), call))
    torch.cuda.synchronize()

    def step(bracket=None):
        # arguments are marshalled once (PreparedGemv), so the host enqueues
        # far faster than the GPU drains; `bracket` = (case index, events)
        # puts an event pair around that one launch
        for i, item in enumerate(setup):
            if bracket is not None and bracket[0] == i:
                bracket[1][0].record()
            item[3]()
            if bracket is not None and bracket[0] == i:
                bracket[1][1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K steps back to back, one HIP event pair on the launch
    # stream around all of them, host clock with a synchronize on both sides
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g0.record()
    for s in range(args.steps):
        step()
    g1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_step_ms = g0.elapsed_time(g1) / args.steps

    # per-case detail (outside the timed region): each case bracketed by its
    # own event pair inside otherwise unmarked steps, so every launch still
    # reads cold weights behind the other cases; the bracket adds the event
    # packets (about 2 us) to the case's time
    detail_reps = 5
    case_ms = [[] for _ in setup]
    for r in range(detail_reps):
        for i in range(len(setup)):
            ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            step((i, ev))
            torch.cuda.synchronize()
            case_ms[i].append(ev[0].elapsed_time(ev[1]))

    read_peak = measured_read_peak(q, torch, dev)

    per_case = []
    tot_w, tot_alg = 0, 0
    for i, (c, w, wb, _) in enumerate(setup):
        med = float(np.median(case_ms[i]))
        tot_w += wb
        tot_alg += algorithmic_bytes(wb, c)
        per_case.append({"format": FMT_NAME[c["fmt"]], "shape": f"{c['n']}x{c['k']}", "m": c["m"],
                         "residual": c["residual"], "us_event_bracketed": round(med * 1e3, 2),
                         "weight_GBps": round(wb / (med * 1e-3) / 1e9, 1),
                         "pct_hbm_peak": round(100 * wb / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 1)})
    step_s = wall / args.steps
    value = tot_w / step_s / 1e9
    launch_s = gpu_step_ms * 1e-3 / len(setup)
    achieved = tot_alg / (gpu_step_ms * 1e-3) / 1e9
    del setup
    torch.cuda.empty_cache()

    extra = {}
    if "prefill" in sections:
        extra["prefill"] = prefill_section(q, torch, dev)
    if "mid" in sections:
        extra["mid"] = mid_section(q, torch, dev)
    if "moe" in sections:
        extra["moe"] = moe_section(q, torch, dev)
    if "fp4" in sections:
        extra["fp4"] = fp4_section(q, torch, dev)
    if "hadamard" in sections:
        extra["hadamard"] = hadamard_section(q, torch, dev)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "decode matvecs, affine4_g64 and q6_k, 17408x5120 and "
                               "5120x17408 (+bf16 residual), M=1,2,4, cold weights",
                   "calls_per_step": len(cases),
                   "weight_bytes_per_step": tot_w},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profile(),
                     "kernel": "qgemv row-streaming kernel (gemv_rows_kernel)",
                     "algorithmic_bytes_per_launch": int(tot_alg / len(cases)),
                     "mean_launch_us": round(launch_s * 1e6, 2),
                     "launch_time": "GPU time of the timed steps (one HIP event pair) / launches",
                     "measured_read_peak": read_peak,
                     "frac_of_measured_read_peak": round(achieved / read_peak["GBps"], 4)},
        "detail": per_case,
        "sections": extra,
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(cases, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
