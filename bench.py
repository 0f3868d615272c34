"""Benchmark of the binary sign-GEMV hot path on one MI355X.

Workload (the metric's configuration): a LLaMA-7B-shaped projection,
M = N = 4096, K = 2 greedy residual binary bases with fp16 column scales,
bf16 activations, batch 1 -- seeded synthetic weights W ~ N(0, 0.02) and
x ~ N(0, 1), packed on the GPU by bsq_pack.  One step is one bs_gemv call,
the whole hot path of this workload (activation staging and tables, the
sign-word scan, row scales and the reduction, the y write).

The packed weights are replicated into enough distinct copies (>= 512 MiB)
that consecutive steps never find their sign words in the 256 MiB
last-level cache: every step streams its operands from HBM.  Activations
and outputs rotate with the weights.  The K timed steps are captured once
into a HIP graph and replayed, so the time is the GPU's, not the host's
launch rate (--eager times plain launches instead).

Prints one JSON line.  `value` is the effective bandwidth (algorithmic
bytes per GEMV / time per GEMV); `roofline` relates it to the 8 TB/s HBM3E
peak, with `traffic` the HBM bytes per launch measured by the FETCH_SIZE /
WRITE_SIZE counters (profiles/bs_gemv_4096x4096_k2_traffic.json, written by
--pmc-summary from two rocprofv3 --pmc runs of this script); cpu_baseline
times the CPU oracle on a sample of the same product.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs/GEMV + effective HBM GB/s (% of peak), 4096×4096 2-base, bs=1"
HBM_PEAK_GBS = 8000.0
ROTATE_BYTES = 512 << 20
CALIB_BYTES = 256 << 20  # size of the plain copy that scales the traffic counters
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "bs_gemv_4096x4096_k2_traffic.json")
KERNEL_SOURCES = ["bsg_gemv.hip", "bsg_prod.h", "bsg_internal.h"]
KERNEL_PREFIX = "bsg::k_prod_f"


def alg_bytes(M, N, K, B, colscale, x_bytes):
    """Bytes the product must read once: sign words, row scales, column scales, x."""
    return K * M * N // 8 + K * M * 4 + (K * N * 2 if colscale else 0) + N * B * x_bytes


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "bit_gemv_packed_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def cpu_baseline(W_bits, alpha, cs, x, M, N, K, budget_s=10.0):
    """Time the oracle (plain C, fp64, one bit at a time) on a bounded sample
    of the same product, on one host thread and then on all host threads
    (row slices in a thread pool; the C call releases the interpreter lock)."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor

    t0 = time.perf_counter()
    oracle.sign_gemv(np.ascontiguousarray(W_bits[:, :64]), K, 64, N, alpha[:, :64], x, cs)
    per_row = (time.perf_counter() - t0) / 64
    rows = M if per_row * M <= budget_s else max(64, int(budget_s / per_row))
    reps = max(1, int(budget_s / (per_row * rows)))
    Wr = np.ascontiguousarray(W_bits[:, :rows])
    ar = np.ascontiguousarray(alpha[:, :rows])
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.sign_gemv(Wr, K, rows, N, ar, x, cs)
    dt1 = (time.perf_counter() - t0) / reps
    sec1 = dt1 * M / rows
    b = alg_bytes(M, N, K, 1, cs is not None, 2)
    out = {"value": round(b / sec1 / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": "%d of %d rows of one %dx%d K=%d GEMV, %d time(s), on one host thread (C fp64 oracle), "
                     "scaled to one full GEMV" % (rows, M, M, N, K, reps),
           "us_per_gemv": round(sec1 * 1e6, 1)}

    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    if threads > 1:
        rows_p = min(M, rows * threads)
        rows_p -= rows_p % threads
        step = rows_p // threads
        parts = [(np.ascontiguousarray(W_bits[:, i * step:(i + 1) * step]),
                  np.ascontiguousarray(alpha[:, i * step:(i + 1) * step])) for i in range(threads)]
        def work(p):
            for _ in range(reps):
                oracle.sign_gemv(p[0], K, step, N, p[1], x, cs)

        with ThreadPoolExecutor(threads) as ex:
            t0 = time.perf_counter()
            list(ex.map(work, parts))
            dtp = (time.perf_counter() - t0) / reps
        secp = dtp * M / rows_p
        out["all_threads"] = {"value": round(b / secp / 1e9, 4), "cores": threads,
                              "sample": "%d rows in %d slices, one host thread each, %d time(s)"
                                        % (rows_p, threads, reps),
                              "us_per_gemv": round(secp * 1e6, 1)}
    return out


# ------------------------------------------------------------------ counters

def _pmc_rows(d):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under %s" % d)
    rows = []
    for f in files:
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def _per_dispatch(rows, counter, pick):
    vals = {}
    for r in rows:
        if r["Counter_Name"] == counter and pick(r["Kernel_Name"]):
            vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return [vals[k] for k in sorted(vals, key=int)]


def pmc_summary(fetch_dir, write_dir):
    """Traffic per launch of the product kernel from two rocprofv3 --pmc runs
    (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each scaled by what the same
    counter reads for the calibration copy of CALIB_BYTES (read and write)."""
    is_prod = lambda n: KERNEL_PREFIX in n
    is_copy = lambda n: KERNEL_PREFIX not in n and "bsg::" not in n
    out = {"kernel": KERNEL_PREFIX, "source_hash": kernel_source_hash(), "calibration_bytes": CALIB_BYTES}
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _pmc_rows(d)
        prod = _per_dispatch(rows, name, is_prod)
        copy = _per_dispatch(rows, name, is_copy)
        copy_big = [v for v in copy if v * 1024 > CALIB_BYTES / 2]  # the calibration copies
        if not prod or not copy_big:
            raise SystemExit("%s: %d product / %d calibration dispatches" % (name, len(prod), len(copy_big)))
        factor = CALIB_BYTES / (float(np.median(copy_big)) * 1024)
        kib = float(np.median(prod[len(prod) // 4:]))  # skip warm-up dispatches
        out[name] = {"kib_per_dispatch_median": round(kib, 2), "dispatches": len(prod),
                     "calibration_kib": round(float(np.median(copy_big)), 1), "scale": round(factor, 4),
                     "bytes_per_launch": int(kib * 1024 * factor)}
    out["bytes_per_launch"] = out["FETCH_SIZE"]["bytes_per_launch"] + out["WRITE_SIZE"]["bytes_per_launch"]
    return out


def load_traffic():
    if not os.path.exists(TRAFFIC_JSON):
        return None
    try:
        t = json.load(open(TRAFFIC_JSON))
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != kernel_source_hash():
        return None  # taken on another version of the kernel
    return t.get("bytes_per_launch")


# ------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--eager", action="store_true", help="time plain launches instead of a graph replay")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--traffic-calib", action="store_true",
                    help="also run a plain %d MiB copy kernel (for scaling the traffic counters)" % (CALIB_BYTES >> 20))
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the traffic summary from two rocprofv3 --pmc output folders and exit")
    args = ap.parse_args()
    if args.pmc_summary:
        t = pmc_summary(*args.pmc_summary)
        with open(TRAFFIC_JSON, "w") as fh:
            json.dump(t, fh, indent=1)
        print(json.dumps(t))
        return
    if args.gpus != 1:
        print("bench.py: the sign-GEMV path runs on one GPU (no collectives, no sharding are built); "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_gemv_packed_amd as bsg
    from bit_gemv_packed_amd import synth

    dev = torch.device("cuda:0")
    w = synth.WORKLOADS[2]
    M, N, K, B = w.shapes[0].M, w.shapes[0].N, w.K, 1
    W = synth.weights(w.wid, 0, M, N)
    bits, alpha, cs = bsg.bsq_pack(torch.from_numpy(W).to(dev), K, colscale=w.colscale)
    torch.cuda.synchronize()

    per_copy = bits.numel() * 4 + alpha.numel() * 4 + (cs.numel() * 2 if cs is not None else 0)
    ncopy = max(2, -(-ROTATE_BYTES // per_copy))
    bits_r = bits.unsqueeze(0).repeat(ncopy, 1).contiguous()
    alpha_r = alpha.unsqueeze(0).repeat(ncopy, 1, 1).contiguous()
    cs_r = cs.unsqueeze(0).repeat(ncopy, 1, 1).contiguous() if cs is not None else None
    xs = torch.from_numpy(np.ascontiguousarray(synth.activations(w, 0, N, ncopy).T)).to(torch.bfloat16).to(dev)
    ys = torch.empty((ncopy, M), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step(i):
        c = i % ncopy
        bsg.bs_gemv(bits_r[c], K, M, N, alpha_r[c], xs[c], colscale=cs_r[c] if cs_r is not None else None,
                    y=ys[c])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    graph = None
    if not args.eager:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(args.steps):
                step(args.warmup + i)
        graph.replay()  # first replay uploads the graph
        torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for i in range(args.steps):
            step(args.warmup + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps

    # eager launches for comparison (includes the host's launch rate)
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    eager_ms = ev0.elapsed_time(ev1) / args.steps

    if args.traffic_calib:
        src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    b_alg = alg_bytes(M, N, K, B, cs is not None, 2)
    gbs = b_alg / (ms_per_step * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded W ~ N(0, 0.02) packed on the GPU, x ~ N(0, 1) in bf16)",
        "config": {"workload": "%s: %dx%d, K=%d, fp16 column scales, bf16 x, batch %d" % (w.name, M, N, K, B),
                   "M": M, "N": N, "K": K, "B": B, "x_dtype": "bf16", "colscale": True,
                   "rotating_copies": ncopy, "rotating_bytes": ncopy * per_copy,
                   "timing": "eager launches" if graph is None else "HIP graph of the timed steps"},
        "us_per_gemv": round(ms_per_step * 1e3, 3),
        "us_per_gemv_eager": round(eager_ms * 1e3, 3),
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "alg_bytes_per_gemv": b_alg,
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": load_traffic()},
    }
    if not args.no_cpu:
        Lb = bsg.bsg_layout_to_logical(bits, K, M, N).cpu().numpy().view(np.uint32)
        xh = synth.activations(w, 0, N, 1)
        out["cpu_baseline"] = cpu_baseline(Lb, alpha.cpu().numpy(), cs.cpu().numpy().view(np.uint16), xh,
                                           M, N, K, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
