"""Benchmark of the binary sign-GEMV hot path on one MI355X.

Workload (the metric's configuration): a LLaMA-7B-shaped projection,
M = N = 4096, K = 2 greedy residual binary bases with fp16 column scales,
bf16 activations, batch 1 -- seeded synthetic weights W ~ N(0, 0.02) and
x ~ N(0, 1), packed on the GPU by bsq_pack.  One step is one bs_gemv call
(the whole hot path of this workload: activation tables, sign-word scan,
row scales, cross-split reduction).

The weights are replicated into enough distinct copies (>= 512 MiB in
total) that consecutive steps never find their sign words in the 256 MiB
last-level cache: every step streams its operands from HBM.  Activations
and outputs rotate with the weights.

Prints one JSON line.  `value` is the effective bandwidth (algorithmic
bytes read per GEMV / time per GEMV); the roofline block relates the same
quantity to the 8 TB/s HBM3E peak; cpu_baseline times the CPU oracle on a
sample of the same product.
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

METRIC = "µs/GEMV + effective HBM GB/s (% of peak), 4096×4096 2-base, bs=1"
HBM_PEAK_GBS = 8000.0
ROTATE_BYTES = 512 << 20


def alg_bytes(M, N, K, B, colscale, x_bytes):
    """Bytes the product must read once: sign words, row scales, column scales, x."""
    return K * M * N // 8 + K * M * 4 + (K * N * 2 if colscale else 0) + N * B * x_bytes


def cpu_baseline(W_bits, alpha, cs, x, M, N, K, budget_s=10.0):
    """Time the oracle (plain C, fp64, one bit at a time, single thread) on a
    bounded sample of the same product: whole-product repetitions, or a row
    sample when one repetition exceeds the budget."""
    import oracle
    t0 = time.perf_counter()
    oracle.sign_gemv(W_bits[:, :64], K, 64, N, alpha[:, :64], x, cs)
    per_row = (time.perf_counter() - t0) / 64
    rows = M if per_row * M <= budget_s else max(64, int(budget_s / per_row))
    reps = max(1, int(budget_s / (per_row * rows)))
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.sign_gemv(np.ascontiguousarray(W_bits[:, :rows]), K, rows, N, alpha[:, :rows], x, cs)
    dt = (time.perf_counter() - t0) / reps
    sec_per_gemv = dt * M / rows
    b = alg_bytes(M, N, K, 1, cs is not None, 2)
    return {"value": round(b / sec_per_gemv / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "%d of %d rows x %d repetition(s), single-threaded C fp64 oracle, scaled to one "
                      "full %dx%d K=%d GEMV" % (rows, M, reps, M, N, K),
            "us_per_gemv": round(sec_per_gemv * 1e6, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only (the sign-GEMV path needs no collectives); "
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
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    ms_per_step = ms / args.steps

    # per-launch durations, each bracketed by its own events on the launch stream
    nper = min(args.steps, 200)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nper)]
    for i in range(nper):
        evs[i][0].record(stream)
        step(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(b) for a, b in evs]) * 1e3  # us
    kernel_us = float(np.median(per))

    b_alg = alg_bytes(M, N, K, B, cs is not None, 2)
    gbs = b_alg / (ms_per_step * 1e-3) / 1e9
    achieved = b_alg / (kernel_us * 1e-6) / 1e9
    traffic = None
    tpath = os.path.join(ROOT, "profiles", "bs_gemv_4096x4096_k2_traffic.json")
    if os.path.exists(tpath):
        try:
            traffic = json.load(open(tpath)).get("bytes_per_launch")
        except Exception:
            traffic = None

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
        "data": "synthetic",
        "config": {"workload": w.name, "M": M, "N": N, "K": K, "B": B, "x_dtype": "bf16", "colscale": True,
                   "rotating_copies": ncopy, "rotating_bytes": ncopy * per_copy},
        "us_per_gemv": round(ms_per_step * 1e3, 3),
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "alg_bytes_per_gemv": b_alg,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel_us_median_events": round(kernel_us, 3)},
    }
    if not args.no_cpu:
        import oracle
        from bit_gemv_packed_amd import synth as _s  # noqa: F401
        Lb = bsg.bsg_layout_to_logical(bits, K, M, N).cpu().numpy().view(np.uint32)
        xh = synth.activations(w, 0, N, 1)
        out["cpu_baseline"] = cpu_baseline(Lb, alpha.cpu().numpy(), cs.cpu().numpy().view(np.uint16), xh,
                                           M, N, K, args.cpu_budget)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
