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
KERNEL_SOURCES = ["bsg_gemv.hip", "bsg_prod_f.h", "bsg_prod.h", "bsg_internal.h"]
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


# ------------------------------------------------------------------ every row of the path

def _graph_us(step, steps, warmup):
    """Mean µs per call of step(i) over `steps` calls replayed from one HIP graph."""
    import torch
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            step(warmup + i)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / steps


def run_rows(steps, warmup):
    """Time every row of the hot path on the pages' projection shapes (synthetic operands, >= 512 MiB
    of rotating weight copies per case, HIP-graph replay).  Prints one JSON line per case."""
    import torch
    import bit_gemv_packed_amd as bsg
    from bit_gemv_packed_amd import synth
    dev = torch.device("cuda:0")
    out = []

    def emit(row, op, shape, us, nbytes, **extra):
        d = {"row": row, "op": op, "shape": shape, "us": round(us, 3), "alg_bytes": int(nbytes),
             "GB_s": round(nbytes / (us * 1e-6) / 1e9, 1), "pct_hbm_peak": round(100 * nbytes / (us * 1e-6) / 8e12, 2)}
        d.update(extra)
        print(json.dumps(d), flush=True)
        out.append(d)

    def copies(nbytes_per_copy):
        return max(2, -(-ROTATE_BYTES // max(1, nbytes_per_copy)))

    def rand_bits(K, M, N, n):
        return torch.randint(-2**31, 2**31 - 1, (n, bsg.layout_words(K, M, N)), dtype=torch.int32, device=dev)

    def xs(N, B, n, dt=torch.bfloat16):
        return torch.randn((n, N, B), device=dev).to(dt)

    # a1-a3, a7: the sign product
    shapes = [("q/o 4096x4096", 4096, 4096, 2, False), ("k/v 1024x4096", 1024, 4096, 2, False),
              ("gate/up 14336x4096", 14336, 4096, 2, False), ("down 4096x14336", 4096, 14336, 2, False),
              ("4096x4096 colscale", 4096, 4096, 2, True), ("5120x5120 K=3", 5120, 5120, 3, False),
              ("13824x5120", 13824, 5120, 2, False), ("5120x13824", 5120, 13824, 2, False),
              ("28672x8192", 28672, 8192, 2, False)]
    for name, M, N, K, cs in shapes:
        for B in ((1, 4, 16) if name.split()[0] in ("q/o", "gate/up", "down") else (1,)):
            wb = K * M * N // 8 + 4 * K * M + (2 * K * N if cs else 0)
            n = copies(wb)
            bits = rand_bits(K, M, N, n)
            alpha = torch.rand((n, K, M), device=dev) * 0.02
            csd = (torch.rand((n, K, N), device=dev) + 0.5).half().view(torch.int16) if cs else None
            x = xs(N, B, n)
            y = torch.empty((n, M, B), device=dev)
            step = lambda i: bsg.bs_gemv(bits[i % n], K, M, N, alpha[i % n], x[i % n],
                                         colscale=csd[i % n] if cs else None, y=y[i % n])
            emit("a1-a3,a7", "bs_gemv", name, _graph_us(step, steps, warmup), wb + 2 * N * B, K=K, B=B, colscale=cs)
            del bits, alpha, csd, x, y
            torch.cuda.empty_cache()

    # f2: projections that share x in one launch, and a whole decoder layer
    layer = [("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
             ("gate", 14336, 4096), ("up", 14336, 4096), ("down", 4096, 14336)]
    for B in (1, 16):
        K = 2
        wbs = {nm: K * M * N // 8 + 4 * K * M for nm, M, N in layer}
        n = copies(sum(wbs.values()))
        W = {nm: (rand_bits(K, M, N, n), torch.rand((n, K, M), device=dev) * 0.02) for nm, M, N in layer}
        Y = {nm: torch.empty((n, M, B), device=dev) for nm, M, N in layer}
        xa, xo, xm = xs(4096, B, n), xs(4096, B, n), xs(14336, B, n)
        xin = {"q": xa, "k": xa, "v": xa, "o": xo, "gate": xa, "up": xa, "down": xm}
        dims = {nm: (M, N) for nm, M, N in layer}

        def proj(nm, c):
            return (W[nm][0][c], dims[nm][0], W[nm][1][c], None, Y[nm][c])

        def fused(names, c):
            bsg.bs_gemv_multi([proj(nm, c) for nm in names], K, dims[names[0]][1], xin[names[0]][c])

        def single(nm, c):
            bsg.bs_gemv(W[nm][0][c], K, dims[nm][0], dims[nm][1], W[nm][1][c], xin[nm][c], y=Y[nm][c])

        for names, label in [(("q", "k", "v"), "q+k+v 6144x4096"), (("gate", "up"), "gate+up 28672x4096")]:
            by = sum(wbs[nm] for nm in names) + 2 * 4096 * B
            emit("f2", "bs_gemv_multi (1 launch)" if B == 1 else "bs_gemv_multi (1 launch, matrix cores)",
                 label, _graph_us(lambda i: fused(names, i % n), steps, warmup), by, K=K, B=B)
            emit("f2", "bs_gemv, one call per projection", label,
                 _graph_us(lambda i: [single(nm, i % n) for nm in names], steps, warmup), by, K=K, B=B)

        def layer_fused(i):
            c = i % n
            fused(("q", "k", "v"), c)
            single("o", c)
            fused(("gate", "up"), c)
            single("down", c)
        by = sum(wbs.values()) + 2 * B * (4096 * 4 + 14336)
        emit("f2", "decoder layer, 4 calls (q+k+v, o, gate+up, down)", "LLaMA-3-8B layer",
             _graph_us(layer_fused, steps, warmup), by, K=K, B=B)
        emit("f2", "decoder layer, 7 bs_gemv calls", "LLaMA-3-8B layer",
             _graph_us(lambda i: [single(nm, i % n) for nm, _, _ in layer], steps, warmup), by, K=K, B=B)
        del W, Y, xa, xo, xm, xin
        torch.cuda.empty_cache()

    # f3: group-wise fp16 row scales (FluxBin Kb-g128) and the salient columns read through the
    # Virtual Columnar Mapping (Kb-sS-g128), on LLaMA-2-7B projection shapes, fp16 x (FluxBin's
    # models run in fp16); batch 16 on the matrix cores
    for name, M, N in [("q/o 4096x4096", 4096, 4096), ("gate/up 11008x4096", 11008, 4096),
                       ("down 4096x11008", 4096, 11008)]:
        K, g = 2, 128
        G = N // g
        for B in (1, 16):
            for s in (0, 8, 16):
                S = s * G
                nds = (S + 31) // 32
                gpw = 32 // s if s else 1
                wb = K * M * N // 8 + 2 * K * M * G + 2 * K * N
                if s:
                    wb += 4 * K * M * nds + 2 * K * nds * M * gpw + 2 * K * S + 4 * S
                n = copies(wb)
                bits = rand_bits(K, M, N, n)
                al = (torch.rand((n, K, G, M), device=dev) * 0.02).half().view(torch.int16)
                csd = (torch.rand((n, K, N), device=dev) + 0.5).half().view(torch.int16)
                x = xs(N, B, n, torch.float16)
                y = torch.empty((n, M, B), device=dev)
                if s:
                    sb = rand_bits(K, M, nds * 32, n)
                    sa = (torch.rand((n,) + bsg.salient_scale_shape(K, M, N, g, s), device=dev) * 0.01).half() \
                        .view(torch.int16)
                    sc = (torch.rand((n, K, S), device=dev) + 0.5).half().view(torch.int16)
                    # s distinct columns of every group of g per copy (seeded, drawn on the host)
                    keys = np.random.default_rng([7, M, N, s]).random((n, G, g))
                    pick = np.sort(np.argsort(keys, axis=2)[:, :, :s], axis=2) + (np.arange(G) * g)[None, :, None]
                    idx = torch.from_numpy(pick.reshape(n, S).astype(np.int32)).to(dev)
                    step = lambda i: bsg.bs_gemv_hybrid(bits[i % n], K, M, N, g, al[i % n], x[i % n],
                                                        colscale=csd[i % n], sbits=sb[i % n], s=s, idx=idx[i % n],
                                                        salpha=sa[i % n], scolscale=sc[i % n], y=y[i % n])
                    op = "bs_gemv_hybrid (2b-s%d-g128, %s)" % (s, "1 launch" if B == 1 else "2 launches, matrix cores")
                else:
                    step = lambda i: bsg.bs_gemv_grouped(bits[i % n], K, M, N, g, al[i % n], x[i % n],
                                                         colscale=csd[i % n], y=y[i % n])
                    op = "bs_gemv_grouped (2b-g128%s)" % ("" if B == 1 else ", matrix cores")
                emit("f3", op, name, _graph_us(step, steps, warmup), wb + 2 * N * B, K=K, B=B, g=g, s=s)
                del bits, al, csd, x, y
                if s:
                    del sb, sa, sc, idx
                torch.cuda.empty_cache()

    # f2 x f3: the query, key and value projections in the 2b-g128 format in one launch, B = 1
    K, g, N = 2, 128, 4096
    G = N // g
    qkv = [("q", 4096), ("k", 1024), ("v", 1024)]
    wbs = {nm: K * M * N // 8 + 2 * K * M * G + 2 * K * N for nm, M in qkv}
    n = copies(sum(wbs.values()))
    P = {nm: (rand_bits(K, M, N, n), (torch.rand((n, K, G, M), device=dev) * 0.02).half().view(torch.int16),
              (torch.rand((n, K, N), device=dev) + 0.5).half().view(torch.int16), torch.empty((n, M, 1), device=dev))
         for nm, M in qkv}
    x = xs(N, 1, n, torch.float16)
    Mof = dict(qkv)

    def gm_fused(i):
        c = i % n
        bsg.bs_gemv_grouped_multi([(P[nm][0][c], Mof[nm], P[nm][1][c], P[nm][2][c], P[nm][3][c]) for nm, _ in qkv],
                                  K, N, g, x[c])

    def gm_single(i):
        c = i % n
        for nm, M in qkv:
            bsg.bs_gemv_grouped(P[nm][0][c], K, M, N, g, P[nm][1][c], x[c], colscale=P[nm][2][c], y=P[nm][3][c])
    by = sum(wbs.values()) + 2 * N
    emit("f3", "bs_gemv_grouped_multi (2b-g128, 1 launch)", "q+k+v 6144x4096", _graph_us(gm_fused, steps, warmup), by,
         K=K, B=1, g=g)
    emit("f3", "bs_gemv_grouped, one call per projection", "q+k+v 6144x4096", _graph_us(gm_single, steps, warmup), by,
         K=K, B=1, g=g)
    del P, x
    torch.cuda.empty_cache()

    # a4, a5: the fused layer (bases + binary low-rank + protected int8 rows) and its parts; at
    # B = 16 columns of bf16 x every part runs on the matrix cores except the protected rows
    for name, M, N, K, r, frac, B in [("5120x5120 K=3 r=512", 5120, 5120, 3, 512, 0.0, 1),
                                      ("13824x5120 r=512 1% rows", 13824, 5120, 2, 512, 0.01, 1),
                                      ("5120x13824 r=512 1% rows", 5120, 13824, 2, 512, 0.01, 1),
                                      ("28672x8192 r=512 1% rows", 28672, 8192, 2, 512, 0.01, 1),
                                      ("13824x5120 r=512 1% rows B=16", 13824, 5120, 2, 512, 0.01, 16),
                                      ("28672x8192 r=512 1% rows B=16", 28672, 8192, 2, 512, 0.01, 16)]:
        ns = synth.n_salient(M, frac) if frac else 0
        wb = K * M * N // 8 + 4 * K * M
        lrb = r * N // 8 + M * r // 8 + 2 * r
        sb = ns * N + 6 * ns
        n = copies(wb + lrb + sb)
        bits = rand_bits(K, M, N, n)
        alpha = torch.rand((n, K, M), device=dev) * 0.02
        U = rand_bits(1, M, r, n)
        V = rand_bits(1, r, N, n)
        ar = (torch.rand((n, r), device=dev) * 0.01).half().view(torch.int16)
        rows = torch.stack([torch.sort(torch.randperm(M, device=dev)[:ns])[0] for _ in range(n)]).to(torch.int32) \
            if ns else None
        q = torch.randint(-127, 128, (n, ns, N), dtype=torch.int8, device=dev) if ns else None
        sv = (torch.rand((n, ns), device=dev) * 1e-3).half().view(torch.int16) if ns else None
        x = xs(N, B, n)
        y = torch.empty((n, M, B), device=dev)
        ws = bsg.new_workspace(bsg.lib().bsg_linear_workspace_bytes(r, B), dev)
        launches = "2 launches" if B == 1 else "matrix cores"

        def step(i):
            c = i % n
            bsg.bsg_linear(bits[c], K, M, N, alpha[c], x[c], lowrank=(U[c], V[c], ar[c], r),
                           salient=(rows[c], q[c], sv[c]) if ns else None, y=y[c], workspace=ws)
        emit("a2-a5", "bsg_linear (%s)" % launches, name, _graph_us(step, steps, warmup),
             wb + lrb + sb + 2 * N * B, K=K, r=r, ns=ns, B=B)
        step = lambda i: bsg.binlr_apply(U[i % n], V[i % n], ar[i % n], r, M, N, x[i % n], y[i % n], workspace=ws)
        emit("a4", "binlr_apply alone (2 launches)", name, _graph_us(step, steps, warmup), lrb + 2 * N * B, r=r, B=B)
        if ns:
            step = lambda i: bsg.salient_int8_apply(rows[i % n], q[i % n], sv[i % n], M, N, x[i % n], y[i % n])
            emit("a5", "salient_int8_apply alone", name, _graph_us(step, steps, warmup), sb + 2 * N * B, ns=ns, B=B)
        del bits, alpha, U, V, ar, rows, q, sv, x, y, ws
        torch.cuda.empty_cache()

    # a6: int8 activations, exact int32
    for name, M, N, K in [("4096x4096", 4096, 4096, 2), ("gate/up 14336x4096", 14336, 4096, 2)]:
        wb = K * M * N // 8 + 4 * K * M
        n = copies(wb)
        bits = rand_bits(K, M, N, n)
        alpha = torch.rand((n, K, M), device=dev) * 0.02
        xq = torch.randint(-127, 128, (n, N, 1), dtype=torch.int8, device=dev)
        sx = torch.rand((n, 1), device=dev)
        y = torch.empty((n, M, 1), device=dev)
        step = lambda i: bsg.bs_gemv_i8(bits[i % n], K, M, N, alpha[i % n], xq[i % n], sx[i % n], want_acc=False,
                                        y=y[i % n])
        emit("a6", "bs_gemv_i8 (y)", name, _graph_us(step, steps, warmup), wb + N + 4, K=K)
        xf = xs(N, 1, 2)
        step = lambda i: bsg.bsq_quantize_i8(xf[i % 2])
        emit("a6", "bsq_quantize_i8", "x of %d" % N, _graph_us(step, steps, warmup), 2 * N)
        del bits, alpha, xq, sx, y, xf
        torch.cuda.empty_cache()

    # f4: the offline binary low-rank fit (greedy alternating signs, joint refit), eager, one call each
    for name, M, N, r in [("5120x5120 r=512", 5120, 5120, 512), ("4096x4096 r=128", 4096, 4096, 128)]:
        W = torch.randn((M, N), device=dev) * 0.02
        vinit = torch.from_numpy(synth.random_bits(1, 1, r, N)[0].view("int32")).to(dev)
        ws = bsg.new_workspace(int(bsg.lib().binlr_fit_workspace_bytes(M, N, r)) + 256, dev)
        bsg.binlr_fit(W[:64], min(r, 32), vinit[:min(r, 32)], workspace=ws)   # first-call costs
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        res = bsg.binlr_fit(W, r, vinit, workspace=ws)
        torch.cuda.synchronize()
        us = (time.perf_counter() - t0) * 1e6
        # per component: 5 rounds x 2 passes over the fp64 residual + the rank-one update (read + write),
        # then one fp32 pass over W per component for the refit
        passes = r * (5 * 2 * 8 * M * N + 16 * M * N + 4 * M * N)
        emit("f4", "binlr_fit (offline, eager, one call)", name, us, passes, r=r,
             sse_greedy_over_w2=round(res[6][0] / float((W.double() ** 2).sum()), 4),
             sse_refit_over_w2=round(res[6][1] / float((W.double() ** 2).sum()), 4))
        del W, vinit, ws, res
        torch.cuda.empty_cache()

    # a0: packing (offline), eager
    W = torch.randn((4096, 4096), device=dev) * 0.02
    bsg.bsq_pack(W, 2, colscale=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(5):
        bsg.bsq_pack(W, 2, colscale=True)
    torch.cuda.synchronize()
    emit("a0", "bsq_pack (offline, eager)", "4096x4096 K=2 colscale", (time.perf_counter() - t0) / 5 * 1e6,
         4096 * 4096 * 4, K=2)
    return out


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
    ap.add_argument("--rows", action="store_true",
                    help="time every row of the path on the pages' shapes (one JSON line per case) and exit")
    args = ap.parse_args()
    if args.rows:
        run_rows(min(args.steps, 200), min(args.warmup, 20))
        return
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
