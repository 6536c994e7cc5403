"""Benchmark of the MI355X factorized linear layer Y = (X.A).B.

Default (one GPU): the Llama-3-8B-shaped q_proj at decode, X[8 x 4096],
A[4096 x 1637], B[1637 x 4096] bf16 -- a misaligned rank -- through the
fused decode kernel.  One step = one lr_linear_run (plan/dispatch, split-K
GEMM1, rank padding and edge masking, T hand-off, GEMM2, deterministic
reduction, bf16 epilogue).  The factors rotate over enough copies (>= 1 GiB)
that every step streams them from HBM, not from the 256 MB last-level
cache.  value = algorithmic bytes per step / time per step (TB/s).

A second object reports the prefill workload (MLP up-projection,
X[4096 x 4096], r = 2867, N = 14336) in TFLOP/s against the dense bf16
MFMA peak, and a third one a whole decoder layer of factorized projections
at M = 1 (TB/s) and M = 2048 (TFLOP/s).  The CPU oracle is timed on a
bounded sample as a baseline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-prefill] [--no-cpu]
                    [--no-layer] [--calib-copy] [--sweep]
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
METRIC = "low-rank linear: decode TB/s and prefill TFLOP/s vs roofline, across rank r"
_CSRC = "rank_linear_layer_amd/csrc/"
DECODE_SOURCES = [_CSRC + f for f in ("lr_decode.hip", "lr_decode_res.hip", "lr_decode_split.hip", "lr_decode_xcd.hip",
                                       "lr_device.h", "lr_kernels.h", "lr_ldsops.h")]
PREFILL_SOURCES = [_CSRC + f for f in ("lr_prefill.hip", "lr_prefill_w4.hip", "lr_device.h", "lr_kernels.h",
                                       "lr_validate.h", "lr_linear.cpp")]
PREFILL_KERNELS = {0: "lr_prefill_gemm_kernel", 1: "lr_prefill_w4_kernel"}


def kernel_source_hash(sources=None) -> str:
    """Hash of the kernel sources a counter summary was taken on (decode
    sources by default)."""
    h = hashlib.sha256()
    for p in sources or DECODE_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def prefill_kernels(plan):
    """Kernel names of the two prefill phases from a describe() string."""
    import re
    m = re.search(r"phase1 kind=(-?\d+) nb=\d+ splits=(\d+), phase2 kind=(-?\d+) nb=\d+ splits=(\d+)", plan)
    if not m:
        return None
    names = []
    for kind, splits in ((int(m.group(1)), int(m.group(2))), (int(m.group(3)), int(m.group(4)))):
        names.append(PREFILL_KERNELS.get(kind, "?") + (" + lr_prefill_reduce_kernel" if splits > 1 else ""))
    return names


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def dev_bf16(torch, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def time_steps(torch, fn, steps, warmup, stream, warm_seconds=0.0):
    """Event-timed average step.  Python's cyclic garbage collector is run
    once before the warm-up and held off until the timed region ends: a
    collection that starts inside the launch loop stalls the host for about
    a millisecond, the GPU runs dry, and a short step reads up to 1.7x
    slower (seen as a one-point dip at a fixed place of the rank sweep).
    The collection itself takes tens of milliseconds, so it must not sit
    between the warm-up and the timed region either: after that long an
    idle gap the first compute-bound prefill steps run through a clock
    transient (up to 1.3x slower for a few milliseconds).  `warm_seconds`
    keeps running warm-up steps until that much time has passed: the
    compute-bound prefill steps otherwise start timing before the GPU clock
    has settled from the lighter load before them."""
    gc.collect()
    gc.disable()
    try:
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        if warm_seconds > 0:
            t_end = time.time() + warm_seconds
            i = warmup
            while time.time() < t_end:
                for _ in range(8):
                    fn(i)
                    i += 1
                torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
    finally:
        gc.enable()
    return e0.elapsed_time(e1) / steps  # ms per step


def decode_kernel_name(plan):
    for kind, name in (("kind=split_stream", "lr_decode_splits_kernel"), ("kind=split_flat", "lr_decode_splitf_kernel"),
                       ("kind=split", "lr_decode_split_kernel"), ("kind=xcd", "lr_decode_xcd_kernel"),
                       ("kind=resident", "lr_decode_res_kernel")):
        if kind in plan:
            return name
    return "lr_decode_fused_kernel"


def traffic_from_profile(name, sources=None, key="hbm_bytes_per_launch"):
    """HBM bytes from a committed rocprofv3 counter summary, if it was taken
    on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_hash") != kernel_source_hash(sources):
        return None
    return d.get(key)


def bench_decode(torch, lrl, configs, datagen, metrics, steps, warmup, flags=0, context=True):
    """q_proj decode through the kernel that `flags` selects (0: the
    library's default, which reads A and B in place)."""
    c = configs.QPROJ_DECODE
    M, K, r, N = c["M"], c["K"], c["r"], c["N"]
    Xb, Ab, Bb = datagen.factorized_inputs(M, K, r, N, configs.seed_base(c["index"]))
    per = metrics.decode_bytes(M, K, r, N)
    ncopies = max(2, int(np.ceil((1 << 30) / (2 * (K * r + r * N)))))
    A0, B0 = dev_bf16(torch, Ab), dev_bf16(torch, Bb)
    As = [A0] + [A0.clone() for _ in range(ncopies - 1)]
    Bs = [B0] + [B0.clone() for _ in range(ncopies - 1)]
    X = dev_bf16(torch, Xb)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    lins = [lrl.LowRankLinear(a, b, max_M=M, flags=flags) for a, b in zip(As, Bs)]
    stream = torch.cuda.current_stream()
    log("decode plan (flags %d): %s; %d weight copies (%.0f MB)"
        % (flags, lins[0].describe(), ncopies, ncopies * 2 * (K * r + r * N) / 1e6))

    def step(i):
        lins[i % ncopies](X, out=Y)

    ms = time_steps(torch, step, steps, warmup, stream)
    tbs = per / (ms * 1e-3) / 1e12
    out = dict(M=M, K=K, r=r, N=N, ms=ms, tbs=tbs, bytes=per, ncopies=ncopies, plan=lins[0].describe(),
               workspace_bytes=lins[0].workspace_bytes())
    if context:
        # warm-cache figure (same copy every step), and the same rotation
        # replayed from a captured graph
        ms_warm = time_steps(torch, lambda i: lins[0](X, out=Y), max(50, steps // 4), 10, stream)
        out["warm_tbs"] = per / (ms_warm * 1e-3) / 1e12
        out["graph_us"] = replay_us(torch, step, ncopies, steps, warmup)
    del lins
    torch.cuda.empty_cache()
    return out


def replay_us(torch, fn, n, steps, warmup):
    """Microseconds per call of fn(0..n-1) replayed from one captured HIP
    graph (no host launch work between the kernels)."""
    for i in range(n):
        fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    reps = max(1, steps // n)
    ms = time_steps(torch, lambda i: g.replay(), reps, max(1, warmup // n), torch.cuda.current_stream())
    del g
    return ms * 1e3 / n


def bench_dense_decode(torch, lrl, configs, steps, warmup):
    """Dense fallback decode (W = A.B formed at create): the k/v layer shape,
    where the library takes it by itself, and the q_proj shape with
    LR_FLAG_DENSE.  Bytes per launch are what the kernel reads and writes,
    2 (MK + KN + MN); W copies rotate over >= 1 GiB.  A single launch is
    shorter than the host's work per call, so the figure is taken from a
    captured graph of one launch per copy (the eager figure is kept for
    context)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(configs.seed_base(configs.LAYER_INDEX, 1))
    out = {}
    for name, (M, K, r, N, flags) in (("kv_auto", (8, 4096, 817, 1024, 0)),
                                      ("qproj_forced", (8, 4096, 1637, 4096, lrl.LR_FLAG_DENSE))):
        A = (torch.randn((K, r), generator=g, device="cuda") / np.sqrt(K)).to(torch.bfloat16)
        B = (torch.randn((r, N), generator=g, device="cuda") / np.sqrt(r)).to(torch.bfloat16)
        X = torch.randn((M, K), generator=g, device="cuda").to(torch.bfloat16)
        Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        ncop = max(2, int(np.ceil((1 << 30) / (2 * K * N))))
        lins = [lrl.LowRankLinear(A, B, max_M=M, flags=flags) for _ in range(ncop)]
        assert "dense=1" in lins[0].describe()
        call = lambda i: lins[i % ncop](X, out=Y)  # noqa: E731
        eager = time_steps(torch, call, steps, warmup, torch.cuda.current_stream()) * 1e3
        us = replay_us(torch, call, ncop, steps, warmup)
        byts = 2 * (M * K + K * N + M * N)
        out[name] = {"M": M, "K": K, "r": r, "N": N, "us_per_launch": round(us, 3), "us_per_launch_eager": round(eager, 3),
                     "hbm_bytes_per_launch": byts, "tbs": round(byts / (us * 1e-6) / 1e12, 4),
                     "roofline_frac_hbm": round(byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "kernel": "lr_dense_decode_kernel", "w_copies": ncop}
        log("dense decode %s: %.2f us/launch from a graph (%.2f eager), %.3f TB/s of W bytes (%d copies)"
            % (name, us, eager, out[name]["tbs"], ncop))
        del lins
        torch.cuda.empty_cache()
    return out


def bench_prefill(torch, lrl, configs, metrics, steps, warmup, r=None, warm_seconds=0.0):
    """MLP up-projection prefill (the rank `r` overrides the workload's)."""
    c = configs.MLP_UP_PREFILL
    M, K, N = c["M"], c["K"], c["N"]
    r = r or c["r"]
    g = torch.Generator(device="cuda")
    g.manual_seed(configs.seed_base(c["index"]))
    X = torch.randn((M, K), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    A = (torch.randn((K, r), generator=g, device="cuda", dtype=torch.float32) / np.sqrt(K)).to(torch.bfloat16)
    B = (torch.randn((r, N), generator=g, device="cuda", dtype=torch.float32) / np.sqrt(r)).to(torch.bfloat16)
    # four copies of the whole working set (X, A, B, Y: about 280 MB each,
    # above the 256 MB last-level cache) rotate, so every step starts cold
    ncop = 4
    Xs = [X] + [X.clone() for _ in range(ncop - 1)]
    lins = [lrl.LowRankLinear(A.clone() if i else A, B.clone() if i else B, max_M=M) for i in range(ncop)]
    Ys = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for _ in range(ncop)]
    stream = torch.cuda.current_stream()
    ms = time_steps(torch, lambda i: lins[i % ncop](Xs[i % ncop], out=Ys[i % ncop]), steps, warmup, stream,
                    warm_seconds=warm_seconds)
    fl = metrics.lowrank_flops(M, K, r, N)
    plan = lins[0].describe()
    del lins, Xs, Ys
    torch.cuda.empty_cache()
    return dict(M=M, K=K, r=r, N=N, ms=ms, tflops=fl / (ms * 1e-3) / 1e12, flops=fl, plan=plan, copies=ncop)


def bench_layer(torch, lrl, configs, metrics, M, steps, warmup, grouped=True, graph=False, warm_seconds=0.0):
    """One decoder layer of factorized projections (q, k, v, o, packed
    gate/up, down) at M rows: the layer's span per step.  q, k and v share X
    in one group call (or three separate calls with grouped=False).  Weights
    rotate over enough copies (>= 1 GiB) that every step streams them from
    HBM."""
    g = torch.Generator(device="cuda")
    g.manual_seed(configs.seed_base(configs.LAYER_INDEX))
    projs = {p.name: p for p in configs.LAYER_PROJS}
    wbytes = sum(2 * (p.K * p.r + p.r * p.N) for p in configs.LAYER_PROJS)
    ncop = max(1, int(np.ceil((1 << 30) / wbytes))) if M <= 16 else 1
    sets = []
    for _ in range(ncop):
        lins = {}
        for name, p in projs.items():
            A = (torch.randn((p.K, p.r), generator=g, device="cuda") / np.sqrt(p.K)).to(torch.bfloat16)
            B = (torch.randn((p.r, p.N), generator=g, device="cuda") / np.sqrt(p.r)).to(torch.bfloat16)
            lins[name] = lrl.LowRankLinear(A, B, max_M=M)
        sets.append(lins)
    X = torch.randn((M, 4096), generator=g, device="cuda").to(torch.bfloat16)
    H = torch.randn((M, 14336), generator=g, device="cuda").to(torch.bfloat16)
    outs = {name: torch.empty((M, p.N), dtype=torch.bfloat16, device="cuda") for name, p in projs.items()}

    def step(i):
        L = sets[i % ncop]
        if grouped:
            lrl.group_run([L["q"], L["k"], L["v"]], X, outs=[outs["q"], outs["k"], outs["v"]])
        else:
            for name in ("q", "k", "v"):
                L[name](X, out=outs[name])
        L["o"](X, out=outs["o"])
        lrl.mlp_packed(L["gate"], L["up"], X, out_gate=outs["gate"], out_up=outs["up"])
        L["down"](H, out=outs["down"])

    if graph:
        # one captured graph holds a layer step per weight copy; a replay is
        # ncop layers with no host launch work between the kernels
        for i in range(ncop):
            step(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(ncop):
                step(i)
        reps = max(1, steps // ncop)
        ms = time_steps(torch, lambda i: g.replay(), reps, max(1, warmup // ncop), torch.cuda.current_stream(),
                        warm_seconds=warm_seconds) / ncop
        del g
    else:
        ms = time_steps(torch, step, steps, warmup, torch.cuda.current_stream(), warm_seconds=warm_seconds)
    byts = sum(metrics.decode_bytes(M, p.K, p.r, p.N) for p in configs.LAYER_PROJS)
    fl = sum(metrics.lowrank_flops(M, p.K, p.r, p.N) for p in configs.LAYER_PROJS)
    dense = [nm for nm, lin in sets[0].items() if "dense=1" in lin.describe()]
    return dict(M=M, ms=ms, tbs=byts / (ms * 1e-3) / 1e12, tflops=fl / (ms * 1e-3) / 1e12, bytes=byts, flops=fl,
                calls=4 if grouped else 6, copies=ncop, dense=dense)


def cpu_baseline(configs, datagen, metrics, budget_s=12.0):
    import oracle
    c = configs.QPROJ_DECODE
    M, K, r, N = c["M"], c["K"], c["r"], c["N"]
    Xb, Ab, Bb = datagen.factorized_inputs(M, K, r, N, configs.seed_base(c["index"]))
    threads = oracle.default_threads()
    oracle.lowrank_bf16(Xb[:1], Ab, Bb, nthreads=threads)  # load + warm
    n = 0
    t0 = time.perf_counter()
    while True:
        oracle.lowrank_bf16(Xb, Ab, Bb, nthreads=threads)
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = (time.perf_counter() - t0) / n
    return {"value": metrics.decode_bytes(M, K, r, N) / dt / 1e12, "unit": "TB/s", "cores": threads,
            "kind": "oracle",
            "sample": "q_proj decode M=8 K=4096 r=1637 N=4096, full output, %d oracle forwards in %.1f s "
                      "(%.3f s each, float64, sequential sums)" % (n, n * dt, dt)}


def calib_copy(torch):
    """A plain device copy of known size, for scaling rocprofv3 FETCH_SIZE /
    WRITE_SIZE counters (run under --pmc)."""
    nbytes = 256 << 20
    a = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log("calibration copy: 3 x %d bytes read and written" % nbytes)


def run_sweep(torch, lrl, configs, metrics, steps, stride=1, ranks=None):
    """Throughput against rank at K = 4096 for both widths N and both M of
    the alignment sweep (the no-cliff check).  Every point is printed as a
    JSON line on stderr; the summary per (N, M) series goes into the result:
    min / median / max, and the ranks whose throughput falls more than 10%
    below the median of their +-8 neighbours (a cliff)."""
    rows = []
    K = configs.SWEEP_K
    for N in configs.SWEEP_N:
        for r in (ranks if ranks is not None else configs.SWEEP_R[::stride]):
            g = torch.Generator(device="cuda")
            g.manual_seed(configs.sweep_seed(N, r))
            wb = 2 * (K * r + r * N)
            A = (torch.randn((K, r), generator=g, device="cuda") / np.sqrt(K)).to(torch.bfloat16)
            B = (torch.randn((r, N), generator=g, device="cuda") / np.sqrt(r)).to(torch.bfloat16)
            for M in configs.SWEEP_M:
                # decode streams >= 1 GiB of weight copies; prefill >= 256 MB
                ncop = max(2, int(np.ceil(((1 << 30) if M <= 16 else (256 << 20)) / wb)))
                As = [A] + [A.clone() for _ in range(ncop - 1)]
                Bs = [B] + [B.clone() for _ in range(ncop - 1)]
                X = torch.randn((M, K), generator=g, device="cuda").to(torch.bfloat16)
                Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
                lins = [lrl.LowRankLinear(a, b, max_M=M) for a, b in zip(As, Bs)]
                ms = time_steps(torch, lambda i: lins[i % ncop](X, out=Y), steps, 10, torch.cuda.current_stream())
                row = dict(N=N, r=r, M=M, us=round(ms * 1e3, 3),
                           tbs=round(metrics.decode_bytes(M, K, r, N) / (ms * 1e-3) / 1e12, 4),
                           tflops=round(metrics.lowrank_flops(M, K, r, N) / (ms * 1e-3) / 1e12, 2))
                rows.append(row)
                print(json.dumps({"sweep": row}), file=sys.stderr, flush=True)
                del lins, As, Bs
            del A, B
    summary = {}
    for N in configs.SWEEP_N:
        for M in configs.SWEEP_M:
            ser = [x for x in rows if x["N"] == N and x["M"] == M]
            key = "tbs" if M <= 16 else "tflops"
            v = np.array([x[key] for x in ser])
            cliffs = []
            for i, x in enumerate(ser):
                nb = np.concatenate([v[max(0, i - 8):i], v[i + 1:i + 9]])
                if len(nb) and x[key] < 0.9 * np.median(nb):
                    cliffs.append(x["r"])
            peak = HBM_PEAK_GBS / 1e3 if M <= 16 else BF16_PEAK_TFLOPS
            summary["N%d_M%d" % (N, M)] = {"unit": "TB/s" if M <= 16 else "TFLOP/s", "points": len(ser),
                                           "ranks": [x["r"] for x in ser],
                                           "residues_mod8": sorted({x["r"] % 8 for x in ser}),
                                           "min": float(v.min()), "median": float(np.median(v)),
                                           "max": float(v.max()), "min_frac": round(float(v.min()) / peak, 4),
                                           "max_over_min": round(float(v.max() / v.min()), 4),
                                           "cliff_ranks": cliffs}
    return summary, rows


def gac_from_sweep(rows, configs):
    """GAC's rank re-selection ("Why Smaller Is Slower?", section 4) driven
    by the measured sweep: a synthetic compressed model of 16 weights of the
    sweep shape (K = 4096, N = 4096 / 3999 alternating) with continuous ranks
    d* in (1030, 1070) and random importance scores; candidates are the
    multiples of 8 within 4% below / 6% above d* that the measured latency
    table does not mark as a cliff; the budget is the misaligned model's
    parameter count.  Reports, per M, how many aligned candidates the table
    rejected and the summed latency of the misaligned ranks against the
    selected aligned ones."""
    from rank_linear_layer_amd import gac
    rng = np.random.default_rng(2026)
    K = configs.SWEEP_K
    n = 16
    Ns = [configs.SWEEP_N[i % len(configs.SWEEP_N)] for i in range(n)]
    dstar = rng.uniform(1030, 1070, n)
    scores = rng.uniform(0.5, 2.0, n)
    costs = [K + N for N in Ns]
    budget = int(sum(c * d for c, d in zip(costs, dstar)))
    out = {"weights": n, "d_star_range": [1030, 1070], "budget_params": budget}
    for M in configs.SWEEP_M:
        lat = {(x["N"], x["r"]): x["us"] for x in rows if x["M"] == M}
        cands, rejected, total = [], 0, 0
        for d, N in zip(dstar, Ns):
            table = {r: lat.get((N, r)) for r in range(900, 1200)}
            c_all = gac.candidates(d, table, window=(0.96, 1.06))
            c_aligned = [r for r in range(8 * int(np.ceil(0.96 * d / 8)), int(1.06 * d) + 1, 8) if table.get(r)]
            rejected += len(c_aligned) - len(c_all)
            total += len(c_aligned)
            cands.append(c_all)
        dims, obj = gac.select(list(scores), costs, list(dstar), cands, budget)
        def nearest(N, d):
            return lat[min((k for k in lat if k[0] == N), key=lambda k: abs(k[1] - d))]
        t_mis = sum(nearest(N, d) for d, N in zip(dstar, Ns))
        t_gac = sum(lat[(N, d)] for d, N in zip(dims, Ns))
        out["M%d" % M] = {"aligned_candidates": total, "rejected_as_cliffs": rejected,
                          "us_misaligned_ranks": round(t_mis, 2), "us_gac_ranks": round(t_gac, 2),
                          "gac_speedup": round(t_mis / t_gac, 4),
                          "params_misaligned": budget, "params_gac": int(sum(c * d for c, d in zip(costs, dims)))}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-layer", action="store_true")
    ap.add_argument("--calib-copy", action="store_true")
    ap.add_argument("--sweep", action="store_true", help="the full rank sweep (every r of the sweep range)")
    ap.add_argument("--no-sweep", action="store_true", help="skip the default strided rank sweep")
    ap.add_argument("--no-alternatives", action="store_true", help="skip the opt-in decode kernels")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only the prefill leg (for profiling it): prints its JSON object")
    ap.add_argument("--prefill-ranks", default=None,
                    help="with --prefill-only: a rank range lo-hi; the prefill step is timed at every r in it, "
                         "after a few seconds of warm-up, in two passes (ascending, then descending)")
    ap.add_argument("--sweep-steps", type=int, default=100)
    ap.add_argument("--sweep-stride", type=int, default=1)
    ap.add_argument("--gac", action="store_true", help="with --sweep: GAC rank re-selection on the measured table")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the layer would shard along the rank with one all-reduce of Y; not built). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import rank_linear_layer_amd as lrl
    from rank_linear_layer_amd import configs, datagen, metrics

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    lrl.load_library()
    torch.cuda.set_device(0)

    if args.calib_copy:
        calib_copy(torch)

    if args.prefill_only and args.prefill_ranks:
        lo, hi = (int(v) for v in args.prefill_ranks.split("-"))
        ranks = list(range(lo, hi + 1))
        t_end = time.time() + 4.0  # steady clocks before the first timed rank
        while time.time() < t_end:
            bench_prefill(torch, lrl, configs, metrics, 5, 1, r=ranks[0])
        per = {r: [] for r in ranks}
        for order in (ranks, ranks[::-1]):
            for r in order:
                p = bench_prefill(torch, lrl, configs, metrics, max(10, args.steps // 50), 3, r=r)
                per[r].append(p["ms"])
                print(json.dumps({"prefill_r": r, "ms": round(p["ms"], 5), "plan": p["plan"].split("prefill=")[1][:80]}),
                      file=sys.stderr, flush=True)
        ms = {r: float(np.mean(v)) for r, v in per.items()}
        print(json.dumps({"workload": "MLP up-projection prefill M=4096 K=4096 N=14336 across r",
                          "ms_per_step": {str(r): round(v, 5) for r, v in ms.items()},
                          "max_over_min": round(max(ms.values()) / min(ms.values()), 4)}), flush=True)
        return
    if args.prefill_only:
        p = bench_prefill(torch, lrl, configs, metrics, max(10, args.steps // 20), 3, warm_seconds=2.0)
        log("prefill: %.3f ms/step, %.1f TFLOP/s, plan %s" % (p["ms"], p["tflops"], p["plan"]))
        print(json.dumps({"prefill_ms_per_step": round(p["ms"], 5), "tflops": round(p["tflops"], 2),
                          "flops_per_step": p["flops"], "plan": p["plan"]}), flush=True)
        return

    torch.cuda.synchronize()
    d = bench_decode(torch, lrl, configs, datagen, metrics, args.steps, args.warmup)
    alts = {}
    if not args.no_alternatives:
        # the opt-in decode kernels on the same workload, for context: the
        # role-split kernel reads a copy of A and B in its operand block
        # layout (extra workspace bytes), the XCD-sliced one reads them in place
        for name, fl in (("split_copy", lrl.LR_FLAG_DECODE_SPLIT), ("xcd", lrl.LR_FLAG_DECODE_XCD),
                         ("streaming", lrl.LR_FLAG_DECODE_STREAMING)):
            a_ = bench_decode(torch, lrl, configs, datagen, metrics, max(200, args.steps // 2), 50, flags=fl,
                              context=False)
            alts[name] = {"flag": fl, "kernel": decode_kernel_name(a_["plan"]), "us_per_launch": round(a_["ms"] * 1e3, 3),
                          "value": round(a_["tbs"], 4), "roofline_frac_hbm": round(a_["tbs"] * 1e3 / HBM_PEAK_GBS, 4),
                          "workspace_bytes": a_["workspace_bytes"],
                          "reads_factors_in_place": fl != lrl.LR_FLAG_DECODE_SPLIT}
            log("decode %s: %.3f us/step, %.3f TB/s, workspace %d bytes"
                % (name, a_["ms"] * 1e3, a_["tbs"], a_["workspace_bytes"]))
    log("decode: %.3f us/step, %.3f TB/s (warm-cache %.3f TB/s; from a captured graph %.3f us/step)"
        % (d["ms"] * 1e3, d["tbs"], d["warm_tbs"], d["graph_us"]))
    kname = decode_kernel_name(d["plan"])
    # one step is one launch of the decode kernel, launched back to back:
    # the event-timed average step is the kernel's average launch duration
    ach = d["bytes"] / (d["ms"] * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(d["tbs"], 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(d["ms"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,1/fan_in) bf16 factors; %d rotating weight copies, "
                "cold last-level cache)" % d["ncopies"],
        "config": {"workload": "Llama-3-8B-shaped q_proj decode, misaligned rank", "M": d["M"], "K": d["K"],
                   "r": d["r"], "N": d["N"], "path": kname, "weight_copies": d["ncopies"],
                   "factors_read_in_place": True, "workspace_bytes": d["workspace_bytes"]},
        "roofline": {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profile("%s_qproj_decode_pmc.json" % kname),
                     "kernel": kname, "algorithmic_bytes_per_launch": d["bytes"],
                     "us_per_launch": round(d["ms"] * 1e3, 3)},
        "warm_cache_tbs": round(d["warm_tbs"], 4),
        "graph_replay_us_per_step": round(d["graph_us"], 3),
        "decode_alternatives": alts or None,
    }
    if not args.no_prefill:
        p = bench_prefill(torch, lrl, configs, metrics, max(10, args.steps // 20), 3, warm_seconds=2.0)
        log("prefill: %.3f ms/step, %.1f TFLOP/s" % (p["ms"], p["tflops"]))
        kn = prefill_kernels(p["plan"])
        result["prefill"] = {
            "workload": "MLP up-projection prefill M=4096 K=4096 r=2867 N=14336 (%d rotating copies of X, A, B, Y)"
                        % p["copies"],
            "ms_per_step": round(p["ms"], 5), "value": round(p["tflops"], 2), "unit": "TFLOP/s",
            "roofline": {"bound": "mfma", "achieved": round(p["tflops"], 2), "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(p["tflops"] / BF16_PEAK_TFLOPS, 4),
                         "traffic": traffic_from_profile("prefill_mlp_up_pmc.json", PREFILL_SOURCES,
                                                         "hbm_bytes_per_step"),
                         "kernel": "phase 1 %s, phase 2 %s" % tuple(kn) if kn else "prefill (2 launches)",
                         "algorithmic_flops_per_step": p["flops"]},
        }
    if not args.no_layer:
        result["dense_decode"] = bench_dense_decode(torch, lrl, configs, min(args.steps, 400), 20)
        lay = {}
        for M in configs.LAYER_M:
            steps_, warm_, ws_ = (200, 20, 0.0) if M <= 16 else (20, 2, 1.0)
            d_ = bench_layer(torch, lrl, configs, metrics, M, steps_, warm_, warm_seconds=ws_)
            sep = bench_layer(torch, lrl, configs, metrics, M, steps_, warm_, grouped=False, warm_seconds=ws_)
            gr = bench_layer(torch, lrl, configs, metrics, M, steps_, warm_, graph=True, warm_seconds=ws_)
            log("layer M=%d: %.1f us/layer, %.3f TB/s, %.1f TFLOP/s (%d library calls, %d weight copies); "
                "q, k, v as separate calls: %.1f us/layer; replayed as a HIP graph: %.1f us/layer"
                % (M, d_["ms"] * 1e3, d_["tbs"], d_["tflops"], d_["calls"], d_["copies"], sep["ms"] * 1e3,
                   gr["ms"] * 1e3))
            if M <= 16:
                lay["M%d" % M] = {"us_per_layer": round(d_["ms"] * 1e3, 2), "value": round(d_["tbs"], 4),
                                  "unit": "TB/s", "roofline_frac_hbm": round(d_["tbs"] * 1e3 / HBM_PEAK_GBS, 4),
                                  "algorithmic_bytes": d_["bytes"], "library_calls": d_["calls"],
                                  "weight_copies": d_["copies"],
                                  "us_per_layer_qkv_separate": round(sep["ms"] * 1e3, 2),
                                  "us_per_layer_graph": round(gr["ms"] * 1e3, 2),
                                  "value_graph": round(gr["tbs"], 4)}
            else:
                lay["M%d" % M] = {"us_per_layer": round(d_["ms"] * 1e3, 2), "value": round(d_["tflops"], 2),
                                  "unit": "TFLOP/s", "roofline_frac_mfma": round(d_["tflops"] / BF16_PEAK_TFLOPS, 4),
                                  "algorithmic_flops": d_["flops"], "library_calls": d_["calls"],
                                  "us_per_layer_qkv_separate": round(sep["ms"] * 1e3, 2),
                                  "us_per_layer_graph": round(gr["ms"] * 1e3, 2),
                                  "value_graph": round(gr["tflops"], 2)}
        lay["dense_fallback"] = d_["dense"]
        result["layer"] = {"workload": "Llama-3-8B-shaped decoder layer: q,o 4096->4096 r1637; k,v 4096->1024 "
                                       "r817 (q, k, v grouped on a shared X); gate,up 4096->14336 r2867 (packed); "
                                       "down 14336->4096 r2867", **lay}
    if args.sweep:
        result["sweep"], sweep_rows = run_sweep(torch, lrl, configs, metrics, args.sweep_steps, args.sweep_stride)
    elif not args.no_sweep:
        # strided: 16 ranks, stride 3, so every residue of r mod 8 appears twice
        result["sweep"], sweep_rows = run_sweep(torch, lrl, configs, metrics, args.sweep_steps,
                                                ranks=configs.SWEEP_R_DEFAULT)
    if args.sweep or not args.no_sweep:
        log("sweep: %s" % json.dumps(result["sweep"]))
        if args.gac:
            result["gac"] = gac_from_sweep(sweep_rows, configs)
            log("gac: %s" % json.dumps(result["gac"]))
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(configs, datagen, metrics)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
