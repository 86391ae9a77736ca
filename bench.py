#!/usr/bin/env python3
"""Throughput of the pipelined tiled GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-secondary] [--no-cpu]

A step is one call of the pipelined GEMM on the headline workload: C = A.B with
M = N = K = 8192, A row-major bf16, B stored transposed (N x K) bf16, entries N(0,1)/sqrt(K),
fp32 accumulation, bf16 output (seeded synthetic data, resident in HBM before timing).
W untimed steps (continued until at least --warm-s seconds of calls have run, so that the part
is at its clock under load), then exactly K timed steps between two device synchronisations;
one JSON line is printed.

value            whole-job TFLOP/s over the timed steps (algorithmic 2 M N K flops per step)
roofline         the GEMM kernel against MI355X's dense bf16 MFMA peak (2500 TFLOP/s); its
                 duration comes from HIP events recorded on the stream the library launches
                 on; `traffic` is the HBM bytes per launch measured by rocprofv3 counters when
                 a summary for the current kernel sources exists under profiles/, else null
cpu_baseline     the fp64 CPU oracle on a bounded sample of the same workload (some output
                 rows), on all host cores it uses, in the same unit
secondary        the 256^3 single GEMM (per-call latency in microseconds), grouped (mixture-of-
                 experts) forward and weight gradient, broadcast, IKBO attention and batched
                 workloads: TFLOP/s, % of peak, GB/s of compulsory traffic from per-call
                 cold-cache times (median, min, p90; a 512 MB scratch write before every call)
                 as the primary figures of the memory-relevant workloads, warm back-to-back
                 figures beside them (labelled), and the oracle timed on a sample of each
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TFLOP/s and % of MI355X bf16 MFMA peak (dense, grouped, broadcast GEMM)"
PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_GBS = 8000.0         # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_8192_nk_bf16.txt")


def kernel_sources_digest() -> str:
    """sha256 over the kernel sources and the build script that holds their compile flags."""
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "pipelined_tiled_gemm_amd")
    csrc = os.path.join(pkg, "csrc")
    files = [os.path.join(csrc, n) for n in sorted(os.listdir(csrc))
             if n.endswith((".hip", ".hpp", ".h", ".cpp"))]
    for path in files + [os.path.join(pkg, "build.py")]:
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode())
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch from the committed counter summary, if it matches the sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.lstrip().startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_sources_sha256") != kernel_sources_digest():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def to_dev(bits, torch, np):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)


def time_calls(fn, steps, warmup, torch, min_warm_s=0.0):
    """Untimed warmup (`warmup` calls, continued until at least `min_warm_s` seconds of calls
    have run), then `steps` calls between device synchronisations.
    Returns (wall seconds per call, event milliseconds per call on the current stream)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    if min_warm_s > 0:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < min_warm_s:
            for _ in range(8):
                fn()
            torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return (t1 - t0) / steps, e0.elapsed_time(e1) / steps


def time_each(fn, reps, torch):
    """Per-call durations of back-to-back calls (an event pair around each call on the current
    stream).  Returns {median, min, p90} in milliseconds."""
    stream = torch.cuda.current_stream()
    pairs = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in pairs)
    return {"median": t[len(t) // 2], "min": t[0], "p90": t[min(len(t) - 1, (9 * len(t)) // 10)], "reps": reps}


def time_cold(fn, reps, torch, flush_bytes=512 << 20):
    """Per-call durations with the caches cold: before each call a 512 MB scratch buffer is
    written (outside the event pair), which evicts the 256 MB last-level cache and the L2s.
    Returns {median, min, p90} in milliseconds."""
    scratch = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    fn()
    pairs = []
    for i in range(reps):
        scratch.fill_(i & 0xFF)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in pairs)
    del scratch
    return {"median": round(t[len(t) // 2], 4), "min": round(t[0], 4),
            "p90": round(t[min(len(t) - 1, (9 * len(t)) // 10)], 4), "reps": reps}


def figures(f, b, ms):
    """TFLOP/s, % of the MFMA peak, GB/s of compulsory traffic and % of HBM peak at `ms`."""
    return {"ms": round(ms, 4), "tflops": round(f / ms / 1e9, 2),
            "pct_peak": round(100 * f / ms / 1e9 / PEAK_TFLOPS, 2),
            "gbs": round(b / ms / 1e6, 1), "pct_hbm": round(100 * b / ms / 1e6 / PEAK_GBS, 2)}


def entry(f, b, warm_ms, cold, primary="cold", **extra):
    """One workload's line.  The top-level figures are the primary ones: cold-cache (median
    of per-call times after a cache flush) for the memory-relevant workloads, warm (back-to-back
    calls) otherwise; the other set follows, labelled."""
    e = {"primary": primary}
    e.update(figures(f, b, cold["median"] if primary == "cold" else warm_ms))
    e["cold_ms"] = cold
    e["warm"] = figures(f, b, warm_ms)
    e.update(extra)
    return e


def oracle_timed(make_sample, n_all, budget_s, threads=None):
    """The CPU oracle, untuned, on a bounded sample: `make_sample(n)` runs it on n units (rows
    or problems) of a workload of `n_all`; a probe of a few units sizes the timed sample to
    about `budget_s` seconds.  Returns (units, seconds, threads used)."""
    import oracle
    oracle.build(force=False)
    prev = oracle.max_threads()
    if threads:
        oracle.set_threads(threads)
    try:
        make_sample(min(n_all, 2))                       # thread pool and page-in
        n = min(n_all, 8)
        t0 = time.perf_counter()
        make_sample(n)
        dt = time.perf_counter() - t0
        n = int(max(n, min(n_all, n * budget_s / max(dt, 1e-4))))
        t0 = time.perf_counter()
        make_sample(n)
        dt = time.perf_counter() - t0
        cores = oracle.max_threads()
    finally:
        oracle.set_threads(prev)
    return n, dt, cores


def cpu_entry(n, dt, cores, unit_flops, what):
    return {"value": round(n * unit_flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle", "seconds": round(dt, 3), "sample": what}


def secondary(torch, np, ptg, wl, steps, warmup, cold_reps=20, warm_s=0.2, cpu=True, cpu_budget_s=2.0):
    """Each secondary workload: warm-cache throughput (back-to-back calls, as for the headline
    GEMM) and per-call cold-cache times (median, min, p90) with a cache flush before every
    call; the cold figures are the primary ones for the memory-relevant workloads.  Each
    workload's inputs are drawn on the host for several seconds while the GPU idles; its warm
    timing starts after at least `warm_s` seconds of calls, once the part has come back to its
    clock under load (the first tens of milliseconds after idling run several percent slower).
    With `cpu`, the oracle is timed on a bounded sample of the same workload."""
    import oracle
    out = {}

    # the 256^3 single GEMM (fp32 out): launch-latency bound, so per-call times in microseconds
    w = wl.config1()
    A, B = to_dev(w.A, torch, np), to_dev(w.B, torch, np)
    C = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
    call = lambda: ptg.gemm(A, B, b_layout=w.b_layout, out=C)  # noqa: E731
    time_calls(call, 10, 10, torch, min_warm_s=warm_s)
    warm = time_each(call, 200, torch)
    cold = time_cold(call, cold_reps, torch)
    f, b = wl.dense_flops(w.M, w.N, w.K), wl.dense_bytes(w.M, w.N, w.K, "f32")
    e = {"primary": "warm per-call latency",
         "us_median": round(1e3 * warm["median"], 2), "us_min": round(1e3 * warm["min"], 2),
         "us_p90": round(1e3 * warm["p90"], 2), "calls": warm["reps"],
         "tflops": round(f / warm["median"] / 1e9, 3), "gbs": round(b / warm["median"] / 1e6, 1),
         "cold_us": {k: (round(1e3 * v, 2) if k != "reps" else v) for k, v in cold.items()},
         "roofline": "not meaningful: launch-latency bound (0.013 us of MFMA work, 0.07 us of HBM traffic)"}
    if cpu:
        # the whole GEMM, repeated: unit r is the r-th call on all 256 rows
        def whole(n):
            for _ in range(n):
                oracle.gemm(w.A, w.B, w.b_layout)
        for threads, key in ((None, "cpu_baseline"), (1, "cpu_baseline_1core")):
            n, dt, cores = oracle_timed(whole, 1 << 20, 0.5, threads=threads)
            e[key] = cpu_entry(n, dt, cores, f, f"{n} calls of the whole 256^3 GEMM ({1e6 * dt / n:.0f} us each)")
    out["config1_gemm_256_f32"] = e
    del A, B, C, w

    # grouped: 64 experts, 16384 rows, K=4096, N=1536, Zipf(1.1) routing under both readings
    # of the weights: rank-Zipf (expert e weighted (e+1)^-1.1; every expert gets rows) and
    # Zipf-sampled weights (most experts empty, one or a few take nearly every row)
    for reading, name in (("rank", "grouped_moe_64x16384x4096x1536"),
                          ("sampled", "grouped_moe_64x16384x4096x1536_sampled_zipf")):
        w = wl.config3(reading)
        X, W, off = to_dev(w.X, torch, np), to_dev(w.W, torch, np), torch.from_numpy(w.offsets).cuda()
        Y = torch.empty((w.M_total, w.N), dtype=torch.bfloat16, device="cuda")
        # with the split workspace: a last round of idle workgroups runs its tiles as two units
        gws = torch.empty(ptg.grouped_gemm_split_workspace(), dtype=torch.uint8, device="cuda")
        call = lambda: ptg.grouped_gemm(X, W, off, out=Y, workspace=gws)  # noqa: E731
        _, ms = time_calls(call, steps, warmup, torch, min_warm_s=warm_s)
        f, b = wl.grouped_flops(w), wl.grouped_bytes(w)
        e = entry(f, b, ms, time_cold(call, cold_reps, torch), live_groups=int((w.counts > 0).sum()),
                  entry_point="ptg_grouped_gemm_split")
        if cpu and reading == "rank":
            rows = np.random.default_rng(0).permutation(w.M_total)
            n, dt, cores = oracle_timed(lambda n: oracle.grouped_gemm(
                w.X, w.W, w.w_layout, w.offsets, rows=np.sort(rows[:n])), w.M_total, cpu_budget_s)
            e["cpu_baseline"] = cpu_entry(n, dt, cores, 2.0 * w.N * w.K,
                                          f"{n} random rows of {w.M_total} (all {w.N} columns)")
        out[name] = e
        del X, W, off, Y, gws
    # weight gradient of the same MoE layer: dW_g = X_g^T . dY_g, 64 x 4096 x 1536 bf16
    w = wl.moe_wgrad()
    X, dY, off = to_dev(w.X, torch, np), to_dev(w.dY, torch, np), torch.from_numpy(w.offsets).cuda()
    dW = torch.empty((w.G, w.K, w.N), dtype=torch.bfloat16, device="cuda")
    wq = torch.empty(ptg.grouped_gemm_wgrad_workspace(), dtype=torch.uint8, device="cuda")
    call = lambda: ptg.grouped_gemm_wgrad(X, dY, off, out=dW, workspace=wq)  # noqa: E731
    _, ms = time_calls(call, steps, warmup, torch, min_warm_s=warm_s)
    f, b = wl.wgrad_flops(w), wl.wgrad_bytes(w)
    e = entry(f, b, ms, time_cold(call, cold_reps, torch))
    if cpu:
        rows = np.random.default_rng(0).permutation(w.G * w.K)
        n, dt, cores = oracle_timed(lambda n: oracle.grouped_wgrad(
            w.X, w.dY, w.offsets, rows=np.sort(rows[:n])), w.G * w.K, cpu_budget_s)
        # a row g*K + i of dW costs 2 * count_g * N flops; over random rows the mean is
        # 2 * N * M_total / G
        e["cpu_baseline"] = cpu_entry(n, dt, cores, 2.0 * w.M_total * w.N / w.G,
                                      f"{n} random rows of the {w.G * w.K} rows of dW (flops at the mean row cost)")
    out["grouped_wgrad_moe_64x16384x4096x1536"] = e
    del X, dY, off, dW, wq, w
    # broadcast: 64 users, sum C_u = 81403 candidates, [2048 | 512] -> 1024
    w = wl.config4()
    Xu, Xc, idx, W = (to_dev(w.Xu, torch, np), to_dev(w.Xc, torch, np),
                      torch.from_numpy(w.idx).cuda(), to_dev(w.W, torch, np))
    Y = torch.empty((w.Mc, w.N), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(ptg.broadcast_gemm_workspace(w.U, w.N), dtype=torch.uint8, device="cuda")
    call = lambda: ptg.broadcast_gemm(Xu, Xc, idx, W, out=Y, workspace=ws)  # noqa: E731
    _, ms = time_calls(call, steps, warmup, torch, min_warm_s=warm_s)
    f, fm, b = wl.broadcast_flops(w), wl.broadcast_flops_materialised(w), wl.broadcast_bytes(w)
    cold = time_cold(call, cold_reps, torch)
    e = entry(f, b, ms, cold, effective_tflops_materialised_equivalent=round(fm / cold["median"] / 1e9, 1))
    if cpu:
        rows = np.random.default_rng(0).permutation(w.Mc)
        n, dt, cores = oracle_timed(lambda n: oracle.broadcast_gemm(
            w.Xu, w.Xc, w.idx, w.W, w.w_layout, rows=np.sort(rows[:n])), w.Mc, cpu_budget_s)
        # the oracle computes the materialised definition: (Ku + Kc) per output element
        e["cpu_baseline"] = cpu_entry(n, dt, cores, 2.0 * (w.Ku + w.Kc) * w.N,
                                      f"{n} random candidate rows of {w.Mc}, materialised [Xu[idx] | Xc] . W "
                                      f"(flops as computed)")
    out["broadcast_ikbo_64users_81403cand"] = e
    # the same workload through the one-launch form (ptg_broadcast_gemm_fused)
    wsf = torch.empty(ptg.broadcast_gemm_fused_workspace(w.U, w.N), dtype=torch.uint8, device="cuda")
    call = lambda: ptg.broadcast_gemm_fused(Xu, Xc, idx, W, out=Y, workspace=wsf)  # noqa: E731
    _, ms = time_calls(call, steps, warmup, torch, min_warm_s=warm_s)
    out["broadcast_ikbo_64users_81403cand_fused"] = entry(
        f, b, ms, time_cold(call, cold_reps, torch), entry_point="ptg_broadcast_gemm_fused",
        note="one persistent launch; the stream-ordered ptg_broadcast_gemm above is the faster path")
    del Xu, Xc, idx, W, Y, ws, wsf
    # IKBO attention: 64 users (C_u ~ U{256..2048}), context of 1024 keys, 4 heads of 128
    w = wl.ikbo_attention_workload()
    Q, K, V = (to_dev(w.Q.reshape(w.Mc, -1), torch, np).view(w.Mc, w.H, w.D),
               to_dev(w.K.reshape(w.U, -1), torch, np).view(w.U, w.L, w.H, w.D),
               to_dev(w.V.reshape(w.U, -1), torch, np).view(w.U, w.L, w.H, w.D))
    off = torch.from_numpy(w.offsets).cuda()
    O = torch.empty((w.Mc, w.H, w.D), dtype=torch.bfloat16, device="cuda")
    call = lambda: ptg.ikbo_attention(Q, K, V, off, scale=w.scale, out=O)  # noqa: E731
    _, ms = time_calls(call, steps, warmup, torch, min_warm_s=warm_s)
    f, b = wl.attention_flops(w), wl.attention_bytes(w)
    e = entry(f, b, ms, time_cold(call, cold_reps, torch), primary="warm")
    if cpu:
        rows = np.random.default_rng(0).permutation(w.Mc)
        n, dt, cores = oracle_timed(lambda n: oracle.ikbo_attention(
            w.Q, w.K, w.V, w.offsets, w.scale, rows=np.sort(rows[:n])), w.Mc, cpu_budget_s)
        e["cpu_baseline"] = cpu_entry(n, dt, cores, 4.0 * w.H * w.L * w.D,
                                      f"{n} random candidates of {w.Mc} (all heads)")
    out["ikbo_attention_64users_77801cand_L1024_H4_D128"] = e
    del Q, K, V, off, O, w
    # batch: 1024 independent GEMMs with fused bias + SiLU, one persistent launch
    pl = wl.config5()
    probs = []
    for p in pl.problems:
        probs.append((to_dev(p.A, torch, np), to_dev(p.B, torch, np),
                      torch.empty((p.M, p.N), dtype=torch.bfloat16, device="cuda"),
                      torch.from_numpy(p.bias).cuda()))
    ws = torch.empty(ptg.grouped_gemm_ptr_array_workspace(len(probs)), dtype=torch.uint8, device="cuda")
    ptg.grouped_gemm_ptr_array_prepare(probs, pl.epi, ws)
    call = lambda: ptg.grouped_gemm_ptr_array_run(len(probs), ws, torch.bfloat16, pl.epi)  # noqa: E731
    _, ms = time_calls(call, steps, warmup, torch, min_warm_s=warm_s)
    f, b = wl.problem_list_flops(pl), wl.problem_list_bytes(pl)
    e = entry(f, b, ms, time_cold(call, cold_reps, torch))
    if cpu:
        order = np.random.default_rng(0).permutation(len(pl.problems))
        pf = [2.0 * p.M * p.N * p.K for p in pl.problems]

        def run(n):
            for i in order[:n]:
                q = pl.problems[i]
                oracle.gemm(q.A, q.B, wl.B_KN, q.bias, pl.epi)
        for threads, key in ((None, "cpu_baseline"), (1, "cpu_baseline_1core")):
            n, dt, cores = oracle_timed(run, len(pl.problems), cpu_budget_s, threads=threads)
            fl = sum(pf[i] for i in order[:n])
            e[key] = {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
                      "seconds": round(dt, 3),
                      "sample": f"{n} random problems of {len(pl.problems)}, whole (every row)"}
    out["batch_recsys_1024_bias_silu"] = e
    return out


def cpu_baseline(w, np, budget_s=15.0):
    """The oracle, untuned, on a bounded sample of output rows of the headline GEMM."""
    import oracle
    oracle.build(force=False)
    M, N, K = w.M, w.N, w.K
    oracle.gemm(w.A, w.B, w.b_layout, rows=np.arange(8))  # thread pool and page-in
    t0 = time.perf_counter()
    oracle.gemm(w.A, w.B, w.b_layout, rows=np.arange(64))
    dt = time.perf_counter() - t0
    rows = int(max(64, min(M, 64 * budget_s / max(dt, 1e-3))))
    t0 = time.perf_counter()
    oracle.gemm(w.A, w.B, w.b_layout, rows=np.arange(rows))
    dt = time.perf_counter() - t0
    return {"value": 2.0 * rows * N * K / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"{rows} of {M} output rows (all {N} columns) of the {M}x{N}x{K} GEMM, "
                      f"fp64 on the same bf16 inputs, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The warmup brings the GPU to the clock it holds under sustained load (the first tens of
    # milliseconds of a GPU that was idle run several percent slower): 150 steps take ~0.12 s,
    # and the 200 timed steps ~0.17 s.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=150)
    # ... and, whatever the step count, at least this many seconds of untimed calls
    ap.add_argument("--warm-s", type=float, default=0.5)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device-to-device copy (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import pipelined_tiled_gemm_amd as ptg
    import workloads as wl

    torch.cuda.set_device(0)
    w = wl.config2()
    A, B = to_dev(w.A, torch, np), to_dev(w.B, torch, np)
    C = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
    flops = wl.dense_flops(w.M, w.N, w.K)
    ptg.watchdog(clear=True)
    step = lambda: ptg.gemm(A, B, b_layout=wl.B_NK, out=C)  # noqa: E731
    wall_s, ev_ms = time_calls(step, args.steps, args.warmup, torch, min_warm_s=args.warm_s)
    if ptg.watchdog(clear=True) != 0:
        raise RuntimeError("a pipeline wait timed out during the benchmark")
    value = flops / wall_s / 1e12
    achieved = flops / (ev_ms * 1e-3) / 1e12
    cfg = ptg.describe_config(w.M, w.N, w.K, wl.B_NK)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warm_s": args.warm_s,
        "ms_per_step": round(wall_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "dense GEMM M=N=K=8192, A row-major, B stored N x K, bf16 inputs "
                               "N(0,1)/sqrt(K), fp32 accumulation, bf16 output",
                   "M": w.M, "N": w.N, "K": w.K, "tile": cfg, "pct_peak": round(100 * value / PEAK_TFLOPS, 2)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS, 4),
                     "traffic": measured_traffic(), "kernel_ms": round(ev_ms, 4)},
    }
    # Context, not the target: the vendor GEMM (torch.mm, which calls hipBLASLt) on the same
    # inputs and output, timed the same way right after, on the same part at the same clock.
    vendor = lambda: torch.mm(A, B.t(), out=C)  # noqa: E731
    v_wall, v_ev = time_calls(vendor, args.steps, args.warmup, torch, min_warm_s=args.warm_s)
    line["vendor_reference"] = {"library": "torch.mm (hipBLASLt)", "ms_per_step": round(v_wall * 1e3, 4),
                                "tflops": round(flops / v_wall / 1e12, 2),
                                "pct_peak": round(100 * flops / v_wall / 1e12 / PEAK_TFLOPS, 2)}
    del A, B, C
    torch.cuda.empty_cache()
    if args.copy_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        line["copy_probe_bytes"] = 1 << 30
        del src, dst
        torch.cuda.empty_cache()
    if not args.no_secondary:
        line["secondary"] = secondary(torch, np, ptg, wl, max(50, args.steps // 2), max(3, args.warmup),
                                      cpu=not args.no_cpu)
        if ptg.watchdog(clear=True) != 0:
            raise RuntimeError("a pipeline wait timed out during the secondary workloads")
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(w, np)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
