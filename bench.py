"""All-reduce busbw / HBM bandwidth of the emulated data path on one GPU.

Headline workload: 8 virtual ranks on one node (the tree is the intra-node
chain), 12 channels, 512 KiB chunks, float32 sum, 16 Mi elements (64 MiB)
per rank drawn from N(0, 1), all buffers resident in HBM before timing
starts.  By default the 16 rank buffers are carved from one pool at
emu_buffer_layout's offsets, the placement the library provides for its
virtual ranks; --placement torch gives each buffer its own torch allocation.

One step = one pass of the whole path over the batch: ring and tree, each in
the fused single-pass mode and in the stepwise mode (4 all-reduces, each
reading every rank's 64 MiB input and writing every rank's output).  Events
on the launch stream between the legs of every timed step give each leg's
average duration inside the timed region; the roofline is taken for the
slowest leg from those.

Beside the headline line (printed as ONE JSON line) the same run measures,
in "configs": the other full-size workloads (16 and 15 single-rank nodes
bf16; 4 x 8 ranks f16, i64 and f32 max; ring and tree, fused and stepwise)
and the message-size sweep's points from 16 MiB per rank up (8 ranks, f32,
1/4/12/32 channels); in "stream": the same-run HBM ceilings of the
library's own 128-bit read-only, write-only and copy kernels; and the oracle
timed on the host, on one core and with its channels spread over the host's
cores ("cpu_baseline").  Those extra inputs are drawn on the GPU from seeded
generators (their values are checked by the parity tests, not here).

value = aggregate bus bandwidth of the headline step, busbw = algbw *
2(N-1)/N with algbw = S / t per all-reduce (GB = 1e9 B).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "all-reduce busbw & HBM GB/s (% of peak) vs msg size, N virtual ranks, 1 GPU"
WORKLOAD = "chain8_f32"
LEGS = (("ring", "fused"), ("tree", "fused"), ("ring", "stepwise"), ("tree", "stepwise"))
KERNEL_NAMES = {("ring", "fused"): "fused_collective (all-reduce, rotated ring fold)",
                ("tree", "fused"): "fused_collective (all-reduce, rotated chain fold)",
                ("ring", "stepwise"): "step_ring (all-reduce)", ("tree", "stepwise"): "step_tree"}
KERNEL_SOURCES = ("double_binary_tree_amd/csrc/fused.hip", "double_binary_tree_amd/csrc/stepwise.hip",
                  "double_binary_tree_amd/csrc/device_ops.h", "double_binary_tree_amd/csrc/common.h")
EXTRA_WORKLOADS = ("dtree16_bf16", "dtree15_bf16", "hier4x8_f16", "hier4x8_i64", "hier4x8_f32max")
SWEEP_MIB = (16, 32, 64, 128, 256)
SWEEP_CHANNELS = (1, 4, 12, 32)
TORCH_DTYPES = {"i32": "int32", "i64": "int64", "f32": "float32", "f16": "float16", "bf16": "bfloat16"}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(leg_key: str):
    """HBM bytes per launch measured with rocprofv3 counters, if the summary
    in profiles/ was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_chain8_f32.json")
    if not os.path.exists(path):
        return None
    with open(path, encoding="utf-8") as f:
        data = json.load(f)
    if data.get("kernel_source_hash") != kernel_source_hash():
        return None
    entry = data.get("legs", {}).get(leg_key)
    return None if entry is None else entry.get("hbm_bytes_per_launch")


# --- the oracle on the host ---------------------------------------------------

def host_info() -> dict:
    import numpy as np
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "cores_available": len(os.sched_getaffinity(0)),
            "numpy": np.__version__, "python": platform.python_version()}


def _oracle_step(xs, w, threads: int) -> None:
    """One ring + tree all-reduce of the oracle; with threads > 1 its
    channels (disjoint element ranges) are computed by a thread pool."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    from oracle import allreduce as A
    from oracle import topology as T
    for algo in ("ring", "tree"):
        if threads <= 1:
            A.allreduce(xs, w.nnodes, algo, w.nchannels, w.chunk_bytes, w.dtype, w.op)
            continue
        outs = [np.array(x, copy=True) for x in xs]
        topo = T.build_topology(w.nranks, w.nnodes, w.nchannels)
        with ThreadPoolExecutor(max_workers=threads) as pool:
            list(pool.map(lambda c: A.allreduce_channel(xs, outs, c, topo, algo, w.chunk_bytes, w.dtype, w.op),
                          range(w.nchannels)))


def cpu_baseline(w, n_sample: int, reps: int = 3, xs=None, min_seconds: float = 0.0) -> dict:
    """The oracle as it stands, timed on the host: ring + tree all-reduce of
    the workload (n_sample elements per rank), median of at least `reps`
    runs (more until min_seconds have passed), on one core (oracle-1c) and
    with the channels over the host's cores (oracle-mc; numpy releases the
    GIL inside its array operations)."""
    from double_binary_tree_amd import inputs as I
    if xs is None or len(xs[0]) != n_sample:
        xs = I.rank_inputs(w, count=n_sample)
    s_bytes = n_sample * w.itemsize
    info = host_info()
    variants = {}
    for name, threads in (("oracle-1c", 1), ("oracle-mc", min(info["cores_available"], w.nchannels))):
        runs = []
        while len(runs) < reps or sum(runs) < min_seconds:
            t0 = time.perf_counter()
            _oracle_step(xs, w, threads)
            runs.append(time.perf_counter() - t0)
        t = statistics.median(runs)
        # one step = 2 all-reduces (ring + tree); busbw and HBM-equivalent rate per all-reduce
        t_ar = t / 2
        variants[name] = {"cores": threads, "seconds_per_step_median": round(t, 3),
                          "runs_s": [round(r, 3) for r in runs],
                          "busbw_GBps": round(s_bytes * 2 * (w.nranks - 1) / w.nranks / t_ar / 1e9, 4),
                          "hbm_equiv_GBps": round(2 * w.nranks * s_bytes / t_ar / 1e9, 4)}
    best = variants["oracle-mc"]
    return {"value": best["busbw_GBps"], "unit": "GB/s", "cores": best["cores"], "kind": "oracle",
            "sample": f"oracle (numpy) ring + tree all-reduce of the bench workload, {n_sample} "
                      f"{w.dtype} elements per rank x {w.nranks} ranks, {w.nchannels} channels; median of "
                      f"{len(variants['oracle-1c']['runs_s'])} (1c) and {len(best['runs_s'])} (mc) runs; value = oracle-mc (channels over {best['cores']} threads), busbw of one "
                      f"all-reduce as in the GPU legs; oracle-1c is the single-thread run",
            "variants": variants, "host": info}


# --- GPU helpers --------------------------------------------------------------

def fill_seeded(bufs, w, seed: int) -> None:
    """Values of workload w's distribution, drawn on the GPU from a seeded
    generator (perf-only inputs)."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    kind = w.dist[0]
    for b in bufs:
        if kind == "int":
            b.copy_(torch.randint(w.dist[1], w.dist[2] + 1, b.shape, generator=g, device="cuda", dtype=torch.int64))
        elif kind == "normal":
            b.copy_(torch.randn(b.shape, generator=g, device="cuda") * w.dist[1])
        else:
            b.copy_(torch.rand(b.shape, generator=g, device="cuda") * (w.dist[2] - w.dist[1]) + w.dist[1])


def time_launches(fn, stream, iters: int, warm: int = 3) -> float:
    """Average seconds per launch of `iters` back-to-back launches, events on
    the launch stream."""
    import torch
    for _ in range(warm):
        fn()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(iters):
        fn()
    b.record(stream)
    b.synchronize()
    return a.elapsed_time(b) / 1e3 / iters


def leg_record(t: float, n: int, s_bytes: int, kernel: str | None = None) -> dict:
    algbw = s_bytes / t / 1e9
    hbm = 2 * n * s_bytes / t / 1e9
    rec = {"us": round(t * 1e6, 2), "algbw_GBps": round(algbw, 2), "busbw_GBps": round(algbw * 2 * (n - 1) / n, 2),
           "hbm_GBps": round(hbm, 1), "hbm_frac": round(hbm / HBM_PEAK_GBPS, 4)}
    if kernel:
        rec["kernel"] = kernel
    return rec


def measure_workload(E, torch, w, count: int, nch: int, legs, stream, iters: int, seed: int) -> dict:
    """Full-size legs of one workload shape: buffers from one pool at the
    library's layout, inputs drawn on the GPU; fused and stepwise results
    of one algorithm must agree bit for bit."""
    dt = getattr(torch, TORCH_DTYPES[w.dtype])
    pool, sends, recvs = E.rank_buffers(w.nranks, count, dt)
    fill_seeded(sends, w, seed)
    sptr = [t.data_ptr() for t in sends]
    rptr = [t.data_ptr() for t in recvs]
    out = {}
    ref = {}
    for algo, mode in legs:
        E.comm_init(w.nranks, w.nnodes, algo, nch, w.chunk_bytes, mode=mode)

        def fn():
            E.allreduce(sptr, rptr, count, w.dtype, w.op, stream.cuda_stream)
        fn()
        torch.cuda.synchronize()
        got = recvs[0].view(torch.uint8).clone()
        if algo in ref and not torch.equal(ref[algo], got):
            raise RuntimeError(f"{w.name} {nch} ch {algo}: {mode} differs from the other mode")
        ref[algo] = got
        t = time_launches(fn, stream, iters)
        out[f"{algo}_{mode}"] = leg_record(t, w.nranks, count * w.itemsize)
    del pool, sends, recvs, ref
    torch.cuda.empty_cache()
    return out


def measure_stream(E, torch, nbytes: int, stream, iters: int) -> dict:
    """The library's read-only, write-only and copy kernels over nbytes of
    traffic each (the headline all-reduce's 2*N*S)."""
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").uniform_()
    b = torch.empty_like(a)
    half = nbytes // 2
    out = {}
    for kind, src, dst, size in (("read", a.data_ptr(), b.data_ptr(), nbytes),
                                 ("write", 0, b.data_ptr(), nbytes),
                                 ("copy", a.data_ptr(), b.data_ptr(), half)):
        t = time_launches(lambda: E.stream_probe(kind, src, dst, size, stream.cuda_stream), stream, iters)
        moved = size * (2 if kind == "copy" else 1)
        out[kind] = {"us": round(t * 1e6, 2), "bytes": moved, "GBps": round(moved / t / 1e9, 1),
                     "frac": round(moved / t / 1e9 / HBM_PEAK_GBPS, 4)}
    r, wr = out["read"]["GBps"], out["write"]["GBps"]
    ceiling = 2.0 / (1.0 / r + 1.0 / wr)
    out["read_write_ceiling"] = {"GBps": round(ceiling, 1), "frac": round(ceiling / HBM_PEAK_GBPS, 4),
                                 "what": "harmonic mean of the read-only and write-only rates: the rate of a "
                                         "pass whose bytes are half reads and half writes, were reads and "
                                         "writes not overlapped"}
    del a, b
    torch.cuda.empty_cache()
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--leg-iters", type=int, default=20)
    ap.add_argument("--cpu-sample", type=int, default=16 * 1024 * 1024)
    ap.add_argument("--cpu-reps", type=int, default=3, help="at least this many oracle runs per variant")
    ap.add_argument("--cpu-seconds", type=float, default=5.0, help="and more until this many seconds per variant")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the other workloads and the sweep points")
    ap.add_argument("--placement", choices=("library", "torch"), default="library",
                    help="library: the 2N rank buffers carved from one pool at emu_buffer_layout's offsets; "
                         "torch: one torch allocation per buffer (all sends, then all receives)")
    ap.add_argument("--calibration-kernel", action="store_true",
                    help="also run one elementwise multiply over 512 MiB (read) + 512 MiB (write), "
                         "the known-size kernel that scales rocprofv3 FETCH_SIZE/WRITE_SIZE")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the emulated ranks all live in one GPU's HBM; "
              "--gpus above 1 is not supported.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from double_binary_tree_amd import emucomm as E
    from double_binary_tree_amd import inputs as I

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    E.lib()
    try:
        return run(args, np, torch, E, I)
    finally:
        E.release()


def run(args, np, torch, E, I) -> int:
    w = I.WORKLOADS[WORKLOAD]
    n, count = w.nranks, w.count
    s_bytes = count * w.itemsize
    log(f"generating {n} x {count} f32 inputs")
    xs = I.rank_inputs(w)
    if args.placement == "library":
        pool, sends, recvs = E.rank_buffers(n, count, torch.float32)
        for s_, x in zip(sends, xs):
            s_.copy_(torch.from_numpy(x))
    else:
        pool = None
        sends = [torch.from_numpy(x).cuda() for x in xs]
        recvs = [torch.empty_like(s) for s in sends]
    stream = torch.cuda.current_stream()
    sptr = [t.data_ptr() for t in sends]
    rptr = [t.data_ptr() for t in recvs]

    def run_leg(algo, mode):
        E.comm_init(n, w.nnodes, algo, w.nchannels, w.chunk_bytes, mode=mode)
        E.allreduce(sptr, rptr, count, w.dtype, w.op, stream.cuda_stream)

    # Warm every leg once (builds the per-shape plans), check the legs agree.
    refs = {}
    for algo, mode in LEGS:
        run_leg(algo, mode)
        torch.cuda.synchronize()
        cur = torch.stack([r.view(torch.int32) for r in recvs])
        if algo in refs and not torch.equal(cur, refs[algo]):
            log(f"ERROR: {algo} {mode} differs from {algo} fused")
            return 1
        refs[algo] = cur.clone()
    del refs

    # Spread of single launches per leg (median, P95, CV), outside the timed region.
    spread = {}
    for algo, mode in LEGS:
        samples = []
        for _ in range(args.leg_iters):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            run_leg(algo, mode)
            b.record(stream)
            b.synchronize()
            samples.append(a.elapsed_time(b) * 1e3)
        samples = np.array(samples)
        spread[(algo, mode)] = {"median": round(float(np.median(samples)), 2),
                                "p95": round(float(np.percentile(samples, 95)), 2),
                                "cv": round(float(samples.std() / samples.mean()), 4)}

    # Copy ceiling of the same byte count (torch's copy kernel), context only.
    big = torch.empty(n * count, dtype=torch.float32, device="cuda")
    big2 = torch.empty_like(big)
    t_copy = time_launches(lambda: big2.copy_(big), stream, 10, warm=1)
    copy_gbps = 2 * n * s_bytes / t_copy / 1e9
    if args.calibration_kernel:
        torch.mul(big, 1.0, out=big2)
        torch.cuda.synchronize()
    del big, big2

    # The timed steps: an event before every leg and one after the last.
    for _ in range(args.warmup):
        for algo, mode in LEGS:
            run_leg(algo, mode)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(LEGS) + 1)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s in range(args.steps):
        for i, (algo, mode) in enumerate(LEGS):
            evs[s][i].record(stream)
            run_leg(algo, mode)
        evs[s][len(LEGS)].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_step = evs[0][0].elapsed_time(evs[-1][len(LEGS)]) / 1e3 / args.steps
    t_step = max(t_step, wall / args.steps)
    busbw = len(LEGS) * s_bytes * 2 * (n - 1) / n / t_step / 1e9
    legs = {}
    for i, (algo, mode) in enumerate(LEGS):
        t = sum(evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(args.steps)) / 1e3 / args.steps
        rec = leg_record(t, n, s_bytes, KERNEL_NAMES[(algo, mode)])
        rec["single_launch_us"] = spread[(algo, mode)]
        legs[f"{algo}_{mode}"] = rec
        log(f"{algo:4s} {mode:8s} {t * 1e6:9.1f} us  hbm {rec['hbm_GBps']:8.1f} GB/s "
            f"({100 * rec['hbm_frac']:.1f}%)")

    dominant = max(legs, key=lambda k: legs[k]["us"])
    d = legs[dominant]
    achieved = 2 * n * s_bytes / (d["us"] * 1e-6) / 1e9
    traffic = traffic_from_profiles(dominant)
    out = {
        "metric": METRIC, "value": round(busbw, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(t_step * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{WORKLOAD}: {n} virtual ranks x 1 node, {w.nchannels} channels, "
                               f"{w.chunk_bytes // 1024} KiB chunks, f32 sum, {count} elements "
                               f"({s_bytes // (1024 * 1024)} MiB) per rank, N(0,1); step = ring + tree, "
                               f"fused + stepwise",
                   "nranks": n, "nnodes": w.nnodes, "nchannels": w.nchannels,
                   "chunk_bytes": w.chunk_bytes, "count_per_rank": count, "global_batch": n * count,
                   "parallelism": "single GPU, virtual ranks",
                   "placement": "emu_buffer_layout pool" if args.placement == "library"
                                else "one torch allocation per buffer"},
        "roofline": {"bound": "hbm", "kernel": d["kernel"], "leg": dominant,
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic,
                     "algorithmic_bytes_per_launch": 2 * n * s_bytes,
                     "timing": "average duration of the leg inside the timed region (events between legs)"},
        "legs": legs,
        "copy_ceiling_GBps": round(copy_gbps, 1),
    }
    del pool, sends, recvs
    torch.cuda.empty_cache()

    log("streaming ceilings")
    out["stream"] = measure_stream(E, torch, 2 * n * s_bytes, stream, args.leg_iters)

    if not args.no_configs:
        configs = {}
        for name in EXTRA_WORKLOADS:
            wk = I.WORKLOADS[name]
            log(f"workload {name}")
            configs[name] = {"nranks": wk.nranks, "nnodes": wk.nnodes, "nchannels": wk.nchannels,
                             "dtype": wk.dtype, "op": wk.op, "count_per_rank": wk.count,
                             "legs": measure_workload(E, torch, wk, wk.count, wk.nchannels, LEGS, stream,
                                                      args.leg_iters, I.SEED_BASE + wk.seed_index)}
        sw = I.WORKLOADS["sweep8_f32"]
        sweep = {}
        for mib in SWEEP_MIB:
            cnt = mib * (1 << 20) // sw.itemsize
            for nch in SWEEP_CHANNELS:
                log(f"sweep {mib} MiB {nch} ch")
                sweep[f"{mib}MiB_{nch}ch"] = measure_workload(E, torch, sw, cnt, nch, LEGS, stream,
                                                              args.leg_iters, I.SEED_BASE + sw.seed_index)
        fused = [leg["hbm_frac"] for pts in sweep.values() for k, leg in pts.items() if k.endswith("fused")]
        best_fused = [max(pts["ring_fused"]["hbm_frac"], pts["tree_fused"]["hbm_frac"]) for pts in sweep.values()]
        out["configs"] = configs
        out["sweep_ge16MiB"] = {"nranks": sw.nranks, "dtype": sw.dtype, "points": sweep,
                                "fused_frac_min": round(min(fused), 4),
                                "best_fused_frac_min": round(min(best_fused), 4)}
    if not args.no_cpu_baseline:
        log("timing the oracle on the host")
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_sample, args.cpu_reps,
                                           xs if args.cpu_sample == count else None, args.cpu_seconds)
    del xs
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
