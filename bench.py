"""All-reduce busbw / HBM bandwidth of the emulated data path on one GPU.

Workload: 8 virtual ranks on one node (the tree is the intra-node chain),
12 channels, 512 KiB chunks, float32 sum, 16 Mi elements (64 MiB) per rank
drawn from N(0, 1), all buffers resident in HBM before timing starts.  By
default the 16 rank buffers are carved from one pool at emu_buffer_layout's
offsets, the placement the library provides for its virtual ranks;
--placement torch gives each buffer its own torch allocation instead.

One step = one pass of the whole path over the batch: ring and tree, each in
the fused single-pass mode and in the stepwise mode (4 all-reduces, each
reading every rank's 64 MiB input and writing every rank's output).

Prints ONE JSON line.  value = aggregate bus bandwidth of the step,
busbw = algbw * 2(N-1)/N with algbw = S / t per all-reduce (GB = 1e9 B).
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

HBM_PEAK_GBPS = 8000.0
METRIC = "all-reduce busbw & HBM GB/s (% of peak) vs msg size, N virtual ranks, 1 GPU"
WORKLOAD = "chain8_f32"
LEGS = (("ring", "fused"), ("tree", "fused"), ("ring", "stepwise"), ("tree", "stepwise"))
KERNEL_NAMES = {("ring", "fused"): "fused_collective (all-reduce, rotated ring fold)",
                ("tree", "fused"): "fused_collective (all-reduce, rotated chain fold)",
                ("ring", "stepwise"): "step_ring (all-reduce)", ("tree", "stepwise"): "step_tree"}
KERNEL_SOURCES = ("double_binary_tree_amd/csrc/fused.hip", "double_binary_tree_amd/csrc/stepwise.hip",
                  "double_binary_tree_amd/csrc/device_ops.h", "double_binary_tree_amd/csrc/common.h")


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


def cpu_baseline(w, n_sample: int, min_seconds: float) -> dict:
    """The oracle as it stands, timed on the host: ring + tree all-reduce of
    the workload (n_sample elements per rank), repeated until min_seconds
    have passed (at least once)."""
    from double_binary_tree_amd import inputs as I
    from oracle import allreduce as A

    xs = I.rank_inputs(w, count=n_sample)
    reps = 0
    t0 = time.perf_counter()
    while True:
        for algo in ("ring", "tree"):
            A.allreduce(xs, w.nnodes, algo, w.nchannels, w.chunk_bytes, w.dtype, w.op)
        reps += 1
        t = time.perf_counter() - t0
        if t >= min_seconds:
            break
    s_bytes = n_sample * w.itemsize
    busbw = reps * 2 * s_bytes * 2 * (w.nranks - 1) / w.nranks / t / 1e9
    return {"value": round(busbw, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"oracle (numpy, one thread) ring + tree all-reduce of the bench workload, "
                      f"{n_sample} f32 elements per rank x {w.nranks} ranks, {w.nchannels} channels; "
                      f"{reps} repetition(s) in {t:.1f} s; busbw of the same step definition"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--leg-iters", type=int, default=20)
    ap.add_argument("--cpu-sample", type=int, default=16 * 1024 * 1024)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
        sends = [torch.from_numpy(x).cuda() for x in xs]
        recvs = [torch.empty_like(s) for s in sends]
    del xs
    stream = torch.cuda.current_stream()
    sptr = [t.data_ptr() for t in sends]
    rptr = [t.data_ptr() for t in recvs]

    def run(algo, mode):
        E.comm_init(n, w.nnodes, algo, w.nchannels, w.chunk_bytes, mode=mode)
        E.allreduce(sptr, rptr, count, w.dtype, w.op, stream.cuda_stream)

    # Warm every leg once (builds the per-shape plans), check the legs agree.
    ref = None
    for algo, mode in LEGS:
        run(algo, mode)
        torch.cuda.synchronize()
        if mode == "fused":
            cur = torch.stack([r.view(torch.int32) for r in recvs])
            if algo == "ring":
                ref_ring = cur.clone()
            else:
                ref_tree = cur.clone()
        else:
            cur = torch.stack([r.view(torch.int32) for r in recvs])
            ref = ref_ring if algo == "ring" else ref_tree
            if not torch.equal(cur, ref):
                log(f"ERROR: {algo} stepwise differs from {algo} fused")
                return 1

    # Per-leg timing: events on the stream the kernels are launched on.
    legs = {}
    for algo, mode in LEGS:
        E.comm_init(n, w.nnodes, algo, w.nchannels, w.chunk_bytes, mode=mode)
        for _ in range(3):
            E.allreduce(sptr, rptr, count, w.dtype, w.op, stream.cuda_stream)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(args.leg_iters):
            E.allreduce(sptr, rptr, count, w.dtype, w.op, stream.cuda_stream)
        end.record(stream)
        end.synchronize()
        t = start.elapsed_time(end) / 1e3 / args.leg_iters
        # spread: the same launches timed one by one (median, P95, CV)
        samples = []
        for _ in range(args.leg_iters):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            E.allreduce(sptr, rptr, count, w.dtype, w.op, stream.cuda_stream)
            b.record(stream)
            b.synchronize()
            samples.append(a.elapsed_time(b) * 1e3)
        samples = np.array(samples)
        algbw = s_bytes / t / 1e9
        hbm = 2 * n * s_bytes / t / 1e9
        legs[f"{algo}_{mode}"] = {
            "us": round(t * 1e6, 2), "algbw_GBps": round(algbw, 2),
            "busbw_GBps": round(algbw * 2 * (n - 1) / n, 2),
            "hbm_GBps": round(hbm, 1), "hbm_frac": round(hbm / HBM_PEAK_GBPS, 4),
            "single_launch_us": {"median": round(float(np.median(samples)), 2),
                                 "p95": round(float(np.percentile(samples, 95)), 2),
                                 "cv": round(float(samples.std() / samples.mean()), 4)},
            "kernel": KERNEL_NAMES[(algo, mode)],
        }
        log(f"{algo:4s} {mode:8s} {t * 1e6:9.1f} us  hbm {hbm:8.1f} GB/s ({100 * hbm / HBM_PEAK_GBPS:.1f}%)")

    # Copy ceiling of the same byte count (torch copy kernel), context only.
    big = torch.empty(n * count, dtype=torch.float32, device="cuda")
    big2 = torch.empty_like(big)
    big2.copy_(big)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(10):
        big2.copy_(big)
    end.record(stream)
    end.synchronize()
    t_copy = start.elapsed_time(end) / 1e3 / 10
    copy_gbps = 2 * n * s_bytes / t_copy / 1e9
    if args.calibration_kernel:
        torch.mul(big, 1.0, out=big2)
        torch.cuda.synchronize()
    del big, big2

    # The timed steps.
    for _ in range(args.warmup):
        for algo, mode in LEGS:
            run(algo, mode)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        for algo, mode in LEGS:
            run(algo, mode)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_step = start.elapsed_time(end) / 1e3 / args.steps
    t_step = max(t_step, wall / args.steps)
    busbw = len(LEGS) * s_bytes * 2 * (n - 1) / n / t_step / 1e9

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
                     "algorithmic_bytes_per_launch": 2 * n * s_bytes},
        "legs": legs,
        "copy_ceiling_GBps": round(copy_gbps, 1),
    }
    if not args.no_cpu_baseline:
        log("timing the oracle on the host")
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_sample, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    E.comm_destroy()
    return 0


if __name__ == "__main__":
    sys.exit(main())
