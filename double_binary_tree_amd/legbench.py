"""One all-reduce leg at full size, for profiling: a workload's shape (or
the size sweep's 8-rank f32 shape at a given size and channel count), one
algorithm and mode, rank buffers from one pool at emu_buffer_layout's
offsets, inputs drawn on the GPU from a seeded generator; `--iters`
back-to-back launches after 3 warm-up launches, timed with events on the
launch stream.  Prints one line per leg: mean us per launch and HBM GB/s
(2*N*S / t).  Several --leg arguments run one after the other in one
process, so that one profiler run covers them.

    python -m double_binary_tree_amd.legbench --leg hier4x8_f16:tree:stepwise \\
        --leg sweep8_f32@256:ring:fused:32 [--iters 20]

A leg is WORKLOAD[@MIB]:ALGO:MODE[:CHANNELS]; @MIB sets the per-rank size
in MiB (default: the workload's own), CHANNELS the channel count (default:
the workload's own).  A leg stream:KIND:MIB runs the library's streaming
kernel KIND (read, write or copy) over MIB MiB of HBM traffic (a copy reads
and writes half of it each), the same-run yardstick at that size.
"""

from __future__ import annotations

import argparse
import sys

TORCH_DTYPES = {"i32": "int32", "i64": "int64", "f32": "float32", "f16": "float16", "bf16": "bfloat16"}


def parse_leg(spec: str):
    from double_binary_tree_amd import inputs as I
    parts = spec.split(":")
    if len(parts) not in (3, 4):
        raise ValueError(f"bad leg {spec!r}: WORKLOAD[@MIB]:ALGO:MODE[:CHANNELS]")
    name, _, mib = parts[0].partition("@")
    w = I.WORKLOADS[name]
    count = int(mib) * (1 << 20) // w.itemsize if mib else w.count
    nch = int(parts[3]) if len(parts) == 4 else w.nchannels
    return w, count, parts[1], parts[2], nch


def _main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--leg", action="append", required=True)
    ap.add_argument("--iters", type=int, default=20)
    ap.add_argument("--calibrate", action="store_true",
                    help="first copy 512 MiB into another 512 MiB with the library's copy kernel (5 launches): "
                         "the known-size kernel that scales FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()

    import torch

    from double_binary_tree_amd import emucomm as E
    from double_binary_tree_amd import inputs as I

    if not torch.cuda.is_available():
        print("needs a GPU", file=sys.stderr)
        return 2
    E.lib()
    stream = torch.cuda.current_stream()
    if args.calibrate:
        nbytes = 512 << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            E.stream_probe("copy", src.data_ptr(), dst.data_ptr(), nbytes, stream.cuda_stream)
        torch.cuda.synchronize()
        print(f"calibration: 5 copies of {nbytes} bytes (stream_kernel<2>)", flush=True)
        del src, dst
        torch.cuda.empty_cache()
    for spec in args.leg:
        if spec.startswith("stream:"):
            _, kind, mib = spec.split(":")
            nbytes = int(mib) << 20
            size = nbytes // 2 if kind == "copy" else nbytes
            src = torch.ones(size // 4, dtype=torch.float32, device="cuda")
            dst = torch.empty_like(src)
            for _ in range(3):
                E.stream_probe(kind, src.data_ptr(), dst.data_ptr(), size, stream.cuda_stream)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(args.iters):
                E.stream_probe(kind, src.data_ptr(), dst.data_ptr(), size, stream.cuda_stream)
            b.record(stream)
            b.synchronize()
            us = a.elapsed_time(b) * 1e3 / args.iters
            print(f"{spec}: {us:.1f} us per launch, {nbytes / us / 1e3:.0f} GB/s ({nbytes / us / 1e3 / 80:.1f}% of "
                  f"8 TB/s)", flush=True)
            del src, dst
            torch.cuda.empty_cache()
            continue
        w, count, algo, mode, nch = parse_leg(spec)
        dt = getattr(torch, TORCH_DTYPES[w.dtype])
        pool, sends, recvs = E.rank_buffers(w.nranks, count, dt)
        g = torch.Generator(device="cuda")
        g.manual_seed(I.SEED_BASE + w.seed_index)
        for b in sends:
            if w.dist[0] == "int":
                b.copy_(torch.randint(w.dist[1], w.dist[2] + 1, b.shape, generator=g, device="cuda",
                                      dtype=torch.int64))
            else:
                b.copy_(torch.randn(b.shape, generator=g, device="cuda"))
        sptr = [t.data_ptr() for t in sends]
        rptr = [t.data_ptr() for t in recvs]
        E.comm_init(w.nranks, w.nnodes, algo, nch, w.chunk_bytes, mode=mode)
        for _ in range(3):
            E.allreduce(sptr, rptr, count, w.dtype, w.op, stream.cuda_stream)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(args.iters):
            E.allreduce(sptr, rptr, count, w.dtype, w.op, stream.cuda_stream)
        b.record(stream)
        b.synchronize()
        us = a.elapsed_time(b) * 1e3 / args.iters
        hbm = 2 * w.nranks * count * w.itemsize / us / 1e3
        print(f"{spec}: {us:.1f} us per launch, {hbm:.0f} GB/s ({hbm / 80:.1f}% of 8 TB/s)", flush=True)
        del pool, sends, recvs
        torch.cuda.empty_cache()
    if E.protocol_status():
        print("an LL or device-transport call was abandoned", file=sys.stderr)
        return 1
    return 0


def main() -> int:
    from double_binary_tree_amd import emucomm as E
    try:
        return _main()
    finally:
        E.release()


if __name__ == "__main__":
    sys.exit(main())
