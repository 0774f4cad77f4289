"""Buffer placement: all-reduce time with the rank buffers where torch puts
them (each buffer its own allocation, sends first, then receives) against
one pool laid out by emu_buffer_layout (slots staggered by 4 KiB modulo
64 KiB), for the workloads of the measurement plan at full size.

Per workload, algorithm and mode: the mean time of 20 back-to-back launches
(events on the launch stream) and the HBM GB/s = 2*N*S / t.  The two
placements of a leg give bit-identical results (checked).

    python -m double_binary_tree_amd.placebench [--out report.md]
"""

from __future__ import annotations

import argparse
import sys

WORKLOADS = ("chain8_f32", "dtree16_bf16", "dtree15_bf16", "hier4x8_f16", "hier4x8_i64", "hier4x8_f32max")
MODES = ("fused", "stepwise")
ITERS = 20


def _main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=None)
    args = ap.parse_args()

    import torch

    from double_binary_tree_amd import emucomm as E
    from double_binary_tree_amd import inputs as I

    if not torch.cuda.is_available():
        print("needs a GPU", file=sys.stderr)
        return 2
    E.lib()
    stream = torch.cuda.current_stream()
    rows = []
    for name in WORKLOADS:
        w = I.WORKLOADS[name]
        n, count = w.nranks, w.count
        tdt = {"i32": torch.int32, "i64": torch.int64, "f32": torch.float32, "f16": torch.float16,
               "bf16": torch.bfloat16}[w.dtype]
        g = torch.Generator(device="cuda")
        g.manual_seed(20261208)
        data = []
        for _ in range(n):
            if w.dtype in ("i32", "i64"):
                data.append(torch.randint(-1000, 1000, (count,), device="cuda", dtype=tdt, generator=g))
            else:
                data.append(torch.randn(count, device="cuda", generator=g).to(tdt))
        placements = {}
        sends = [d.clone() for d in data]
        recvs = [torch.empty_like(s) for s in sends]
        placements["torch"] = (None, sends, recvs)
        pool, ls, lr = E.rank_buffers(n, count, tdt)
        for s, d in zip(ls, data):
            s.copy_(d)
        placements["layout"] = (pool, ls, lr)
        del data
        for algo in w.algos:
            for mode in MODES:
                E.comm_init(n, w.nnodes, algo, w.nchannels, w.chunk_bytes, mode=mode)
                res = {}
                row = {"workload": name, "algo": algo, "mode": mode}
                for pname, (_, ss, rr) in placements.items():
                    sp, rp = [t.data_ptr() for t in ss], [t.data_ptr() for t in rr]
                    for _ in range(3):
                        E.allreduce(sp, rp, count, w.dtype, w.op, stream.cuda_stream)
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    for _ in range(ITERS):
                        E.allreduce(sp, rp, count, w.dtype, w.op, stream.cuda_stream)
                    b.record(stream)
                    b.synchronize()
                    row[pname] = a.elapsed_time(b) * 1e3 / ITERS
                    res[pname] = rr[0].view(torch.uint8).clone()
                if not torch.equal(res["torch"], res["layout"]):
                    print(f"MISMATCH {name} {algo} {mode}", file=sys.stderr)
                    return 1
                del res
                hbm = 2 * n * count * w.itemsize / 1e3
                print(f"{name:15s} {algo:4s} {mode:8s} torch {row['torch']:8.1f} us ({hbm / row['torch']:6.0f} GB/s)"
                      f"  layout {row['layout']:8.1f} us ({hbm / row['layout']:6.0f} GB/s)", flush=True)
                row["hbm_bytes"] = 2 * n * count * w.itemsize
                rows.append(row)
        del placements, sends, recvs, pool, ls, lr
        torch.cuda.empty_cache()
    if args.out:
        lines = ["# Buffer placement: torch allocations vs emu_buffer_layout (full-size workloads, one MI355X)\n\n",
                 "Command: `python -m double_binary_tree_amd.placebench --out <this file>`. Mean of "
                 f"{ITERS} back-to-back launches (events on the launch stream); HBM GB/s = 2·N·S/t; "
                 "% of 8 TB/s. torch: every rank buffer its own allocation, sends first, then receives "
                 "(the bench's placement). layout: one pool, buffer i at i·slot, slot = size rounded up to "
                 "64 KiB plus 4 KiB. Same bits in both placements.\n\n",
                 "| workload | algo | mode | torch µs | torch GB/s (%) | layout µs | layout GB/s (%) |\n"
                 "|---|---|---|---|---|---|---|\n"]
        for r in rows:
            gt, gl = r["hbm_bytes"] / r["torch"] / 1e3, r["hbm_bytes"] / r["layout"] / 1e3
            lines.append(f"| {r['workload']} | {r['algo']} | {r['mode']} | {r['torch']:.1f} | {gt:.0f} "
                         f"({gt / 80:.1f}) | {r['layout']:.1f} | {gl:.0f} ({gl / 80:.1f}) |\n")
        with open(args.out, "w", encoding="utf-8") as f:
            f.writelines(lines)
    return 0


def main() -> int:
    from double_binary_tree_amd import emucomm as E
    try:
        return _main()
    finally:
        E.release()


if __name__ == "__main__":
    sys.exit(main())
