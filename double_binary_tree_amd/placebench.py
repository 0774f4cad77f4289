"""Buffer placement: all-reduce time with the rank buffers where torch puts
them (each buffer its own allocation, sends first, then receives) against
one pool laid out by emu_buffer_layout (slots staggered by 6 KiB modulo
64 KiB), for the workloads of the measurement plan at full size.

Per workload, algorithm and mode: the mean time of 20 back-to-back launches
(events on the launch stream) and the HBM GB/s = 2*N*S / t.  The two
placements of a leg give bit-identical results (checked).

With --staggers, a sweep of the stagger instead: for each case (a workload
at its full size, or the 8-rank f32 sweep shape at a given size and channel
count) the 2N buffers sit in one 2 MiB-aligned pool at i * (S rounded up to
64 KiB + stagger), sends first, and all four legs (ring and tree, fused and
stepwise) run on them; the staggers alternate within each of --rounds
rounds.  Reported: % of 8 TB/s per leg (mean over the rounds), and per
stagger the worst fused leg, the worst stepwise leg and the mean of all.

    python -m double_binary_tree_amd.placebench [--out report.md]
    python -m double_binary_tree_amd.placebench --staggers 0,2048,4096,6144,8192,65536 [--rounds 2] [--out report.md]
"""

from __future__ import annotations

import argparse
import sys

WORKLOADS = ("chain8_f32", "dtree16_bf16", "dtree15_bf16", "hier4x8_f16", "hier4x8_i64", "hier4x8_f32max")
MODES = ("fused", "stepwise")
ITERS = 20


# (workload, MiB per rank or None for the workload's own size, channels or None)
STAGGER_CASES = (("sweep8_f32", 16, 12), ("sweep8_f32", 32, 12), ("sweep8_f32", 64, 12), ("sweep8_f32", 128, 12),
                 ("sweep8_f32", 256, 12), ("sweep8_f32", 64, 1), ("sweep8_f32", 64, 32), ("sweep8_f32", 128, 1),
                 ("sweep8_f32", 128, 32), ("dtree16_bf16", None, None), ("dtree15_bf16", None, None),
                 ("hier4x8_f16", None, None), ("hier4x8_i64", None, None), ("hier4x8_f32max", None, None))
STAGGER_LEGS = (("ring", "fused"), ("ring", "stepwise"), ("tree", "fused"), ("tree", "stepwise"))


def stagger_sweep(staggers, rounds, out) -> int:
    import torch

    from double_binary_tree_amd import emucomm as E
    from double_binary_tree_amd import inputs as I

    stream = torch.cuda.current_stream()
    align = 1 << 21
    pct = {}   # (case, leg, stagger) -> [% per round]
    for rnd in range(rounds):
        for case in STAGGER_CASES:
            name, mib, nch = case
            w = I.WORKLOADS[name]
            n = w.nranks
            count = mib * (1 << 20) // w.itemsize if mib else w.count
            nch = nch or w.nchannels
            nb = count * w.itemsize
            tdt = getattr(torch, {"i32": "int32", "i64": "int64", "f32": "float32", "f16": "float16",
                                  "bf16": "bfloat16"}[w.dtype])
            refs = {}
            for st in staggers:
                slot = (nb + 65535) // 65536 * 65536 + st
                pool = torch.empty(2 * n * slot + align, dtype=torch.uint8, device="cuda")
                base = (-pool.data_ptr()) % align
                bufs = [pool[base + k * slot: base + k * slot + nb].view(tdt) for k in range(2 * n)]
                g = torch.Generator(device="cuda")
                g.manual_seed(20261208)
                for b in bufs[:n]:
                    if w.dtype in ("i32", "i64"):
                        b.copy_(torch.randint(-1000, 1000, b.shape, device="cuda", dtype=tdt, generator=g))
                    else:
                        b.copy_(torch.randn(b.shape, device="cuda", generator=g).to(tdt))
                sp, rp = [b.data_ptr() for b in bufs[:n]], [b.data_ptr() for b in bufs[n:]]
                cells = []
                for algo, mode in STAGGER_LEGS:
                    E.comm_init(n, w.nnodes, algo, nch, w.chunk_bytes, mode=mode)
                    for _ in range(2):
                        E.allreduce(sp, rp, count, w.dtype, w.op, stream.cuda_stream)
                    iters = 10 if nb * n >= (512 << 20) else 20
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    for _ in range(iters):
                        E.allreduce(sp, rp, count, w.dtype, w.op, stream.cuda_stream)
                    b.record(stream)
                    b.synchronize()
                    us = a.elapsed_time(b) * 1e3 / iters
                    res = bufs[n].view(torch.uint8).clone()
                    if algo in refs and not torch.equal(refs[algo], res):
                        print(f"MISMATCH {case} {algo} {mode} stagger {st}", file=sys.stderr)
                        return 1
                    refs.setdefault(algo, res)
                    p = 2 * n * nb / us / 1e3 / 80
                    pct.setdefault((case, (algo, mode), st), []).append(p)
                    cells.append(f"{algo[0]}{mode[0]} {p:.1f}")
                print(f"round {rnd + 1} {name} {mib or ''} {nch}ch stagger {st:6d}: " + "  ".join(cells), flush=True)
                del bufs, pool
                torch.cuda.empty_cache()
            del refs
    mean = {k: sum(v) / len(v) for k, v in pct.items()}
    if out:
        lines = ["# Buffer placement: slot stagger sweep (every workload, one MI355X)\n\n",
                 "Command: `python -m double_binary_tree_amd.placebench --staggers "
                 f"{','.join(str(s) for s in staggers)} --rounds {rounds} --out <this file>`. Per case the 2N rank "
                 "buffers (sends first) in one 2 MiB-aligned pool, buffer i at i·(S rounded up to 64 KiB + "
                 "stagger); the staggers alternate within each round; per leg the mean over the rounds of "
                 "2·N·S / t as % of 8 TB/s (t: mean of 10–20 back-to-back launches). Every stagger gives the "
                 "same bits (checked). emu_buffer_layout uses 6144.\n\n",
                 "| case | leg | " + " | ".join(f"{s} B" for s in staggers) + " |\n",
                 "|---|---|" + "---|" * len(staggers) + "\n"]
        for case in STAGGER_CASES:
            name, mib, nch = case
            w = I.WORKLOADS[name]
            label = f"{name} {mib} MiB {nch} ch" if mib else name
            for leg in STAGGER_LEGS:
                lines.append(f"| {label} | {leg[0]} {leg[1]} | " +
                             " | ".join(f"{mean[(case, leg, s)]:.1f}" for s in staggers) + " |\n")
        for what, pick in (("worst fused", lambda leg: leg[1] == "fused"),
                           ("worst stepwise", lambda leg: leg[1] == "stepwise")):
            lines.append(f"| **{what}** | | " + " | ".join(
                f"**{min(v for (c, leg, s2), v in mean.items() if s2 == s and pick(leg)):.1f}**"
                for s in staggers) + " |\n")
        lines.append("| **mean** | | " + " | ".join(
            f"**{sum(v for (c, leg, s2), v in mean.items() if s2 == s) / (len(STAGGER_CASES) * len(STAGGER_LEGS)):.2f}**"
            for s in staggers) + " |\n")
        with open(out, "w", encoding="utf-8") as f:
            f.writelines(lines)
    return 0


def _main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=None)
    ap.add_argument("--staggers", default=None, help="comma-separated slot staggers in bytes (a sweep instead)")
    ap.add_argument("--rounds", type=int, default=2, help="rounds of the stagger sweep")
    args = ap.parse_args()

    import torch

    from double_binary_tree_amd import emucomm as E
    from double_binary_tree_amd import inputs as I

    if not torch.cuda.is_available():
        print("needs a GPU", file=sys.stderr)
        return 2
    E.lib()
    if args.staggers:
        return stagger_sweep([int(x) for x in args.staggers.split(",")], args.rounds, args.out)
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
                 "64 KiB plus 6 KiB. Same bits in both placements.\n\n",
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
