"""Message-size sweep: ring vs tree, fused vs stepwise, per channel count.

8 virtual ranks on one node, f32 sum, per-rank sizes 8 B .. 256 MiB in
powers of two, channels in {1, 4, 12, 32}, values uniform in [-1, 1]
(drawn on the device with a seeded generator; every point also checks that
the fused and stepwise results of each algorithm are bit-identical).

Reports per point the median time over repeated launches, algbw = S/t,
busbw = algbw * 2(N-1)/N and HBM GB/s = 2*N*S/t, and per channel count the
size intervals where ring or tree wins, with the practical-tie rule of the
course page ("NCCL 专家课程 13", section "性能结果的判定规则": a loser within
5% of the winner is a tie).

    python -m double_binary_tree_amd.sweep [--max-pow 26] [--out report.md]
"""

from __future__ import annotations

import argparse
import json
import statistics
import sys

N = 8
CHANNELS = (1, 4, 12, 32)
CHUNK = 512 * 1024
LEGS = (("ring", "fused"), ("tree", "fused"), ("ring", "stepwise"), ("tree", "stepwise"))
TIE = 0.05


def human(nbytes: int) -> str:
    for unit, div in (("GiB", 1 << 30), ("MiB", 1 << 20), ("KiB", 1 << 10)):
        if nbytes >= div:
            return f"{nbytes // div} {unit}"
    return f"{nbytes} B"


def time_point(E, sptr, rptr, count, stream, torch, reps: int) -> float:
    """Median of per-launch times (us) measured with events on the stream."""
    for _ in range(3):
        E.allreduce(sptr, rptr, count, "f32", "sum", stream.cuda_stream)
    samples = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        E.allreduce(sptr, rptr, count, "f32", "sum", stream.cuda_stream)
        b.record(stream)
        b.synchronize()
        samples.append(a.elapsed_time(b) * 1e3)
    return statistics.median(samples)


def intervals(rows, key_a, key_b):
    """Winner intervals between two legs over increasing sizes."""
    out = []
    for r in rows:
        ta, tb = r[key_a], r[key_b]
        winner = key_a if ta < tb else key_b
        loser_t, winner_t = max(ta, tb), min(ta, tb)
        verdict = "tie" if loser_t / winner_t - 1 < TIE else winner
        if out and out[-1][0] == verdict:
            out[-1][2] = r["bytes"]
        else:
            out.append([verdict, r["bytes"], r["bytes"]])
    return out


def _main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--max-pow", type=int, default=26, help="largest count = 2**max_pow elements")
    ap.add_argument("--min-pow", type=int, default=1)
    ap.add_argument("--reps", type=int, default=15)
    ap.add_argument("--out", default=None, help="write a markdown report here")
    ap.add_argument("--jsonl", default=None, help="write one JSON line per point here")
    args = ap.parse_args()

    import torch

    from double_binary_tree_amd import emucomm as E

    if not torch.cuda.is_available():
        print("the sweep needs a GPU", file=sys.stderr)
        return 2
    E.lib()
    maxc = 1 << args.max_pow
    g = torch.Generator(device="cuda")
    g.manual_seed(20261206)
    sends = [torch.rand(maxc, device="cuda", generator=g) * 2 - 1 for _ in range(N)]
    recvs = [torch.empty_like(s) for s in sends]
    stream = torch.cuda.current_stream()
    sptr = [t.data_ptr() for t in sends]
    rptr = [t.data_ptr() for t in recvs]
    rows = {c: [] for c in CHANNELS}
    jl = open(args.jsonl, "w") if args.jsonl else None
    for nch in CHANNELS:
        for p in range(args.min_pow, args.max_pow + 1):
            count = 1 << p
            row = {"nch": nch, "count": count, "bytes": 4 * count}
            results = {}
            for algo, mode in LEGS:
                E.comm_init(N, 1, algo, nch, CHUNK, mode=mode)
                reps = args.reps if count < (1 << 24) else max(5, args.reps // 3)
                t = time_point(E, sptr, rptr, count, stream, torch, reps)
                results[(algo, mode)] = torch.cat([r[:count] for r in recvs]).view(torch.int32).clone()
                key = f"{algo}_{mode}"
                row[key] = t
            for algo in ("ring", "tree"):
                if not torch.equal(results[(algo, "fused")], results[(algo, "stepwise")]):
                    print(f"MISMATCH {algo} fused vs stepwise at count {count} nch {nch}", file=sys.stderr)
                    return 1
            del results
            rows[nch].append(row)
            line = {**row, **{f"{k}_busbw": row["bytes"] / (row[k] * 1e-6) / 1e9 * 2 * (N - 1) / N
                              for k in ("ring_fused", "tree_fused", "ring_stepwise", "tree_stepwise")}}
            if jl:
                jl.write(json.dumps(line) + "\n")
            print(f"nch {nch:2d} {human(4 * count):>8s}: " +
                  "  ".join(f"{k} {row[k]:9.1f}us" for k in ("ring_fused", "tree_fused", "ring_stepwise",
                                                            "tree_stepwise")), flush=True)
    if jl:
        jl.close()
    if args.out:
        write_report(args.out, rows)
    return 0


def write_report(path, rows):
    lines = ["# Message-size sweep: ring vs tree, fused vs stepwise (8 ranks, f32 sum, one MI355X)\n\n",
             "Command: `python -m double_binary_tree_amd.sweep --out <this file>`. Median of per-launch times "
             "(events on the launch stream, warm launches, buffers resident in HBM; no cache flush between "
             "launches, so sizes whose 2·N·S fits the 256 MB Infinity Cache run partly from cache). "
             "busbw = S/t · 2(N−1)/N; HBM = 2·N·S/t.\n\n"]
    for nch, rs in rows.items():
        lines.append(f"## {nch} channel(s)\n\n")
        lines.append("| S per rank | ring fused µs | tree fused µs | ring stepwise µs | tree stepwise µs | "
                     "best busbw GB/s | best HBM GB/s |\n|---|---|---|---|---|---|---|\n")
        for r in rs:
            best = min(r["ring_fused"], r["tree_fused"], r["ring_stepwise"], r["tree_stepwise"])
            busbw = r["bytes"] / (best * 1e-6) / 1e9 * 2 * (N - 1) / N
            hbm = 2 * N * r["bytes"] / (best * 1e-6) / 1e9
            lines.append(f"| {human(r['bytes'])} | {r['ring_fused']:.1f} | {r['tree_fused']:.1f} | "
                         f"{r['ring_stepwise']:.1f} | {r['tree_stepwise']:.1f} | {busbw:.1f} | {hbm:.0f} |\n")
        for mode in ("fused", "stepwise"):
            iv = intervals(rs, f"ring_{mode}", f"tree_{mode}")
            desc = "; ".join(f"{v.replace('_' + mode, '')} {human(a)}–{human(b)}" for v, a, b in iv)
            lines.append(f"\nRing vs tree ({mode}, 5% tie): {desc}\n")
        lines.append("\n")
    with open(path, "w", encoding="utf-8") as f:
        f.writelines(lines)


def main() -> int:
    from double_binary_tree_amd import emucomm as E
    try:
        return _main()
    finally:
        E.release()


if __name__ == "__main__":
    sys.exit(main())
